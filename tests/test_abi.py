"""The C-ABI library: it loads, exports every entry point that
include/moe_route.h declares, and rejects bad arguments on the host before
any launch. Every call here either fails validation or returns before a
launch (T = 0 router / finalize calls), so no kernel ever sees the fake
pointers; these tests run on the CPU."""
import ctypes
import os
import re

import pytest
import torch  # the binding must share torch's HIP runtime

from permutation_group_limited_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_route.h")

OK, INVALID, UNSUPPORTED, ALIGNMENT, WORKSPACE = 0, 1, 2, 3, 4


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        from permutation_group_limited_amd import build
        build.build()
    return binding.load_library()


def test_header_declares_the_three_stages():
    names = declared_functions()
    for fn in ("moe_router_group_limited", "moe_create_indices",
               "moe_create_indices_workspace_size", "moe_finalize"):
        assert fn in names


def test_every_declared_symbol_is_exported(lib):
    for fn in declared_functions():
        assert hasattr(lib, fn), fn


PROBE_HEADER = os.path.join(ROOT, "include", "moe_probe.h")


@pytest.fixture(scope="module")
def probe_lib():
    from permutation_group_limited_amd import probe
    if not os.path.exists(probe._LIB_PATH):
        from permutation_group_limited_amd import build
        build.build()
    return probe.load_library()


def test_probe_library_exports_its_header(probe_lib):
    src = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(moe_probe_\w+)\s*\(", src)))
    assert names == ["moe_probe_consume", "moe_probe_empty", "moe_probe_gather", "moe_probe_read",
                     "moe_probe_write"]
    for fn in names:
        assert hasattr(probe_lib, fn), fn


def test_probe_validation(probe_lib):
    # sizes that are not whole waves, missing pointers, misalignment: nothing launched
    assert probe_lib.moe_probe_read(FAKE, 8191, FAKE, None) == INVALID
    assert probe_lib.moe_probe_read(None, 8192, FAKE, None) == INVALID
    assert probe_lib.moe_probe_read(FAKE_ODD, 8192, FAKE, None) == ALIGNMENT
    assert probe_lib.moe_probe_read(FAKE, (1 << 40) + 8192, FAKE, None) == INVALID
    assert probe_lib.moe_probe_read(None, 0, None, None) == OK
    assert probe_lib.moe_probe_write(FAKE, 1000, 0, 0, None) == INVALID
    assert probe_lib.moe_probe_write(FAKE_ODD, 1024, 0, 1, None) == ALIGNMENT
    assert probe_lib.moe_probe_gather(FAKE, FAKE, -1, 8, 14336, FAKE, None) == INVALID
    assert probe_lib.moe_probe_gather(FAKE, FAKE, 4, 0, 14336, FAKE, None) == INVALID
    assert probe_lib.moe_probe_gather(FAKE, FAKE, 4, 8, 14330, FAKE, None) == INVALID
    assert probe_lib.moe_probe_empty(0, None) == INVALID
    assert probe_lib.moe_probe_empty(65536, None) == INVALID
    assert probe_lib.moe_probe_consume(FAKE, 16384 + 16, FAKE, None) == INVALID
    assert probe_lib.moe_probe_consume(FAKE, 17 * 16384, FAKE, None) == INVALID
    assert probe_lib.moe_probe_consume(None, 16384, FAKE, None) == INVALID
    assert probe_lib.moe_probe_consume(FAKE_ODD, 16384, FAKE, None) == ALIGNMENT
    assert probe_lib.moe_probe_consume(None, 0, None, None) == OK
    assert probe_lib.moe_probe_gather(FAKE_ODD, FAKE, 4, 8, 14336, FAKE, None) == ALIGNMENT
    assert probe_lib.moe_probe_gather(None, None, 0, 8, 14336, None, None) == OK


def test_status_strings(lib):
    for code in range(6):
        assert lib.moe_status_string(code)
    assert lib.moe_last_hip_error() == 0


P = ctypes.c_void_p
FAKE = P(0x10000)  # 16-byte aligned, never dereferenced: validation fails first
FAKE_MIS = P(0x10004)
FAKE_ODD = P(0x10002)


def router(lib, T=4, E=256, K=8, G=8, TG=4, norm=1, mode=0, ptrs=None, sd=0, bd=0):
    p = ptrs or (FAKE, FAKE, FAKE, FAKE)
    return lib.moe_router_group_limited(p[0], p[1], p[2], p[3], sd, bd, T, E, K, G, TG, norm,
                                        ctypes.c_float(1.0), mode, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID), (dict(E=0), INVALID), (dict(G=3), INVALID),
    (dict(G=128, E=256, TG=4), INVALID), (dict(TG=0), INVALID), (dict(TG=9), INVALID),
    (dict(K=0), INVALID), (dict(K=129, TG=4), INVALID), (dict(E=256, G=8, TG=1, K=33), INVALID),
    (dict(E=1024, G=1, TG=1, K=65), INVALID), (dict(mode=2), INVALID), (dict(sd=7), INVALID),
    (dict(sd=1, bd=2), UNSUPPORTED), (dict(bd=1), UNSUPPORTED), (dict(sd=2, bd=1), UNSUPPORTED),
    # any E up to 1024 is supported (T = 0: validated, nothing launched)
    (dict(E=96, G=8, TG=4, T=0), OK), (dict(E=1000, G=8, TG=4, T=0), OK),
    (dict(E=160, G=8, TG=3, K=6, ptrs=(FAKE, FAKE, FAKE_MIS, FAKE)), ALIGNMENT),
    (dict(E=2048, G=8, TG=4), UNSUPPORTED),
    (dict(ptrs=(None, FAKE, FAKE, FAKE)), INVALID),
    (dict(ptrs=(FAKE, FAKE, FAKE_MIS, FAKE)), ALIGNMENT),
    (dict(T=0, ptrs=(None, None, None, None)), OK),
])
def test_router_validation(lib, kw, code):
    assert router(lib, **kw) == code


def indices(lib, N=1000, E=256, ws=None, ws_bytes=1 << 20, scales=None, ptrs=None):
    p = ptrs or (FAKE,) * 6
    return lib.moe_create_indices(p[0], p[1], p[2], p[3], p[4], p[5], N, E,
                                  FAKE if ws is None else ws, ws_bytes, scales, None)


def test_workspace_size(lib):
    assert lib.moe_create_indices_workspace_size(0, 256) == 0
    assert lib.moe_create_indices_workspace_size(1024, 256) == 0  # one chunk: no workspace
    big = lib.moe_create_indices_workspace_size(524288, 256)
    assert big >= 256 * 4 and big % 4 == 0
    assert lib.moe_create_indices_workspace_size(-1, 256) == 0
    # one workgroup (no workspace) up to 5 rounds of 1024 slots; 8 rounds for
    # E <= 16 and for E > 256 (rounds of 256 slots)
    # past that, room for the counts of up to 64 chunks, whatever N
    ws = lib.moe_create_indices_workspace_size
    assert ws(5120, 256) == 0 and ws(5121, 256) == 256 * 4 * 64
    assert ws(8192, 8) == 0 and ws(8193, 8) == 8 * 4 * 64
    assert ws(2048, 512) == 0 and ws(2049, 512) == 512 * 4 * 64
    assert ws(1 << 31, 1024) == 1024 * 4 * 64


@pytest.mark.parametrize("E", [1, 8, 160, 256, 512, 1024])
def test_workspace_sizes_never_decrease(lib, E):
    """A workspace sized for the largest batch must serve every smaller one:
    both size functions are non-decreasing in the problem size, checked over
    every N up to 20,000 slots and around every chunk-count change of the
    index plan (N = c * 64 * rounds-of-slots boundaries) up to 2^31."""
    ci = lib.moe_create_indices_workspace_size
    ri = lib.moe_route_and_index_workspace_size
    ns = list(range(0, 20001))
    for per_round in (256, 1024):
        for r in range(1, 1 << 15, 97):
            b = 64 * per_round * r
            ns += [b - 1, b, b + 1, b + per_round * r + 1]
    ns = sorted(set(n for n in ns if 0 <= n < (1 << 31)))
    prev_c = prev_r = 0
    for n in ns:
        c = ci(n, E)
        assert c >= prev_c, (n, c, prev_c)
        prev_c = c
    for n in ns:
        if n % 8:
            continue
        r = ri(n // 8, 8, E)
        assert r >= prev_r, (n, r, prev_r)
        prev_r = r


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), INVALID), (dict(N=1 << 32), INVALID), (dict(E=0), INVALID),
    (dict(E=1025), INVALID), (dict(scales=FAKE), UNSUPPORTED),
    (dict(N=65536, ws_bytes=16), WORKSPACE),
    (dict(ptrs=(None,) + (FAKE,) * 5), INVALID),
    (dict(ptrs=(FAKE_ODD,) + (FAKE,) * 5, N=100), ALIGNMENT),
])
def test_indices_validation(lib, kw, code):
    assert indices(lib, **kw) == code


def test_no_alloc_scratch_size(lib):
    # 64 chunks x 1024 experts of uint32: the largest counts matrix any plan needs
    assert lib.moe_create_indices_no_alloc_max_scratch_bytes() == 64 * 1024 * 4
    ws = lib.moe_create_indices_workspace_size
    assert ws((1 << 32) - 1, 1024) <= lib.moe_create_indices_no_alloc_max_scratch_bytes()


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), INVALID), (dict(N=1 << 32), INVALID), (dict(E=0), INVALID),
    (dict(E=1025), INVALID), (dict(ptrs=(FAKE, None) + (FAKE,) * 4), INVALID),
    (dict(ptrs=(FAKE_ODD,) + (FAKE,) * 5, N=100), ALIGNMENT),
])
def test_no_alloc_validation(lib, kw, code):
    p = kw.get("ptrs", (FAKE,) * 6)
    assert lib.moe_create_indices_no_alloc(*p, kw.get("N", 100), kw.get("E", 256), None) == code


def finalize(lib, T=4, K=2, H=64, od=1, dd=1, wd=0, ptrs=None):
    p = ptrs or (FAKE,) * 4
    return lib.moe_finalize(p[0], od, p[1], dd, p[2], p[3], wd, T, K, H, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID), (dict(K=0), INVALID), (dict(H=-8), INVALID), (dict(od=3), INVALID),
    (dict(dd=3), INVALID), (dict(wd=-1), INVALID), (dict(T=1 << 31, K=2), INVALID),
    (dict(H=12, dd=1), ALIGNMENT),  # 24-byte rows
    (dict(H=20, dd=2), ALIGNMENT),  # 40-byte rows
    (dict(H=6, dd=0), ALIGNMENT),
    (dict(ptrs=(FAKE_MIS, FAKE, FAKE, FAKE)), ALIGNMENT),
    (dict(ptrs=(FAKE, FAKE, FAKE, None)), INVALID),
    (dict(T=0, ptrs=(None,) * 4), OK), (dict(H=0, ptrs=(None,) * 4), OK),
    # output rows of 2^31 bytes or more are not supported
    (dict(H=1 << 29, od=0), UNSUPPORTED), (dict(H=1 << 30, od=1), UNSUPPORTED),
    (dict(H=1 << 40), UNSUPPORTED),
    # more than 2^32 - 2^18 waves (one per token and 1 KiB of the row), in
    # both launch shapes: rows past the memory-side cache (these) take
    # one-wave workgroups, and the limit is the same just past it
    (dict(T=(1 << 32) - 2, K=1, H=8), UNSUPPORTED),
    (dict(T=(1 << 32) - (1 << 18), K=1, H=8), UNSUPPORTED),
    (dict(T=(1 << 32) - (1 << 17), K=1, H=8), UNSUPPORTED),
    (dict(T=1 << 31, K=1, H=1024), UNSUPPORTED),
])
def test_finalize_validation(lib, kw, code):
    assert finalize(lib, **kw) == code


def test_binding_rejects_host_tensors(lib):
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        binding.moe_finalize(x, torch.zeros(8, 8), torch.zeros(8, dtype=torch.int32),
                             torch.zeros(4, 2))


@pytest.mark.parametrize("fn,code", [(0, INVALID), (3, INVALID)])
def test_logits_router_rejects_bad_score_fn(lib, fn, code):
    assert lib.moe_router_group_limited_logits(FAKE, FAKE, FAKE, FAKE, 0, 0, fn, 4, 256, 8, 8, 4,
                                               1, ctypes.c_float(1.0), 0, None) == code


def test_logits_router_validates_like_router(lib):
    # same shape checks as the plain router (E % n_groups != 0)
    assert lib.moe_router_group_limited_logits(FAKE, FAKE, FAKE, FAKE, 0, 0, 1, 4, 256, 8, 3, 1,
                                               1, ctypes.c_float(1.0), 0, None) == INVALID


def test_aligned_indices_validation(lib):
    args = [FAKE] * 6 + [100, 256, FAKE, 1 << 20]
    assert lib.moe_create_indices_aligned(*args, None, 4, None) == INVALID  # no output
    assert lib.moe_create_indices_aligned(*args, FAKE, 0, None) == INVALID  # align 0
    big = [FAKE] * 6 + [(1 << 32) - 10, 256, FAKE, 1 << 30]
    assert lib.moe_create_indices_aligned(*big, FAKE, 2, None) == INVALID  # padded total overflows
    assert lib.moe_create_indices_aligned(*args, FAKE_ODD, 4, None) == ALIGNMENT
    # the plain entry point still refuses scales_offset_p
    assert lib.moe_create_indices(*args, FAKE, None) == UNSUPPORTED


def route_index(lib, T=16, E=256, K=8, G=8, TG=4, fn=0, sd=0, bd=0, mode=0, ws=FAKE,
                ws_bytes=1 << 20, scales=None, align=0, ptrs=None):
    p = ptrs or (FAKE,) * 9
    return lib.moe_route_and_index(p[0], p[1], p[2], p[3], p[4], p[5], p[6], scales, align,
                                   p[7], p[8], sd, bd, fn, T, E, K, G, TG, 1,
                                   ctypes.c_float(1.0), mode, ws, ws_bytes, None)


def test_route_and_index_workspace_size(lib):
    ws = lib.moe_route_and_index_workspace_size

    def ranked(T, E):  # header, 64 rows of counts, fine rows (stride E rounded up to 4)
        Ep = (E + 3) // 4 * 4
        return 256 + 64 * Ep * 4 + min((T + 3) // 4, 64 * 512) * Ep * 4

    # one launch (T <= 16 at E = 256, 128 at E = 8): the 256-byte header only
    assert ws(16, 8, 256) == 256 and ws(128, 2, 8) == 256
    # two launches, E <= 256: header, counts matrix and the router's fine rows
    assert ws(17, 8, 256) == ranked(17, 256)
    assert ws(128, 8, 256) == ranked(128, 256)
    assert ws(8192, 8, 256) == ranked(8192, 256)
    assert ws(100, 6, 160) == ranked(100, 160)
    assert ws(4096, 2, 8) == ranked(4096, 8)
    assert ws(1 << 20, 8, 256) == ranked(1 << 20, 256)  # fine rows capped at 64 * 512
    # E > 256 (chunked form only): the counts matrix once several chunks are possible
    assert ws(256, 8, 512) == 256 and ws(257, 8, 512) == 256 + 512 * 4 * 64
    # the case that once shrank: 8200 tokens needed less than 8192
    assert ws(8200, 8, 256) >= ws(8192, 8, 256)
    assert ws(-1, 8, 256) == 0 and ws(8, 0, 256) == 0 and ws(8, 8, 2048) == 0


@pytest.mark.parametrize("kw,code", [
    # router checks
    (dict(T=-1), INVALID), (dict(G=3), INVALID), (dict(K=0), INVALID), (dict(TG=9), INVALID),
    (dict(mode=2), INVALID), (dict(fn=3), INVALID), (dict(sd=1, bd=2), UNSUPPORTED),
    (dict(E=2048, G=8), UNSUPPORTED),
    (dict(ptrs=(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE_MIS, FAKE)), ALIGNMENT),
    (dict(ptrs=(None,) + (FAKE,) * 8), INVALID),
    # index-output checks
    (dict(ptrs=(FAKE, FAKE, None) + (FAKE,) * 6), INVALID),
    (dict(ptrs=(FAKE, FAKE, FAKE, None) + (FAKE,) * 5), INVALID),
    (dict(ptrs=(FAKE,) * 6 + (FAKE_ODD, FAKE, FAKE)), ALIGNMENT),
    (dict(scales=FAKE, align=0), INVALID), (dict(scales=FAKE_ODD, align=4), ALIGNMENT),
    # workspace
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=255), WORKSPACE), (dict(ws=FAKE_ODD), ALIGNMENT),
    (dict(T=8192, ws_bytes=256), WORKSPACE),  # several index chunks need the counts matrix
])
def test_route_and_index_validation(lib, kw, code):
    assert route_index(lib, **kw) == code


def test_route_and_index_binding_rejects_host_tensors(lib):
    z = torch.zeros
    with pytest.raises(ValueError):
        binding.moe_route_and_index(z(4, 2, dtype=torch.int32), z(4, 2), z(8, dtype=torch.int32),
                                    z(9, dtype=torch.int32), z(8, dtype=torch.int32),
                                    z(8, dtype=torch.int32), z(2, dtype=torch.int32), z(4, 8),
                                    z(8), z(1, dtype=torch.int32), 1, 1, True, 1.0)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the HIP library there is no other path: the loader and every
    entry point raise before touching any tensor (nothing falls back to the
    CPU or to the oracle)."""
    from permutation_group_limited_amd import binding, probe
    monkeypatch.setattr(binding, "_LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        binding.load_library()
    x = torch.zeros(4, 8)
    calls = [
        lambda: binding.moe_finalize(x, torch.zeros(8, 8), torch.zeros(8, dtype=torch.int32),
                                     torch.zeros(4, 2)),
        lambda: binding.moe_router_group_limited(torch.zeros(4, 2, dtype=torch.int32),
                                                 torch.zeros(4, 2), x, torch.zeros(8), 1, 1,
                                                 True, 1.0),
        lambda: binding.moe_create_indices_workspace_size(8, 8),
    ]
    for call in calls:
        with pytest.raises(RuntimeError, match="not built"):
            call()
    monkeypatch.setattr(probe, "_LIB_PATH", str(tmp_path / "absent_probe.so"))
    monkeypatch.setattr(probe, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        probe.load_library()


def test_route_and_index_workspace_formula():
    """The header's size formula, ranked form (E <= 256, two launches):
    256-byte header + 64 count rows + min(ceil(T / 4), 32768) fine rows, of
    E rounded up to 4 words each."""
    def expected(T, E):
        e4 = (E + 3) // 4 * 4
        return 256 + 64 * e4 * 4 + min((T + 3) // 4, 32768) * e4 * 4
    for T, K, E in ((8192, 8, 256), (8200, 8, 256), (65536, 8, 256), (4096, 2, 8),
                    (1 << 20, 8, 256), (3000, 6, 64)):
        assert binding.moe_route_and_index_workspace_size(T, K, E) == expected(T, E), (T, K, E)
