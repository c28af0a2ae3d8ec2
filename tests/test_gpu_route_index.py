"""GPU parity of moe_route_and_index (router and index creation with fewer
launches: one when a single workgroup routes the whole batch, e.g. T <= 16
at E = 256, else the router filling the index step's histogram, then the
scatter) against the oracle's router
followed by its index creation, and bit-identity with the two separate GPU
entry points on the same inputs; the workspace is all zero after each call.

Acceptance as for the separate stages: indices, weights and every index
output bit-exact against the oracle, and bit-identical to the separate
calls. Marked gpu."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from permutation_group_limited_amd import binding
from permutation_group_limited_amd import workloads as wl

from _gpu import (DEV, assert_indices_equal, assert_weights_equal,
                  bf16_bits, encode, log, to_np_u32)

pytestmark = pytest.mark.gpu

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
FNS = {"none": (binding.SCORE_NONE, oracle.SCORE_LOAD),
       "sigmoid": (binding.SCORE_SIGMOID, oracle.SCORE_SIGMOID),
       "softmax": (binding.SCORE_SOFTMAX, oracle.SCORE_SOFTMAX)}
POISON = 0x5A5A5A5A


class Outputs:
    """Device output buffers of one fused call, poisoned before the call."""

    def __init__(self, T, E, K, dtype, aligned):
        n = T * K
        full = lambda *shape: torch.full(shape, POISON, dtype=torch.int32, device=DEV)  # noqa
        self.idx = full(T, K)
        self.w = torch.full((T, K), float("nan"), dtype=dtype, device=DEV)
        self.order, self.restore = full(n), full(n)
        self.starts, self.eids, self.stats = full(E + 1), full(E), full(2)
        self.scales = full(E + 1) if aligned else None

    def host(self):
        wh = self.w.cpu()
        return {
            "idx": self.idx.cpu().numpy(),
            "w": wh.numpy() if wh.dtype == torch.float32 else wh,
            "ind": {"token_expert_order": to_np_u32(self.order),
                    "expert_start_indices": to_np_u32(self.starts),
                    "restore_token_order": to_np_u32(self.restore),
                    "expert_ids": self.eids.cpu().numpy(),
                    "expert_usage_stats": to_np_u32(self.stats)},
            "scales": None if self.scales is None else to_np_u32(self.scales),
        }


def launch(o, x, b, ws, G, TG, norm, scale, fn, mode=0, align=0, stream=None):
    binding.moe_route_and_index(o.idx, o.w, o.order, o.starts, o.restore, o.eids, o.stats, x, b,
                                ws, G, TG, norm, scale, group_score=mode, score_fn=fn,
                                scales_offset=o.scales, scale_align=align, stream=stream)


def workspace(T, K, E):
    n = binding.moe_route_and_index_workspace_size(T, K, E)
    assert n >= 256 and n % 4 == 0
    return torch.zeros(n // 4, dtype=torch.int32, device=DEV)


def zero_part(ws, E):
    """The header and the counts matrix: the part of the workspace every
    call leaves zero (the rest is scratch)."""
    return ws[:(256 + 64 * ((E + 3) // 4 * 4) * 4) // 4]


def assert_zero(ws, E, what=""):
    nz = int(torch.count_nonzero(zero_part(ws, E)).item())
    assert nz == 0, "workspace header / counts not left zero (%d words set) %s" % (nz, what)


def fused(x, b, K, G, TG, norm, scale, fn="none", mode=0, align=0, ws=None):
    """One fused call on host inputs; checks the workspace is left zero."""
    T, E = x.shape
    o = Outputs(T, E, K, x.dtype, align > 0)
    ws = workspace(T, K, E) if ws is None else ws
    launch(o, x.to(DEV), b.to(DEV), ws, G, TG, norm, scale, FNS[fn][0], mode, align)
    torch.cuda.synchronize()
    assert_zero(ws, E)
    return o.host()


def separate(x, b, K, G, TG, norm, scale, fn="none", mode=0, align=0):
    """The same step through the two separate entry points."""
    T, E = x.shape
    o = Outputs(T, E, K, x.dtype, align > 0)
    xd, bd = x.to(DEV), b.to(DEV)
    if fn == "none":
        binding.moe_router_group_limited(o.idx, o.w, xd, bd, G, TG, norm, scale, mode)
    else:
        binding.moe_router_group_limited_logits(o.idx, o.w, xd, bd, FNS[fn][0], G, TG, norm,
                                                scale, mode)
    n = binding.moe_create_indices_workspace_size(T * K, E)
    ws = torch.empty(max(n, 4) // 4, dtype=torch.int32, device=DEV)
    if align:
        binding.moe_create_indices_aligned(o.order, o.starts, o.restore, o.eids, o.stats, o.idx,
                                           ws, o.scales, align)
    else:
        binding.moe_create_indices(o.order, o.starts, o.restore, o.eids, o.stats, o.idx, ws)
    torch.cuda.synchronize()
    return o.host()


def check_against_oracle(got, x, b, K, G, TG, norm, scale, fn="none", mode=0, align=0):
    E = x.shape[1]
    xn, xcode = encode(x)
    bn, bcode = encode(b)
    oi, ow = oracle.router(xn, bn, K, G, TG, norm, scale, group_score=mode, scores_dtype=xcode,
                           bias_dtype=None if b.dtype == torch.float32 else bcode,
                           score_fn=FNS[fn][1])
    assert np.array_equal(got["idx"], oi), \
        "indices differ in %d tokens" % np.sum(np.any(got["idx"] != oi, 1))
    if x.dtype == torch.float32:
        assert_weights_equal(got["w"], ow)
    else:
        assert_weights_equal(bf16_bits(got["w"]), ow)
    assert_indices_equal(got["ind"], oracle.create_indices(oi, E))
    if align:
        assert np.array_equal(got["scales"], oracle.scale_offsets(oi, E, align))


def check_same(a, b_):
    assert np.array_equal(a["idx"], b_["idx"])
    wa = a["w"] if isinstance(a["w"], np.ndarray) else bf16_bits(a["w"])
    wb = b_["w"] if isinstance(b_["w"], np.ndarray) else bf16_bits(b_["w"])
    assert np.array_equal(np.asarray(wa).view(np.uint8), np.asarray(wb).view(np.uint8))
    assert_indices_equal(a["ind"], b_["ind"])
    if a["scales"] is not None:
        assert np.array_equal(a["scales"], b_["scales"])


@pytest.mark.parametrize("name,T", [("decode", 128), ("tiny", 64), ("mixtral", 2048),
                                    ("dsv3", 2048), ("dsv3", 1), ("decode", 97),
                                    ("mixtral", 4096), ("dsv3", 8192), ("dsv3", 3001),
                                    ("skewed", 65536)])
@pytest.mark.parametrize("from_logits", [False, True])
def test_workload_shapes(name, T, from_logits):
    wk = wl.WORKLOADS[name].with_tokens(T)
    log("route_and_index", wk.describe(), "logits" if from_logits else "scores")
    b = wl.make_bias(wk)
    if from_logits:
        x, fn = wl.make_logits(wk), wk.score_fn
    else:
        x, fn = wl.make_scores(wk), "none"
    args = (wk.K, wk.n_groups, wk.topk_group, wk.norm_weights, wk.scale, fn)
    got = fused(x, b, *args)
    check_against_oracle(got, x, b, *args)
    check_same(got, separate(x, b, *args))


@pytest.mark.parametrize("T,E,G,TG,K", [# one launch: a single workgroup routes every token
                                        (1, 1, 1, 1, 1), (1024, 1, 1, 1, 1), (33, 2, 1, 1, 2),
                                        (512, 2, 1, 1, 2), (128, 8, 4, 2, 3), (127, 8, 4, 2, 4),
                                        (32, 32, 8, 4, 6), (16, 64, 8, 3, 6), (16, 128, 8, 4, 8),
                                        (16, 256, 8, 4, 8), (9, 256, 8, 4, 8), (8, 512, 16, 4, 8),
                                        (4, 1024, 16, 4, 8), (3, 1024, 16, 4, 8),
                                        (16, 256, 8, 8, 64), (4, 1024, 16, 16, 64),
                                        (32, 32, 1, 1, 32),
                                        # two launches: one chunk or several, E a power of two
                                        # or not, just above the one-launch limits included
                                        (1025, 1, 1, 1, 1), (129, 8, 4, 2, 3), (33, 32, 8, 4, 6),
                                        (17, 256, 8, 4, 8), (9, 512, 16, 4, 8),
                                        (5, 1024, 16, 4, 8), (300, 32, 8, 4, 6),
                                        (77, 64, 8, 3, 6), (511, 128, 8, 4, 8),
                                        (1000, 256, 8, 4, 8), (61, 512, 16, 4, 8),
                                        (2048, 1024, 16, 4, 8), (4095, 256, 8, 4, 8),
                                        # router filling the histogram with two tokens per
                                        # wave from T = 4096 (E = 64 ... 256, G <= 32)
                                        (4096, 256, 8, 4, 8), (4101, 128, 32, 4, 8),
                                        (4099, 64, 8, 4, 8), (4099, 256, 64, 8, 8),
                                        (4099, 256, 8, 4, 40),
                                        (5000, 1024, 16, 4, 8), (2500, 8, 1, 1, 8),
                                        (100, 160, 8, 3, 6), (4096, 160, 8, 3, 6),
                                        (777, 20, 4, 3, 6), (3000, 1000, 8, 4, 8),
                                        # ranked form with E not a multiple of 4
                                        # (rows of counts padded to 8 and 12)
                                        (1500, 6, 2, 1, 2), (900, 10, 5, 2, 3)])
@pytest.mark.parametrize("levels", [0, 3])
def test_random_shapes(T, E, G, TG, K, levels):
    log("route_and_index random", T, E, G, TG, K, levels)
    x = wl.random_scores(T, E, seed=T + E + levels, levels=levels)
    b = wl.random_bias(E, seed=E + 5, std=0.02, levels=levels)
    for norm, mode in ((True, 0), (False, 1)):
        args = (K, G, TG, norm, 2.5, "none", mode)
        got = fused(x, b, *args)
        check_against_oracle(got, x, b, *args)
        check_same(got, separate(x, b, *args))


@pytest.mark.parametrize("sd,bd", [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16"),
                                   ("f16", "f32")])
@pytest.mark.parametrize("fn", ["none", "sigmoid", "softmax"])
def test_16bit_inputs(sd, bd, fn):
    T, E, G, TG, K = 300, 256, 8, 4, 8
    log("route_and_index dtypes", sd, bd, fn)
    g = torch.Generator().manual_seed(11)
    if fn == "none":
        x = wl.random_scores(T, E, seed=12, levels=5).to(DTYPES[sd])
    else:
        x = (torch.randn(T, E, generator=g) * 3).to(DTYPES[sd])
    b = wl.random_bias(E, seed=13, std=0.02).to(DTYPES[bd])
    args = (K, G, TG, True, 2.5, fn)
    got = fused(x, b, *args)
    check_against_oracle(got, x, b, *args)
    check_same(got, separate(x, b, *args))


@pytest.mark.parametrize("align", [1, 16, 128])
def test_aligned_scale_offsets(align):
    wk = wl.WORKLOADS["decode"]
    log("route_and_index aligned", align)
    x, b = wl.make_scores(wk), wl.make_bias(wk)
    args = (wk.K, wk.n_groups, wk.topk_group, True, wk.scale, "none", 0, align)
    got = fused(x, b, *args)
    check_against_oracle(got, x, b, *args)
    check_same(got, separate(x, b, *args))


def test_empty_batch():
    log("route_and_index T=0")
    E, K = 256, 8
    x = torch.zeros(0, E)
    got = fused(x, torch.zeros(E), K, 8, 4, True, 1.0)
    assert got["ind"]["expert_start_indices"].tolist() == [0] * (E + 1)
    assert got["ind"]["expert_ids"].tolist() == [-1] * E
    assert got["ind"]["expert_usage_stats"].tolist() == [0, 0]


def test_back_to_back_calls_share_the_counter():
    """Calls queued without synchronisation on one workspace, with sizes
    going down and up and switching between the one- and two-launch forms:
    each must see the counter and counts the previous one left."""
    wk = wl.WORKLOADS["decode"]
    log("route_and_index back to back")
    ws = workspace(8192, wk.K, wk.E)
    Ts = [128, 3, 2000, 8192, 17, 5000, 128, 1, 8192]
    cases = []
    for i, T in enumerate(Ts):
        x = wl.random_scores(T, wk.E, seed=100 + i, levels=4 if i % 2 else 0)
        b = wl.random_bias(wk.E, seed=7)
        o = Outputs(T, wk.E, wk.K, torch.float32, False)
        launch(o, x.to(DEV), b.to(DEV), ws, 8, 4, True, 2.5, binding.SCORE_NONE)
        cases.append((x, b, o))
    torch.cuda.synchronize()
    assert_zero(ws, wk.E)
    for x, b, o in cases:
        check_against_oracle(o.host(), x, b, wk.K, 8, 4, True, 2.5)


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", 16), ("decode", None),
                                    ("mixtral", None), ("dsv3", None)])
def test_graph_replay(name, T):
    """Captured once, replayed several times with eager work in between;
    every replay gives the eager result and leaves the workspace zero (the
    one-launch form at T = 64, E = 8 and T = 16, E = 256, the two-launch
    form with one chunk and with several, at E = 8 and E = 256)."""
    wk = wl.WORKLOADS[name]
    if T is not None:
        wk = replace(wk, T=T)
    log("route_and_index graph replay", wk.describe())
    x = wl.make_scores(wk).to(DEV)
    b = wl.make_bias(wk).to(DEV)
    ws = workspace(wk.T, wk.K, wk.E)
    eager = Outputs(wk.T, wk.E, wk.K, torch.float32, True)
    launch(eager, x, b, ws, 8, 4, True, 2.5, binding.SCORE_NONE, align=16)
    torch.cuda.synchronize()
    ref = eager.host()
    o = Outputs(wk.T, wk.E, wk.K, torch.float32, True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch(o, x, b, ws, 8, 4, True, 2.5, binding.SCORE_NONE, align=16)  # warm-up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(o, x, b, ws, 8, 4, True, 2.5, binding.SCORE_NONE, align=16,
               stream=torch.cuda.current_stream())
    for rep in range(4):
        for t in (o.idx, o.order, o.restore, o.starts, o.eids, o.stats, o.scales):
            t.fill_(POISON)
        o.w.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_zero(ws, wk.E, "after replay %d" % rep)
        check_same(o.host(), ref)


def test_huge_batch_matches_separate():
    """2^22 + 3 tokens of the DSv3 shape (4 GiB of scores; 33.5M slots in 64
    index chunks): every output equal, bit for bit and compared on the GPU,
    to the two separate entry points (whose own parity at this size is
    covered by the sampled router test and the index-property tests), and
    the workspace left zero."""
    T, E, K, G, TG = (1 << 22) + 3, 256, 8, 8, 4
    log("route_and_index huge batch", T)
    g = torch.Generator(device=DEV).manual_seed(21)
    x = torch.sigmoid(torch.randn(T, E, generator=g, device=DEV))
    b = wl.random_bias(E, seed=22).to(DEV)
    ws = workspace(T, K, E)
    fo = Outputs(T, E, K, torch.float32, True)
    launch(fo, x, b, ws, G, TG, True, 2.5, binding.SCORE_NONE, align=16)
    so = Outputs(T, E, K, torch.float32, True)
    binding.moe_router_group_limited(so.idx, so.w, x, b, G, TG, True, 2.5)
    n = binding.moe_create_indices_workspace_size(T * K, E)
    ws2 = torch.empty(max(n, 4) // 4, dtype=torch.int32, device=DEV)
    binding.moe_create_indices_aligned(so.order, so.starts, so.restore, so.eids, so.stats,
                                       so.idx, ws2, so.scales, 16)
    torch.cuda.synchronize()
    assert_zero(ws, E)
    for name in ("idx", "order", "restore", "starts", "eids", "stats", "scales"):
        assert torch.equal(getattr(fo, name), getattr(so, name)), name
    assert torch.equal(fo.w.view(torch.int32), so.w.view(torch.int32))


def test_workspace_sized_for_a_larger_batch():
    """A workspace sized for T = 8200 tokens (E = 256, K = 8) serves the
    smaller batches 8192, 4097 and 600 after it, queued back to back: the
    size function never decreases in T (at 8192 the plan has more chunks
    than at 8200, which once made the smaller call need more)."""
    E, K, G, TG = 256, 8, 8, 4
    log("route_and_index workspace sized for 8200 tokens")
    ws = workspace(8200, K, E)
    assert ws.numel() * 4 >= binding.moe_route_and_index_workspace_size(8192, K, E)
    cases = []
    for i, T in enumerate((8200, 8192, 4097, 600)):
        x = wl.random_scores(T, E, seed=300 + i)
        b = wl.random_bias(E, seed=301)
        o = Outputs(T, E, K, torch.float32, False)
        launch(o, x.to(DEV), b.to(DEV), ws, G, TG, True, 2.5, binding.SCORE_NONE)
        cases.append((x, b, o))
    torch.cuda.synchronize()
    assert_zero(ws, E)
    for x, b, o in cases:
        check_against_oracle(o.host(), x, b, K, G, TG, True, 2.5)


def test_dirty_workspace_is_reported():
    """A counts matrix that is not zero on entry is detected: the index step
    finds that the counts do not add up to T * K, stores
    MOE_STATUS_COUNTS_MISMATCH in the workspace's status word, and still
    clears the matrix (every kernel exits normally). The next call on the
    same workspace, with the status word reset, is correct again. DSv3
    shape (8192 tokens: 64 index chunks, every row of the matrix in use)."""
    wk = wl.WORKLOADS["dsv3"]
    T, E, K = wk.T, wk.E, wk.K
    log("route_and_index dirty workspace", wk.describe())
    x, b = wl.make_scores(wk), wl.make_bias(wk)
    ws = workspace(T, K, E)
    status = binding.ROUTE_INDEX_STATUS_OFFSET // 4
    header = 256 // 4
    ws[header:] = 1  # every count off by one (and the scratch past the matrix dirty too)
    o = Outputs(T, E, K, torch.float32, False)
    launch(o, x.to(DEV), b.to(DEV), ws, wk.n_groups, wk.topk_group, True, wk.scale,
           binding.SCORE_NONE)
    torch.cuda.synchronize()
    assert int(ws[status].item()) == binding.STATUS_COUNTS_MISMATCH
    zp = zero_part(ws, E)
    rest = torch.cat([zp[:status], zp[status + 1:]])
    assert int(torch.count_nonzero(rest).item()) == 0, "matrix or ticket not cleared"
    # the router's own outputs do not depend on the workspace
    got = o.host()
    ref = separate(x, b, K, wk.n_groups, wk.topk_group, True, wk.scale)
    assert np.array_equal(got["idx"], ref["idx"])
    # reset the status word: the next call is clean
    ws[status] = 0
    got = fused(x, b, K, wk.n_groups, wk.topk_group, True, wk.scale, ws=ws)
    assert int(ws[status].item()) == 0
    check_against_oracle(got, x, b, K, wk.n_groups, wk.topk_group, True, wk.scale)


@pytest.mark.parametrize("name,T", [("dsv3", 8192), ("decode", 128), ("mixtral", 4096)])
def test_workspace_4_byte_aligned(name, T):
    """A workspace that is 4-byte but not 16-byte aligned takes the chunked
    form (the ranked form moves rows of counts in 16-byte pieces): same
    outputs, header and counts left zero."""
    wk = wl.WORKLOADS[name].with_tokens(T)
    log("route_and_index 4-byte aligned workspace", wk.describe())
    x, b = wl.make_scores(wk), wl.make_bias(wk)
    n = binding.moe_route_and_index_workspace_size(wk.T, wk.K, wk.E) // 4
    base = torch.zeros(n + 4, dtype=torch.int32, device=DEV)
    ws = base[1:1 + n]
    assert ws.data_ptr() % 16 == 4
    args = (wk.K, wk.n_groups, wk.topk_group, wk.norm_weights, wk.scale)
    got = fused(x, b, *args, ws=ws)
    check_against_oracle(got, x, b, *args)
    check_same(got, fused(x, b, *args))
