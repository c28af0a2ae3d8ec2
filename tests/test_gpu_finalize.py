"""GPU parity: moe_finalize vs the CPU oracle (moe_finalize page:
description, Args), bit for bit for every dtype combination: both run one
fmaf per k in ascending k from +0 in fp32 and round once to the output
type. Marked gpu."""
import numpy as np
import pytest
import torch

import oracle
from permutation_group_limited_amd import binding
from permutation_group_limited_amd import workloads as wl

from _gpu import (DEV, assert_finalize_equal, assert_finalize_matches_in_blocks, bf16_bits,
                  gpu_finalize, log, oracle_finalize_from, term_magnitude)

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _inputs(T, K, H, ddt, wdt, seed):
    g = torch.Generator().manual_seed(seed)
    down = torch.randn(T * K, H, generator=g).to(ddt)
    w = (torch.rand(T, K, generator=g) * 2.0).to(wdt)
    restore = torch.randperm(T * K, generator=g).numpy().astype(np.uint32)
    return down, w, restore


@pytest.mark.parametrize("ddt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("wdt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("T,K,H", [(1, 1, 8), (5, 2, 136), (33, 8, 520), (17, 3, 1032),
                                   (9, 9, 264), (4, 16, 64), (40, 6, 7168), (3, 1, 4096),
                                   (3, 64, 520)])
def test_random_shapes(ddt, wdt, odt, T, K, H):
    if ddt == "f32" and H % 4 or ddt != "f32" and H % 8:
        pytest.skip("row not a multiple of 16 bytes")
    log("finalize case", ddt, wdt, odt, T, K, H)
    down, w, restore = _inputs(T, K, H, DT[ddt], DT[wdt], seed=T * 100 + K * 10 + H)
    got = gpu_finalize(down.to(DEV), restore, w, DT[odt])
    exp = oracle_finalize_from(down, restore, w, DT[odt])
    assert_finalize_equal(got, exp, term_magnitude(down, restore, w))


def test_cancellation_is_judged_against_term_magnitude():
    T, K, H = 8, 2, 64
    down = torch.randn(T * K, H)
    down[1::2] = -down[0::2]
    w = torch.ones(T, K)
    restore = np.arange(T * K, dtype=np.uint32)
    got = gpu_finalize(down.to(DEV), restore, w, torch.float32)
    assert torch.all(got.cpu() == 0)


@pytest.mark.parametrize("name", ["tiny", "mixtral", "dsv3", "decode"])
def test_workload_full_size(name):
    wk = wl.WORKLOADS[name]
    log("finalize workload", wk.describe())
    s, b = wl.make_scores(wk), wl.make_bias(wk)
    ids, wts = oracle.router(s.numpy(), b.numpy(), wk.K, wk.n_groups, wk.topk_group,
                             wk.norm_weights, wk.scale)
    restore = oracle.create_indices(ids, wk.E)["restore_token_order"]
    down = wl.make_down(wk, device=DEV)
    w = torch.from_numpy(wts)
    got = gpu_finalize(down, restore, w, wk.out_dtype)
    down_h = down.cpu()
    exp = oracle_finalize_from(down_h, restore, w, wk.out_dtype)
    mag = term_magnitude(down_h, restore, w) if wk.out_dtype == torch.float32 else None
    assert_finalize_equal(got, exp, mag)


def test_skewed_full_size():
    # full-size launch (7 GiB of down); every one of the 65,536 output rows
    # is compared with the oracle, 4,096 tokens (470 MB of gathered rows) at
    # a time
    wk = wl.WORKLOADS["skewed"]
    log("finalize workload", wk.describe(), "(all tokens, in blocks)")
    s, b = wl.make_scores(wk), wl.make_bias(wk)
    ids, wts = oracle.router(s.numpy(), b.numpy(), wk.K, wk.n_groups, wk.topk_group,
                             wk.norm_weights, wk.scale)
    restore = oracle.create_indices(ids, wk.E)["restore_token_order"]
    down = wl.make_down(wk, device=DEV)
    got = gpu_finalize(down, restore, torch.from_numpy(wts), wk.out_dtype)
    worst = assert_finalize_matches_in_blocks(got, down, restore, torch.from_numpy(wts),
                                              wk.out_dtype)
    log("skewed finalize: largest difference %s ulp" % worst)
    del down, got
    torch.cuda.empty_cache()


def test_deterministic():
    T, K, H = 512, 8, 7168
    down, w, restore = _inputs(T, K, H, torch.bfloat16, torch.float32, seed=1)
    dd = down.to(DEV)
    a = gpu_finalize(dd, restore, w, torch.bfloat16).cpu()
    for _ in range(3):
        assert torch.equal(gpu_finalize(dd, restore, w, torch.bfloat16).cpu().view(torch.int16),
                           a.view(torch.int16))


def test_more_than_2_32_work_items():
    """2^26 + 5 tokens, K = 1, H = 8 (one wave per token): more work-items
    than one grid dimension holds, so the launch is laid out as rows of
    workgroups. Sampled tokens (first, last, around 2^26, 4,096 random)
    against the oracle; every output row written."""
    T, K, H = (1 << 26) + 5, 1, 8
    log("finalize 2-D grid", T)
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(3)
    down = torch.randn(T * K, H, generator=g, device=dev).to(torch.bfloat16)
    w = torch.rand(T, K, generator=g, device=dev) * 2.0
    restore = torch.randperm(T * K, generator=g, device=dev).to(torch.int32)
    out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)
    binding.moe_finalize(out, down, restore, w)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(out).any())
    ts = torch.randperm(T, generator=torch.Generator().manual_seed(4))[:4096]
    edge = torch.tensor([0, 1, (1 << 26) - 1, 1 << 26, (1 << 26) + 1, T - 2, T - 1])
    ts = torch.sort(torch.cat([ts, edge])).values.to(dev)
    rows = restore.view(T, K)[ts].reshape(-1).long()
    sub_down = down[rows].cpu()
    exp = oracle_finalize_from(sub_down, np.arange(rows.numel(), dtype=np.uint32),
                               w[ts].cpu(), torch.bfloat16)
    assert_finalize_equal(out[ts], exp, None)
    del down, out, restore
    torch.cuda.empty_cache()


@pytest.mark.parametrize("odt", ["f16", "bf16", "f32"])
def test_overflow_to_infinity(odt):
    """Sums past the output format's largest finite value round to +-inf
    (round to nearest), equal bit for bit to the oracle: f16 past 65504,
    bf16 and f32 past about 3.4e38 (fp32 accumulation overflows there)."""
    T, K, H = 6, 2, 64
    g = torch.Generator().manual_seed(9)
    big = 3.0e38 if odt != "f16" else 4.0e4
    down = torch.randn(T * K, H, generator=g)
    down[:, :8] = big  # both terms large and of one sign: certain overflow
    down[:, 8:16] = -big
    w = torch.full((T, K), 1.5)
    restore = np.arange(T * K, dtype=np.uint32)
    got = gpu_finalize(down.to(DEV), restore, w, DT[odt])
    exp = oracle_finalize_from(down, restore, w, DT[odt])
    g_np = got.cpu()
    assert torch.isinf(g_np[:, :16]).all()
    if odt == "f32":
        assert np.array_equal(g_np.numpy().view(np.uint32), np.asarray(exp).view(np.uint32))
    else:
        assert np.array_equal(bf16_bits(got), np.asarray(exp, np.uint16))


# ---- large shapes ----------------------------------------------------------
# Millions of outputs per case, so the fp32 sums include thousands that sit
# exactly halfway between two binary16 (or bf16) values: rounding them once
# more, to the output type, must follow the fp32 rounding, as in the oracle
# (a mixed-precision fma rounding the exact sum straight to binary16 would
# differ there). Ragged H (7160: the last 16-byte column of a 512-element
# chunk missing), long rows (14336, 16384), every K up to 8, all 16-bit
# dtype combinations; both launch shapes (gathered rows below 256 MiB: four
# waves per workgroup, sc1 output stores; above: one wave per workgroup with
# the LDS reservation that caps the waves per compute unit, non-temporal
# stores), the latter at K = 2 (no cap), 3, 4, 5, 6, 7, 8 and 16 (batches
# of 8 rows).
LARGE_CASES = [
    # T, K, H, down, weight, out
    (8200, 8, 7168, "bf16", "f32", "bf16"),
    (4101, 3, 7160, "f16", "f16", "bf16"),
    (2051, 5, 14336, "bf16", "f32", "f16"),
    (2053, 1, 16384, "f16", "bf16", "f16"),
    (4113, 4, 7168, "f16", "f32", "f16"),
    (8197, 6, 4096, "bf16", "f16", "bf16"),
    (4099, 7, 8192, "bf16", "f32", "f16"),
    (8195, 2, 4096, "f16", "bf16", "bf16"),
    # fp32 rows past the 256 MiB memory-side cache (non-temporal output
    # stores): two 16-byte stores per lane, and one 8-byte store
    (2100, 8, 4096, "f32", "f32", "f32"),
    (4500, 4, 4096, "f32", "bf16", "bf16"),
    # more streaming shapes: K above 8, K = 2 and 3, a ragged last chunk
    (1100, 16, 8192, "bf16", "f32", "bf16"),
    (8200, 2, 8192, "bf16", "bf16", "bf16"),
    (5000, 3, 9216, "f16", "f32", "f16"),
    (4097, 8, 4104, "bf16", "f32", "bf16"),
]


@pytest.mark.parametrize("T,K,H,ddt,wdt,odt", LARGE_CASES,
                         ids=["T%d-K%d-H%d-%s-%s-%s" % c for c in LARGE_CASES])
def test_large_shapes_equal_oracle(T, K, H, ddt, wdt, odt):
    log("finalize large shape", T, K, H, ddt, wdt, odt)
    down, w, restore = _inputs(T, K, H, DT[ddt], DT[wdt], seed=T + K + H)
    got = gpu_finalize(down.to(DEV), restore, w, DT[odt])
    exp = oracle_finalize_from(down, restore, w, DT[odt])
    assert_finalize_equal(got, exp)


@pytest.mark.parametrize("T,K,H", [(4100, 8, 4096), (64, 2, 4104)])
def test_out_of_range_restore_entries_stay_in_bounds(T, K, H):
    """Precondition violated on purpose (restore entries >= T*K): the call
    completes, no access leaves `down` (such an entry reads row 0 with
    weight 0), and every token whose entries are all in range is exact."""
    log("finalize out-of-range restore", T, K, H)
    down, w, restore = _inputs(T, K, H, torch.bfloat16, torch.float32, seed=5)
    bad_slots = np.array([1, 7, 2 * K + 1, T * K - 1])
    restore = restore.copy()
    restore[bad_slots] = np.array([T * K, 0xFFFFFFFF, T * K + 12345, 0x80000000],
                                  dtype=np.uint32)
    got = gpu_finalize(down.to(DEV), restore, w, torch.bfloat16)
    good = np.ones(T, dtype=bool)
    good[bad_slots // K] = False
    ok_rest = np.where(restore < T * K, restore, 0).astype(np.uint32)
    exp = oracle_finalize_from(down, ok_rest, w, torch.bfloat16)
    assert_finalize_equal(got[torch.from_numpy(good).to(DEV)], np.asarray(exp)[good])
