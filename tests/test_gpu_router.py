"""GPU parity: moe_router_group_limited vs the CPU oracle (router page:
description, Parameters, Args). Indices and weights bit-exact (the
required weight bound is 1e-6 relative; both sides normalise in binary64 and
round once, so they agree exactly). Marked gpu: needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle
from permutation_group_limited_amd import binding
from permutation_group_limited_amd import workloads as wl

from _gpu import (assert_weights_equal, bf16_bits, encode,
                  gpu_router, log)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "mixtral", "dsv3", "decode", "skewed"])
def test_workload_full_size(name):
    w = wl.WORKLOADS[name]
    log("router workload", w.describe())
    s, b = wl.make_scores(w), wl.make_bias(w)
    for mode in (oracle.GROUP_TOP2_SUM, oracle.GROUP_MAX):
        gi, gw = gpu_router(s, b, w.K, w.n_groups, w.topk_group, w.norm_weights, w.scale, mode)
        oi, ow = oracle.router(s.numpy(), b.numpy(), w.K, w.n_groups, w.topk_group,
                               w.norm_weights, w.scale, mode)
        assert np.array_equal(gi, oi), "indices differ in %d tokens" % np.sum(np.any(gi != oi, 1))
        assert_weights_equal(gw, ow)


CASES = [
    # (T, E, G, TG, K)
    (1, 1, 1, 1, 1), (5, 2, 1, 1, 2), (7, 4, 2, 1, 2), (33, 8, 1, 1, 2), (33, 8, 4, 2, 3),
    (65, 8, 8, 3, 3), (100, 16, 4, 2, 4), (129, 32, 8, 4, 6), (257, 64, 8, 4, 8),
    (1000, 64, 64, 7, 5), (300, 128, 8, 4, 8), (300, 128, 4, 1, 16), (511, 256, 8, 4, 8),
    (77, 256, 1, 1, 8), (77, 256, 16, 5, 10), (77, 256, 64, 32, 64), (77, 256, 256 // 4, 2, 8),
    (130, 512, 8, 4, 8), (130, 512, 32, 3, 12), (61, 1024, 8, 4, 8), (61, 1024, 64, 64, 64),
]


@pytest.mark.parametrize("T,E,G,TG,K", CASES)
@pytest.mark.parametrize("levels", [0, 3])
def test_random_shapes(T, E, G, TG, K, levels):
    log("router case", T, E, G, TG, K, "levels", levels)
    s = wl.random_scores(T, E, seed=T + E + K, levels=levels)
    b = wl.random_bias(E, seed=G + TG, std=0.02, levels=levels)
    for mode in (oracle.GROUP_TOP2_SUM, oracle.GROUP_MAX):
        for norm in (True, False):
            gi, gw = gpu_router(s, b, K, G, TG, norm, 1.75, mode)
            oi, ow = oracle.router(s.numpy(), b.numpy(), K, G, TG, norm, 1.75, mode)
            assert np.array_equal(gi, oi), (mode, norm)
            assert_weights_equal(gw, ow)


def test_all_ties():
    # every score equal: selection is decided by the index rule alone
    T, E = 50, 256
    s = torch.full((T, E), 0.5)
    b = torch.zeros(E)
    gi, _ = gpu_router(s, b, 8, 8, 4, True, 1.0)
    oi, _ = oracle.router(s.numpy(), b.numpy(), 8, 8, 4, True, 1.0)
    assert np.array_equal(gi, oi)
    assert gi[0].tolist() == list(range(8))


def test_signed_zero_scores_tie():
    # -0 and +0 compare equal: lower index wins
    T, E = 4, 8
    s = torch.zeros(T, E)
    s[:, ::2] = -0.0
    b = torch.zeros(E)
    gi, _ = gpu_router(s, b, 3, 1, 1, False, 1.0)
    oi, _ = oracle.router(s.numpy(), b.numpy(), 3, 1, 1, False, 1.0)
    assert np.array_equal(gi, oi)
    assert gi[0].tolist() == [0, 1, 2]


def test_empty_batch():
    gi, gw = gpu_router(torch.zeros(0, 256), torch.zeros(256), 8, 8, 4, True, 1.0)
    assert gi.shape == (0, 8) and gw.shape == (0, 8)


def test_deterministic():
    w = wl.WORKLOADS["dsv3"]
    s, b = wl.make_scores(w), wl.make_bias(w)
    a = gpu_router(s, b, 8, 8, 4, True, 2.5)
    for _ in range(3):
        c = gpu_router(s, b, 8, 8, 4, True, 2.5)
        assert np.array_equal(a[0], c[0]) and np.array_equal(a[1].view(np.uint32),
                                                             c[1].view(np.uint32))


DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.mark.parametrize("sd,bd", [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16"),
                                   ("f16", "f32")])
@pytest.mark.parametrize("T,E,G,TG,K", [(300, 256, 8, 4, 8), (129, 8, 1, 1, 2),
                                        (77, 64, 8, 3, 6), (65, 1024, 16, 4, 8)])
def test_16bit_scores(sd, bd, T, E, G, TG, K):
    log("router dtypes", sd, bd, T, E, G, TG, K)
    for levels in (0, 3):
        s = wl.random_scores(T, E, seed=E + T, levels=levels).to(DTYPES[sd])
        b = wl.random_bias(E, seed=G, std=0.02, levels=levels).to(DTYPES[bd])
        gi, gw = gpu_router(s, b, K, G, TG, True, 2.5)
        sn, scode = encode(s)
        bn, bcode = encode(b)
        oi, ow = oracle.router(sn, bn, K, G, TG, True, 2.5, scores_dtype=scode,
                               bias_dtype=None if bd == "f32" else bcode)
        assert np.array_equal(gi, oi)
        assert_weights_equal(bf16_bits(gw), ow)


def gpu_router_logits(logits, bias, fn, K, G, TG, norm, scale, mode=0):
    T, E = logits.shape
    x = logits.to("cuda:0")
    b = bias.to("cuda:0")
    idx = torch.full((T, K), -7, dtype=torch.int32, device="cuda:0")
    w = torch.full((T, K), float("nan"), dtype=logits.dtype, device="cuda:0")
    binding.moe_router_group_limited_logits(idx, w, x, b, fn, G, TG, norm, scale, mode)
    torch.cuda.synchronize()
    wh = w.cpu()
    return idx.cpu().numpy(), (wh.numpy() if wh.dtype == torch.float32 else wh)


FNS = {"sigmoid": (binding.SCORE_SIGMOID, oracle.SCORE_SIGMOID),
       "softmax": (binding.SCORE_SOFTMAX, oracle.SCORE_SOFTMAX)}


@pytest.mark.parametrize("name", ["tiny", "mixtral", "dsv3", "decode", "skewed"])
def test_logits_workload_full_size(name):
    w = wl.WORKLOADS[name]
    log("router logits workload", w.describe(), w.score_fn)
    x, b = wl.make_logits(w), wl.make_bias(w)
    gfn, ofn = FNS[w.score_fn]
    gi, gw = gpu_router_logits(x, b, gfn, w.K, w.n_groups, w.topk_group, w.norm_weights,
                               w.scale)
    oi, ow = oracle.router(x.numpy(), b.numpy(), w.K, w.n_groups, w.topk_group,
                           w.norm_weights, w.scale, score_fn=ofn)
    assert np.array_equal(gi, oi), "indices differ in %d tokens" % np.sum(np.any(gi != oi, 1))
    assert_weights_equal(gw, ow)


@pytest.mark.parametrize("fn", ["sigmoid", "softmax"])
@pytest.mark.parametrize("T,E,G,TG,K", [(33, 8, 4, 2, 3), (129, 32, 8, 4, 6), (300, 128, 8, 4, 8),
                                        (511, 256, 8, 4, 8), (61, 1024, 64, 8, 16),
                                        (77, 64, 1, 1, 6)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_logits_random_shapes(fn, T, E, G, TG, K, dt):
    log("router logits", fn, T, E, G, TG, K, dt)
    g = torch.Generator().manual_seed(T * E + K)
    x = (torch.randn(T, E, generator=g) * 3).to(DTYPES[dt])
    b = (torch.randn(E, generator=g) * 0.02)
    gfn, ofn = FNS[fn]
    for norm in (True, False):
        gi, gw = gpu_router_logits(x, b, gfn, K, G, TG, norm, 1.5)
        xn, xcode = encode(x)
        oi, ow = oracle.router(xn, b.numpy(), K, G, TG, norm, 1.5, scores_dtype=xcode,
                               score_fn=ofn)
        assert np.array_equal(gi, oi)
        if dt == "f32":
            assert_weights_equal(gw, ow)
        else:
            assert_weights_equal(bf16_bits(gw), ow)


def test_huge_batch_sampled():
    """2^22 + 3 tokens of the DSv3 shape (4 GiB of scores, so byte offsets
    past 2^32), routed in one call; each token's result depends on its own
    row only, so the oracle checks 4,099 of them (random rows, the first and
    the last)."""
    T, E, K, G, TG = (1 << 22) + 3, 256, 8, 8, 4
    log("router huge batch", T)
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(11)
    s = torch.sigmoid(torch.randn(T, E, generator=g, device=dev))
    b = wl.random_bias(E, seed=12).to(dev)
    idx = torch.full((T, K), -7, dtype=torch.int32, device=dev)
    w = torch.full((T, K), float("nan"), device=dev)
    binding.moe_router_group_limited(idx, w, s, b, G, TG, True, 2.5)
    torch.cuda.synchronize()
    rows = torch.randperm(T, generator=torch.Generator().manual_seed(13))[:4096]
    rows = torch.cat([rows, torch.tensor([0, 1, T - 1])]).to(dev)
    oi, ow = oracle.router(s[rows].cpu().numpy(), b.cpu().numpy(), K, G, TG, True, 2.5)
    assert np.array_equal(idx[rows].cpu().numpy(), oi)
    assert_weights_equal(w[rows].cpu().numpy(), ow)


@pytest.mark.parametrize("E,G,TG,K", [(64, 8, 4, 8), (96, 8, 4, 8)])
def test_more_than_2_32_work_items(E, G, TG, K):
    """2^26 + 5 tokens of 64 lanes each: more work-items than one grid
    dimension holds, so the launch is laid out as rows of workgroups (the
    power-of-two form at E = 64, the general form at E = 96). Sampled
    tokens against the oracle: the first and last, those around token 2^26
    and 4,096 random ones."""
    T = (1 << 26) + 5
    log("router 2-D grid", T, "E", E)
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(E)
    s = torch.rand(T, E, generator=g, device=dev)
    b = wl.random_bias(E, seed=E + 1).to(dev)
    idx = torch.full((T, K), -7, dtype=torch.int32, device=dev)
    w = torch.full((T, K), float("nan"), device=dev)
    binding.moe_router_group_limited(idx, w, s, b, G, TG, True, 2.5)
    torch.cuda.synchronize()
    rows = torch.randperm(T, generator=torch.Generator().manual_seed(E))[:4096]
    edge = torch.tensor([0, 1, (1 << 26) - 1, 1 << 26, (1 << 26) + 1, T - 2, T - 1])
    rows = torch.cat([rows, edge]).to(dev)
    oi, ow = oracle.router(s[rows].cpu().numpy(), b.cpu().numpy(), K, G, TG, True, 2.5)
    assert np.array_equal(idx[rows].cpu().numpy(), oi)
    assert_weights_equal(w[rows].cpu().numpy(), ow)
    assert int((idx < 0).sum()) == 0  # every token written
    del s, idx, w
    torch.cuda.empty_cache()


# Large batches at E = 64 ... 256 with at most 32 groups and K <= 32 take the
# two-tokens-per-wave form (T >= 8192, or >= 4096 when the histogram is
# filled too); 64 groups or K > 32 keep one token per wave. Ragged T leaves
# the last wave half used.
WIDE = [(8195, 64, 8, 4, 8), (8195, 64, 32, 8, 16), (8192, 128, 1, 1, 8),
        (8195, 128, 16, 4, 8), (8195, 256, 8, 4, 8), (8195, 256, 32, 4, 12),
        (9001, 256, 16, 5, 10), (8195, 256, 64, 8, 8), (8195, 256, 8, 4, 32),
        (8195, 256, 8, 4, 33), (8195, 128, 4, 4, 64), (8195, 64, 2, 2, 48)]


@pytest.mark.parametrize("T,E,G,TG,K", WIDE)
@pytest.mark.parametrize("levels", [0, 3])
def test_two_tokens_per_wave(T, E, G, TG, K, levels):
    log("router wide", T, E, G, TG, K, "levels", levels)
    s = wl.random_scores(T, E, seed=T + E + K + levels, levels=levels)
    b = wl.random_bias(E, seed=G + TG, std=0.02, levels=levels)
    for mode in (oracle.GROUP_TOP2_SUM, oracle.GROUP_MAX):
        for norm in (True, False):
            gi, gw = gpu_router(s, b, K, G, TG, norm, 1.75, mode)
            oi, ow = oracle.router(s.numpy(), b.numpy(), K, G, TG, norm, 1.75, mode)
            assert np.array_equal(gi, oi)
            assert_weights_equal(gw, ow)


@pytest.mark.parametrize("sd,bd", [("bf16", "bf16"), ("f16", "f32")])
def test_two_tokens_per_wave_16bit(sd, bd):
    T, E, G, TG, K = 8195, 256, 8, 4, 8
    log("router wide dtypes", sd, bd)
    s = wl.random_scores(T, E, seed=3, levels=4).to(DTYPES[sd])
    b = wl.random_bias(E, seed=4, std=0.02, levels=4).to(DTYPES[bd])
    gi, gw = gpu_router(s, b, K, G, TG, True, 2.5)
    sn, scode = encode(s)
    bn, bcode = encode(b)
    oi, ow = oracle.router(sn, bn, K, G, TG, True, 2.5, scores_dtype=scode,
                           bias_dtype=None if bd == "f32" else bcode)
    assert np.array_equal(gi, oi)
    assert_weights_equal(bf16_bits(gw), ow)


@pytest.mark.parametrize("fn", ["sigmoid", "softmax"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_two_tokens_per_wave_logits(fn, dt):
    T, E, G, TG, K = 8195, 128, 8, 4, 8
    log("router wide logits", fn, dt)
    g = torch.Generator().manual_seed(17)
    x = (torch.randn(T, E, generator=g) * 3).to(DTYPES[dt])
    b = torch.randn(E, generator=g) * 0.02
    gfn, ofn = FNS[fn]
    gi, gw = gpu_router_logits(x, b, gfn, K, G, TG, True, 1.5)
    xn, xcode = encode(x)
    oi, ow = oracle.router(xn, b.numpy(), K, G, TG, True, 1.5, scores_dtype=xcode, score_fn=ofn)
    assert np.array_equal(gi, oi)
    if dt == "f32":
        assert_weights_equal(gw, ow)
    else:
        assert_weights_equal(bf16_bits(gw), ow)


@pytest.mark.parametrize("row", [0, 1])
@pytest.mark.parametrize("T", [1, 8192])
def test_softmax_sum_order_rows(row, T):
    # logits on which another order of the softmax denominator's additions
    # changes a binary32 score (tests/golden/softmax_sum_order_logits.txt):
    # the kernel must add in the oracle's pairwise order. No normalisation
    # and scale 1, so the weights are the scores; the bias makes the flipping
    # expert one of the K selected. T = 8192 at E = 256 takes the
    # two-tokens-per-wave form.
    from test_oracle_scorefn import sum_order_rows
    E, flip, x1 = sum_order_rows()[row]
    log("router softmax sum-order row", E, flip, T)
    x = torch.from_numpy(np.repeat(x1, T, axis=0))
    if E == 4:
        K, bias = 4, torch.zeros(E)
    else:
        K = 32
        bias = torch.zeros(E)
        lo = flip - flip % K
        bias[lo:lo + K] = 10.0
    gfn, ofn = FNS["softmax"]
    gi, gw = gpu_router_logits(x, bias, gfn, K, 1, 1, False, 1.0)
    oi, ow = oracle.router(x.numpy(), bias.numpy(), K, 1, 1, False, 1.0, score_fn=ofn)
    assert np.array_equal(gi, oi)
    assert_weights_equal(gw, ow)
    assert np.any(gi[0] == flip)
