"""GPU parity of the router for expert counts that are not powers of two
(any E up to 1024 with E % n_groups == 0; the router page leaves E to the
caller). These take the kernel's general form: one wave per token, group
stage through LDS. Indices and weights (fp32 and 16-bit) bit-exact against the
oracle. Marked gpu."""
import numpy as np
import pytest
import torch

import oracle
from permutation_group_limited_amd import binding
from permutation_group_limited_amd import workloads as wl

from _gpu import (DEV, assert_indices_equal, assert_weights_equal,
                  bf16_bits, encode, gpu_indices, log)

pytestmark = pytest.mark.gpu

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

# (T, E, G, TG, K): odd and even E, groups of odd size, one group, E near
# the 64-lane and 1024 limits, and a DeepSeek-V2-like 160 experts in 8 groups
SHAPES = [(129, 3, 1, 1, 2), (77, 6, 3, 2, 3), (200, 12, 4, 2, 4), (65, 20, 4, 3, 6),
          (300, 40, 8, 4, 8), (64, 60, 6, 2, 5), (257, 96, 8, 4, 8), (33, 100, 4, 2, 8),
          (511, 160, 8, 3, 6), (97, 384, 8, 4, 8), (50, 640, 16, 4, 8), (40, 1000, 8, 4, 8),
          (31, 1023, 3, 2, 8), (1, 72, 9, 9, 1)]


def gpu_route(x, b, K, G, TG, norm, scale, mode=0, fn=None):
    T, E = x.shape
    idx = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, K), float("nan"), dtype=x.dtype, device=DEV)
    if fn is None:
        binding.moe_router_group_limited(idx, w, x.to(DEV), b.to(DEV), G, TG, norm, scale, mode)
    else:
        binding.moe_router_group_limited_logits(idx, w, x.to(DEV), b.to(DEV), fn, G, TG, norm,
                                                scale, mode)
    torch.cuda.synchronize()
    wh = w.cpu()
    return idx.cpu().numpy(), (wh.numpy() if wh.dtype == torch.float32 else wh)


def check(gi, gw, x, b, K, G, TG, norm, scale, mode=0, ofn=oracle.SCORE_LOAD):
    xn, xcode = encode(x)
    bn, bcode = encode(b)
    oi, ow = oracle.router(xn, bn, K, G, TG, norm, scale, group_score=mode, scores_dtype=xcode,
                           bias_dtype=None if b.dtype == torch.float32 else bcode, score_fn=ofn)
    assert np.array_equal(gi, oi), "indices differ in %d tokens" % np.sum(np.any(gi != oi, 1))
    if x.dtype == torch.float32:
        assert_weights_equal(gw, ow)
    else:
        assert_weights_equal(bf16_bits(gw), ow)
    return oi


@pytest.mark.parametrize("T,E,G,TG,K", SHAPES)
@pytest.mark.parametrize("levels", [0, 3])
def test_any_e_shapes(T, E, G, TG, K, levels):
    log("router any E", T, E, G, TG, K, levels)
    x = wl.random_scores(T, E, seed=T * 7 + E, levels=levels)
    b = wl.random_bias(E, seed=E + 3, std=0.02, levels=levels)
    for norm, mode, scale in ((True, 0, 2.5), (False, 1, 1.0), (True, 1, 1.5)):
        gi, gw = gpu_route(x, b, K, G, TG, norm, scale, mode)
        check(gi, gw, x, b, K, G, TG, norm, scale, mode)


@pytest.mark.parametrize("sd,bd", [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16"),
                                   ("f16", "f32")])
@pytest.mark.parametrize("T,E,G,TG,K", [(300, 160, 8, 3, 6), (65, 20, 4, 3, 6)])
def test_any_e_16bit(sd, bd, T, E, G, TG, K):
    log("router any E dtypes", sd, bd, T, E)
    x = wl.random_scores(T, E, seed=E, levels=5).to(DTYPES[sd])
    b = wl.random_bias(E, seed=E + 1, std=0.02).to(DTYPES[bd])
    gi, gw = gpu_route(x, b, K, G, TG, True, 2.5)
    check(gi, gw, x, b, K, G, TG, True, 2.5)


@pytest.mark.parametrize("fn", ["sigmoid", "softmax"])
@pytest.mark.parametrize("T,E,G,TG,K", [(257, 160, 8, 3, 6), (100, 12, 4, 2, 4),
                                        (40, 1000, 8, 4, 8)])
def test_any_e_logits(fn, T, E, G, TG, K):
    log("router any E logits", fn, T, E)
    g = torch.Generator().manual_seed(T + E)
    x = torch.randn(T, E, generator=g) * 3
    b = torch.randn(E, generator=g) * 0.02
    gfn = binding.SCORE_SIGMOID if fn == "sigmoid" else binding.SCORE_SOFTMAX
    ofn = oracle.SCORE_SIGMOID if fn == "sigmoid" else oracle.SCORE_SOFTMAX
    for norm in (True, False):
        gi, gw = gpu_route(x, b, K, G, TG, norm, 1.5, fn=gfn)
        check(gi, gw, x, b, K, G, TG, norm, 1.5, ofn=ofn)


def test_any_e_then_indices():
    """DeepSeek-V2-like routing (160 experts, 8 groups, 3 kept, top-6) on a
    decode-sized batch, then index creation on its output."""
    T, E, G, TG, K = 128, 160, 8, 3, 6
    log("router any E -> create_indices", T, E)
    x = wl.random_scores(T, E, seed=5)
    b = wl.random_bias(E, seed=6)
    gi, gw = gpu_route(x, b, K, G, TG, True, 16.0)
    oi = check(gi, gw, x, b, K, G, TG, True, 16.0)
    assert_indices_equal(gpu_indices(gi, E), oracle.create_indices(oi, E))


def test_any_e_empty_batch():
    idx = torch.empty(0, 6, dtype=torch.int32, device=DEV)
    w = torch.empty(0, 6, device=DEV)
    binding.moe_router_group_limited(idx, w, torch.empty(0, 160, device=DEV),
                                     torch.zeros(160, device=DEV), 8, 3, True, 1.0)
    torch.cuda.synchronize()
