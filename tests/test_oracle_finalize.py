"""Pins of the CPU oracle's finalize (moe_finalize page: description, Args
output, down, restore_order, router_weight).

Checked against a float64 numpy reference within the error bound of a
K-term fp32 fused multiply-add chain, exact gather special cases, the
hand-worked fixture (including a case where the fp32, k-ordered
accumulation the page prescribes differs from a wider sum), and the bf16
rounding helper against torch's own fp32 -> bf16 conversion.
"""
import json
import os

import numpy as np
import pytest
import torch

U = 2.0 ** -24  # unit roundoff of binary32


def f64_reference(down_f32, restore, w_f32):
    T, K = w_f32.shape
    rows = down_f32.astype(np.float64)[restore.astype(np.int64)].reshape(T, K, -1)
    terms = w_f32.astype(np.float64)[:, :, None] * rows
    return terms.sum(1), np.abs(terms).sum(1)


def _case(T, K, H, seed, dtype_down, dtype_w):
    rng = np.random.default_rng(seed)
    down = rng.standard_normal((T * K, H)).astype(np.float32)
    w = rng.random((T, K)).astype(np.float32) * 2.0
    restore = rng.permutation(T * K).astype(np.uint32)
    return down, w, restore


@pytest.mark.parametrize("T,K,H", [(1, 1, 8), (5, 2, 128), (64, 8, 72), (33, 3, 40),
                                   (16, 16, 24)])
def test_fp32_within_fma_chain_bound(oracle, T, K, H):
    down, w, restore = _case(T, K, H, T * K + H, "f32", "f32")
    out = oracle.finalize(down, oracle.F32, restore, w, oracle.F32, oracle.F32)
    ref, mag = f64_reference(down, restore, w)
    gamma = K * U / (1 - K * U)
    assert np.all(np.abs(out.astype(np.float64) - ref) <= gamma * mag + 1e-300)


@pytest.mark.parametrize("T,K,H", [(7, 2, 64), (50, 8, 96)])
def test_bf16_within_bound(oracle, T, K, H):
    down, w, restore = _case(T, K, H, 99 + T, "bf16", "f32")
    down_b = oracle.f32_to_bf16(down)
    down_bf = oracle.bf16_to_f32(down_b)
    out = oracle.finalize(down_b, oracle.BF16, restore, w, oracle.F32, oracle.BF16)
    got = oracle.bf16_to_f32(out).astype(np.float64)
    ref, mag = f64_reference(down_bf, restore, w)
    gamma = K * U / (1 - K * U)
    # fp32 chain error, then one bf16 rounding (at most half a bf16 ulp, i.e.
    # 2^-8 of the value, relative)
    bound = gamma * mag + (np.abs(ref) + gamma * mag) * 2.0 ** -8
    assert np.all(np.abs(got - ref) <= bound)


def test_bf16_weights_widen_exactly(oracle):
    down, w, restore = _case(9, 4, 32, 3, "f32", "bf16")
    wb = oracle.f32_to_bf16(w)
    a = oracle.finalize(down, oracle.F32, restore, wb, oracle.BF16, oracle.F32)
    b = oracle.finalize(down, oracle.F32, restore, oracle.bf16_to_f32(wb), oracle.F32, oracle.F32)
    assert np.array_equal(a, b)


def test_k1_unit_weight_is_gather(oracle):
    T, H = 40, 48
    rng = np.random.default_rng(1)
    down = rng.standard_normal((T, H)).astype(np.float32)
    restore = rng.permutation(T).astype(np.uint32)
    out = oracle.finalize(down, oracle.F32, restore, np.ones((T, 1), np.float32), oracle.F32,
                          oracle.F32)
    assert np.array_equal(out, down[restore.astype(np.int64)])


def test_one_hot_weights_gather(oracle):
    T, K, H = 30, 4, 16
    rng = np.random.default_rng(2)
    down = rng.standard_normal((T * K, H)).astype(np.float32)
    restore = rng.permutation(T * K).astype(np.uint32)
    pick = rng.integers(0, K, T)
    w = np.zeros((T, K), np.float32)
    w[np.arange(T), pick] = 1.0
    out = oracle.finalize(down, oracle.F32, restore, w, oracle.F32, oracle.F32)
    exp = down[restore.astype(np.int64).reshape(T, K)[np.arange(T), pick]]
    assert np.array_equal(out, exp)


def test_identity_restore_is_weighted_row_sum(oracle):
    T, K, H = 12, 3, 20
    rng = np.random.default_rng(3)
    down = rng.standard_normal((T * K, H)).astype(np.float32)
    w = rng.random((T, K)).astype(np.float32)
    out = oracle.finalize(down, oracle.F32, np.arange(T * K, dtype=np.uint32), w, oracle.F32,
                          oracle.F32)
    ref = np.einsum("tk,tkh->th", w.astype(np.float64),
                    down.astype(np.float64).reshape(T, K, H))
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-6)


def test_empty(oracle):
    out = oracle.finalize(np.zeros((0, 16), np.float32), oracle.F32, np.zeros(0, np.uint32),
                          np.zeros((0, 2), np.float32), oracle.F32, oracle.F32)
    assert out.shape == (0, 16)


def test_hand_worked_fixture(oracle, golden_dir):
    with open(os.path.join(golden_dir, "finalize_worked_example.json")) as f:
        fx = json.load(f)
    out = oracle.finalize(np.array(fx["down"], np.float32), oracle.F32,
                          np.array(fx["restore_order"], np.uint32),
                          np.array(fx["router_weight"], np.float32), oracle.F32, oracle.F32)
    assert out.tolist() == fx["output_f32"]
    oc = fx["order_case"]
    out = oracle.finalize(np.array(oc["down"], np.float32), oracle.F32,
                          np.array(oc["restore_order"], np.uint32),
                          np.array(oc["router_weight"], np.float32), oracle.F32, oracle.F32)
    assert out.tolist() == oc["output_f32"]
    fc = fx["fma_case"]
    out = oracle.finalize(np.array(fc["down"], np.float32), oracle.F32,
                          np.array(fc["restore_order"], np.uint32),
                          np.array(fc["router_weight"], np.float32), oracle.F32, oracle.F32)
    assert out.tolist() == fc["output_f32"]
    bc = fx["bf16_rounding_case"]
    out = oracle.finalize(np.array(bc["down"], np.float32), oracle.F32,
                          np.array(bc["restore_order"], np.uint32),
                          np.array(bc["router_weight"], np.float32), oracle.F32, oracle.BF16)
    assert oracle.bf16_to_f32(out).tolist() == bc["output_bf16_as_f32"]


def test_bf16_rounding_matches_torch(oracle):
    # all 2^16 high halves, each with the low halves that probe the rounding
    # boundary: exact, just below half, half (tie), just above half, max.
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).reshape(-1)
    x = bits.view(np.float32)
    got = oracle.f32_to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(oracle.bf16_to_f32(got[nan])))


def test_rejects_bad_restore(oracle):
    with pytest.raises(ValueError):
        oracle.finalize(np.zeros((2, 8), np.float32), oracle.F32, np.array([0, 2], np.uint32),
                        np.ones((1, 2), np.float32), oracle.F32, oracle.F32)
