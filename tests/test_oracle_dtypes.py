"""Pins of the oracle's 16-bit float handling (the pages leave scores_type,
bias_type, down_type, weight_type and out_type generic).

binary16 conversions are checked against numpy's float16 casts on every
binary16 value and on binary32 values around each rounding boundary; the
router and finalize on 16-bit data are checked against the already-pinned
fp32 paths on the exactly widened inputs."""
import numpy as np
import pytest

from permutation_group_limited_amd import workloads as wl

U = 2.0 ** -24


def test_f16_widening_matches_numpy(oracle):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.all(np.isnan(got[nan]))


def test_f16_rounding_matches_numpy(oracle):
    # every high half, with low halves straddling the binary16 rounding bit
    # (bit 12 of the binary32 word) and the subnormal range
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x3000, 0x7FFF, 0x8000,
                     0xFFFF], dtype=np.uint32)
    x = (hi[:, None] | lows[None, :]).reshape(-1).view(np.float32)
    got = oracle.f32_to_f16(x)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(got[nan].view(np.float16)))


def test_f16_values_and_midpoints(oracle):
    # every binary16 value is its own rounding (widen, then narrow), and every
    # midpoint between neighbours, max finite to infinity included, rounds as
    # numpy does (ties to even)
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    fin = np.isfinite(v)
    wide = oracle.f16_to_f32(bits[fin])
    assert np.array_equal(oracle.f32_to_f16(wide), bits[fin])
    pos = np.sort(v[fin & (v >= 0)].astype(np.float64))
    nxt = np.append(pos[1:], 65536.0)  # the next value above 65504 is infinity's threshold
    mids = ((pos + nxt) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos + nxt) / 2)  # exact in binary32
    with np.errstate(over="ignore"):
        ref = mids.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f32_to_f16(mids), ref)
    assert np.array_equal(oracle.f32_to_f16(-mids), ref | 0x8000)


@pytest.mark.parametrize("sd,bd", [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16"),
                                   ("f16", "f32")])
def test_router_16bit_equals_fp32_on_widened_values(oracle, sd, bd):
    code = {"f32": oracle.F32, "bf16": oracle.BF16, "f16": oracle.F16}
    T, E, G, TG, K = 200, 64, 8, 3, 6
    s32 = wl.random_scores(T, E, seed=3, levels=0).numpy()
    b32 = wl.random_bias(E, seed=4, std=0.05).numpy()
    s16 = oracle.from_f32(s32, code[sd])
    b16 = oracle.from_f32(b32, code[bd])
    idx, w = oracle.router(s16, b16, K, G, TG, True, 2.5, scores_dtype=code[sd],
                           bias_dtype=code[bd] if bd != "f32" else None)
    idx_ref, w_ref = oracle.router(oracle.to_f32(s16, code[sd]), oracle.to_f32(b16, code[bd]),
                                   K, G, TG, True, 2.5)
    assert np.array_equal(idx, idx_ref)
    assert np.array_equal(w, oracle.from_f32(w_ref, code[sd]))


@pytest.mark.parametrize("dd,wd,od", [("f16", "f32", "f16"), ("f16", "f16", "f32"),
                                      ("bf16", "f16", "f16"), ("f32", "f16", "bf16")])
def test_finalize_16bit_within_bound(oracle, dd, wd, od):
    code = {"f32": oracle.F32, "bf16": oracle.BF16, "f16": oracle.F16}
    T, K, H = 40, 5, 48
    rng = np.random.default_rng(7)
    down = oracle.from_f32(rng.standard_normal((T * K, H)).astype(np.float32), code[dd])
    w = oracle.from_f32((rng.random((T, K)) * 2).astype(np.float32), code[wd])
    restore = rng.permutation(T * K).astype(np.uint32)
    out = oracle.finalize(down, code[dd], restore, w, code[wd], code[od])
    got = oracle.to_f32(out, code[od]).astype(np.float64)
    d = oracle.to_f32(down, code[dd]).astype(np.float64)[restore.astype(np.int64)].reshape(T, K, H)
    terms = oracle.to_f32(w, code[wd]).astype(np.float64)[:, :, None] * d
    ref, mag = terms.sum(1), np.abs(terms).sum(1)
    rel = {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}[od]
    bound = K * U * mag + (np.abs(ref) + K * U * mag) * rel + 2.0 ** -24
    assert np.all(np.abs(got - ref) <= bound)
