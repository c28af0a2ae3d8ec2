"""Pins of the oracle's score functions (router page, Parameters:
scores_input_fn). The scores are recovered through the router itself: with
one group, K = E, no normalisation and scale 1, slot k's weight is exactly
the score of the expert in slot k.

Checked against torch's float64 sigmoid / softmax rounded to float32 (at
most one float32 ulp apart, almost always equal: both are binary64
evaluations rounded once), exact special values, and the softmax
normalisation. The two primitives they are built from are pinned on their
own: the binary64 exponential against a correctly rounded exp (decimal
arithmetic at 60 digits), the pairwise sum against hand-worked sums whose
value depends on the order of the additions and against exact sums."""
import math
import os
import random
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

F32 = np.float32


def oracle_scores(oracle, logits, fn):
    T, E = logits.shape
    idx, w = oracle.router(logits.astype(F32), np.zeros(E, F32), E, 1, 1, False, 1.0,
                           score_fn=fn)
    s = np.empty_like(w)
    np.put_along_axis(s, idx.astype(np.int64), w, axis=1)
    return s


def ulp_distance(a, b):
    ia = a.astype(F32).view(np.int32).astype(np.int64)
    ib = b.astype(F32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def test_sigmoid_matches_float64_reference(oracle):
    g = torch.Generator().manual_seed(1)
    x = (torch.randn(512, 64, generator=g, dtype=torch.float64) * 6).to(torch.float32)
    got = oracle_scores(oracle, x.numpy(), oracle.SCORE_SIGMOID)
    ref = torch.sigmoid(x.to(torch.float64)).to(torch.float32).numpy()
    d = ulp_distance(got, ref)
    assert d.max() <= 1 and np.mean(d == 0) > 0.9999


def test_softmax_matches_float64_reference(oracle):
    g = torch.Generator().manual_seed(2)
    x = (torch.randn(512, 32, generator=g, dtype=torch.float64) * 4).to(torch.float32)
    got = oracle_scores(oracle, x.numpy(), oracle.SCORE_SOFTMAX)
    ref = torch.softmax(x.to(torch.float64), dim=1).to(torch.float32).numpy()
    d = ulp_distance(got, ref)
    assert d.max() <= 1 and np.mean(d == 0) > 0.999
    np.testing.assert_allclose(got.astype(np.float64).sum(1), 1.0, rtol=1e-6)


def test_special_values(oracle):
    x = np.array([[0.0, 200.0, -200.0, 0.0]], F32)
    s = oracle_scores(oracle, x, oracle.SCORE_SIGMOID)
    assert s[0, 0] == 0.5 and s[0, 1] == 1.0 and 0.0 <= s[0, 2] < 1e-40
    # equal logits: exactly 1/E for a power of two E
    s = oracle_scores(oracle, np.full((3, 8), 1.25, F32), oracle.SCORE_SOFTMAX)
    assert np.all(s == F32(0.125))
    # one dominant logit: one-hot
    x = np.zeros((1, 4), F32)
    x[0, 2] = 1000.0
    s = oracle_scores(oracle, x, oracle.SCORE_SOFTMAX)
    assert s.tolist() == [[0.0, 0.0, 1.0, 0.0]]


@pytest.mark.parametrize("fn", ["sigmoid", "softmax"])
def test_routing_on_logits_equals_routing_on_scores(oracle, fn):
    # the score function is a loader: routing from logits is routing on the
    # scores it produces
    code = oracle.SCORE_SIGMOID if fn == "sigmoid" else oracle.SCORE_SOFTMAX
    g = torch.Generator().manual_seed(3)
    x = torch.randn(300, 64, generator=g).numpy()
    bias = (torch.randn(64, generator=g) * 0.05).numpy()
    s = oracle_scores(oracle, x, code)
    a = oracle.router(x, bias, 6, 8, 3, True, 2.5, score_fn=code)
    b = oracle.router(s, bias, 6, 8, 3, True, 2.5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _ulps64(a, b):
    ia = struct.unpack("<q", struct.pack("<d", a))[0]
    ib = struct.unpack("<q", struct.pack("<d", b))[0]
    return abs(ia - ib)


def _correctly_rounded_exp(x):
    getcontext().prec = 60
    return float(Fraction(Decimal(x).exp()))


def test_exp_against_correctly_rounded(oracle):
    # within one binary64 ulp everywhere, and correctly rounded on most
    # arguments (a Taylor series one term short, or a reduction without
    # the low part of ln 2, falls below this)
    rng = random.Random(11)
    xs = ([rng.uniform(-745.0, 709.7) for _ in range(1500)]
          + [rng.uniform(-30.0, 0.0) for _ in range(1500)]
          + [rng.uniform(-0.6, 0.6) for _ in range(1000)])
    d = []
    for x in xs:
        ref = _correctly_rounded_exp(x)
        if ref < 2.2250738585072014e-308:  # subnormal results: not compared in ulps
            continue
        d.append(_ulps64(oracle.exp(x), ref))
    d = np.array(d)
    assert d.max() <= 1
    assert np.mean(d == 0) >= 0.92


def test_exp_special_values(oracle):
    assert oracle.exp(0.0) == 1.0 and oracle.exp(-0.0) == 1.0
    assert oracle.exp(1.0) == math.e  # e rounded to nearest
    assert oracle.exp(-746.0) == 0.0 and oracle.exp(-1e300) == 0.0
    assert oracle.exp(710.0) == math.inf and oracle.exp(1e300) == math.inf
    assert math.isnan(oracle.exp(math.nan))
    # results in the subnormal range: within one ulp of the correct value
    for x in (-709.0, -720.5, -740.0, -745.0):
        ref = _correctly_rounded_exp(x)
        assert abs(oracle.exp(x) - ref) <= 5e-324 * 1.0 + abs(ref) * 2.0 ** -52


def test_pairwise_sum_order(oracle):
    u = 2.0 ** -53  # half an ulp of 1
    # left to right: 1 + 0 = 1, 1 + u = 1 (tie to even), 1 + u = 1;
    # pairwise: (1 + 0) + (u + u) = 1 + 2u, which is representable
    assert oracle.pairwise_sum([1.0, 0.0, u, u]) == 1.0 + 2 * u
    # padding to 8: ((1 + 0) + (0 + 0)) + ((u + u) + (0 + 0)) = 1 + 2u
    assert oracle.pairwise_sum([1.0, 0.0, 0.0, 0.0, u, u]) == 1.0 + 2 * u
    # (1 + u) + (u + 0): both halves round the tie to even, 1
    assert oracle.pairwise_sum([1.0, u, u]) == 1.0
    # (u + u) + (1 + u) = 2u + 1 (1 + u rounds to 1 first)
    assert oracle.pairwise_sum([u, u, 1.0, u]) == 1.0 + 2 * u
    assert oracle.pairwise_sum([3.5]) == 3.5


def test_pairwise_sum_exact_and_bounded(oracle):
    rng = np.random.default_rng(12)
    for n in (1, 2, 3, 7, 8, 64, 160, 256, 1000, 1024):
        ints = rng.integers(0, 1000, n).astype(np.float64)
        assert oracle.pairwise_sum(ints) == float(ints.sum())  # exact either way
        v = rng.random(n)
        bound = max(1, math.ceil(math.log2(n))) * 2.0 ** -53 * float(np.abs(v).sum())
        assert abs(oracle.pairwise_sum(v) - math.fsum(v)) <= bound


def sum_order_rows():
    """Rows of tests/golden/softmax_sum_order_logits.txt: (E, flipping
    expert, float32 logits [1, E])."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "softmax_sum_order_logits.txt")
    rows = []
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        E, flip = int(f[0]), int(f[1])
        x = np.array([float.fromhex(v) for v in f[2:]], dtype=F32).reshape(1, E)
        assert x.shape[1] == E
        rows.append((E, flip, x))
    return rows


def _softmax_from_primitives(oracle, row):
    m = float(max(float(v) for v in row))
    ex = [oracle.exp(float(v) - m) for v in row]
    den = oracle.pairwise_sum(ex)
    return ex, np.array([e / den for e in ex], dtype=np.float64).astype(F32)


def test_softmax_built_from_the_pinned_primitives(oracle):
    # the score function is exp of the max-shifted logits over their
    # pairwise sum, rounded once to binary32
    g = torch.Generator().manual_seed(13)
    x = (torch.randn(40, 24, generator=g) * 5).numpy().astype(F32)
    got = oracle_scores(oracle, x, oracle.SCORE_SOFTMAX)
    for t in range(x.shape[0]):
        _, exp_row = _softmax_from_primitives(oracle, x[t])
        assert np.array_equal(got[t].view(np.uint32), exp_row.view(np.uint32))


@pytest.mark.parametrize("row", [0, 1])
def test_softmax_sum_order_rows(oracle, row):
    # inputs on which another order of the denominator's additions changes a
    # binary32 score: the oracle must give the pairwise-order scores
    E, flip, x = sum_order_rows()[row]
    got = oracle_scores(oracle, x, oracle.SCORE_SOFTMAX)[0]
    ex, exp_row = _softmax_from_primitives(oracle, x[0])
    assert np.array_equal(got.view(np.uint32), exp_row.view(np.uint32))
    # the row still separates the orders it was chosen for
    if E == 4:
        other = 0.0
        for e in ex:
            other += e
    else:
        blocks = [sum_left_to_right(ex[i:i + 4]) for i in range(0, E, 4)]
        other = oracle.pairwise_sum(blocks)
    assert F32(ex[flip] / other) != exp_row[flip]


def sum_left_to_right(v):
    s = 0.0
    for e in v:
        s += e
    return s
    got = oracle_scores(oracle, x, oracle.SCORE_SIGMOID)
    ref = np.array([[1.0 / (1.0 + oracle.exp(-float(v))) for v in row] for row in x]).astype(F32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
