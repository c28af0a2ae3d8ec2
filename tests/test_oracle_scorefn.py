"""Pins of the oracle's score functions (router page, Parameters:
scores_input_fn). The scores are recovered through the router itself: with
one group, K = E, no normalisation and scale 1, slot k's weight is exactly
the score of the expert in slot k.

Checked against torch's float64 sigmoid / softmax rounded to float32 (at
most one float32 ulp apart, almost always equal: both are binary64
evaluations rounded once), exact special values, and the softmax
normalisation."""
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
