"""Helpers shared by the GPU parity tests: run one stage of the HIP library
through the C ABI on host inputs, and the acceptance comparisons.

Acceptance:
  * expert indices, token_expert_order, restore_token_order,
    expert_start_indices, expert_ids, expert_usage_stats: bit-exact;
  * router weights: bit-exact (both sides normalise and scale in binary64
    and round once; the required bound, 1e-6 relative, is reported beside
    a mismatch);
  * finalize, every output dtype: bit-exact. The moe_finalize page fixes
    the arithmetic (the sum held in fp32), read as one fused multiply-add
    per k in ascending k from +0 and one rounding to the output type; the
    kernels and the oracle both do exactly that. The chained pipeline feeds
    finalize the GPU's own weights, which equal the oracle's bit for bit,
    so the same bar holds there. A mismatch is reported with its size
    (ulps of the 16-bit output, or the absolute difference against
    1e-5 * sum_k |w_k * down_k| for fp32).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from permutation_group_limited_amd import binding

DEV = "cuda:0"


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np_u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int32).numpy().view(np.uint32)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """16-bit float tensor (bf16 or fp16) -> uint16 bit patterns."""
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_code(dtype) -> int:
    return {torch.float32: oracle.F32, torch.bfloat16: oracle.BF16,
            torch.float16: oracle.F16}[dtype]


def encode(t: torch.Tensor):
    """Host tensor -> (numpy array for the oracle, dtype code)."""
    if t.dtype == torch.float32:
        return t.contiguous().numpy(), oracle.F32
    return bf16_bits(t), oracle_code(t.dtype)


def gpu_router(scores, bias, K, G, TG, norm, scale, mode=0):
    """Router on the GPU; weights come back as a host tensor in the scores'
    dtype (numpy float32 for fp32 scores)."""
    T, E = scores.shape
    s = scores.to(DEV)
    b = bias.to(DEV)
    idx = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, K), float("nan"), dtype=scores.dtype, device=DEV)
    binding.moe_router_group_limited(idx, w, s, b, G, TG, norm, scale, mode)
    torch.cuda.synchronize()
    wh = w.cpu()
    return idx.cpu().numpy(), (wh.numpy() if wh.dtype == torch.float32 else wh)


def gpu_indices(ids, E, poison=True):
    ids = torch.as_tensor(ids).reshape(-1).to(torch.int32)
    n = ids.numel()
    d = ids.to(DEV)
    fill = 0x5A5A5A5A if poison else 0
    order = torch.full((n,), fill, dtype=torch.int32, device=DEV)
    restore = torch.full((n,), fill, dtype=torch.int32, device=DEV)
    starts = torch.full((E + 1,), fill, dtype=torch.int32, device=DEV)
    eids = torch.full((E,), fill, dtype=torch.int32, device=DEV)
    stats = torch.full((2,), fill, dtype=torch.int32, device=DEV)
    ws_bytes = binding.moe_create_indices_workspace_size(n, E)
    ws = torch.full((max(ws_bytes, 4) // 4,), fill, dtype=torch.int32, device=DEV)
    binding.moe_create_indices(order, starts, restore, eids, stats, d, ws)
    torch.cuda.synchronize()
    return {
        "token_expert_order": to_np_u32(order),
        "expert_start_indices": to_np_u32(starts),
        "restore_token_order": to_np_u32(restore),
        "expert_ids": eids.cpu().numpy(),
        "expert_usage_stats": to_np_u32(stats),
    }


def gpu_finalize(down_dev, restore, weight, out_dtype):
    T, K = weight.shape
    H = down_dev.shape[1]
    r = torch.as_tensor(np.asarray(restore, dtype=np.uint32).view(np.int32)).to(DEV)
    w = weight.to(DEV)
    out = torch.full((T, H), float("nan"), dtype=out_dtype, device=DEV)
    binding.moe_finalize(out, down_dev, r, w)
    torch.cuda.synchronize()
    return out


def oracle_finalize_from(down_host, restore, weight, out_dtype):
    """Oracle finalize on host tensors (float32, bfloat16 or float16)."""
    d, dd = encode(down_host)
    w, wd = encode(weight)
    return oracle.finalize(d, dd, np.asarray(restore, dtype=np.uint32), w, wd,
                           oracle_code(out_dtype))


def term_magnitude(down_host, restore, weight):
    """sum_k |w_k * down[restore[t*K+k]]| in float64, [T, H]."""
    T, K = weight.shape
    d = down_host.to(torch.float64)
    rows = d[torch.as_tensor(np.asarray(restore, dtype=np.int64))].reshape(T, K, -1)
    return (weight.to(torch.float64).abs()[:, :, None] * rows.abs()).sum(1).numpy()


def assert_indices_equal(got, exp):
    for key in ("token_expert_order", "expert_start_indices", "restore_token_order",
                "expert_ids", "expert_usage_stats"):
        g, e = np.asarray(got[key]), np.asarray(exp[key])
        if not np.array_equal(g, e):
            bad = np.nonzero(g.reshape(-1) != e.reshape(-1))[0]
            raise AssertionError("%s differs at %d places, first %s: gpu %s oracle %s"
                                 % (key, bad.size, bad[:5], g.reshape(-1)[bad[:5]],
                                    e.reshape(-1)[bad[:5]]))


def assert_weights_equal(got, exp):
    """Router weights bit for bit: float32 arrays, or 16-bit patterns
    (uint16) for bf16 / fp16 weights."""
    got, exp = np.asarray(got), np.asarray(exp)
    assert got.shape == exp.shape, (got.shape, exp.shape)
    if exp.dtype == np.uint16:
        gb, eb = got.astype(np.uint16), exp
    else:
        gb = got.astype(np.float32).view(np.uint32)
        eb = exp.astype(np.float32).view(np.uint32)
    bad = gb != eb
    if bad.any():
        i = np.argwhere(bad)[:5]
        msg = "router weights differ from the oracle at %d places, first %s" % (
            int(bad.sum()), i.tolist())
        if exp.dtype != np.uint16:
            g64, e64 = got.astype(np.float64), exp.astype(np.float64)
            msg += "; within 1e-6 relative: %s" % bool(
                np.all(np.abs(g64 - e64) <= 1e-6 * np.abs(e64)))
        raise AssertionError(msg)


def _bf16_ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_finalize_equal(got_dev, exp_np, mag=None):
    """Finalize acceptance: the output equals the oracle's bit for bit. On a
    mismatch the message gives its size: ulps for 16-bit outputs, for fp32
    the absolute difference and whether it stays within 1e-5 of the term
    magnitude `mag` (when given)."""
    if got_dev.dtype in (torch.bfloat16, torch.float16):
        gb, eb = bf16_bits(got_dev), np.asarray(exp_np, np.uint16)
        bad = gb != eb
        if bad.any():
            diff = np.abs(_bf16_ordered(gb) - _bf16_ordered(eb))
            i = np.argwhere(bad)[:5]
            raise AssertionError("16-bit output differs from the oracle at %d places (largest "
                                 "%d ulp), first %s" % (int(bad.sum()), int(diff.max()),
                                                        i.tolist()))
        return 0
    g = got_dev.cpu().numpy()
    e = np.asarray(exp_np, np.float32)
    bad = g.view(np.uint32) != e.view(np.uint32)
    if bad.any():
        err = np.abs(g.astype(np.float64) - e.astype(np.float64))
        i = np.argwhere(bad)[:5]
        msg = ("fp32 output differs from the oracle at %d places (largest %g), first %s"
               % (int(bad.sum()), float(err[bad].max()), i.tolist()))
        if mag is not None:
            msg += "; within 1e-5 of the term magnitude: %s" % bool(np.all(err <= 1e-5 * mag))
        raise AssertionError(msg)
    return 0


def assert_finalize_matches_in_blocks(got_dev, down_dev, restore, weight, out_dtype,
                                      block_tokens=4096):
    """Every output row of a finalize launch against the oracle, token block
    by token block: output row t depends only on its own K rows of `down`,
    so each block's rows are gathered on the device (in restore order),
    copied to the host and fed to the oracle with an identity restore. This
    compares the whole output of problems whose `down` is too large to
    hand to the oracle at once, bit for bit."""
    T, K = weight.shape
    rest = np.asarray(restore, dtype=np.uint32).reshape(T, K)
    worst = 0
    for t0 in range(0, T, block_tokens):
        t1 = min(T, t0 + block_tokens)
        rows = torch.from_numpy(rest[t0:t1].reshape(-1).astype(np.int64)).to(down_dev.device)
        sub_down = down_dev[rows].cpu()
        ident = np.arange((t1 - t0) * K, dtype=np.uint32)
        sub_w = weight[t0:t1]
        exp = oracle_finalize_from(sub_down, ident, sub_w, out_dtype)
        mag = term_magnitude(sub_down, ident, sub_w) if out_dtype == torch.float32 else None
        d = assert_finalize_equal(got_dev[t0:t1], exp, mag)
        worst = max(worst, d)
        del sub_down, rows
    return worst
