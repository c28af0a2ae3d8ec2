"""CPU oracle for the group-limited MoE routing data path (ctypes wrapper).

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package. The
product (``permutation_group_limited_amd``) never imports it, and the two
share no code: the oracle is plain C in ``moe_oracle.c``, compiled with gcc
(``-O2 -ffp-contract=off``, OpenMP across tokens only), and takes host numpy
arrays.

Conventions of this wrapper:
  * bf16 and fp16 arrays are passed and returned as ``numpy.uint16`` bit
    patterns, with a dtype code (BF16 or F16) saying which;
  * fp32 arrays as ``numpy.float32``; index arrays as int32 / uint32.

Each function names the page passage it follows; the C file holds the
step-by-step definitions and the readings of the pages' silent points.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

F32 = 0
BF16 = 1
F16 = 2
GROUP_TOP2_SUM = 0
GROUP_MAX = 1
SCORE_LOAD = 0
SCORE_SIGMOID = 1
SCORE_SOFTMAX = 2
_ERRORS = {1: "invalid argument", 2: "input violates a precondition", 3: "out of memory"}

_lib = None


def _lib_path() -> str:
    # MOE_ORACLE_LIB points the wrapper at another build of moe_oracle.c; the
    # mutation tests use it to check that the pins catch planted mistakes.
    return os.environ.get("MOE_ORACLE_LIB", _LIB_PATH)


def build(force: bool = True) -> str:
    """Compile ``moe_oracle.c`` into ``libmoe_oracle.so`` with gcc."""
    global _lib
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        path = _lib_path()
        if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.moe_oracle_router.argtypes = [p, p, p, p, i32, i32, i64, i32, i32, i32, i32, i32,
                                          ctypes.c_float, i32, i32]
        lib.moe_oracle_router.restype = ctypes.c_int
        lib.moe_oracle_create_indices.argtypes = [p, p, p, p, p, p, i64, i32]
        lib.moe_oracle_create_indices.restype = ctypes.c_int
        lib.moe_oracle_scale_offsets.argtypes = [p, p, i64, i32, ctypes.c_uint32]
        lib.moe_oracle_scale_offsets.restype = ctypes.c_int
        lib.moe_oracle_finalize.argtypes = [p, i32, p, i32, p, p, i32, i64, i32, i64]
        lib.moe_oracle_finalize.restype = ctypes.c_int
        for fn in ("moe_oracle_f32_to_bf16_array", "moe_oracle_f32_to_f16_array",
                   "moe_oracle_f16_to_f32_array"):
            getattr(lib, fn).argtypes = [p, p, i64]
            getattr(lib, fn).restype = None
        lib.moe_oracle_num_threads.argtypes = []
        lib.moe_oracle_num_threads.restype = ctypes.c_int
        lib.moe_oracle_exp.argtypes = [ctypes.c_double]
        lib.moe_oracle_exp.restype = ctypes.c_double
        lib.moe_oracle_pairwise_sum.argtypes = [p, i64]
        lib.moe_oracle_pairwise_sum.restype = ctypes.c_double
        lib.moe_oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.moe_oracle_set_num_threads.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s: %s" % (what, _ERRORS.get(rc, "error %d" % rc)))


def set_num_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on (results do not
    depend on it: the loops split whole tokens or chunks)."""
    _load().moe_oracle_set_num_threads(int(n))


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().moe_oracle_num_threads())


def _encoded(a, dtype):
    """(contiguous array, dtype code): float32 arrays are F32; uint16 bit
    patterns need an explicit BF16 or F16 code."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        assert dtype in (None, F32)
        return a, F32
    assert a.dtype == np.uint16 and dtype in (BF16, F16), "uint16 data needs BF16 or F16"
    return a, dtype


def router(scores, bias, k: int, n_groups: int, topk_group: int, norm_weights: bool,
           routed_scaling_factor: float, group_score: int = GROUP_TOP2_SUM,
           scores_dtype=None, bias_dtype=None, score_fn: int = SCORE_LOAD):
    """Group-limited top-k router (group_limited_router_kernel page, description,
    Parameters and Args). With score_fn SCORE_SIGMOID or SCORE_SOFTMAX the
    `scores` argument holds logits and the scores are computed from them
    (Parameters: scores_input_fn). Returns (expert_indices int32 [T, K],
    expert_weights [T, K] in the scores' dtype)."""
    s, sd = _encoded(scores, scores_dtype)
    b, bd = _encoded(bias, bias_dtype)
    T, E = s.shape
    assert b.shape == (E,)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32 if sd == F32 else np.uint16)
    rc = _load().moe_oracle_router(_ptr(idx), _ptr(w), _ptr(s), _ptr(b), sd, bd, T, E, k,
                                   n_groups, topk_group, int(bool(norm_weights)),
                                   ctypes.c_float(routed_scaling_factor), group_score, score_fn)
    _check(rc, "router")
    return idx, w


def create_indices(topk_ids, n_experts: int):
    """Bucket sort of routed slots by expert (moe_create_indices page, description
    and Args). Returns a dict with token_expert_order, expert_start_indices,
    restore_token_order (uint32), expert_ids (int32), expert_usage_stats (uint32)."""
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32).reshape(-1)
    n = ids.shape[0]
    out = {
        "token_expert_order": np.empty(n, dtype=np.uint32),
        "expert_start_indices": np.empty(n_experts + 1, dtype=np.uint32),
        "restore_token_order": np.empty(n, dtype=np.uint32),
        "expert_ids": np.empty(n_experts, dtype=np.int32),
        "expert_usage_stats": np.empty(2, dtype=np.uint32),
    }
    rc = _load().moe_oracle_create_indices(
        _ptr(out["token_expert_order"]), _ptr(out["expert_start_indices"]),
        _ptr(out["restore_token_order"]), _ptr(out["expert_ids"]),
        _ptr(out["expert_usage_stats"]), _ptr(ids), n, n_experts)
    _check(rc, "create_indices")
    return out


def scale_offsets(topk_ids, n_experts: int, align: int) -> np.ndarray:
    """Aligned scale offsets [E + 1] uint32 (moe_create_indices page, Args:
    scales_offset_p; TokenFormat page, pad_expert_offsets): start of each
    active expert's scale rows when every active expert's row count is
    rounded up to a multiple of `align`."""
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32).reshape(-1)
    out = np.empty(n_experts + 1, dtype=np.uint32)
    rc = _load().moe_oracle_scale_offsets(_ptr(out), _ptr(ids), ids.shape[0], n_experts, align)
    _check(rc, "scale_offsets")
    return out


def finalize(down, down_dtype: int, restore_order, router_weight, weight_dtype: int,
             out_dtype: int):
    """Fused unpermute gather plus weighted top-k sum (moe_finalize page,
    description and Args). ``down`` is [T*K, H] and ``router_weight`` [T, K]
    (float32, or uint16 bit patterns for BF16 / F16). Returns [T, H] as float32
    or uint16 bit patterns."""
    d = np.ascontiguousarray(down)
    w = np.ascontiguousarray(router_weight)
    r = np.ascontiguousarray(restore_order, dtype=np.uint32).reshape(-1)
    assert d.dtype == (np.float32 if down_dtype == F32 else np.uint16)
    assert w.dtype == (np.float32 if weight_dtype == F32 else np.uint16)
    T, K = w.shape
    N, H = d.shape
    assert N == T * K and r.shape[0] == N
    out = np.empty((T, H), dtype=np.float32 if out_dtype == F32 else np.uint16)
    rc = _load().moe_oracle_finalize(_ptr(out), out_dtype, _ptr(d), down_dtype, _ptr(r), _ptr(w),
                                     weight_dtype, T, K, H)
    _check(rc, "finalize")
    return out


def exp(x: float) -> float:
    """The score functions' binary64 exponential (one value)."""
    return float(_load().moe_oracle_exp(float(x)))


def pairwise_sum(v) -> float:
    """The softmax denominator's binary64 pairwise sum of v, in index order."""
    a = np.ascontiguousarray(v, dtype=np.float64)
    return float(_load().moe_oracle_pairwise_sum(_ptr(a), a.size))


def f32_to_bf16(x) -> np.ndarray:
    """Round binary32 values to bf16 (nearest, ties to even); uint16 bits."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().moe_oracle_f32_to_bf16_array(_ptr(out), _ptr(a), a.size)
    return out


def bf16_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_f16(x) -> np.ndarray:
    """Round binary32 values to binary16 (nearest, ties to even); uint16 bits."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().moe_oracle_f32_to_f16_array(_ptr(out), _ptr(a), a.size)
    return out


def f16_to_f32(bits) -> np.ndarray:
    """Widen binary16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    _load().moe_oracle_f16_to_f32_array(_ptr(out), _ptr(b), b.size)
    return out


def to_f32(bits, dtype: int) -> np.ndarray:
    """Widen an array in dtype code `dtype` to float32."""
    if dtype == F32:
        return np.ascontiguousarray(bits, dtype=np.float32)
    return bf16_to_f32(bits) if dtype == BF16 else f16_to_f32(bits)


def from_f32(x, dtype: int) -> np.ndarray:
    """Round float32 values to dtype code `dtype` (bit patterns for 16-bit)."""
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    return f32_to_bf16(x) if dtype == BF16 else f32_to_f16(x)
