"""ctypes binding of ``libmoe_route.so`` (C ABI in ``include/moe_route.h``).

Argument marshalling only: every step of the routing path runs in the HIP
kernels of the library. torch supplies device memory and the stream; the
library must run on torch's HIP runtime, so torch is imported before the
library is loaded and the process is checked to hold exactly one HIP
runtime. There is no fallback: if the library is missing or fails to load,
every entry point raises.

Entry points keep the C names and argument order (outputs, inputs,
scalars); shapes are taken from the tensors. ``stream`` defaults to torch's
current stream on the tensors' device.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_route.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_F16 = 2
GROUP_TOP2_SUM = 0
GROUP_MAX = 1
SCORE_NONE = 0
SCORE_SIGMOID = 1
SCORE_SOFTMAX = 2

# moe_route_and_index workspace: byte offset of the status word, and the
# value the index step stores there when the router's counts do not add up
ROUTE_INDEX_STATUS_OFFSET = 4
STATUS_COUNTS_MISMATCH = 1

_STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
           3: "MOE_ERR_ALIGNMENT", 4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_HIP"}

_lib = None


class MoeError(RuntimeError):
    """A non-zero moe_status_t from the library."""

    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = "%s returned %s" % (fn, _STATUS.get(status, str(status)))
        if status == 5:
            msg += " (hipError_t %d)" % hip_error
        super().__init__(msg)


def library_path() -> str:
    return _LIB_PATH


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    except OSError:
        return []


def load_library(check_runtime: bool = True):
    """Load the library (once). Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libmoe_route.so is not built (run __graft_entry__.build() or "
                           "python -m permutation_group_limited_amd.build)")
    lib = ctypes.CDLL(_LIB_PATH)
    if check_runtime:
        rts = _hip_runtimes_mapped()
        if len(rts) > 1:
            raise RuntimeError("two HIP runtimes are mapped (%s); torch and libmoe_route.so "
                               "must share one" % ", ".join(rts))
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.moe_router_group_limited.argtypes = [p, p, p, p, i32, i32, i64, i32, i32, i32, i32, i32,
                                             ctypes.c_float, i32, p]
    lib.moe_router_group_limited.restype = ctypes.c_int
    lib.moe_router_group_limited_logits.argtypes = [p, p, p, p, i32, i32, i32, i64, i32, i32,
                                                    i32, i32, i32, ctypes.c_float, i32, p]
    lib.moe_router_group_limited_logits.restype = ctypes.c_int
    lib.moe_create_indices_workspace_size.argtypes = [i64, i32]
    lib.moe_create_indices_workspace_size.restype = ctypes.c_size_t
    lib.moe_create_indices.argtypes = [p, p, p, p, p, p, i64, i32, p, ctypes.c_size_t, p, p]
    lib.moe_create_indices.restype = ctypes.c_int
    lib.moe_create_indices_aligned.argtypes = [p, p, p, p, p, p, i64, i32, p, ctypes.c_size_t, p,
                                               ctypes.c_uint32, p]
    lib.moe_create_indices_aligned.restype = ctypes.c_int
    lib.moe_create_indices_no_alloc.argtypes = [p, p, p, p, p, p, i64, i32, p]
    lib.moe_create_indices_no_alloc.restype = ctypes.c_int
    lib.moe_create_indices_no_alloc_max_scratch_bytes.argtypes = []
    lib.moe_create_indices_no_alloc_max_scratch_bytes.restype = ctypes.c_size_t
    lib.moe_route_and_index_workspace_size.argtypes = [i64, i32, i32]
    lib.moe_route_and_index_workspace_size.restype = ctypes.c_size_t
    lib.moe_route_and_index.argtypes = [p, p, p, p, p, p, p, p, ctypes.c_uint32, p, p, i32, i32,
                                        i32, i64, i32, i32, i32, i32, i32, ctypes.c_float, i32,
                                        p, ctypes.c_size_t, p]
    lib.moe_route_and_index.restype = ctypes.c_int
    lib.moe_finalize.argtypes = [p, i32, p, i32, p, p, i32, i64, i32, i64, p]
    lib.moe_finalize.restype = ctypes.c_int
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_hip_error.argtypes = []
    lib.moe_last_hip_error.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status, _lib.moe_last_hip_error() if status == 5 else 0)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float16:
        return DTYPE_F16
    raise TypeError("unsupported dtype %s (float32, bfloat16 or float16)" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, *tensors):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    dev = next((t.device for t in tensors if t is not None and t.is_cuda), None)
    if dev is None:
        raise ValueError("device tensors required")
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dev(*tensors):
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _int32_like(t, name):
    if t.dtype not in (torch.int32, torch.uint32):
        raise TypeError("%s must be int32/uint32" % name)


def moe_router_group_limited(expert_indices: torch.Tensor, expert_weights: torch.Tensor,
                             expert_scores: torch.Tensor, expert_bias: torch.Tensor,
                             n_groups: int, topk_group: int, norm_weights: bool,
                             routed_scaling_factor: float, group_score: int = GROUP_TOP2_SUM,
                             stream=None) -> None:
    """expert_indices int32 [T, K], expert_weights [T, K] (scores dtype) <-
    expert_scores [T, E], expert_bias [E]."""
    lib = load_library()
    _dev(expert_indices, expert_weights, expert_scores, expert_bias)
    T, E = expert_scores.shape
    K = expert_indices.shape[1]
    if expert_indices.dtype != torch.int32 or tuple(expert_indices.shape) != (T, K):
        raise ValueError("expert_indices must be int32 [T, K]")
    if tuple(expert_weights.shape) != (T, K) or expert_weights.dtype != expert_scores.dtype:
        raise ValueError("expert_weights must be [T, K] with the scores' dtype")
    if tuple(expert_bias.shape) != (E,):
        raise ValueError("expert_bias must be [E]")
    st = lib.moe_router_group_limited(
        _ptr(expert_indices), _ptr(expert_weights), _ptr(expert_scores), _ptr(expert_bias),
        _dtype_code(expert_scores), _dtype_code(expert_bias), T, E, K, n_groups, topk_group,
        int(bool(norm_weights)), ctypes.c_float(routed_scaling_factor), int(group_score),
        _stream(stream, expert_scores))
    _check("moe_router_group_limited", st)


def moe_router_group_limited_logits(expert_indices: torch.Tensor, expert_weights: torch.Tensor,
                                    router_logits: torch.Tensor, expert_bias: torch.Tensor,
                                    score_fn: int, n_groups: int, topk_group: int,
                                    norm_weights: bool, routed_scaling_factor: float,
                                    group_score: int = GROUP_TOP2_SUM, stream=None) -> None:
    """As moe_router_group_limited, with the scores computed from router_logits
    [T, E] by score_fn (SCORE_SIGMOID or SCORE_SOFTMAX); expert_weights take
    the logits' dtype."""
    lib = load_library()
    _dev(expert_indices, expert_weights, router_logits, expert_bias)
    T, E = router_logits.shape
    K = expert_indices.shape[1]
    if expert_indices.dtype != torch.int32 or tuple(expert_indices.shape) != (T, K):
        raise ValueError("expert_indices must be int32 [T, K]")
    if tuple(expert_weights.shape) != (T, K) or expert_weights.dtype != router_logits.dtype:
        raise ValueError("expert_weights must be [T, K] with the logits' dtype")
    if tuple(expert_bias.shape) != (E,):
        raise ValueError("expert_bias must be [E]")
    st = lib.moe_router_group_limited_logits(
        _ptr(expert_indices), _ptr(expert_weights), _ptr(router_logits), _ptr(expert_bias),
        _dtype_code(router_logits), _dtype_code(expert_bias), int(score_fn), T, E, K, n_groups,
        topk_group, int(bool(norm_weights)), ctypes.c_float(routed_scaling_factor),
        int(group_score), _stream(stream, router_logits))
    _check("moe_router_group_limited_logits", st)


def moe_create_indices_workspace_size(n: int, n_experts: int) -> int:
    """Device workspace bytes moe_create_indices needs for n slots."""
    return int(load_library().moe_create_indices_workspace_size(n, n_experts))


def moe_create_indices(token_expert_order: torch.Tensor, expert_start_indices: torch.Tensor,
                       restore_token_order: torch.Tensor, expert_ids: torch.Tensor,
                       expert_usage_stats: torch.Tensor, topk_ids: torch.Tensor,
                       workspace: torch.Tensor = None, scales_offset_p=None,
                       stream=None) -> None:
    """Bucket sort of the flat topk_ids [N] (or [T, K]) by expert. Buffers:
    token_expert_order [N], expert_start_indices [E+1], restore_token_order
    [N], expert_usage_stats [2] (uint32 or int32 storage), expert_ids [E]
    int32. workspace: a device byte buffer of at least
    moe_create_indices_workspace_size(N, E) bytes."""
    lib = load_library()
    _dev(token_expert_order, expert_start_indices, restore_token_order, expert_ids,
         expert_usage_stats, topk_ids, workspace)
    for t, name in ((token_expert_order, "token_expert_order"),
                    (expert_start_indices, "expert_start_indices"),
                    (restore_token_order, "restore_token_order"), (expert_ids, "expert_ids"),
                    (expert_usage_stats, "expert_usage_stats"), (topk_ids, "topk_ids")):
        _int32_like(t, name)
    n = topk_ids.numel()
    E = expert_ids.numel()
    if token_expert_order.numel() != n or restore_token_order.numel() != n:
        raise ValueError("token_expert_order and restore_token_order need N entries")
    if expert_start_indices.numel() != E + 1 or expert_usage_stats.numel() != 2:
        raise ValueError("expert_start_indices needs E+1 entries, expert_usage_stats 2")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.moe_create_indices(
        _ptr(token_expert_order), _ptr(expert_start_indices), _ptr(restore_token_order),
        _ptr(expert_ids), _ptr(expert_usage_stats), _ptr(topk_ids), n, E, _ptr(workspace),
        ws_bytes, scales_offset_p, _stream(stream, topk_ids, expert_ids))
    _check("moe_create_indices", st)


def moe_create_indices_no_alloc(token_expert_order: torch.Tensor,
                                expert_start_indices: torch.Tensor,
                                restore_token_order: torch.Tensor, expert_ids: torch.Tensor,
                                expert_usage_stats: torch.Tensor, topk_ids: torch.Tensor,
                                stream=None) -> None:
    """moe_create_indices without a workspace: the counts matrix lives in the
    library's own device array (for callers that cannot allocate). Calls
    that may overlap on one GPU race on that array."""
    lib = load_library()
    _dev(token_expert_order, expert_start_indices, restore_token_order, expert_ids,
         expert_usage_stats, topk_ids)
    for t, name in ((token_expert_order, "token_expert_order"),
                    (expert_start_indices, "expert_start_indices"),
                    (restore_token_order, "restore_token_order"), (expert_ids, "expert_ids"),
                    (expert_usage_stats, "expert_usage_stats"), (topk_ids, "topk_ids")):
        _int32_like(t, name)
    n = topk_ids.numel()
    E = expert_ids.numel()
    if token_expert_order.numel() != n or restore_token_order.numel() != n:
        raise ValueError("token_expert_order and restore_token_order need N entries")
    if expert_start_indices.numel() != E + 1 or expert_usage_stats.numel() != 2:
        raise ValueError("expert_start_indices needs E+1 entries, expert_usage_stats 2")
    st = lib.moe_create_indices_no_alloc(
        _ptr(token_expert_order), _ptr(expert_start_indices), _ptr(restore_token_order),
        _ptr(expert_ids), _ptr(expert_usage_stats), _ptr(topk_ids), n, E,
        _stream(stream, topk_ids, expert_ids))
    _check("moe_create_indices_no_alloc", st)


def moe_create_indices_aligned(token_expert_order: torch.Tensor,
                               expert_start_indices: torch.Tensor,
                               restore_token_order: torch.Tensor, expert_ids: torch.Tensor,
                               expert_usage_stats: torch.Tensor, topk_ids: torch.Tensor,
                               workspace: torch.Tensor, scales_offset: torch.Tensor,
                               scale_align: int, stream=None) -> None:
    """moe_create_indices plus scales_offset [E+1]: per active expert, the start
    of its scale rows with every expert's row count rounded up to scale_align."""
    lib = load_library()
    _dev(token_expert_order, expert_start_indices, restore_token_order, expert_ids,
         expert_usage_stats, topk_ids, workspace, scales_offset)
    for t, name in ((token_expert_order, "token_expert_order"),
                    (expert_start_indices, "expert_start_indices"),
                    (restore_token_order, "restore_token_order"), (expert_ids, "expert_ids"),
                    (expert_usage_stats, "expert_usage_stats"), (topk_ids, "topk_ids"),
                    (scales_offset, "scales_offset")):
        _int32_like(t, name)
    n = topk_ids.numel()
    E = expert_ids.numel()
    if token_expert_order.numel() != n or restore_token_order.numel() != n:
        raise ValueError("token_expert_order and restore_token_order need N entries")
    if expert_start_indices.numel() != E + 1 or expert_usage_stats.numel() != 2 or \
            scales_offset.numel() != E + 1:
        raise ValueError("expert_start_indices and scales_offset need E+1 entries, "
                         "expert_usage_stats 2")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.moe_create_indices_aligned(
        _ptr(token_expert_order), _ptr(expert_start_indices), _ptr(restore_token_order),
        _ptr(expert_ids), _ptr(expert_usage_stats), _ptr(topk_ids), n, E, _ptr(workspace),
        ws_bytes, _ptr(scales_offset), int(scale_align), _stream(stream, topk_ids, expert_ids))
    _check("moe_create_indices_aligned", st)


def moe_route_and_index_workspace_size(T: int, K: int, n_experts: int) -> int:
    """Device workspace bytes moe_route_and_index needs for T tokens, K slots
    per token and n_experts experts (a counter and, for batches the index
    step splits into chunks, its counts matrix)."""
    return int(load_library().moe_route_and_index_workspace_size(T, K, n_experts))


def moe_route_and_index(expert_indices: torch.Tensor, expert_weights: torch.Tensor,
                        token_expert_order: torch.Tensor, expert_start_indices: torch.Tensor,
                        restore_token_order: torch.Tensor, expert_ids: torch.Tensor,
                        expert_usage_stats: torch.Tensor, router_input: torch.Tensor,
                        expert_bias: torch.Tensor, workspace: torch.Tensor, n_groups: int,
                        topk_group: int, norm_weights: bool, routed_scaling_factor: float,
                        group_score: int = GROUP_TOP2_SUM, score_fn: int = SCORE_NONE,
                        scales_offset: torch.Tensor = None, scale_align: int = 0,
                        stream=None) -> None:
    """Router and index creation in one or two launches. router_input [T, E]
    holds scores (score_fn SCORE_NONE) or logits; the outputs are those of
    moe_router_group_limited(_logits) and moe_create_indices(_aligned).
    workspace: at least moe_route_and_index_workspace_size(T, K, E) bytes,
    zero before the first call (each call leaves it zero)."""
    lib = load_library()
    _dev(expert_indices, expert_weights, token_expert_order, expert_start_indices,
         restore_token_order, expert_ids, expert_usage_stats, router_input, expert_bias,
         workspace, scales_offset)
    T, E = router_input.shape
    K = expert_indices.shape[1]
    if expert_indices.dtype != torch.int32 or tuple(expert_indices.shape) != (T, K):
        raise ValueError("expert_indices must be int32 [T, K]")
    if tuple(expert_weights.shape) != (T, K) or expert_weights.dtype != router_input.dtype:
        raise ValueError("expert_weights must be [T, K] with the router input's dtype")
    if tuple(expert_bias.shape) != (E,):
        raise ValueError("expert_bias must be [E]")
    for t, name in ((token_expert_order, "token_expert_order"),
                    (expert_start_indices, "expert_start_indices"),
                    (restore_token_order, "restore_token_order"), (expert_ids, "expert_ids"),
                    (expert_usage_stats, "expert_usage_stats")):
        _int32_like(t, name)
    if scales_offset is not None:
        _int32_like(scales_offset, "scales_offset")
        if scales_offset.numel() != E + 1:
            raise ValueError("scales_offset needs E+1 entries")
    n = T * K
    if token_expert_order.numel() != n or restore_token_order.numel() != n:
        raise ValueError("token_expert_order and restore_token_order need T*K entries")
    if expert_start_indices.numel() != E + 1 or expert_ids.numel() != E or \
            expert_usage_stats.numel() != 2:
        raise ValueError("expert_start_indices needs E+1 entries, expert_ids E, "
                         "expert_usage_stats 2")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.moe_route_and_index(
        _ptr(expert_indices), _ptr(expert_weights), _ptr(token_expert_order),
        _ptr(expert_start_indices), _ptr(restore_token_order), _ptr(expert_ids),
        _ptr(expert_usage_stats), _ptr(scales_offset), int(scale_align), _ptr(router_input),
        _ptr(expert_bias), _dtype_code(router_input), _dtype_code(expert_bias), int(score_fn), T,
        E, K, n_groups, topk_group, int(bool(norm_weights)), ctypes.c_float(routed_scaling_factor),
        int(group_score), _ptr(workspace), ws_bytes, _stream(stream, router_input))
    _check("moe_route_and_index", st)


def moe_finalize(output: torch.Tensor, down: torch.Tensor, restore_order: torch.Tensor,
                 router_weight: torch.Tensor, stream=None) -> None:
    """output [T, H] <- down [T*K, H], restore_order [T*K], router_weight [T, K]."""
    lib = load_library()
    _dev(output, down, restore_order, router_weight)
    _int32_like(restore_order, "restore_order")
    T, K = router_weight.shape
    H = output.shape[1]
    if tuple(output.shape) != (T, H) or tuple(down.shape) != (T * K, H) or \
            restore_order.numel() != T * K:
        raise ValueError("shapes: output [T, H], down [T*K, H], restore_order [T*K], "
                         "router_weight [T, K]")
    st = lib.moe_finalize(_ptr(output), _dtype_code(output), _ptr(down), _dtype_code(down),
                          _ptr(restore_order), _ptr(router_weight), _dtype_code(router_weight),
                          T, K, H, _stream(stream, output, down))
    _check("moe_finalize", st)
