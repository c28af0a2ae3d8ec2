"""MI355X (gfx950) group-limited MoE routing path.

Python binding of the C-ABI library ``libmoe_route.so`` (declared in
``include/moe_route.h``). Importing the package is cheap; the library is
loaded on the first call of an entry point, after torch (whose HIP runtime
the library must share).
"""
from .binding import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_F16,
    DTYPE_F32,
    GROUP_MAX,
    GROUP_TOP2_SUM,
    SCORE_NONE,
    SCORE_SIGMOID,
    SCORE_SOFTMAX,
    MoeError,
    library_path,
    load_library,
    moe_create_indices,
    moe_create_indices_aligned,
    moe_create_indices_no_alloc,
    moe_create_indices_workspace_size,
    moe_finalize,
    moe_route_and_index,
    moe_route_and_index_workspace_size,
    moe_router_group_limited,
    moe_router_group_limited_logits,
)
