"""placeholder"""
DTYPE_F32 = 0
DTYPE_BF16 = 1
GROUP_TOP2_SUM = 0
GROUP_MAX = 1
class MoeError(RuntimeError):
    pass
def library_path(): raise NotImplementedError
def load_library(): raise NotImplementedError
def moe_create_indices(*a, **k): raise NotImplementedError
def moe_create_indices_workspace_size(*a, **k): raise NotImplementedError
def moe_finalize(*a, **k): raise NotImplementedError
def moe_router_group_limited(*a, **k): raise NotImplementedError
