"""GPU: moe_create_indices_no_alloc (counts matrix in the library's own
device array) against moe_create_indices with a caller workspace, through
the C ABI on the same ids: every output bit-identical, on pairs of calls in
a row where the second is smaller (it finds the first call's counts still in
the array, which must not matter), and against the oracle. Marked gpu."""
import numpy as np
import pytest
import torch

import oracle
from permutation_group_limited_amd import binding

from _gpu import DEV, assert_indices_equal, log, to_np_u32

pytestmark = pytest.mark.gpu

POISON = 0x5A5A5A5A


def _ids(n, E, seed, skew=False):
    g = torch.Generator().manual_seed(seed)
    if skew:  # Zipf-like: expert 0 hottest
        w = 1.0 / torch.arange(1, E + 1, dtype=torch.float64) ** 1.2
        return torch.multinomial(w, n, replacement=True, generator=g).to(torch.int32)
    return torch.randint(0, E, (n,), generator=g, dtype=torch.int32)


def _outputs(n, E):
    full = lambda k: torch.full((k,), POISON, dtype=torch.int32, device=DEV)  # noqa: E731
    return [full(n), full(E + 1), full(n), full(E), full(2)]


def _host(o):
    return {"token_expert_order": to_np_u32(o[0]), "expert_start_indices": to_np_u32(o[1]),
            "restore_token_order": to_np_u32(o[2]), "expert_ids": o[3].cpu().numpy(),
            "expert_usage_stats": to_np_u32(o[4])}


def _no_alloc(ids_dev, E):
    o = _outputs(ids_dev.numel(), E)
    binding.moe_create_indices_no_alloc(o[0], o[1], o[2], o[3], o[4], ids_dev)
    return o


def _with_workspace(ids_dev, E):
    n = ids_dev.numel()
    o = _outputs(n, E)
    ws = torch.full((max(binding.moe_create_indices_workspace_size(n, E), 4) // 4,), POISON,
                    dtype=torch.int32, device=DEV)
    binding.moe_create_indices(o[0], o[1], o[2], o[3], o[4], ids_dev, ws)
    return o


@pytest.mark.parametrize("first,second", [
    ((524288, 256, True), (65536, 256, False)),   # both several chunks, same E
    ((100000, 1000, False), (9000, 8, True)),     # smaller matrix over stale rows
    ((65536, 256, False), (1000, 256, False)),    # several chunks, then one workgroup
])
def test_no_alloc_matches_workspace_entry_point(first, second):
    calls = []
    for k, (n, E, skew) in enumerate((first, second)):
        log("no_alloc call %d: N=%d E=%d skew=%s" % (k, n, E, skew))
        ids = _ids(n, E, seed=n + E + k, skew=skew)
        d = ids.to(DEV)
        calls.append((ids, E, _no_alloc(d, E), _with_workspace(d, E)))
    torch.cuda.synchronize()
    for ids, E, got, ref in calls:
        g, r = _host(got), _host(ref)
        assert_indices_equal(g, r)
        assert_indices_equal(g, oracle.create_indices(ids.numpy(), E))
