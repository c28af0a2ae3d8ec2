"""GPU parity of the chained path router -> create_indices -> finalize, all
on the GPU from the same inputs, against the chained oracle: indices and
weights bit-exact, every finalize output row within 1 bf16 ulp (1e-5 of the
term magnitude for fp32). Marked gpu."""
import numpy as np
import pytest
import torch

import oracle
from permutation_group_limited_amd import binding
from permutation_group_limited_amd import workloads as wl

from _gpu import (DEV, assert_finalize_matches_in_blocks, assert_indices_equal,
                  assert_weights_equal, log, to_np_u32)

pytestmark = pytest.mark.gpu



def run_pipeline(wk, down):
    T, E, K = wk.T, wk.E, wk.K
    s = wl.make_scores(wk).to(DEV)
    b = wl.make_bias(wk).to(DEV)
    idx = torch.empty(T, K, dtype=torch.int32, device=DEV)
    w = torch.empty(T, K, dtype=torch.float32, device=DEV)
    order = torch.empty(T * K, dtype=torch.int32, device=DEV)
    restore = torch.empty(T * K, dtype=torch.int32, device=DEV)
    starts = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    eids = torch.empty(E, dtype=torch.int32, device=DEV)
    stats = torch.empty(2, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(binding.moe_create_indices_workspace_size(T * K, E), 4) // 4,
                     dtype=torch.int32, device=DEV)
    out = torch.empty(T, wk.H, dtype=wk.out_dtype, device=DEV)
    binding.moe_router_group_limited(idx, w, s, b, wk.n_groups, wk.topk_group, wk.norm_weights,
                                     wk.scale)
    binding.moe_create_indices(order, starts, restore, eids, stats, idx, ws)
    binding.moe_finalize(out, down, restore, w)
    torch.cuda.synchronize()
    return idx, w, {"token_expert_order": to_np_u32(order),
                    "expert_start_indices": to_np_u32(starts),
                    "restore_token_order": to_np_u32(restore),
                    "expert_ids": eids.cpu().numpy(),
                    "expert_usage_stats": to_np_u32(stats)}, out


@pytest.mark.parametrize("name", ["tiny", "mixtral", "dsv3", "decode", "skewed"])
def test_pipeline(name):
    wk = wl.WORKLOADS[name]
    log("pipeline workload", wk.describe())
    down = wl.make_down(wk, device=DEV)
    idx, w, ind, out = run_pipeline(wk, down)
    s, b = wl.make_scores(wk), wl.make_bias(wk)
    oi, ow = oracle.router(s.numpy(), b.numpy(), wk.K, wk.n_groups, wk.topk_group,
                           wk.norm_weights, wk.scale)
    assert np.array_equal(idx.cpu().numpy(), oi)
    assert_weights_equal(w.cpu().numpy(), ow)
    oind = oracle.create_indices(oi, wk.E)
    assert_indices_equal(ind, oind)
    restore = oind["restore_token_order"]
    # the GPU finalize ran on the GPU's weights, which equal the oracle's bit
    # for bit (checked above); every output row is compared, in token blocks
    worst = assert_finalize_matches_in_blocks(out, down, restore, torch.from_numpy(ow),
                                              wk.out_dtype)
    log("pipeline %s: largest finalize difference %s" % (name, worst))
    del down, out
    torch.cuda.empty_cache()
