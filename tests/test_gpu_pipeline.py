"""GPU parity of the chained path router -> create_indices -> finalize, all
on the GPU from the same inputs, against the chained oracle. Marked gpu."""
import numpy as np
import pytest
import torch

import oracle
from permutation_group_limited_amd import binding
from permutation_group_limited_amd import workloads as wl

from _gpu import (DEV, assert_finalize_close, assert_indices_equal, assert_weights_close,
                  bf16_bits, log, oracle_finalize_from, term_magnitude, to_np_u32)

pytestmark = pytest.mark.gpu



def chained_tol(K):
    """Router weight tolerance plus two K-term fp32 FMA chains."""
    return 1e-6 + 2 * K * 2.0 ** -24


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
    assert_weights_close(w.cpu().numpy(), ow)
    oind = oracle.create_indices(oi, wk.E)
    assert_indices_equal(ind, oind)
    restore = oind["restore_token_order"]
    # the oracle's finalize takes the oracle's own weights
    wt = torch.from_numpy(ow)
    if name == "skewed":
        ts = np.sort(np.random.default_rng(1).choice(wk.T, 1024, replace=False))
        rows = restore.reshape(wk.T, wk.K)[ts].reshape(-1).astype(np.int64)
        sub = down[torch.from_numpy(rows).to(DEV)].cpu()
        sub_r = np.arange(rows.size, dtype=np.uint32)
        exp = oracle_finalize_from(sub, sub_r, wt[ts], wk.out_dtype)
        assert_finalize_close(out[torch.from_numpy(ts).to(DEV)], exp,
                              term_magnitude(sub, sub_r, wt[ts]), chained_tol(wk.K))
    else:
        dh = down.cpu()
        exp = oracle_finalize_from(dh, restore, wt, wk.out_dtype)
        assert_finalize_close(out, exp, term_magnitude(dh, restore, wt), chained_tol(wk.K))
