"""GPU parity: moe_create_indices vs the CPU oracle (moe_create_indices
page: description, Args). Every output bit-exact. Marked gpu."""
import numpy as np
import pytest
import torch

import oracle
from permutation_group_limited_amd import binding
from permutation_group_limited_amd import workloads as wl

from _gpu import assert_indices_equal, gpu_indices, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "mixtral", "dsv3", "decode", "skewed"])
def test_workload_router_output(name):
    w = wl.WORKLOADS[name]
    log("indices workload", w.describe())
    s, b = wl.make_scores(w), wl.make_bias(w)
    ids, _ = oracle.router(s.numpy(), b.numpy(), w.K, w.n_groups, w.topk_group,
                           w.norm_weights, w.scale)
    got = gpu_indices(ids, w.E)
    exp = oracle.create_indices(ids, w.E)
    assert_indices_equal(got, exp)
    if name == "skewed":
        assert exp["expert_usage_stats"][0] > 8192  # the skew this workload is for


SIZES = [0, 1, 2, 63, 64, 65, 255, 256, 257, 1000, 4095, 4096, 4097, 4352, 8192, 65536,
         65537, 100000, 524288, 1 << 20]


@pytest.mark.parametrize("N", SIZES)
@pytest.mark.parametrize("E", [1, 3, 8, 256, 1000, 1024])
def test_random_ids(N, E):
    if N > 100000 and E not in (8, 256):
        pytest.skip("large N covered for E = 8 and 256")
    log("indices case N", N, "E", E)
    ids = wl.random_ids(N, E, seed=N * 31 + E).numpy()
    assert_indices_equal(gpu_indices(ids, E), oracle.create_indices(ids, E))


@pytest.mark.parametrize("N", [5000, 524288])
def test_skewed_ids(N):
    ids = wl.random_ids(N, 256, seed=N, skew=1.5).numpy()
    assert_indices_equal(gpu_indices(ids, 256), oracle.create_indices(ids, 256))


def test_single_expert_everywhere():
    ids = np.full(70000, 17, np.int32)
    assert_indices_equal(gpu_indices(ids, 256), oracle.create_indices(ids, 256))


def test_sorted_and_reversed_ids():
    ids = np.sort(wl.random_ids(30000, 256, seed=3).numpy())
    assert_indices_equal(gpu_indices(ids, 256), oracle.create_indices(ids, 256))
    ids = ids[::-1].copy()
    assert_indices_equal(gpu_indices(ids, 256), oracle.create_indices(ids, 256))


def test_deterministic_skewed():
    w = wl.WORKLOADS["skewed"]
    s, b = wl.make_scores(w), wl.make_bias(w)
    ids, _ = oracle.router(s.numpy(), b.numpy(), 8, 8, 4, True, 2.5)
    first = gpu_indices(ids, 256)
    for _ in range(5):
        assert_indices_equal(gpu_indices(ids, 256), first)


def test_out_of_range_ids_stay_contained():
    # precondition violated on purpose: the kernels skip such slots (they
    # never form an address from them) and mark their restore entry
    ids = wl.random_ids(3000, 64, seed=9).numpy()
    bad = np.array([5, 77, 1500, 2999])
    ids[bad] = [64, -1, 1000, 2 ** 31 - 1]
    got = gpu_indices(ids, 64)
    assert np.all(got["restore_token_order"][bad] == 0xFFFFFFFF)
    keep = np.setdiff1d(np.arange(ids.size), bad)
    ref = oracle.create_indices(ids[keep], 64)
    n = keep.size
    assert np.array_equal(got["expert_ids"], ref["expert_ids"])
    assert np.array_equal(got["expert_usage_stats"], ref["expert_usage_stats"])
    assert np.array_equal(got["expert_start_indices"], ref["expert_start_indices"])
    # the valid slots keep their own (uncompacted) indices
    assert np.array_equal(got["token_expert_order"][:n], keep[ref["token_expert_order"]])
    assert np.array_equal(got["restore_token_order"][keep], ref["restore_token_order"])


def gpu_indices_aligned(ids, E, align):
    ids = torch.as_tensor(ids).reshape(-1).to(torch.int32)
    n = ids.numel()
    d = ids.to("cuda:0")
    mk = lambda m: torch.full((m,), 0x5A5A5A5A, dtype=torch.int32, device="cuda:0")
    order, restore, starts, eids, stats, scales = mk(n), mk(n), mk(E + 1), mk(E), mk(2), mk(E + 1)
    ws = mk(max(binding.moe_create_indices_workspace_size(n, E), 4) // 4)
    binding.moe_create_indices_aligned(order, starts, restore, eids, stats, d, ws, scales, align)
    torch.cuda.synchronize()
    return {"token_expert_order": order.cpu().numpy().view(np.uint32),
            "expert_start_indices": starts.cpu().numpy().view(np.uint32),
            "restore_token_order": restore.cpu().numpy().view(np.uint32),
            "expert_ids": eids.cpu().numpy(),
            "expert_usage_stats": stats.cpu().numpy().view(np.uint32)}, \
        scales.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("align", [1, 3, 32, 128])
@pytest.mark.parametrize("N,E", [(0, 8), (100, 8), (1024, 256), (65536, 256), (524288, 256),
                                 (5000, 1000)])
def test_aligned_scale_offsets(N, E, align):
    log("aligned indices N", N, "E", E, "align", align)
    ids = wl.random_ids(N, E, seed=N + align, skew=1.2).numpy()
    got, scales = gpu_indices_aligned(ids, E, align)
    assert_indices_equal(got, oracle.create_indices(ids, E))
    assert np.array_equal(scales, oracle.scale_offsets(ids, E, align))


@pytest.mark.parametrize("N,E", [((1 << 28) + 12345, 256), ((1 << 27) + 7, 1000)])
def test_huge_n_properties(N, E):
    """Far past what the oracle finishes: 2^28 + 12345 slots (outputs are
    uint32, so N may go up to 2^32 - 1). Checked on the GPU through the
    properties that define the result: token_expert_order is a permutation
    and restore_token_order its inverse; read through the order, the ids are
    non-decreasing and, within one expert, the slot indices ascend (stable);
    expert_start_indices, expert_ids and expert_usage_stats equal what
    torch.bincount gives."""
    log("indices huge N", N, "E", E)
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(N % 1000003)
    ids = torch.randint(0, E, (N,), generator=g, dtype=torch.int32, device=dev)
    order = torch.full((N,), -1, dtype=torch.int32, device=dev)
    restore = torch.full((N,), -1, dtype=torch.int32, device=dev)
    starts = torch.full((E + 1,), -1, dtype=torch.int32, device=dev)
    eids = torch.full((E,), -7, dtype=torch.int32, device=dev)
    stats = torch.full((2,), -1, dtype=torch.int32, device=dev)
    ws = torch.empty(max(binding.moe_create_indices_workspace_size(N, E), 4) // 4,
                     dtype=torch.int32, device=dev)
    binding.moe_create_indices(order, starts, restore, eids, stats, ids, ws)
    torch.cuda.synchronize()
    o = order.long()
    assert int(o.min()) == 0 and int(o.max()) == N - 1
    assert torch.equal(restore.long()[o], torch.arange(N, device=dev))
    seg = ids[o]
    assert bool((seg[1:] >= seg[:-1]).all())
    same = seg[1:] == seg[:-1]
    assert bool((o[1:] > o[:-1])[same].all())
    del seg, same
    cnt = torch.bincount(ids.long(), minlength=E)
    active = torch.nonzero(cnt).flatten()
    A = active.numel()
    csum = torch.cat([torch.zeros(1, dtype=torch.long, device=dev), torch.cumsum(cnt, 0)])
    exp_starts = torch.full((E + 1,), N, dtype=torch.long, device=dev)
    exp_starts[:A] = csum[active]
    assert torch.equal(starts.long(), exp_starts)
    exp_ids = torch.full((E,), -1, dtype=torch.long, device=dev)
    exp_ids[:A] = active
    assert torch.equal(eids.long(), exp_ids)
    assert stats.tolist() == [int(cnt.max()), A]


def test_max_n_properties():
    """The largest problem the uint32 outputs allow: N = 2^32 - 1 slots over
    E = 256 (16 GiB per [N] array). Same defining properties as above,
    checked in slices of 2^28 slots on the GPU, with uint32 values read
    through int64 (positions above 2^31 - 1 are negative as int32)."""
    N, E = (1 << 32) - 1, 256
    log("indices max N", N, "E", E)
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(5)
    ids = torch.randint(0, E, (N,), generator=g, dtype=torch.int32, device=dev)
    order = torch.full((N,), -1, dtype=torch.int32, device=dev)
    restore = torch.full((N,), -1, dtype=torch.int32, device=dev)
    starts = torch.full((E + 1,), -1, dtype=torch.int32, device=dev)
    eids = torch.full((E,), -7, dtype=torch.int32, device=dev)
    stats = torch.full((2,), -1, dtype=torch.int32, device=dev)
    ws = torch.empty(max(binding.moe_create_indices_workspace_size(N, E), 4) // 4,
                     dtype=torch.int32, device=dev)
    binding.moe_create_indices(order, starts, restore, eids, stats, ids, ws)
    torch.cuda.synchronize()
    log("indices max N: kernels done, checking")
    u32 = lambda t: t.long() & 0xFFFFFFFF  # noqa: E731
    cnt = torch.zeros(E, dtype=torch.long, device=dev)
    step = 1 << 28
    prev_id, prev_slot = -1, -1
    for a in range(0, N, step):
        b = min(a + step, N)
        o = u32(order[a:b])
        assert int(o.max()) < N
        # restore(order(i)) == i for every i makes order injective, hence a
        # permutation of [0, N), and restore its inverse
        assert torch.equal(u32(restore[o]), torch.arange(a, b, device=dev))
        seg = ids[o].long()
        assert int(seg[0]) >= prev_id and (int(seg[0]) > prev_id or int(o[0]) > prev_slot)
        assert bool((seg[1:] >= seg[:-1]).all())
        same = seg[1:] == seg[:-1]
        assert bool((o[1:] > o[:-1])[same].all())
        prev_id, prev_slot = int(seg[-1]), int(o[-1])
        cnt += torch.bincount(ids[a:b].long(), minlength=E)
        del o, seg, same
    active = torch.nonzero(cnt).flatten()
    A = active.numel()
    csum = torch.cat([torch.zeros(1, dtype=torch.long, device=dev), torch.cumsum(cnt, 0)])
    exp_starts = torch.full((E + 1,), N, dtype=torch.long, device=dev)
    exp_starts[:A] = csum[active]
    assert torch.equal(u32(starts), exp_starts)
    exp_ids = torch.full((E,), -1, dtype=torch.long, device=dev)
    exp_ids[:A] = active
    assert torch.equal(eids.long(), exp_ids)
    assert u32(stats).tolist() == [int(cnt.max()), A]
    del ids, order, restore
    torch.cuda.empty_cache()
