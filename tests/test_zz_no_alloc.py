"""hstu_encode_static, the entry point that allocates nothing (its workspace is a fixed
device array, its planner fixed host arrays), against hstu_encode on the same inputs:
two calls in a row, the second on a smaller batch, with and without a key/value cache.
The two share their plan and kernels, so the outputs (and cached rows) agree bit for
bit; the oracle's bf16 bar (2e-2 normwise) is checked too."""
import numpy as np
import pytest

import hstu_silu_attention_amd as hsa
import workloads
from gpu_util import BF16_TOL, make_model, normwise_per_user, oracle_encode, say, to_dev, to_np, torch_cuda

pytestmark = pytest.mark.gpu


def _run(torch, wl, model, static, cache=None):
    du, dc = to_dev(torch, wl.uih, wl.dtype), to_dev(torch, wl.cand, wl.dtype)
    uo = workloads.lengths_to_offsets(wl.uih_lengths)
    co = workloads.lengths_to_offsets(wl.cand_lengths)
    say(f"  {'static' if static else 'workspace'} entry: users {wl.users}, rows {du.shape[0] + dc.shape[0]}")
    f = hsa.encode_static if static else hsa.encode
    gu, gc = f(model, du, uo, dc, co, cache=cache)
    torch.cuda.synchronize()
    return to_np(gu), to_np(gc)


@pytest.mark.parametrize("with_cache", [False, True])
def test_static_entry_matches_workspace_entry(with_cache):
    torch = torch_cuda()
    big = workloads.make_custom(seed=1301, dtype="bf16", layers=2, d_model=512, heads=4, max_len=1200,
                                uih_lengths=[700, 0, 129, 1000, 64], cand_lengths=[300, 8, 0, 129, 1])
    small = workloads.make_custom(seed=1302, dtype="bf16", layers=2, d_model=512, heads=4, max_len=1200,
                                  uih_lengths=[33, 200], cand_lengths=[5, 0])
    small.params = big.params      # the same model for both calls
    model = make_model(torch, big)
    for wl in (big, small):
        caches = [None, None]
        if with_cache:
            caches = [hsa.KVCache(model, slots=6, capacity=1100) for _ in range(2)]
            for cch in caches:
                cch.slot_of_user = np.arange(wl.users, dtype=np.int32)[::-1].copy()
                cch.cached_len = np.zeros(wl.users, dtype=np.int32)
        ws_u, ws_c = _run(torch, wl, model, False, caches[0])
        st_u, st_c = _run(torch, wl, model, True, caches[1])
        assert np.array_equal(ws_u, st_u) and np.array_equal(ws_c, st_c)
        if with_cache:
            assert caches[0].cached_len.tolist() == caches[1].cached_len.tolist() == wl.uih_lengths.tolist()
            assert torch.equal(caches[0].k, caches[1].k) and torch.equal(caches[0].v, caches[1].v)
        ru, rc, _ = oracle_encode(wl, "bf16")
        eu, ec = normwise_per_user(st_u, ru, wl.uih_lengths), normwise_per_user(st_c, rc, wl.cand_lengths)
        say(f"  static entry vs oracle: uih {eu:.3e} cand {ec:.3e}")
        assert eu <= BF16_TOL and ec <= BF16_TOL


def test_static_entry_rejects_a_batch_beyond_its_scratch():
    torch = torch_cuda()
    wl = workloads.make_custom(seed=1303, dtype="bf16", layers=1, d_model=512, heads=4, max_len=20000,
                               uih_lengths=[16000], cand_lengths=[2048])
    model = make_model(torch, wl)
    du, dc = to_dev(torch, wl.uih, "bf16"), to_dev(torch, wl.cand, "bf16")
    with pytest.raises(hsa.HstuError) as e:
        hsa.encode_static(model, du, [0, 16000], dc, [0, 2048])
    assert e.value.status == hsa.HSTU_ERR_TOO_LARGE
