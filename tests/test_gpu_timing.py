"""The per-kernel timing aid on the GPU: launch counts per kernel kind, positive device
times that fit inside the wall time, records consumed by a read, and results that do
not depend on whether timing is on."""
import time

import numpy as np
import pytest

import hstu_silu_attention_amd as hsa
import workloads
from gpu_util import gpu_encode, make_model, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _workload(dtype):
    return workloads.make_custom(seed=77, dtype=dtype, layers=3, d_model=128 if dtype == "bf16" else 64,
                                 heads=2, max_len=300, uih_lengths=[200, 0, 129], cand_lengths=[5, 17, 0])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_timing_counts_and_bounds(dtype):
    torch = torch_cuda()
    wl = _workload(dtype)
    model = make_model(torch, wl)
    uih = to_dev(torch, wl.uih.reshape(-1, wl.d_model), wl.dtype)
    cand = to_dev(torch, wl.cand.reshape(-1, wl.d_model), wl.dtype)
    base_u, base_c = gpu_encode(wl, model=model, uih=uih, cand=cand)

    calls = 3
    torch.cuda.synchronize()
    assert hsa.hstu_timing_enable(True) == 0
    t0 = time.perf_counter()
    for _ in range(calls):
        got_u, got_c = gpu_encode(wl, model=model, uih=uih, cand=cand)
    wall_ms = (time.perf_counter() - t0) * 1e3
    assert hsa.hstu_timing_enable(False) == 0
    st, rec = hsa.hstu_timing_read()
    assert st == 0
    L = wl.layers
    norm = 2 if dtype == "bf16" else L          # bf16: row and column sums once per call
    # plan: the plan's transfer (its upload kernels, one record) and the plan kernel
    expect = {"plan": 2, "uvqk": L, "attention": L, "out": L, "norm": norm}
    total = 0.0
    for kind, n in expect.items():
        ms, launches = rec[kind]
        say(f"  {dtype} {kind}: {launches} launches, {ms:.4f} ms")
        assert launches == calls * n
        assert ms > 0.0
        total += ms
    assert total <= wall_ms
    # timing changes no result
    assert np.array_equal(got_u, base_u) and np.array_equal(got_c, base_c)
    # a read consumes the records
    st, rec = hsa.hstu_timing_read()
    assert st == 0 and all(n == 0 and ms == 0.0 for ms, n in rec.values())


def test_timing_select_limits_the_kinds():
    """With a kind mask, only launches of those kinds are recorded; the mask is kept until
    changed and None restores all kinds."""
    torch = torch_cuda()
    wl = _workload("bf16")
    model = make_model(torch, wl)
    uih = to_dev(torch, wl.uih.reshape(-1, wl.d_model), wl.dtype)
    cand = to_dev(torch, wl.cand.reshape(-1, wl.d_model), wl.dtype)
    try:
        assert hsa.hstu_timing_select(("attention", "out")) == 0
        assert hsa.hstu_timing_enable(True) == 0
        gpu_encode(wl, model=model, uih=uih, cand=cand)
        gpu_encode(wl, model=model, uih=uih, cand=cand)
        assert hsa.hstu_timing_enable(False) == 0
        st, rec = hsa.hstu_timing_read()
        assert st == 0
        L = wl.layers
        assert rec["attention"][1] == 2 * L and rec["out"][1] == 2 * L
        assert all(rec[k][1] == 0 for k in ("plan", "uvqk", "norm", "pack", "score"))
        assert rec["attention"][0] > 0.0 and rec["out"][0] > 0.0
    finally:
        hsa.hstu_timing_select(None)
        hsa.hstu_timing_enable(False)
        hsa.hstu_timing_read()
