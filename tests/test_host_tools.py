"""Host logic around the kernels, on the CPU: the replay driver's batching, and the
benchmark's per-launch flop and byte accounting against the oracle's counter and the
closed forms the design states."""
import numpy as np

import bench
import oracle
import workloads
from hstu_silu_attention_amd.replay import Replayer, Request


def test_batches_keep_time_order_and_distinct_users():
    reqs = [Request(t, u, 10 * (i + 1), np.zeros((1, 4), np.float32))
            for i, (t, u) in enumerate([(0, 1), (1, 2), (1, 1), (2, 3), (5, 4), (5, 5), (6, 6), (9, 2)])]
    rep = Replayer.__new__(Replayer)
    batches = rep.batches_of(reqs[4:] + reqs[:4], max_users=3)   # served in time order whatever the input order
    flat = [r for b in batches for r in b]
    assert [r.time for r in flat] == sorted(r.time for r in reqs)
    for b in batches:
        assert 1 <= len(b) <= 3 and len({r.user for r in b}) == len(b)
    # a repeated user closes the batch: user 1 at t=1 starts a new one
    assert [[r.user for r in b] for b in batches] == [[1, 2], [1, 3, 4], [5, 6, 2]]


def test_kernel_flops_match_the_oracle_counter():
    wl = workloads.make_custom(seed=61, dtype="f32", layers=1, d_model=8, heads=2, max_len=64,
                               uih_lengths=[7, 0, 12], cand_lengths=[3, 5, 0], cached_lengths=[4, 9, 0])
    got = bench.kernel_flops_per_launch(wl)
    want = {"uvqk": 0, "out": 0, "attention": 0}
    for n, c, m in zip(wl.uih_lengths, wl.cand_lengths, wl.cached_lengths):
        macs = oracle.count_macs(8, 1, int(n), int(c), int(m))
        want["uvqk"] += 2 * macs["gemm_uvqk"]
        want["out"] += 2 * macs["gemm_out"]
        want["attention"] += 2 * (macs["attn_qk"] + macs["attn_pv"] + macs["attn_self"])
    assert {k: got[k] for k in want} == want


def test_kernel_bytes_closed_forms():
    wl = workloads.make_workload("d512_uih2k_c2k", users=2, layers=1)
    T = int(wl.uih_lengths.sum() + wl.cand_lengths.sum())
    D = 512
    b = bench.kernel_bytes_per_launch(wl)
    assert b["uvqk"] == 2 * (T * D + 4 * D * D + 4097 * 3 * D + 4 * T * D)
    assert b["attention"] == 2 * 4 * T * D
    assert b["out"] == 2 * (4 * T * D + 3 * D * D)
    # interleaving doubles the history rows the kernels see
    il = workloads.make_workload("d512_uih2k_c2k_interleaved", users=2, layers=1)
    assert bench.token_lengths(il).tolist() == (2 * il.uih_lengths).tolist()


def test_head_flops():
    wl = workloads.make_custom(seed=3, dtype="bf16", layers=1, d_model=128, heads=1, max_len=8,
                               uih_lengths=[0, 0], cand_lengths=[5, 7], head=(256, 128, 2))
    assert bench.head_flops(wl) == 2 * 12 * (128 * 256 + 256 * 128 + 128 * 2)
