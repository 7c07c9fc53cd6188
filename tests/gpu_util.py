"""Helpers for the GPU parity tests: run the HIP path through the C ABI on workloads and
measure normwise errors against the oracle. No fallback: a missing GPU or library fails."""
import os
import sys
import time

import numpy as np

import hstu_silu_attention_amd as hsa
import workloads

BF16_TOL = 2e-2
F32_TOL = 1e-4


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (torch.cuda.is_available() is False)")
    hsa.load_library()
    return torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(torch, a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def make_model(torch, wl, params=None):
    return hsa.Model(wl.params if params is None else params, d_model=wl.d_model, heads=wl.heads,
                     max_len=wl.max_len, dtype=wl.dtype)


def gpu_encode(wl, *, model=None, uih=None, cand=None, uih_lengths=None, cand_lengths=None,
               cache=None, keep_device=False):
    """hstu_encode over a workload's (or given) tokens. Returns numpy float64 (uih_out, cand_out)."""
    torch = torch_cuda()
    model = model or make_model(torch, wl)
    uih = wl.uih if uih is None else uih
    cand = wl.cand if cand is None else cand
    ul = wl.uih_lengths if uih_lengths is None else uih_lengths
    cl = wl.cand_lengths if cand_lengths is None else cand_lengths
    du = uih if hasattr(uih, "data_ptr") else to_dev(torch, uih.reshape(-1, wl.d_model), wl.dtype)
    dc = cand if hasattr(cand, "data_ptr") else to_dev(torch, cand.reshape(-1, wl.d_model), wl.dtype)
    out = hsa.encode(model, du, workloads.lengths_to_offsets(ul), dc, workloads.lengths_to_offsets(cl),
                     cache=cache)
    torch.cuda.synchronize()
    if keep_device:
        return out
    return to_np(out[0]), to_np(out[1])


def normwise_per_user(got, ref, lengths):
    """max over users of max|g - r| / max|r| (users with rows only)."""
    offs = workloads.lengths_to_offsets(lengths)
    worst = 0.0
    for b in range(len(lengths)):
        g, r = got[offs[b]:offs[b + 1]], ref[offs[b]:offs[b + 1]]
        if r.size == 0:
            continue
        assert np.all(np.isfinite(g)), f"non-finite output for user {b}"
        worst = max(worst, float(np.max(np.abs(g - r)) / max(float(np.max(np.abs(r))), 1e-30)))
    return worst


def oracle_encode(wl, mode, users=None, cache=None, uih_lengths=None, cand_lengths=None, uih=None, cand=None):
    import oracle
    ul = wl.uih_lengths if uih_lengths is None else uih_lengths
    cl = wl.cand_lengths if cand_lengths is None else cand_lengths
    t0 = time.perf_counter()
    res = oracle.encode(wl.uih if uih is None else uih, workloads.lengths_to_offsets(ul),
                        wl.cand if cand is None else cand, workloads.lengths_to_offsets(cl), wl.params,
                        heads=wl.heads, max_len=wl.max_len, mode=mode, cache=cache, users=users)
    say(f"  oracle ({mode}, users={'all' if users is None else list(users)}) {time.perf_counter() - t0:.1f}s")
    return res


def select_users(a, lengths, users):
    offs = workloads.lengths_to_offsets(lengths)
    return np.concatenate([a[offs[b]:offs[b + 1]] for b in users]) if len(users) else a[:0]
