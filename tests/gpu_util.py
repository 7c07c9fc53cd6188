"""Helpers for the GPU parity tests: run the HIP path through the C ABI on workloads and
measure normwise errors against the oracle. No fallback: a missing GPU or library fails."""
import json
import multiprocessing
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


# ---------------------------------------------------------------- oracle over many users

_POOL_JOB = None      # (wl, uih, uih_lengths, cand, cand_lengths), read by forked workers


def _oracle_one_user(task):
    from threadpoolctl import threadpool_limits
    import oracle
    b, mode = task
    wl, uih, ul, cand, cl = _POOL_JOB
    with threadpool_limits(limits=1):
        uo, co = workloads.lengths_to_offsets(ul), workloads.lengths_to_offsets(cl)
        ru, rc, _ = oracle.encode(uih, uo, cand, co, wl.params, heads=wl.heads, max_len=wl.max_len, mode=mode,
                                  users=[b])
    return b, mode, ru[uo[b]:uo[b + 1]].copy(), rc[co[b]:co[b + 1]].copy()


_RESULTS = {}         # (inputs digest, user, mode) -> the oracle's rows, for workloads that repeat
                      # another's encoder inputs (the scored workload repeats the headline's)


def _job_key(job):
    """Digest of everything the oracle's result for a user depends on."""
    import hashlib
    wl, uih, ul, cand, cl = job
    h = hashlib.sha1()
    for a in [uih, cand, ul, cl] + [x for p in wl.params for x in (p.w1, p.w2, p.pos, getattr(p, "rel", None))]:
        h.update(b"none" if a is None else np.ascontiguousarray(a).tobytes())
    h.update(repr((wl.heads, wl.max_len)).encode())
    return h.hexdigest()


def pool_workers():
    """Worker processes for the oracle (one BLAS thread each): the host's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def oracle_users(wl, users, mode="bf16", uih=None, uih_lengths=None, cand=None, cand_lengths=None,
                 extra=()):
    """The oracle's outputs of each listed user, computed one user per task in forked worker
    processes (users are independent; the oracle's elementwise steps are single-threaded).
    ``extra`` lists more (user, mode) tasks run in the same pool. Returns
    {user: (uih_rows, cand_rows)} for ``mode``, or {(user, mode): ...} when ``extra`` is
    given. The workers only run NumPy: they never touch the GPU and end with os._exit
    (multiprocessing's fork start method)."""
    global _POOL_JOB
    ul = wl.uih_lengths if uih_lengths is None else uih_lengths
    cl = wl.cand_lengths if cand_lengths is None else cand_lengths
    job = (wl, wl.uih if uih is None else uih, ul, wl.cand if cand is None else cand, cl)
    key = _job_key(job)
    tasks = [(int(b), mode) for b in users] + [(int(b), m) for b, m in extra]
    done = {t: _RESULTS[(key,) + t] for t in tasks if (key,) + t in _RESULTS}
    tasks = [t for t in tasks if t not in done]
    if not tasks:
        out = dict(done)
        return out if extra else {b: v for (b, _), v in out.items()}
    _POOL_JOB = job
    # longest users first so the pool ends on short ones
    tasks.sort(key=lambda t: -int(ul[t[0]] + cl[t[0]]))
    t0 = time.perf_counter()
    out = dict(done)
    try:
        ctx = multiprocessing.get_context("fork")
        with ctx.Pool(min(pool_workers(), len(tasks))) as pool:
            for b, m, ru, rc in pool.imap_unordered(_oracle_one_user, tasks):
                out[(b, m)] = (ru, rc)
                _RESULTS[(key, b, m)] = (ru, rc)
                say(f"    oracle user {b} ({m}) done at {time.perf_counter() - t0:.0f}s")
    finally:
        _POOL_JOB = None
    say(f"  oracle: {len(tasks)} user tasks on {min(pool_workers(), len(tasks))} workers: "
        f"{time.perf_counter() - t0:.1f}s")
    return out if extra else {b: v for (b, _), v in out.items()}


def error_stats(got, ref, tol):
    """Normwise error max|g - r| / max|r| (the gate), and two diagnostics: the elementwise
    maximum of |g - r| / max(|r|, 1e-3 max|r|) and the fraction of elements whose floored
    elementwise error exceeds tol."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if r.size == 0:
        return {"normwise": 0.0, "elem_max": 0.0, "frac_above": 0.0}
    assert np.all(np.isfinite(g)), "non-finite output"
    scale = max(float(np.max(np.abs(r))), 1e-30)
    d = np.abs(g - r)
    el = d / np.maximum(np.abs(r), 1e-3 * scale)
    return {"normwise": float(np.max(d) / scale), "elem_max": float(np.max(el)),
            "frac_above": float(np.mean(el > tol))}


def report(record):
    """Append one JSON line of parity diagnostics to $HSTU_PARITY_REPORT (if set)."""
    path = os.environ.get("HSTU_PARITY_REPORT")
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "a") as f:
            f.write(json.dumps(record) + "\n")
