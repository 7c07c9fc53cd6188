"""Throughput benchmark of the jagged HSTU encoder on one MI355X.

One step = one hstu_encode call over the whole batch through every layer (row
statistics, uvqk projection, target-aware SiLU attention, gated output GEMM), on
seeded synthetic inputs already resident in HBM; for a workload given as per-event
context and action embeddings, the hstu_pack_uih call that makes the tokens is part
of the step, and for a workload with a scoring head, the hstu_score call over every
candidate's output (its flops are added to the encoder's). The default workload is
"d512_uih2k_c2k": 16 users, UIH lengths lognormal (median 2000, sigma 0.5, clipped
to [512, 4096]), 2048 candidates per user, D=512, 4 heads, 8 layers, bfloat16.

Prints one JSON line: algorithmic TFLOP/s of the whole job (``value``), users/s, the
fraction of the bf16 MFMA peak, per-kernel device times (HIP events recorded by the
library on the launch stream around one group of kernel kinds per timed step, the
groups in turn), the roofline of the dominant kernel and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import hstu_silu_attention_amd as hsa  # noqa: E402
import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = {
    "attention": "hstu_silu_attention_amd/csrc/attn_bf16.hip",
    "uvqk": "hstu_silu_attention_amd/csrc/gemm_bf16.hip",
    "out": "hstu_silu_attention_amd/csrc/gemm_bf16.hip",
}


def token_lengths(wl) -> np.ndarray:
    """History tokens per user as the encoder sees them: a packing workload's event counts
    become two tokens per event when interleaved and one when merged."""
    return wl.uih_lengths.astype(np.int64) * (2 if wl.packing == "interleave" else 1)


def head_flops(wl) -> int:
    """Algorithmic flops of the scoring head over every candidate (2 per multiply-add)."""
    return 2 * int(wl.cand_lengths.sum()) * sum(int(w.shape[0]) * int(w.shape[1]) for w, _ in wl.head)


def kernel_flops_per_launch(wl) -> dict:
    """Algorithmic flops of one launch (one layer) of each kernel, from the lengths."""
    D = wl.d_model
    n = token_lengths(wl)
    c = wl.cand_lengths.astype(np.int64)
    m = np.zeros_like(n) if wl.cached_lengths is None else wl.cached_lengths.astype(np.int64)
    T = int((n + c).sum())
    pairs = int((n * m + n * (n + 1) // 2 + c * (m + n + 1)).sum())
    return {"uvqk": 2 * T * D * 4 * D, "attention": 4 * D * pairs, "out": 2 * T * 3 * D * D,
            "norm": 0, "plan": 0, "pack": 0, "score": head_flops(wl)}


def kernel_bytes_per_launch(wl) -> dict:
    """Algorithmic HBM bytes of one launch (one layer) of each kernel (bf16, 2 B): what the
    kernel must read and write at least once.
    uvqk: the layer input X [T, D], W1 [4D, D] and the position table [max_len, 3D] read;
          U, V, Q, K [T, 4D] written (the appended cache rows are copies of V and K).
    attention: Q, K, V of every computed row read, the cached K and V [m, D] of each user,
          O [T, D] written.
    out: U and O [T, 2D], W2 [D, 3D] and the residual X [T, D] read; Y [T, D] written."""
    D = wl.d_model
    n = token_lengths(wl)
    c = wl.cand_lengths.astype(np.int64)
    m = wl.cached_lengths.astype(np.int64)
    T = int((n + c).sum())
    pos = wl.max_len * 3 * D if wl.params[0].pos is not None else 0
    return {"uvqk": 2 * (T * D + 4 * D * D + pos + 4 * T * D),
            "attention": 2 * (3 * T * D + 2 * int(m.sum()) * D + T * D),
            "out": 2 * (2 * T * D + 3 * D * D + T * D + T * D)}


def gpu_sclk_mhz():
    """The GPU's current shader clock from the driver's DPM table (the level marked with
    '*'), or None where the file is not readable."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(path):
                if line.rstrip().endswith("*"):
                    return int(float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz")))
        except (OSError, ValueError, IndexError):
            continue
    return None


def source_hash(path: str) -> str:
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the kernel source as it is now (its hash matches); otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, min_seconds: float = 10.0):
    """The CPU oracle (as it stands) on a bounded sample of the same workload: users in
    order of closeness to the median history length, each through every layer in
    bf16-mirror mode, until at least ``min_seconds`` of CPU work; scaled to TFLOP/s by
    the sample's algorithmic flops."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    tl = token_lengths(wl)
    med = float(np.median(tl))
    order = sorted(range(wl.users), key=lambda b: (abs(float(tl[b]) - med), b))
    uo = workloads.lengths_to_offsets(wl.uih_lengths)
    co = workloads.lengths_to_offsets(wl.cand_lengths)
    D, L = wl.d_model, wl.layers
    mode = "bf16" if wl.dtype == "bf16" else "f64"
    done, flops, dt = [], 0, 0.0
    for b in order:
        t0 = time.perf_counter()
        if wl.cached_lengths[b] > 0:       # the user's prefix cached first (untimed), as on the GPU
            t_fill = time.perf_counter()
            m = int(wl.cached_lengths[b])
            po = workloads.lengths_to_offsets(wl.cached_lengths)
            oc = oracle.OracleCache(np.zeros((L, 1, m + int(wl.uih_lengths[b]), D)),
                                    np.zeros((L, 1, m + int(wl.uih_lengths[b]), D)), np.zeros(1, np.int64),
                                    np.zeros(1, np.int64))
            _, _, oc = oracle.encode(wl.prefix[po[b]:po[b + 1]], [0, m], np.zeros((0, D)), [0, 0], wl.params,
                                     heads=wl.heads, max_len=wl.max_len, mode=mode, cache=oc)
            t0 += time.perf_counter() - t_fill
            _, cand_out, _ = oracle.encode(wl.uih[uo[b]:uo[b + 1]], [0, uo[b + 1] - uo[b]], wl.cand[co[b]:co[b + 1]],
                                           [0, co[b + 1] - co[b]], wl.params, heads=wl.heads, max_len=wl.max_len,
                                           mode=mode, cache=oc)
        elif wl.packing == "none":
            _, cand_out, _ = oracle.encode(wl.uih, uo, wl.cand, co, wl.params, heads=wl.heads,
                                           max_len=wl.max_len, mode=mode, users=[b])
            cand_out = cand_out[co[b]:co[b + 1]]
        else:                             # this user's events packed, then encoded on their own
            ev = slice(int(uo[b]), int(uo[b + 1]))
            tok, toff = oracle.pack_uih(wl.uih[ev], wl.action[ev], [0, uo[b + 1] - uo[b]], wl.packing,
                                        bf16=(mode == "bf16"))
            _, cand_out, _ = oracle.encode(tok, toff, wl.cand[co[b]:co[b + 1]], [0, co[b + 1] - co[b]],
                                           wl.params, heads=wl.heads, max_len=wl.max_len, mode=mode)
        n, c = int(tl[b]), int(wl.cand_lengths[b])
        if wl.head:                       # the user's encoded candidates scored
            oracle.score_head(cand_out, wl.head, bf16=(mode == "bf16"))
            flops += 2 * c * sum(int(w.shape[0]) * int(w.shape[1]) for w, _ in wl.head)
        dt += time.perf_counter() - t0
        m = int(wl.cached_lengths[b])
        flops += L * (14 * (n + c) * D * D + 4 * D * (n * m + n * (n + 1) // 2 + c * (m + n + 1)))
        done.append(b)
        if dt >= min_seconds:
            break
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"users {done} of {wl.users} (closest to the median UIH length), all {L} layers, "
                      f"float64 with bf16-mirror rounding; {dt:.1f} s; {len(done) / dt:.4f} users/s on this host"}


def graph_replays(torch, step, steps, alg_flops, users, warm=3):
    """One step captured into a HIP graph (on a side stream, after the eager steps: its
    launches, with the plan in their arguments, are recorded once), then `steps` replays
    timed by the wall clock with a synchronize on both sides. The library records no
    events while its timing is off, and the step has no memset or allocation to record."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    return {"steps": steps, "ms_per_step": round(sec * 1e3, 4), "value": round(alg_flops / sec / 1e12, 3),
            "unit": "TFLOP/s", "users_per_s": round(users / sec, 2)}


def replay_bench(args, pages=10240, max_rows=4096, ttl=300, window=3072, batch_users=16, cand_sets=16):
    """Streaming replay: 2048 requests from 192 drawn users in time order (first visit with a
    lognormal history, then 16-128 new events per visit, 2048 candidates per request), served
    in batches of up to 16 distinct users through the page pool and a paged cache of 10240
    pages of 64 rows (655K rows, the memory of 160 users at 4096 rows; a user holds
    ceil(rows / 64) pages, at most 4096 rows; when pages run out the least recently served
    users are evicted). Histories are host bf16 rows (a request's new events, or its latest
    3072 events when the pool says to encode again, cross PCIe per batch); candidate rows
    come from 16 device-resident sets reused in turn. One untimed pass over the first 64
    requests warms up; the timed pass replays all requests from an empty pool."""
    import torch
    from hstu_silu_attention_amd.replay import Replayer, Request
    dev = torch.device("cuda:0")
    rs = workloads.make_replay()
    wl = rs.model
    model = hsa.Model(wl.params, d_model=wl.d_model, heads=wl.heads, max_len=wl.max_len, dtype="bf16", device=dev)
    hist = {u: torch.from_numpy(h).to(torch.bfloat16) for u, h in rs.history.items()}
    sets = [torch.from_numpy(rs.candidates(i)).to(device=dev, dtype=torch.bfloat16) for i in range(cand_sets)]
    reqs = [Request(t, u, e, sets[i % cand_sets]) for i, (t, u, e, _) in enumerate(rs.requests)]
    ppu = (max_rows + hsa.PAGE_ROWS - 1) // hsa.PAGE_ROWS
    cache = hsa.PagedKVCache(model, pages=pages, pages_per_user=ppu, max_users=batch_users, device=dev)

    def run(requests):
        pool = hsa.KvPool(pages, max_rows, ttl)
        rep = Replayer(model, cache, pool, hist, window=window, device=dev, keep_outputs=False)
        for b in rep.batches_of(requests, batch_users):
            rep.serve(b)
        torch.cuda.synchronize()
        return rep, pool

    run(reqs[:64])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    rep, pool = run(reqs)
    dt = time.perf_counter() - t0
    stats = pool.stats()
    held = [pool.lookup(u) for u in rs.history]
    held_rows, held_pages = sum(n for n, _ in held), sum(p for _, p in held)
    print(json.dumps({
        "metric": "HSTU streaming replay requests/s (2K candidates per request)",
        "value": round(len(reqs) / dt, 2), "unit": "requests/s", "n_gpus": 1, "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic (seeded replay stream)",
        "config": {"workload": "replay_192u_2048r_c2k", "users": len(rs.history), "requests": len(reqs),
                   "batch_users": batch_users, "pages": pages, "page_rows": hsa.PAGE_ROWS, "max_rows": max_rows,
                   "ttl": ttl, "window": window,
                   "layers": wl.layers, "d_model": wl.d_model, "heads": wl.heads},
        "seconds": round(dt, 3), "batches": rep.batches, "tflops": round(rep.flops / dt / 1e12, 3),
        "history_rows_sent": rep.rows_sent, "history_rows_without_cache": rep.rows_no_cache, "pool": stats,
        "rows_held_end": held_rows, "pages_held_end": held_pages,
        "page_fill_end": round(held_rows / max(held_pages * hsa.PAGE_ROWS, 1), 4),
        "flops_saved_by_cache": round(1.0 - rep.flops / max(rep.flops_no_cache, 1), 4),
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--warmup-seconds", type=float, default=2.0,
                    help="keep running untimed steps (beyond --warmup) until this much time has "
                         "passed, so the timed steps run at the GPU's steady clocks")
    ap.add_argument("--workload", default="d512_uih2k_c2k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--replay", action="store_true",
                    help="time-ordered streaming replay (page pool + paged cache) instead of the batch encode")
    ap.add_argument("--paged", choices=("shuffled", "ordered"), default=None,
                    help="workloads with a cached prefix: keep it in a paged cache of 64-row pages instead "
                         "of one slot per user, the page ids a random permutation of the pool (shuffled) "
                         "or each user's pages consecutive (ordered)")
    ap.add_argument("--weight-layout", choices=("prepared", "math"), default="prepared",
                    help="weights as the GEMMs read them (prepared once per model) or in the method's "
                         "layout W1 [D][4D], W2 [3D][D], transposed by every call into its workspace")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one step into a HIP graph after the timed steps and report "
                         "the rate of K replays of it beside the eager figures")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (to scale the HBM "
                         "byte counters of a profiler run) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); users are "
              f"independent, so N GPUs would each run this one-GPU workload on their own users.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    hsa.load_library()
    if args.replay:
        replay_bench(args)
        return
    dev = torch.device("cuda:0")
    wl = workloads.make_workload(args.workload)
    if wl.dtype != "bf16" or (wl.cached_lengths.any() and wl.packing != "none"):
        print("bench.py times the bf16 workloads (a cached prefix only with plain tokens)", file=sys.stderr)
        sys.exit(1)
    model = hsa.Model(wl.params, d_model=wl.d_model, heads=wl.heads, max_len=wl.max_len,
                      dtype=wl.dtype, device=dev, weight_layout=args.weight_layout)
    bf = lambda a: torch.from_numpy(a).to(device=dev, dtype=torch.bfloat16)
    cand = bf(wl.cand)
    eo = workloads.lengths_to_offsets(wl.uih_lengths)
    uo = workloads.lengths_to_offsets(token_lengths(wl))
    co = workloads.lengths_to_offsets(wl.cand_lengths)
    if wl.packing == "none":
        uih = bf(wl.uih)
    else:                                 # per-event context and action embeddings
        ctx, act = bf(wl.uih), bf(wl.action)
        uih = torch.empty((int(uo[-1]), wl.d_model), dtype=torch.bfloat16, device=dev)
    out = (torch.empty_like(uih), torch.empty_like(cand))
    ws = torch.empty(hsa.workspace_bytes(model, uo, co), dtype=torch.uint8, device=dev)
    cached = wl.cached_lengths.astype(np.int32)
    cache = None
    if cached.any():
        # streaming: each user's prefix goes into its cache slot once (untimed, no
        # candidates); every step then encodes the new events and the candidates against
        # it, with the cached lengths reset first, so each step rewrites the same rows
        cap = int((wl.cached_lengths + wl.uih_lengths).max())
        if args.paged:
            ppu = (cap + hsa.PAGE_ROWS - 1) // hsa.PAGE_ROWS
            cache = hsa.PagedKVCache(model, pages=wl.users * ppu, pages_per_user=ppu, max_users=wl.users, device=dev)
            ids = np.arange(wl.users * ppu).reshape(wl.users, ppu)
            if args.paged == "shuffled":
                ids = np.random.default_rng(0).permutation(wl.users * ppu).reshape(wl.users, ppu)
            cache.set_table(ids)
        else:
            cache = hsa.KVCache(model, slots=wl.users, capacity=cap, device=dev)
        po = workloads.lengths_to_offsets(wl.cached_lengths)
        hsa.encode(model, bf(wl.prefix), po, cand[:0], np.zeros(wl.users + 1, np.int32), cache=cache)
        torch.cuda.synchronize()
        assert cache.cached_len.tolist() == cached.tolist()
    st, alg_flops, formula_flops = hsa.hstu_flops(model.dims(), wl.users, uo, co, cached if cache else None)
    assert st == 0
    alg_flops += head_flops(wl)
    if wl.head:
        head = hsa.ScoringHead(wl.head, dtype=wl.dtype, device=dev)
        prob = torch.empty((int(co[-1]), head.outcomes), dtype=torch.float32, device=dev)

    def step():
        # the current stream: the default one, or the capture stream of a graph
        stream = torch.cuda.current_stream(dev).cuda_stream
        if wl.packing != "none":
            hsa.pack_uih(model, ctx, act, eo, wl.packing, out=uih, stream=stream)
        if cache is not None:
            cache.cached_len[:] = cached
        hsa.encode(model, uih, uo, cand, co, cache=cache, out=out, workspace=ws, stream=stream)
        if wl.head:
            hsa.score(model, head, out[1], out=prob, stream=stream)

    t_w = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        step()
        done += 1
        if done >= args.warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # Every step is timed by the wall clock. Each step also brackets the launches of one
    # group of kernel kinds with HIP events, the groups taken in turn: events cost device
    # time between kernels, so timing every launch of every step would slow the step.
    phases = [("attention",), ("uvqk",), ("out",), ("plan", "norm", "pack", "score")]
    phase_steps = [0] * len(phases)
    # one event between consecutive steps on the launch stream gives each step's device
    # time (median and minimum reported beside the mean)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    hsa.hstu_timing_enable(True)
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(args.steps):
        hsa.hstu_timing_select(phases[i % len(phases)])
        phase_steps[i % len(phases)] += 1
        step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    sclk = gpu_sclk_mhz()                 # read right after the timed steps
    hsa.hstu_timing_enable(False)
    hsa.hstu_timing_select(None)
    st, ktimes = hsa.hstu_timing_read()
    assert st == 0
    steps_of = {k: phase_steps[j] for j, ph in enumerate(phases) for k in ph}
    finite = bool(torch.isfinite(out[0].float()).all().item() and torch.isfinite(out[1].float()).all().item())
    if wl.head:
        finite = finite and bool(((prob >= 0) & (prob <= 1)).all().item())

    sec = (t1 - t0) / args.steps
    tflops = alg_flops / sec / 1e12
    per_launch = kernel_flops_per_launch(wl)
    per_step = {k: (ms / steps_of[k] if steps_of.get(k) else 0.0) for k, (ms, n) in ktimes.items()}
    kernels = {k: {"avg_ms": (ms / n if n else 0.0), "launches": n, "timed_steps": steps_of.get(k, 0),
                   "share": per_step[k] / max(sum(per_step.values()), 1e-12)}
               for k, (ms, n) in ktimes.items()}
    dominant = max(("uvqk", "attention", "out"), key=lambda k: kernels[k]["avg_ms"])
    avg_s = kernels[dominant]["avg_ms"] / 1e3
    achieved = per_launch[dominant] / avg_s / 1e12
    for k in ("uvqk", "attention", "out", "score"):
        a_ms = kernels[k]["avg_ms"]
        if a_ms:
            kernels[k]["tflops"] = per_launch[k] / (a_ms / 1e3) / 1e12
            # HBM rate from the committed counter summary of this kernel (when it was
            # taken on the current source), over this run's average launch time
            t = read_traffic(k, args.workload) if k in KERNEL_SOURCES else None
            if t:
                kernels[k]["hbm_gbs"] = t / (a_ms / 1e3) / 1e9
    traffic = read_traffic(dominant, args.workload)
    # the bound of the dominant kernel: its algorithmic flops per algorithmic byte against
    # the ridge point of the two peaks
    nbytes = kernel_bytes_per_launch(wl)[dominant]
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if per_launch[dominant] / nbytes >= ridge:
        roof = {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
    else:
        gbs = nbytes / avg_s / 1e9
        roof = {"kernel": dominant, "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                "tflops": round(achieved, 2)}
    result = {
        "metric": "HSTU encoder TFLOP/s (% bf16 MFMA peak) + users/s, D=512 UIH~2K, 2K cands",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": done,
        "ms_per_step": round(sec * 1e3, 4),
        "step_ms": {"median": round(float(np.median(step_ms)), 4), "min": round(float(np.min(step_ms)), 4)},
        "sclk_mhz_after": sclk,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: lognormal UIH lengths, N(0,1) tokens, N(0,1/D) weights, "
                "N(0,0.02) position bias)" + ("" if wl.packing == "none" else
                                              "; N(0,1) context and action embeddings per event"),
        "config": {"workload": args.workload, "users": wl.users, "layers": wl.layers,
                   **({"weight_layout": "math"} if args.weight_layout == "math" else {}),
                   **({"cached_per_user": int(wl.cached_lengths[0]),
                       "cache_layout": f"paged (64-row pages, {args.paged} ids)" if args.paged else "slot"}
                    if cache is not None else {}),
                   "d_model": wl.d_model, "heads": wl.heads, "cands_per_user": int(wl.cand_lengths[0]),
                   "uih_mean": float(token_lengths(wl).mean()),
                   "rows": int(token_lengths(wl).sum() + wl.cand_lengths.sum()),
                   **({} if wl.packing == "none" else
                      {"packing": wl.packing, "events_mean": float(wl.uih_lengths.mean())}),
                   **({"head": [int(w.shape[0]) for w, _ in wl.head]} if wl.head else {})},
        "users_per_s": round(wl.users / sec, 2),
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "formula_tflops": round(formula_flops / sec / 1e12, 3),
        "algorithmic_tflop_per_step": alg_flops / 1e12,
        "outputs_finite": finite,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "roofline": roof,
    }
    if args.graph:
        result["graph"] = graph_replays(torch, step, args.steps, alg_flops, wl.users)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
        result["cpu_baseline"]["value"] = round(result["cpu_baseline"]["value"], 6)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
