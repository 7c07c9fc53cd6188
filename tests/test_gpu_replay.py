"""GPU check of time-ordered request replay over the paged streaming cache and the page
pool: every request's candidate outputs and the outputs of the history rows it sent equal
the oracle's one-shot encode of the user's cached window plus those rows (bfloat16
normwise <= 2e-2). The stream is built so that cache hits, evictions, stale rebuilds and
rebuilds for want of room all occur; every user holds ceil(rows / 64) pages."""
import numpy as np
import pytest

import hstu_silu_attention_amd as hsa
import oracle
import workloads
from gpu_util import BF16_TOL, make_model, say, torch_cuda
from hstu_silu_attention_amd.replay import Replayer, Request

pytestmark = pytest.mark.gpu


def _stream(rng, users, D, requests):
    history = {u: workloads.to_bf16_values(rng.standard_normal((700, D)).astype(np.float32)) for u in range(users)}
    seen = dict.fromkeys(range(users), 0)
    out, t = [], 0
    for _ in range(requests):
        t += int(rng.integers(0, 9))
        u = int(rng.integers(0, users))
        seen[u] = min(700, seen[u] + int(rng.integers(0, 61)))
        c = int(rng.integers(1, 13))
        out.append(Request(t, u, seen[u], workloads.to_bf16_values(rng.standard_normal((c, D)).astype(np.float32))))
    return history, out


def test_replay_matches_one_shot_encodes():
    torch = torch_cuda()
    D, H, L = 256, 2, 2
    wl = workloads.make_custom(seed=501, dtype="bf16", layers=L, d_model=D, heads=H, max_len=400,
                               uih_lengths=[0], cand_lengths=[0], position="both", rel_std=0.3)
    model = make_model(torch, wl)
    cache = hsa.PagedKVCache(model, pages=20, pages_per_user=4, max_users=4)
    pool = hsa.KvPool(pages=20, max_rows=240, ttl=30)
    history, requests = _stream(np.random.default_rng(5), users=14, D=D, requests=80)
    rep = Replayer(model, cache, pool, history, window=200)
    served = []
    for batch in rep.batches_of(requests, max_users=4):
        served += rep.serve(batch)
    stats = pool.stats()
    say(f"  replay: {len(served)} requests in {rep.batches} batches, {rep.rows_sent} rows sent; {stats}")
    assert all(stats[k] > 0 for k in ("hits", "rebuild_new", "rebuild_stale", "rebuild_full", "evictions"))
    held = [pool.lookup(u) for u in history]
    assert all(p == (n + 63) // 64 for n, p in held)
    assert stats["pages_in_use"] == sum(p for _, p in held)
    worst = 0.0
    for s in served:
        r = s.request
        hist = history[r.user][s.window_start:r.events]
        ru, rc, _ = oracle.encode(hist, [0, hist.shape[0]], r.cand, [0, r.cand.shape[0]], wl.params,
                                  heads=H, max_len=400, mode="bf16")
        sent = ru[s.sent_from - s.window_start:]
        assert sent.shape == s.uih_out.shape
        for g, w in ((s.uih_out, sent), (s.cand_out, rc)):
            if w.size:
                worst = max(worst, float(np.max(np.abs(g - w)) / np.max(np.abs(w))))
    say(f"  worst normwise error {worst:.3e}")
    assert worst <= BF16_TOL
