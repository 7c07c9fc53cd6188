"""GPU parity at the workloads' full sizes.

The GPU always runs the whole batch in one hstu_encode call, as the benchmark does.
The oracle recomputes every user of the batch (users are independent, so a user's rows
depend on that user alone; the users are spread over worker processes), or, for the
16-layer long histories, single layers on sampled rows, fed with the GPU's own layer
input. Besides the normwise gate each workload reports the floored elementwise maximum,
the fraction of elements above the tolerance, and the error against the unrounded
float64 oracle for its longest and its median user."""
import numpy as np
import pytest

import hstu_silu_attention_amd as hsa
import oracle
import workloads
from gpu_util import (BF16_TOL, error_stats, gpu_encode, make_model, normwise_per_user, oracle_encode,
                      oracle_users, report, say, select_users, to_dev, to_np, torch_cuda)

pytestmark = pytest.mark.gpu


def compare_all_users(name, wl, gu, gc, *, uih=None, uih_lengths=None):
    """Every user's history and candidate rows against the oracle's bf16 mirror; the
    longest and the median user also against the unrounded float64 oracle (reported)."""
    ul = wl.uih_lengths if uih_lengths is None else uih_lengths
    users = list(range(wl.users))
    order = np.argsort(ul, kind="stable")
    pick = sorted({int(order[-1]), int(order[len(order) // 2])})
    ref = oracle_users(wl, users, "bf16", uih=uih, uih_lengths=uih_lengths, extra=[(b, "f64") for b in pick])
    worst = {"uih": error_stats([], [], BF16_TOL), "cand": error_stats([], [], BF16_TOL)}
    for b in users:
        ru, rc = ref[(b, "bf16")]
        line = []
        for kind, g, r, lens in (("uih", gu, ru, ul), ("cand", gc, rc, wl.cand_lengths)):
            e = error_stats(select_users(g, lens, [b]), r, BF16_TOL)
            line.append(f"{kind} {e['normwise']:.3e} (elem {e['elem_max']:.2e}, >tol {e['frac_above']:.1e})")
            for k in e:
                worst[kind][k] = max(worst[kind][k], e[k])
        say(f"  user {b} (UIH {ul[b]}, {wl.cand_lengths[b]} cand): " + "; ".join(line))
    rec = {"workload": name, "users": len(users), "bf16_mirror": worst, "f64_unrounded": {}}
    for b in pick:
        fu, fc = ref[(b, "f64")]
        eu = error_stats(select_users(gu, ul, [b]), fu, BF16_TOL)["normwise"]
        ec = error_stats(select_users(gc, wl.cand_lengths, [b]), fc, BF16_TOL)["normwise"]
        rec["f64_unrounded"][str(b)] = {"uih_rows": int(ul[b]), "uih": eu, "cand": ec}
        say(f"  user {b} vs unrounded f64 oracle: uih {eu:.3e} cand {ec:.3e}")
    say(f"  {name}: worst {worst}")
    report(rec)
    assert worst["uih"]["normwise"] <= BF16_TOL and worst["cand"]["normwise"] <= BF16_TOL


def compare_users(wl, gu, gc, users):
    ru, rc, _ = oracle_encode(wl, "bf16", users=users)
    worst = 0.0
    for b in users:
        eu = normwise_per_user(select_users(gu, wl.uih_lengths, [b]), select_users(ru, wl.uih_lengths, [b]),
                               [wl.uih_lengths[b]])
        ec = normwise_per_user(select_users(gc, wl.cand_lengths, [b]), select_users(rc, wl.cand_lengths, [b]),
                               [wl.cand_lengths[b]])
        say(f"  user {b} (UIH {wl.uih_lengths[b]}, {wl.cand_lengths[b]} cand): uih {eu:.3e} cand {ec:.3e}")
        worst = max(worst, eu, ec)
    assert worst <= BF16_TOL


@pytest.mark.timeout(900)
def test_headline_workload_all_users():
    """D=512, UIH ~2K (lognormal, up to 4096), 2048 candidates, 8 layers, 16 users: the
    benchmark's inputs and launch; every user recomputed by the oracle."""
    wl = workloads.make_workload("d512_uih2k_c2k")
    gu, gc = gpu_encode(wl)
    compare_all_users("d512_uih2k_c2k", wl, gu, gc)


@pytest.mark.timeout(900)
def test_relative_bias_workload_all_users():
    """The headline workload in the original HSTU form (relative position bias, no absolute
    table): every user recomputed by the oracle."""
    wl = workloads.make_workload("d512_uih2k_c2k_rel")
    gu, gc = gpu_encode(wl)
    compare_all_users("d512_uih2k_c2k_rel", wl, gu, gc)


@pytest.mark.timeout(1200)
def test_interleaved_workload_all_users():
    """The headline workload's users in the original HSTU input form: each event's context
    and action embeddings interleaved by hstu_pack_uih on the GPU (about 3.7K tokens per
    user, up to 8192), the whole batch encoded in one call as the benchmark does; every
    user packed and recomputed by the oracle."""
    torch = torch_cuda()
    wl = workloads.make_workload("d512_uih2k_c2k_interleaved")
    model = make_model(torch, wl)
    eo = workloads.lengths_to_offsets(wl.uih_lengths)
    tok, to = hsa.pack_uih(model, to_dev(torch, wl.uih, "bf16"), to_dev(torch, wl.action, "bf16"), eo,
                           "interleave")
    tl = np.diff(to.astype(np.int64))
    assert tl.tolist() == (2 * wl.uih_lengths).tolist()
    gu, gc = gpu_encode(wl, model=model, uih=tok, uih_lengths=tl)
    del tok
    rtok, _ = oracle.pack_uih(wl.uih, wl.action, eo, "interleave", bf16=True)
    compare_all_users("d512_uih2k_c2k_interleaved", wl, gu, gc, uih=rtok, uih_lengths=tl)


@pytest.mark.timeout(900)
def test_scored_workload():
    """The benchmark's users with the 512-256-1 scoring head, as the benchmark launches it:
    one hstu_score over all 32 768 candidate rows. The head alone is checked on every row
    (the oracle's head fed with the GPU's encoder outputs, to 4e-3), and the whole
    prediction of every user against the oracle's encoder and head (to 2e-2)."""
    torch = torch_cuda()
    wl = workloads.make_workload("d512_uih2k_c2k_scored")
    model = make_model(torch, wl)
    _, dc = gpu_encode(wl, model=model, keep_device=True)
    head = hsa.ScoringHead(wl.head, dtype="bf16")
    prob = hsa.score(model, head, dc)
    torch.cuda.synchronize()
    got = prob.cpu().numpy().astype(np.float64)
    x = dc.float().cpu().numpy().astype(np.float64)
    alone = float(np.max(np.abs(got - oracle.score_head(x, wl.head, bf16=True))))
    say(f"  head alone, {got.shape[0]} rows: max |dp| = {alone:.3e}")
    assert alone <= 4e-3
    ref = oracle_users(wl, list(range(wl.users)), "bf16")
    worst = 0.0
    for b in range(wl.users):
        want = oracle.score_head(ref[b][1], wl.head, bf16=True)
        err = float(np.max(np.abs(select_users(got, wl.cand_lengths, [b]) - want)))
        say(f"  user {b} (UIH {wl.uih_lengths[b]}): encode+score max |dp| = {err:.3e}")
        worst = max(worst, err)
    report({"workload": "d512_uih2k_c2k_scored", "users": wl.users, "head_alone_max_dp": alone,
            "encode_score_max_dp": worst})
    assert worst <= 2e-2


def test_d256_workload_all_users():
    """D=256, 4 layers, 32 users, UIH uniform [256, 1024], 64 candidates: every user checked."""
    wl = workloads.make_workload("d256_uih1k_c64")
    gu, gc = gpu_encode(wl)
    ru, rc, _ = oracle_encode(wl, "bf16")
    eu = normwise_per_user(gu, ru, wl.uih_lengths)
    ec = normwise_per_user(gc, rc, wl.cand_lengths)
    say(f"  d256 all users: uih {eu:.3e} cand {ec:.3e}")
    assert eu <= BF16_TOL and ec <= BF16_TOL


def test_d384_projection_tiles_inside_column_blocks():
    """D=384 (three 128-wide heads) over enough rows that the projection would fill the
    GPU with its widest tiles: D is not a multiple of their width, so those tiles would
    straddle the U/V/Q/K column blocks; every user is checked."""
    wl = workloads.make_custom(seed=384, dtype="bf16", layers=1, d_model=384, heads=3, max_len=4400,
                               uih_lengths=[4000, 3000, 2500, 1500], cand_lengths=[300, 64, 17, 0])
    gu, gc = gpu_encode(wl)
    compare_users(wl, gu, gc, [0, 1, 2, 3])


def test_streaming_workload_sampled_user():
    """64 users, each with a 3000-event cached prefix (filled by hstu_encode with no
    candidates), then 300 new events + 2048 candidates against the cache. One user is
    recomputed by the oracle, prefix fill included, on a one-user batch."""
    torch = torch_cuda()
    wl = workloads.make_workload("stream_3000p300_c2k")
    B, L, D = wl.users, wl.layers, wl.d_model
    model = make_model(torch, wl)
    cap = 3300
    cache = hsa.KVCache(model, slots=B, capacity=cap)
    cache.cached_len = np.zeros(B, dtype=np.int32)
    empty = np.zeros((0, D), np.float32)
    gpu_encode(wl, model=model, uih=wl.prefix, cand=empty, uih_lengths=wl.cached_lengths,
               cand_lengths=np.zeros(B, np.int64), cache=cache)
    assert cache.cached_len.tolist() == [3000] * B
    gu, gc = gpu_encode(wl, model=model, cache=cache)
    assert cache.cached_len.tolist() == [3300] * B
    b = 37
    n, c, m = int(wl.uih_lengths[b]), int(wl.cand_lengths[b]), int(wl.cached_lengths[b])
    pre = wl.prefix[b * m:(b + 1) * m]
    ocache = oracle.OracleCache(np.zeros((L, 1, cap, D)), np.zeros((L, 1, cap, D)), np.array([0]),
                                np.array([0]))
    _, _, ocache = oracle.encode(pre, [0, m], empty, [0, 0], wl.params, heads=wl.heads, max_len=wl.max_len,
                                 mode="bf16", cache=ocache)
    ru, rc, ocache = oracle.encode(wl.uih[b * n:(b + 1) * n], [0, n], wl.cand[b * c:(b + 1) * c], [0, c],
                                   wl.params, heads=wl.heads, max_len=wl.max_len, mode="bf16", cache=ocache)
    eu = normwise_per_user(gu[b * n:(b + 1) * n], ru, [n])
    ec = normwise_per_user(gc[b * c:(b + 1) * c], rc, [c])
    gk = to_np(cache.k[:, b])
    ek = max(float(np.max(np.abs(gk[l, :m + n] - ocache.k[l, 0, :m + n])) / np.max(np.abs(ocache.k[l, 0, :m + n])))
             for l in range(L))
    say(f"  streaming user {b}: uih {eu:.3e} cand {ec:.3e} cached K {ek:.3e}")
    assert eu <= BF16_TOL and ec <= BF16_TOL and ek <= BF16_TOL


def test_streaming_workload_paged_matches_slot():
    """The streaming workload (64 users, 3000 cached + 300 new rows, 2048 candidates, 8
    layers) with its cache in 64-row pages under shuffled page ids, as `bench.py --paged`
    runs it, against the slot layout: every output row and every cached row agree bit for
    bit (the kernels add in the same order; only addresses differ)."""
    torch = torch_cuda()
    wl = workloads.make_workload("stream_3000p300_c2k")
    B, D = wl.users, wl.d_model
    model = make_model(torch, wl)
    empty = np.zeros((0, D), np.float32)
    cap = 3300
    ppu = (cap + 63) // 64
    slot = hsa.KVCache(model, slots=B, capacity=cap)
    paged = hsa.PagedKVCache(model, pages=B * ppu, pages_per_user=ppu, max_users=B)
    ids = np.random.default_rng(0).permutation(B * ppu).reshape(B, ppu).astype(np.int32)
    paged.set_table(ids)
    outs = []
    for cache in (slot, paged):
        cache.cached_len = np.zeros(B, dtype=np.int32)
        gpu_encode(wl, model=model, uih=wl.prefix, cand=empty, uih_lengths=wl.cached_lengths,
                   cand_lengths=np.zeros(B, np.int64), cache=cache)
        outs.append(gpu_encode(wl, model=model, cache=cache))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    idx = torch.from_numpy(ids.astype(np.int64)).to(paged.k.device)
    for name in ("k", "v"):
        ps = getattr(paged, name)[:, idx].reshape(wl.layers, B, ppu * 64, D)[:, :, :cap]
        assert torch.equal(ps, getattr(slot, name))
    say(f"  streaming workload, paged cache ({B * ppu} pages) = slot cache, bit for bit")


@pytest.mark.parametrize("name", ["long_uih16k_c2k", "long_uih16k_c2k_rel"])
def test_long_workload_layerwise_sampled_rows(name):
    """16 layers, 4 users with UIH 8K-16K, 2048 candidates, 8 heads (dh 64), with the
    absolute position table, and in the original HSTU form with a relative table over
    positions up to 16384. The full call equals the chain of 16 one-layer calls bit for
    bit; layers 0, 7 and 15 are then checked row by row against the oracle on sampled
    history and candidate rows of every user, fed with the GPU's own input to that layer."""
    torch = torch_cuda()
    wl = workloads.make_workload(name)
    D = wl.d_model
    full_u, full_c = gpu_encode(wl, keep_device=True)
    full_u, full_c = to_np(full_u), to_np(full_c)
    xs = [(to_dev(torch, wl.uih, "bf16"), to_dev(torch, wl.cand, "bf16"))]
    for l in range(wl.layers):
        m1 = hsa.Model([wl.params[l]], d_model=D, heads=wl.heads, max_len=wl.max_len, dtype="bf16")
        xs.append(gpu_encode(wl, model=m1, uih=xs[-1][0], cand=xs[-1][1], keep_device=True))
        del m1
    assert np.array_equal(to_np(xs[-1][0]), full_u) and np.array_equal(to_np(xs[-1][1]), full_c)
    uo = workloads.lengths_to_offsets(wl.uih_lengths)
    co = workloads.lengths_to_offsets(wl.cand_lengths)
    rng = np.random.default_rng(5)
    worst = 0.0
    for l in (0, 7, 15):
        p = wl.params[l]
        f64 = lambda a: None if a is None else a.astype(np.float64)
        w1, w2, pos, rel = f64(p.w1), f64(p.w2), f64(p.pos), f64(getattr(p, "rel", None))
        xin_u, xin_c = to_np(xs[l][0]), to_np(xs[l][1])
        xo_u, xo_c = to_np(xs[l + 1][0]), to_np(xs[l + 1][1])
        for b in range(wl.users):
            n, c = int(wl.uih_lengths[b]), int(wl.cand_lengths[b])
            rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, n - 2, n - 1], rng.integers(0, n, 24)]))
            crows = np.unique(np.concatenate([[0, c - 1], rng.integers(0, c, 14)]))
            yu, yc, _, _ = oracle.layer_user(xin_u[uo[b]:uo[b + 1]], xin_c[co[b]:co[b + 1]], w1, w2, pos,
                                             k_cached=np.zeros((0, D)), v_cached=np.zeros((0, D)),
                                             heads=wl.heads, max_len=wl.max_len, bf16=True,
                                             uih_rows=rows, cand_rows=crows, rel=rel)
            gu_rows = xo_u[uo[b] + rows]
            gc_rows = xo_c[co[b] + crows]
            eu = float(np.max(np.abs(gu_rows - yu)) / np.max(np.abs(yu)))
            ec = float(np.max(np.abs(gc_rows - yc)) / np.max(np.abs(yc)))
            worst = max(worst, eu, ec)
        say(f"  {name}: layer {l} worst sampled normwise error so far {worst:.3e}")
    assert worst <= BF16_TOL
