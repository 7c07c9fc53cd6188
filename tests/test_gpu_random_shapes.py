"""GPU parity over seeded random configurations, beside the hand-picked cases: dtype, head
width (32, 64, 128) and count, 1-6 users with ragged lengths and empty users, no cache, a
slot cache or a paged cache (shuffled page ids) with cached prefixes, absolute, relative
or both position biases, one or two layers, weights prepared or in the method's layout; the wide draw goes to 8 users, histories of
up to 900 new and 600 cached rows, 400 candidates, 3 or 6 heads and D up to 768. Each
case fills the cache with the prefixes (no candidates), then encodes the new events and
candidates; every user's outputs are held to the oracle's bar (bf16 mirror or float64),
the oracle doing the same two calls. The large draw (one layer, 4-16 users, up to 2500
new and 1500 cached rows, 1200 candidates, D 256-1024) reaches the batch sizes at which
the projection takes its 256 x 128 and 128 x 128 ring tiles and the output GEMM its
256 x 256 tile."""
import numpy as np
import pytest

import hstu_silu_attention_amd as hsa
import workloads
from gpu_util import BF16_TOL, F32_TOL, gpu_encode, normwise_per_user, oracle_encode, say, torch_cuda

pytestmark = pytest.mark.gpu

SEEDS = list(range(9100, 9116))
WIDE_SEEDS = list(range(9200, 9216))
# large draws covering each projection tile and the output GEMM's large tile, with every
# cache layout: 40000 (128 x 128 ring, paged), 40003 and 40007 (256 x 128, 256 x 256, paged),
# 40008 and 40011 (slot cache; the latter 16 heads of 64), 40014 (no cache)
LARGE_SEEDS = [40000, 40003, 40007, 40008, 40011, 40014]


def draw(seed):
    rng = np.random.default_rng(seed)
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    dh = int(rng.choice([32, 64, 128]))
    unit = 128 if dtype == "bf16" else 64            # D must be a multiple of this
    heads = [h for h in (1, 2, 4, 8) if (dh * h) % unit == 0 and dh * h <= 512]
    H = int(rng.choice(heads))
    B = int(rng.integers(1, 7))
    uih = np.where(rng.random(B) < 0.2, 0, rng.integers(1, 400, B))
    cand = np.where(rng.random(B) < 0.25, 0, rng.integers(1, 200, B))
    cache = str(rng.choice(["none", "slot", "paged"]))
    cached = np.zeros(B, np.int64) if cache == "none" else np.where(rng.random(B) < 0.3, 0, rng.integers(1, 300, B))
    position = str(rng.choice(["absolute", "relative", "both"]))
    layers = int(rng.integers(1, 3))
    max_len = int((cached + uih).max()) + 1 + int(rng.integers(0, 100))   # every candidate position fits
    weights = "math" if rng.random() < 0.3 else "prepared"
    return dict(dtype=dtype, D=dh * H, H=H, B=B, uih=uih, cand=cand, cache=cache, cached=cached,
                position=position, layers=layers, max_len=max_len, weights=weights)


def draw_wide(seed):
    rng = np.random.default_rng(seed)
    dtype = "bf16" if rng.random() < 0.8 else "f32"
    dh = int(rng.choice([32, 64, 128]))
    unit = 128 if dtype == "bf16" else 64
    heads = [h for h in (1, 2, 3, 4, 6, 8) if (dh * h) % unit == 0 and dh * h <= 768]
    H = int(rng.choice(heads))
    B = int(rng.integers(1, 9))
    uih = np.where(rng.random(B) < 0.15, 0, rng.integers(1, 900, B))
    cand = np.where(rng.random(B) < 0.2, 0, rng.integers(1, 400, B))
    cache = str(rng.choice(["none", "slot", "paged"]))
    cached = np.zeros(B, np.int64) if cache == "none" else np.where(rng.random(B) < 0.3, 0, rng.integers(1, 600, B))
    position = str(rng.choice(["absolute", "relative", "both"]))
    layers = int(rng.integers(1, 3))
    max_len = int((cached + uih).max()) + 1 + int(rng.integers(0, 300))
    weights = "math" if rng.random() < 0.3 else "prepared"
    return dict(dtype=dtype, D=dh * H, H=H, B=B, uih=uih, cand=cand, cache=cache, cached=cached,
                position=position, layers=layers, max_len=max_len, weights=weights)


def draw_large(seed):
    rng = np.random.default_rng(seed)
    D = int(rng.choice([256, 512, 768, 1024]))
    dh = int(rng.choice([64, 128])) if D != 768 else 128
    B = int(rng.integers(4, 17))
    uih = np.where(rng.random(B) < 0.1, 0, rng.integers(1, 2500, B))
    cand = np.where(rng.random(B) < 0.1, 0, rng.integers(1, 1200, B))
    cache = str(rng.choice(["none", "slot", "paged"]))
    cached = np.zeros(B, np.int64) if cache == "none" else np.where(rng.random(B) < 0.3, 0, rng.integers(1, 1500, B))
    position = str(rng.choice(["absolute", "relative", "both"]))
    max_len = int((cached + uih).max()) + 1 + int(rng.integers(0, 300))
    weights = "math" if rng.random() < 0.3 else "prepared"
    return dict(dtype="bf16", D=D, H=D // dh, B=B, uih=uih, cand=cand, cache=cache, cached=cached,
                position=position, layers=1, max_len=max_len, weights=weights)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_configuration(seed):
    run_configuration(seed, draw(seed))


@pytest.mark.parametrize("seed", WIDE_SEEDS)
def test_random_wide_configuration(seed):
    run_configuration(seed, draw_wide(seed))


@pytest.mark.parametrize("seed", LARGE_SEEDS)
def test_random_large_configuration(seed):
    run_configuration(seed, draw_large(seed))


def run_configuration(seed, c):
    torch = torch_cuda()
    say(f"  seed {seed}: {c['dtype']} D={c['D']} H={c['H']} B={c['B']} layers={c['layers']} cache={c['cache']} "
        f"weights={c.get('weights', 'prepared')} "
        f"{c['position']} uih={c['uih'].tolist()} cand={c['cand'].tolist()} cached={c['cached'].tolist()}")
    wl = workloads.make_custom(seed=seed, dtype=c["dtype"], layers=c["layers"], d_model=c["D"], heads=c["H"],
                               max_len=c["max_len"], uih_lengths=c["uih"], cand_lengths=c["cand"],
                               cached_lengths=c["cached"], position=c["position"], rel_std=0.3)
    B, D, L = wl.users, wl.d_model, wl.layers
    model = hsa.Model(wl.params, d_model=wl.d_model, heads=wl.heads, max_len=wl.max_len, dtype=wl.dtype,
                      weight_layout=c.get("weights", "prepared"))
    total = wl.cached_lengths + wl.uih_lengths
    cap = max(int(total.max()), 1)
    empty = np.zeros((0, D), np.float32)
    if c["cache"] == "none":
        gu, gc = gpu_encode(wl, model=model)
        ocache = None
    else:
        if c["cache"] == "slot":
            cache = hsa.KVCache(model, slots=B + 2, capacity=cap + 5)
            cache.slot_of_user = np.random.default_rng(seed).permutation(B + 2)[:B].astype(np.int32)
        else:
            ppu = (cap + 63) // 64
            npool = B * ppu + 3
            ids = np.random.default_rng(seed).permutation(npool)[:B * ppu].reshape(B, ppu).astype(np.int32)
            cache = hsa.PagedKVCache(model, pages=npool, pages_per_user=ppu, max_users=B)
            cache.set_table(ids)
        cache.cached_len = np.zeros(B, dtype=np.int32)
        gpu_encode(wl, model=model, uih=wl.prefix, cand=empty, uih_lengths=wl.cached_lengths,
                   cand_lengths=np.zeros(B, np.int64), cache=cache)
        assert cache.cached_len[:B].tolist() == wl.cached_lengths.tolist()
        gu, gc = gpu_encode(wl, model=model, cache=cache)
        assert cache.cached_len[:B].tolist() == total.tolist()
        import oracle
        ocache = oracle.OracleCache(np.zeros((L, B, cap, D)), np.zeros((L, B, cap, D)), np.arange(B),
                                    np.zeros(B, np.int64))
    mode = "bf16" if c["dtype"] == "bf16" else "f64"
    tol = BF16_TOL if c["dtype"] == "bf16" else F32_TOL
    if ocache is not None:
        _, _, ocache = oracle_encode(wl, mode, cache=ocache, uih=wl.prefix, uih_lengths=wl.cached_lengths,
                                     cand=empty, cand_lengths=np.zeros(B, np.int64))
    ru, rc, _ = oracle_encode(wl, mode, cache=ocache)
    eu, ec = normwise_per_user(gu, ru, wl.uih_lengths), normwise_per_user(gc, rc, wl.cand_lengths)
    say(f"  normwise error: uih {eu:.3e} cand {ec:.3e} (tol {tol})")
    assert eu <= tol and ec <= tol
