"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element,
on seeded inputs that span several tiles with ragged tails, empty users and the cache path.

bfloat16: normwise error <= 2e-2 per user and output tensor against the oracle's bfloat16
mirror; float32: <= 1e-4 against the float64 oracle."""
import numpy as np
import pytest

import hstu_silu_attention_amd as hsa
import workloads
from gpu_util import (BF16_TOL, F32_TOL, gpu_encode, make_model, normwise_per_user, oracle_encode,
                      say, to_dev, to_np, torch_cuda)

pytestmark = pytest.mark.gpu


def check(wl, got_u, got_c, mode, tol, cache=None, label=""):
    ru, rc, _ = oracle_encode(wl, mode, cache=cache)
    eu = normwise_per_user(got_u, ru, wl.uih_lengths)
    ec = normwise_per_user(got_c, rc, wl.cand_lengths)
    say(f"  {label} normwise err uih={eu:.3e} cand={ec:.3e} (tol {tol})")
    assert eu <= tol and ec <= tol
    return ru, rc


def test_tiny_f32_workload():
    wl = workloads.make_workload("tiny_f32")
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "f64", F32_TOL, label="tiny_f32")


@pytest.mark.parametrize("D,H", [(128, 2), (128, 1), (256, 8)])
def test_f32_ragged(D, H):
    wl = workloads.make_custom(seed=100 + H, dtype="f32", layers=2, d_model=D, heads=H, max_len=300,
                               uih_lengths=[0, 1, 63, 65, 200], cand_lengths=[3, 0, 64, 1, 70])
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "f64", F32_TOL, label=f"f32 D={D} H={H}")


@pytest.mark.parametrize("D,H", [(256, 4), (256, 2), (512, 8), (512, 4), (640, 10), (768, 6), (1024, 8),
                                 (256, 8), (512, 16)])
def test_bf16_ragged(D, H):
    """dh = 32, 64 and 128; histories of 0, 1, 127, 129, 300 rows and candidate sets of 1, 0, 130,
    5, 64 rows cover empty users, single rows and ragged tails of 128-row query tiles and
    64-key blocks. Widths up to D = 1024, including ones whose projection column blocks are
    not whole 256-wide tiles (640, 768)."""
    wl = workloads.make_custom(seed=200 + D + H, dtype="bf16", layers=2, d_model=D, heads=H, max_len=400,
                               uih_lengths=[0, 1, 127, 129, 300], cand_lengths=[1, 0, 130, 5, 64])
    gu, gc = gpu_encode(wl)
    ru, rc = check(wl, gu, gc, "bf16", BF16_TOL, label=f"bf16 D={D} H={H}")
    fu, fc, _ = oracle_encode(wl, "f64")
    say(f"  vs unrounded f64 oracle: uih={normwise_per_user(gu, fu, wl.uih_lengths):.3e} "
        f"cand={normwise_per_user(gc, fc, wl.cand_lengths):.3e}")


@pytest.mark.parametrize("dtype,D,H", [("bf16", 4096, 32), ("bf16", 8192, 64), ("f32", 8128, 127)])
def test_widest_models(dtype, D, H):
    """Wide models, one layer: D = 4096 and 8192 in bfloat16 (32 and 64 heads of 128; the
    projection's N = 4D = 32768 columns, the row statistics of 64 column groups) and the
    most heads the planner takes, 127 heads of 64 in float32 (D = 8128), with both biases,
    ragged users and an empty one."""
    wl = workloads.make_custom(seed=5000 + H, dtype=dtype, layers=1, d_model=D, heads=H, max_len=200,
                               uih_lengths=[70, 0, 129], cand_lengths=[3, 9, 0], position="both")
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "bf16" if dtype == "bf16" else "f64", BF16_TOL if dtype == "bf16" else F32_TOL,
          label=f"{dtype} D={D} H={H}")


@pytest.mark.parametrize("dtype,tol", [("bf16", BF16_TOL), ("f32", F32_TOL)])
def test_history_fills_the_position_table(dtype, tol):
    """m + n + 1 == max_len: the candidates of the long user take the table's last row, its
    history rows every other one; a second user has no history (candidates at position 0)."""
    wl = workloads.make_custom(seed=811, dtype=dtype, layers=2, d_model=256 if dtype == "bf16" else 128,
                               heads=2, max_len=301, uih_lengths=[300, 0], cand_lengths=[4, 2])
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "bf16" if dtype == "bf16" else "f64", tol, label=f"{dtype} full position table")


@pytest.mark.parametrize("position", ["relative", "both"])
@pytest.mark.parametrize("D,H", [(256, 4), (512, 4), (256, 8)])
def test_bf16_relative_bias(D, H, position):
    """The original HSTU form: a relative position bias on every attention weight (alone,
    and with the absolute table), dh = 64 and 128, the ragged lengths of the other tests."""
    wl = workloads.make_custom(seed=900 + D + H, dtype="bf16", layers=2, d_model=D, heads=H, max_len=400,
                               uih_lengths=[0, 1, 127, 129, 300], cand_lengths=[1, 0, 130, 5, 64],
                               position=position, rel_std=0.3)
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "bf16", BF16_TOL, label=f"bf16 {position} bias D={D} H={H}")


@pytest.mark.parametrize("D,H,max_len,uih,cand", [
    (128, 1, 1, [0], [54]),            # a one-entry table: every candidate at position 0
    (128, 1, 3, [2, 0], [5, 3]),       # three entries
    (384, 3, 5, [4, 1], [3, 2]),       # 15 entries: head 2's distance 4 is the last
    (640, 5, 7, [6], [9]),             # 35 entries: head 4's distance 6 is the last
])
def test_bf16_relative_table_end(D, H, max_len, uih, cand):
    """Relative tables with an odd number of entries H * max_len: the last entry shares its
    4-byte word with bytes past the table. The kernel reads the table in 16-byte chunks
    through a buffer range, which returns zero for every word that crosses the range's end;
    the range must reach past the last entry (it ended at the last byte and lost that
    entry). Short histories, so the last distances weigh in every output."""
    wl = workloads.make_custom(seed=61 + max_len + H, dtype="bf16", layers=2, d_model=D, heads=H,
                               max_len=max_len, uih_lengths=uih, cand_lengths=cand, position="relative",
                               rel_std=1.0)
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "bf16", BF16_TOL, label=f"bf16 relative table of {H} x {max_len}")


@pytest.mark.parametrize("D,H", [(64, 2), (128, 2)])
def test_f32_relative_bias(D, H):
    wl = workloads.make_custom(seed=950 + D, dtype="f32", layers=2, d_model=D, heads=H, max_len=300,
                               uih_lengths=[0, 1, 63, 65, 200], cand_lengths=[3, 0, 64, 1, 70],
                               position="relative", rel_std=0.3)
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "f64", F32_TOL, label=f"f32 relative bias D={D} H={H}")


@pytest.mark.parametrize("D,H,max_len,n,m", [(256, 4, 7600, 4500, 0), (512, 4, 12000, 9000, 0),
                                              (256, 4, 12000, 1500, 8001)])
def test_bf16_relative_bias_long_table(D, H, max_len, n, m):
    """Long histories with a relative table of thousands of positions (dh 64 and 128; a
    table longer than one workgroup could hold in LDS; a cached prefix that puts the
    history's positions past 8000): the attention streams the table a slice per key
    block."""
    torch = torch_cuda()
    wl = workloads.make_custom(seed=977 + n, dtype="bf16", layers=1, d_model=D, heads=H, max_len=max_len,
                               uih_lengths=[n, 77], cand_lengths=[2, 130], cached_lengths=[m, 0],
                               position="relative", rel_std=0.3)
    if m == 0:
        gu, gc = gpu_encode(wl)
        check(wl, gu, gc, "bf16", BF16_TOL, label=f"bf16 relative bias, {n} history rows, max_len {max_len}")
        return
    import oracle
    model = make_model(torch, wl)
    cache = hsa.KVCache(model, slots=2, capacity=m + n)
    gu, gc = _fill_and_encode(wl, model, cache)
    ocache = oracle.OracleCache(np.zeros((1, 2, m + n, D)), np.zeros((1, 2, m + n, D)), np.arange(2),
                                np.zeros(2, np.int64))
    empty = np.zeros((0, D), np.float32)
    _, _, ocache = oracle_encode(wl, "bf16", cache=ocache, uih=wl.prefix, uih_lengths=wl.cached_lengths,
                                 cand=empty, cand_lengths=np.zeros(2, np.int64))
    ru, rc, _ = oracle_encode(wl, "bf16", cache=ocache)
    eu, ec = normwise_per_user(gu, ru, wl.uih_lengths), normwise_per_user(gc, rc, wl.cand_lengths)
    say(f"  bf16 relative bias after a {m}-row cached prefix: uih {eu:.3e} cand {ec:.3e}")
    assert eu <= BF16_TOL and ec <= BF16_TOL


@pytest.mark.parametrize("uih,cand", [
    ([1200, 900, 0], [301, 500, 99]),                         # 3000 rows: 128 x 128 tiles, one per CU
    ([3001, 2500, 1700, 0], [1024, 1499, 300, 1]),            # 10025 rows: 128 x 128 ring tiles, three per CU
    ([4000, 3901, 3000, 1999], [2048, 1100, 700, 301]),       # 17049 rows: 256 x 128 ring tiles, two per CU
])
def test_bf16_projection_tiles(uih, cand):
    """D = 512, one layer: batch sizes that select each of the projection's tile shapes (the
    launcher picks by the tile counts), ragged tails and an empty user; every user against
    the oracle."""
    wl = workloads.make_custom(seed=1200 + sum(uih), dtype="bf16", layers=1, d_model=512, heads=4, max_len=4200,
                               uih_lengths=uih, cand_lengths=cand)
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "bf16", BF16_TOL, label=f"bf16 projection tiles, {sum(uih) + sum(cand)} rows")


def test_bf16_single_layer_many_tiles():
    """One layer, long rows: attention work items of up to 16 key blocks per query tile."""
    wl = workloads.make_custom(seed=301, dtype="bf16", layers=1, d_model=256, heads=2, max_len=1100,
                               uih_lengths=[1000, 513], cand_lengths=[257, 3])
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "bf16", BF16_TOL, label="bf16 long rows")


@pytest.mark.parametrize("position", ["absolute", "both"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_streaming_cache(dtype, position):
    """Fill each user's cache slot with its prefix (no candidates), then encode the new events
    plus candidates against the cache; compare with the oracle doing the same, and with the
    GPU's own one-shot encode of prefix + new events. The cached keys are exactly the
    recomputed ones (the history mask is causal), but the two calls sum the attention in a
    different order: the kernel groups keys into 32-key halves counted from a key origin
    shifted by the cached length, so agreement is to the floating-point tolerance, not bit
    for bit."""
    torch = torch_cuda()
    D, H, L = (256, 2, 2) if dtype == "bf16" else (128, 2, 2)
    wl = workloads.make_custom(seed=401, dtype=dtype, layers=L, d_model=D, heads=H, max_len=500,
                               uih_lengths=[40, 0, 130, 7], cand_lengths=[9, 3, 65, 0],
                               cached_lengths=[200, 17, 129, 0], position=position, rel_std=0.3)
    B = wl.users
    model = make_model(torch, wl)
    cache = hsa.KVCache(model, slots=6, capacity=384)
    cache.slot_of_user = np.array([3, 0, 5, 1], dtype=np.int32)
    cache.cached_len = np.zeros(B, dtype=np.int32)
    empty = np.zeros((0, D), np.float32)
    gpu_encode(wl, model=model, uih=wl.prefix, cand=empty, uih_lengths=wl.cached_lengths,
               cand_lengths=np.zeros(B, np.int64), cache=cache)
    assert cache.cached_len.tolist() == wl.cached_lengths.tolist()
    gu, gc = gpu_encode(wl, model=model, cache=cache)
    assert cache.cached_len.tolist() == (wl.cached_lengths + wl.uih_lengths).tolist()

    import oracle
    ocache = oracle.OracleCache(np.zeros((L, 6, 384, D)), np.zeros((L, 6, 384, D)),
                                cache.slot_of_user.astype(np.int64), np.zeros(B, np.int64))
    mode = "bf16" if dtype == "bf16" else "f64"
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    _, _, ocache = oracle_encode(wl, mode, cache=ocache, uih=wl.prefix, uih_lengths=wl.cached_lengths,
                                 cand=empty, cand_lengths=np.zeros(B, np.int64))
    ru, rc, ocache = oracle_encode(wl, mode, cache=ocache)
    eu = normwise_per_user(gu, ru, wl.uih_lengths)
    ec = normwise_per_user(gc, rc, wl.cand_lengths)
    say(f"  streaming {dtype}: uih={eu:.3e} cand={ec:.3e}")
    assert eu <= tol and ec <= tol
    # cached keys/values of every layer against the oracle's
    gk, gv = to_np(cache.k), to_np(cache.v)
    for b in range(B):
        s, n_all = int(cache.slot_of_user[b]), int(cache.cached_len[b])
        if n_all == 0:
            continue
        for l in range(L):
            for g, r in [(gk[l, s, :n_all], ocache.k[l, s, :n_all]), (gv[l, s, :n_all], ocache.v[l, s, :n_all])]:
                assert np.max(np.abs(g - r)) <= tol * np.max(np.abs(r))
    # one-shot recompute on the GPU, no cache
    offs_p = workloads.lengths_to_offsets(wl.cached_lengths)
    offs_u = workloads.lengths_to_offsets(wl.uih_lengths)
    full = np.concatenate([np.concatenate([wl.prefix[offs_p[b]:offs_p[b + 1]], wl.uih[offs_u[b]:offs_u[b + 1]]])
                           for b in range(B)])
    full_len = wl.cached_lengths + wl.uih_lengths
    fu, fc = gpu_encode(wl, model=model, uih=full, uih_lengths=full_len)
    offs_f = workloads.lengths_to_offsets(full_len)
    new_rows = np.concatenate([fu[offs_f[b] + wl.cached_lengths[b]:offs_f[b + 1]] for b in range(B)])
    eu1 = normwise_per_user(gu, new_rows, wl.uih_lengths)
    ec1 = normwise_per_user(gc, fc, wl.cand_lengths)
    say(f"  streaming vs one-shot {dtype}: uih={eu1:.3e} cand={ec1:.3e}")
    assert eu1 <= tol and ec1 <= tol


def _fill_and_encode(wl, model, cache):
    """Prefix into the cache (no candidates), then the new events plus candidates."""
    B = wl.users
    empty = np.zeros((0, wl.d_model), np.float32)
    gpu_encode(wl, model=model, uih=wl.prefix, cand=empty, uih_lengths=wl.cached_lengths,
               cand_lengths=np.zeros(B, np.int64), cache=cache)
    assert cache.cached_len[:B].tolist() == wl.cached_lengths.tolist()
    out = gpu_encode(wl, model=model, cache=cache)
    assert cache.cached_len[:B].tolist() == (wl.cached_lengths + wl.uih_lengths).tolist()
    return out


@pytest.mark.parametrize("dtype,D,H,position", [("bf16", 512, 4, "absolute"), ("bf16", 256, 4, "both"),
                                                ("bf16", 512, 4, "relative"), ("bf16", 256, 8, "both"),
                                                ("f32", 128, 2, "both")])
def test_paged_cache_matches_slot_cache(dtype, D, H, position):
    """The paged layout (64-row pages, shuffled page ids, a device page table) against the
    slot layout on the same calls: the kernels add in the same order, so outputs and
    cached rows agree bit for bit; the outputs are also held to the oracle's bar. Cached
    lengths cross page boundaries mid-block (200, 17, 129, 0 then +40, 0, 130, 7)."""
    torch = torch_cuda()
    L = 2
    wl = workloads.make_custom(seed=1401, dtype=dtype, layers=L, d_model=D, heads=H, max_len=500,
                               uih_lengths=[40, 0, 130, 7], cand_lengths=[9, 3, 65, 0],
                               cached_lengths=[200, 17, 129, 0], position=position, rel_std=0.3)
    B = wl.users
    model = make_model(torch, wl)
    slot = hsa.KVCache(model, slots=4, capacity=400)
    slot.cached_len = np.zeros(B, dtype=np.int32)
    su, sc = _fill_and_encode(wl, model, slot)
    ppu, npool = 7, 40
    rng = np.random.default_rng(3)
    ids = rng.permutation(npool)[:B * ppu].reshape(B, ppu).astype(np.int32)
    paged = hsa.PagedKVCache(model, pages=npool, pages_per_user=ppu, max_users=B)
    paged.set_table(ids)
    paged.cached_len = np.zeros(B, dtype=np.int32)
    pu, pc = _fill_and_encode(wl, model, paged)
    assert np.array_equal(pu, su) and np.array_equal(pc, sc)
    total = wl.cached_lengths + wl.uih_lengths
    for name in ("k", "v"):
        sk, pk = to_np(getattr(slot, name)), to_np(getattr(paged, name))
        for b in range(B):
            rows = np.concatenate([pk[:, ids[b, i]] for i in range(ppu)], axis=1)   # [L][ppu*64][D]
            assert np.array_equal(rows[:, :total[b]], sk[:, b, :total[b]])
    import oracle
    ocache = oracle.OracleCache(np.zeros((L, B, 400, D)), np.zeros((L, B, 400, D)), np.arange(B), np.zeros(B, np.int64))
    mode = "bf16" if dtype == "bf16" else "f64"
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    empty = np.zeros((0, D), np.float32)
    _, _, ocache = oracle_encode(wl, mode, cache=ocache, uih=wl.prefix, uih_lengths=wl.cached_lengths,
                                 cand=empty, cand_lengths=np.zeros(B, np.int64))
    ru, rc, _ = oracle_encode(wl, mode, cache=ocache)
    eu, ec = normwise_per_user(pu, ru, wl.uih_lengths), normwise_per_user(pc, rc, wl.cand_lengths)
    say(f"  paged {dtype} D={D} {position}: bit-identical to the slot layout; vs oracle uih {eu:.3e} cand {ec:.3e}")
    assert eu <= tol and ec <= tol


def test_uih_outputs_bit_identical_for_any_candidate_set():
    """The history's representation must not depend on the candidates: identical bits for the
    candidate sets {}, A, B and A permuted; permuting candidates permutes their outputs."""
    wl = workloads.make_custom(seed=501, dtype="bf16", layers=2, d_model=256, heads=4, max_len=600,
                               uih_lengths=[300, 77, 150], cand_lengths=[40, 40, 40])
    rng = np.random.default_rng(9)
    B_set = workloads.to_bf16_values(rng.standard_normal(wl.cand.shape).astype(np.float32))
    perm = np.concatenate([rng.permutation(40) + 40 * b for b in range(3)])
    empty = np.zeros((0, 256), np.float32)
    ref_u, _ = gpu_encode(wl, cand=empty, cand_lengths=np.zeros(3, np.int64))
    ua, ca = gpu_encode(wl)
    ub, _ = gpu_encode(wl, cand=B_set)
    up, cp = gpu_encode(wl, cand=wl.cand[perm])
    for u in (ua, ub, up):
        assert np.array_equal(u, ref_u)
    assert np.array_equal(cp, ca[perm])
    # a candidate scored alone equals the same candidate within its set
    one_u, one_c = gpu_encode(wl, cand=wl.cand[[5, 45, 85]], cand_lengths=np.array([1, 1, 1]))
    assert np.array_equal(one_c, ca[[5, 45, 85]])


def test_zero_query_gives_zero_attention_on_gpu():
    """Zero Q columns of W1 and the Q slice of the bias table: SiLU(0) = 0, so every attention
    weight and output is exactly 0 and X1 = bf16(X0 + U W2[0:D]). Checked three ways: against
    the oracle's bf16 mirror; bit for bit against a second run whose W2 rows for O and U*O
    (rows D..3D) are other random values (exact zeros times anything add nothing); and,
    with all-zero input rows (then U = 0 too and X1 = bf16(O W2[D:2D])), every output
    exactly zero."""
    torch = torch_cuda()
    wl = workloads.make_custom(seed=601, dtype="bf16", layers=1, d_model=256, heads=4, max_len=300,
                               uih_lengths=[200, 31, 0], cand_lengths=[17, 2, 5])
    D = 256
    wl.params[0].w1[:, 2 * D:3 * D] = 0.0
    wl.params[0].pos[:, D:2 * D] = 0.0
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "bf16", BF16_TOL, label="zero-Q")
    import copy
    params2 = copy.deepcopy(wl.params)
    rng = np.random.default_rng(602)
    params2[0].w2[D:3 * D] = workloads.to_bf16_values(4.0 * rng.standard_normal((2 * D, D)).astype(np.float32))
    gu2, gc2 = gpu_encode(wl, model=make_model(torch, wl, params2))
    assert np.array_equal(gu, gu2) and np.array_equal(gc, gc2)
    zu, zc = np.zeros_like(wl.uih), np.zeros_like(wl.cand)
    gu0, gc0 = gpu_encode(wl, uih=zu, cand=zc)
    assert not np.any(gu0) and not np.any(gc0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_large_row_offsets(dtype):
    """Layer inputs whose rows carry a large common offset (rows of c + N(0, 1), c = 50, 300,
    1000 and -300 for the four users): the row normalisation must not lose the rows' spread
    to the offset. Each of two layers runs as a one-layer call on the GPU's own input to
    that layer (the offset survives the residual, and in bfloat16 a row at 1000 has a
    spacing of 4 against a spread near 1.5, so a single rounding flip of X + Z upstream
    would change the next layer's normalised row: the oracle gets the same bits). The
    cached keys and values of the call are the projection's outputs (normalised input
    times W1, SiLU, position bias) and are compared with the oracle's; the outputs too
    (their scale is the offset, so they pin less)."""
    torch = torch_cuda()
    import oracle
    D, H, L = (512, 4, 2) if dtype == "bf16" else (128, 2, 2)
    offsets = [50.0, 300.0, 1000.0, -300.0]
    ul, cl = [300, 129, 64, 200], [17, 64, 1, 0]
    wl = workloads.make_custom(seed=1201, dtype=dtype, layers=L, d_model=D, heads=H, max_len=400,
                               uih_lengths=ul, cand_lengths=cl)
    uo, co = workloads.lengths_to_offsets(ul), workloads.lengths_to_offsets(cl)
    uih = wl.uih.copy()
    cand = wl.cand.copy()
    for b, c in enumerate(offsets):
        uih[uo[b]:uo[b + 1]] += c
        cand[co[b]:co[b + 1]] += c
    if dtype == "bf16":
        uih, cand = workloads.to_bf16_values(uih), workloads.to_bf16_values(cand)
    mode = "bf16" if dtype == "bf16" else "f64"
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    x_u, x_c = uih.astype(np.float64), cand.astype(np.float64)
    for l in range(L):
        model = hsa.Model([wl.params[l]], d_model=D, heads=H, max_len=wl.max_len, dtype=dtype)
        cache = hsa.KVCache(model, slots=4, capacity=384)
        cache.cached_len = np.zeros(4, dtype=np.int32)
        gu, gc = gpu_encode(wl, model=model, uih=x_u, cand=x_c, cache=cache)
        ocache = oracle.OracleCache(np.zeros((1, 4, 384, D)), np.zeros((1, 4, 384, D)), np.arange(4),
                                    np.zeros(4, np.int64))
        ru, rc, ocache = oracle.encode(x_u, uo, x_c, co, [wl.params[l]], heads=H, max_len=wl.max_len, mode=mode,
                                       cache=ocache)
        gk, gv = to_np(cache.k), to_np(cache.v)
        for b in range(4):
            n = ul[b]
            ek = float(np.max(np.abs(gk[0, b, :n] - ocache.k[0, b, :n])) / np.max(np.abs(ocache.k[0, b, :n])))
            ev = float(np.max(np.abs(gv[0, b, :n] - ocache.v[0, b, :n])) / np.max(np.abs(ocache.v[0, b, :n])))
            say(f"  large row offsets {dtype}, layer {l}, user {b} (offset {offsets[b]}): cached K {ek:.3e} V {ev:.3e}")
            assert ek <= tol and ev <= tol
        eu = normwise_per_user(gu, ru, ul)
        ec = normwise_per_user(gc, rc, cl)
        say(f"  large row offsets {dtype}, layer {l}: outputs uih {eu:.3e} cand {ec:.3e}")
        assert eu <= tol and ec <= tol
        x_u, x_c = gu, gc


def test_two_runs_bitwise_identical():
    wl = workloads.make_custom(seed=701, dtype="bf16", layers=2, d_model=512, heads=4, max_len=700,
                               uih_lengths=[600, 3, 250], cand_lengths=[100, 200, 0])
    torch = torch_cuda()
    model = make_model(torch, wl)
    a = gpu_encode(wl, model=model)
    b = gpu_encode(wl, model=model)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
