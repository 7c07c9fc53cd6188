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


@pytest.mark.parametrize("D,H", [(256, 4), (256, 2), (512, 8), (512, 4), (640, 10), (768, 6), (1024, 8)])
def test_bf16_ragged(D, H):
    """dh = 64 and 128; histories of 0, 1, 127, 129, 300 rows and candidate sets of 1, 0, 130,
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


@pytest.mark.parametrize("dtype,tol", [("bf16", BF16_TOL), ("f32", F32_TOL)])
def test_history_fills_the_position_table(dtype, tol):
    """m + n + 1 == max_len: the candidates of the long user take the table's last row, its
    history rows every other one; a second user has no history (candidates at position 0)."""
    wl = workloads.make_custom(seed=811, dtype=dtype, layers=2, d_model=256 if dtype == "bf16" else 128,
                               heads=2, max_len=301, uih_lengths=[300, 0], cand_lengths=[4, 2])
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "bf16" if dtype == "bf16" else "f64", tol, label=f"{dtype} full position table")


@pytest.mark.parametrize("position", ["relative", "both"])
@pytest.mark.parametrize("D,H", [(256, 4), (512, 4)])
def test_bf16_relative_bias(D, H, position):
    """The original HSTU form: a relative position bias on every attention weight (alone,
    and with the absolute table), dh = 64 and 128, the ragged lengths of the other tests."""
    wl = workloads.make_custom(seed=900 + D + H, dtype="bf16", layers=2, d_model=D, heads=H, max_len=400,
                               uih_lengths=[0, 1, 127, 129, 300], cand_lengths=[1, 0, 130, 5, 64],
                               position=position, rel_std=0.3)
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "bf16", BF16_TOL, label=f"bf16 {position} bias D={D} H={H}")


@pytest.mark.parametrize("D,H", [(64, 2), (128, 2)])
def test_f32_relative_bias(D, H):
    wl = workloads.make_custom(seed=950 + D, dtype="f32", layers=2, d_model=D, heads=H, max_len=300,
                               uih_lengths=[0, 1, 63, 65, 200], cand_lengths=[3, 0, 64, 1, 70],
                               position="relative", rel_std=0.3)
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "f64", F32_TOL, label=f"f32 relative bias D={D} H={H}")


def test_bf16_relative_bias_long_table():
    """One long history: the staged relative table spans several thousand positions."""
    wl = workloads.make_custom(seed=977, dtype="bf16", layers=1, d_model=256, heads=4, max_len=7600,
                               uih_lengths=[4500], cand_lengths=[2], position="relative", rel_std=0.3)
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "bf16", BF16_TOL, label="bf16 relative bias, 4500 history rows")


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
    """Zero Q columns of W1 and the Q slice of the bias table: SiLU(0) = 0, so the attention
    output vanishes and X1 = bf16(X0 + U W2[0:D]); compared with the oracle's bf16 mirror."""
    wl = workloads.make_custom(seed=601, dtype="bf16", layers=1, d_model=256, heads=4, max_len=300,
                               uih_lengths=[200, 31], cand_lengths=[17, 2])
    D = 256
    wl.params[0].w1[:, 2 * D:3 * D] = 0.0
    wl.params[0].pos[:, D:2 * D] = 0.0
    gu, gc = gpu_encode(wl)
    check(wl, gu, gc, "bf16", BF16_TOL, label="zero-Q")


def test_two_runs_bitwise_identical():
    wl = workloads.make_custom(seed=701, dtype="bf16", layers=2, d_model=512, heads=4, max_len=700,
                               uih_lengths=[600, 3, 250], cand_lengths=[100, 200, 0])
    torch = torch_cuda()
    model = make_model(torch, wl)
    a = gpu_encode(wl, model=model)
    b = gpu_encode(wl, model=model)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
