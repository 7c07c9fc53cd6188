"""Pins for the CPU oracle: things other than the oracle itself that fix its results.

Each test names what pins it: brute force on tiny inputs, a closed form, an
invariant that the pages' definition implies, the page's worked jagged example,
or the pages' FLOP formula.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from oracle.hstu_oracle import OracleCache, count_macs
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- helpers

def tiny(seed, *, uih, cand, cached=None, D=4, H=2, L=2, max_len=16, mode="bf16"):
    wl = workloads.make_custom(seed=seed, dtype="bf16" if mode == "bf16" else "f32", layers=L,
                               d_model=D, heads=H, max_len=max_len, uih_lengths=uih,
                               cand_lengths=cand, cached_lengths=cached)
    return wl


def random_cache(wl, seed, capacity, bf16):
    """Arbitrary cached history keys/values (any values are a valid cache state)."""
    rng = np.random.default_rng(seed)
    B, L, D = wl.users, wl.layers, wl.d_model
    k = rng.standard_normal((L, B, capacity, D)).astype(np.float32) * 0.5
    v = rng.standard_normal((L, B, capacity, D)).astype(np.float32) * 0.5
    if bf16:
        k, v = workloads.to_bf16_values(k), workloads.to_bf16_values(v)
    return OracleCache(k.astype(np.float64), v.astype(np.float64),
                       np.arange(B, dtype=np.int64), wl.cached_lengths.astype(np.int64).copy())


def run_oracle(wl, mode, cache=None, counter=None, uih=None, cand=None, cand_lengths=None):
    uih = wl.uih if uih is None else uih
    cand = wl.cand if cand is None else cand
    cl = wl.cand_lengths if cand_lengths is None else cand_lengths
    return oracle.encode(uih, workloads.lengths_to_offsets(wl.uih_lengths), cand,
                         workloads.lengths_to_offsets(cl), wl.params, heads=wl.heads,
                         max_len=wl.max_len, mode=mode, cache=cache, counter=counter)


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)) if a.size else 0.0


# --------------------------------------------------------------------------- jagged offsets

def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            out[key] = [int(v) for v in vals]
    return out


def test_jagged_offsets_page_example():
    """Pin: the worked KeyedJaggedTensor example (10 lengths over 14 values)."""
    g = _read_golden("jagged_offsets_torchrec_example.txt")
    offs = oracle.jagged_offsets(g["lengths"])
    assert offs.tolist() == g["offsets"]
    assert offs[-1] == g["values"][0]
    assert workloads.lengths_to_offsets(g["lengths"]).tolist() == g["offsets"]


# --------------------------------------------------------------------------- bf16 rounding

def test_round_bf16_hand_built_cases():
    """Pin: closed-form rounding cases (ties to even, overflow to inf, signed zero)."""
    ulp1 = 2.0 ** -7                       # spacing of bfloat16 in [1, 2)
    cases = [
        (1.0 + ulp1 / 2, 1.0),             # tie, 1.0 is even
        (1.0 + 3 * ulp1 / 2, 1.0 + 2 * ulp1),   # tie, 1+ulp is odd -> up
        (1.0 + ulp1 / 2 + 2.0 ** -30, 1.0 + ulp1),   # just above a tie -> up
        (1.0 + ulp1 / 2 - 2.0 ** -30, 1.0),          # just below a tie -> down
        (-(1.0 + 3 * ulp1 / 2), -(1.0 + 2 * ulp1)),
        (3.0, 3.0), (0.1, 0.10009765625), (-0.1, -0.10009765625),
        (2.0 ** -134, 0.0),                # half the smallest subnormal, tie to even zero
        (3 * 2.0 ** -134, 2.0 ** -132),    # tie between 1 and 2 quanta -> 2 (even)
        (2.0 ** -133, 2.0 ** -133),
    ]
    bmax = (2.0 - 2.0 ** -7) * 2.0 ** 127
    cases += [(bmax, bmax), (bmax + 2.0 ** 119 - 2.0 ** 100, bmax),
              (bmax + 2.0 ** 119, math.inf), (-bmax - 2.0 ** 119, -math.inf), (1e39, math.inf)]
    xs = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases])
    got = oracle.round_bf16(xs)
    assert np.array_equal(got, want), list(zip(xs, got, want))
    for x, w in cases:
        assert brute.bf16_round(x) == w
    z = oracle.round_bf16(np.array([-0.0, -1e-45, 0.0]))
    assert np.all(z == 0) and np.signbit(z[0]) and np.signbit(z[1]) and not np.signbit(z[2])
    assert np.isnan(oracle.round_bf16(np.nan))


def test_round_bf16_matches_library_on_float32_values():
    """Pin: for float32 inputs, bfloat16 rounding must equal PyTorch's conversion."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 200000),
                        rng.standard_normal(1000).astype(np.float32) * 1e-39]).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), lib)
    assert np.array_equal(workloads.to_bf16_values(x).astype(np.float64), lib)


def test_round_bf16_brute_agrees_on_float64():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(5000) * 10.0 ** rng.integers(-40, 38, 5000)
    got = oracle.round_bf16(x)
    assert all(brute.bf16_round(float(a)) == float(b) for a, b in zip(x, got))


# --------------------------------------------------------------------------- SiLU

def test_silu_closed_forms():
    """Pin: SiLU(0)=0, SiLU(x)-SiLU(-x)=x, limits at +-inf without NaN."""
    x = np.linspace(-30, 30, 1001)
    assert oracle.silu(0.0) == 0.0
    assert np.max(np.abs(oracle.silu(x) - oracle.silu(-x) - x)) < 1e-13
    y = oracle.silu(np.array([-1e4, -800.0, 800.0]))
    assert y[0] == 0 and np.signbit(y[0]) and y[1] == 0 and y[2] == 800.0
    assert not np.any(np.isnan(y))
    # x * logistic(x) at a point computed by hand: SiLU(1) = 1 / (1 + 1/e)
    assert abs(float(oracle.silu(1.0)) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


# --------------------------------------------------------------------------- input normalisation

def test_normalize_rows_closed_forms():
    """Pin (closed form): a row (1, 3) has mean 2 and variance 1, so it maps to
    (-1, 1)/sqrt(1 + eps); every row ends with mean 0 and variance 1/(1 + eps/var); the map is
    invariant to a positive scale and a shift of the row."""
    eps = oracle.NORM_EPS
    assert np.allclose(oracle.normalize_rows(np.array([[1.0, 3.0]])),
                       np.array([[-1.0, 1.0]]) / math.sqrt(1 + eps), rtol=1e-15)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 64)) * 3.0 + 1.5
    y = oracle.normalize_rows(x)
    var = x.var(axis=1)
    assert np.max(np.abs(y.mean(axis=1))) < 1e-14
    assert np.allclose(y.var(axis=1), var / (var + eps), rtol=1e-13)
    assert np.allclose(oracle.normalize_rows(7.0 * x - 4.0), oracle.normalize_rows(x), atol=1e-6)
    assert oracle.normalize_rows(np.zeros((0, 8))).shape == (0, 8)


# --------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("mode", ["f64", "bf16"])
def test_oracle_matches_brute_force(mode):
    """Pin: every output of the stack re-derived with scalar loops (tiny inputs), including a
    user with cached history, a user with no new history and a user without candidates."""
    uih, cand, cached = [3, 0, 5], [2, 3, 0], [2, 3, 0]
    wl = tiny(11, uih=uih, cand=cand, cached=cached, mode=mode)
    cache = random_cache(wl, 5, capacity=8, bf16=(mode == "bf16"))
    got_u, got_c, new_cache = run_oracle(wl, mode, cache=cache)
    ck = [[[list(map(float, cache.k[l, b, j])) for j in range(cached[b])] for b in range(3)]
          for l in range(wl.layers)]
    cv = [[[list(map(float, cache.v[l, b, j])) for j in range(cached[b])] for b in range(3)]
          for l in range(wl.layers)]
    params = [(p.w1.astype(np.float64).tolist(), p.w2.astype(np.float64).tolist(),
               p.pos.astype(np.float64).tolist()) for p in wl.params]
    bu, bc = brute.encode_brute(wl.uih.astype(np.float64).tolist(),
                                workloads.lengths_to_offsets(uih).tolist(),
                                wl.cand.astype(np.float64).tolist(),
                                workloads.lengths_to_offsets(cand).tolist(), params,
                                heads=wl.heads, max_len=wl.max_len, bf16=(mode == "bf16"),
                                cached_k=ck, cached_v=cv, cached_len=cached)
    assert rel(got_u, np.array(bu)) <= 1e-12
    assert rel(got_c, np.array(bc)) <= 1e-12
    # the cache now holds prefix + new keys/values for every layer
    for l in range(wl.layers):
        for b in range(3):
            n_all = cached[b] + uih[b]
            assert new_cache.cached_len[b] == n_all
            assert rel(new_cache.k[l, b, :n_all], np.array(ck[l][b]).reshape(n_all, -1)) <= 1e-12
            assert rel(new_cache.v[l, b, :n_all], np.array(cv[l][b]).reshape(n_all, -1)) <= 1e-12


def test_oracle_matches_brute_force_no_cache_four_heads():
    wl = tiny(12, uih=[6, 1], cand=[3, 1], D=8, H=4, L=1, max_len=9, mode="bf16")
    got_u, got_c, _ = run_oracle(wl, "bf16")
    params = [(p.w1.astype(np.float64).tolist(), p.w2.astype(np.float64).tolist(),
               p.pos.astype(np.float64).tolist()) for p in wl.params]
    bu, bc = brute.encode_brute(wl.uih.astype(np.float64).tolist(), [0, 6, 7],
                                wl.cand.astype(np.float64).tolist(), [0, 3, 4], params,
                                heads=4, max_len=9, bf16=True)
    assert rel(got_u, np.array(bu)) <= 1e-12 and rel(got_c, np.array(bc)) <= 1e-12


# --------------------------------------------------------------------------- closed forms

def _qkv(rng, rows, D, scale=0.7):
    return [rng.standard_normal((rows, D)) * scale for _ in range(3)]


@pytest.mark.parametrize("bf16", [False, True])
def test_attention_single_history_token(bf16):
    """Pin (closed form): one history token, no candidates: O = SiLU(q.k) v / max_len per head."""
    rng = np.random.default_rng(3)
    D, H, max_len = 8, 2, 10
    q, k, v = _qkv(rng, 1, D)
    if bf16:
        q, k, v = (oracle.round_bf16(a) for a in (q, k, v))
    o_u, o_c = oracle.attention_user(q, k, v, np.zeros((0, D)), np.zeros((0, D)), np.zeros((0, D)),
                                     m=0, heads=H, inv=1.0 / max_len, bf16=bf16)
    assert o_c.shape == (0, D)
    for h in range(H):
        s = slice(h * 4, h * 4 + 4)
        dot = sum(q[0, t] * k[0, t] for t in range(h * 4, h * 4 + 4))
        a = dot / (1 + math.exp(-dot))
        if bf16:
            a = brute.bf16_round(a)
            want = [brute.bf16_round(a * x / max_len) for x in v[0, s]]
        else:
            want = [a * x / max_len for x in v[0, s]]
        assert np.allclose(o_u[0, s], want, rtol=1e-15, atol=0)


def test_attention_candidate_with_empty_history():
    """Pin (closed form): n = 0, one candidate: it sees only itself."""
    rng = np.random.default_rng(4)
    D, H, max_len = 8, 2, 10
    q, k, v = _qkv(rng, 1, D)
    o_u, o_c = oracle.attention_user(np.zeros((0, D)), np.zeros((0, D)), np.zeros((0, D)), q, k, v,
                                     m=0, heads=H, inv=1.0 / max_len, bf16=False)
    for h in range(H):
        s = slice(h * 4, h * 4 + 4)
        dot = float(np.dot(q[0, s], k[0, s]))
        assert np.allclose(o_c[0, s], dot / (1 + math.exp(-dot)) * v[0, s] / max_len, rtol=1e-14)


def test_attention_two_tokens_causal_closed_form():
    """Pin (closed form): two history tokens; row 0 sees key 0, row 1 sees keys 0 and 1."""
    rng = np.random.default_rng(5)
    D, max_len = 4, 7
    q, k, v = _qkv(rng, 2, D)
    o_u, _ = oracle.attention_user(q, k, v, np.zeros((0, D)), np.zeros((0, D)), np.zeros((0, D)),
                                   m=0, heads=1, inv=1.0 / max_len, bf16=False)
    sl = lambda x: x / (1 + math.exp(-x))
    want0 = sl(q[0] @ k[0]) * v[0] / max_len
    want1 = (sl(q[1] @ k[0]) * v[0] + sl(q[1] @ k[1]) * v[1]) / max_len
    assert np.allclose(o_u[0], want0, rtol=1e-14) and np.allclose(o_u[1], want1, rtol=1e-14)


@pytest.mark.parametrize("mode", ["f64", "bf16"])
def test_zero_query_gives_zero_attention(mode):
    """Pin (invariant, SiLU(0)=0): zero the Q columns of W1 and the Q slice of the position
    table; then every attention output is exactly 0 and X1 = X0 + U W2[0:D]."""
    wl = workloads.make_custom(seed=21, dtype="bf16" if mode == "bf16" else "f32", layers=1, d_model=16,
                               heads=2, max_len=40, uih_lengths=[7, 12], cand_lengths=[5, 0])
    D = wl.d_model
    p = wl.params[0]
    p.w1[:, 2 * D:3 * D] = 0.0
    p.pos[:, D:2 * D] = 0.0
    xu = wl.uih.astype(np.float64)
    w1, w2, pos = (a.astype(np.float64) for a in (p.w1, p.w2, p.pos))
    bf16 = mode == "bf16"
    x_u, x_c, _, _ = oracle.layer_user(xu[:7], wl.cand[:5].astype(np.float64), w1, w2, pos,
                                       k_cached=np.zeros((0, D)), v_cached=np.zeros((0, D)),
                                       heads=2, max_len=40, bf16=bf16)
    # attention outputs directly
    xn = oracle.normalize_rows(xu[:7])
    s = oracle.silu(xn @ w1)   # the normalised rows are never stored, so never rounded
    q = s[:, 2 * D:3 * D] + pos[:7, D:2 * D]
    assert np.all(q == 0)
    kk = s[:, 3 * D:] + pos[:7, 2 * D:]
    vv = s[:, D:2 * D] + pos[:7, :D]
    o_u, _ = oracle.attention_user(q, kk, vv, np.zeros((0, D)), np.zeros((0, D)), np.zeros((0, D)),
                                   m=0, heads=2, inv=1 / 40, bf16=bf16)
    assert np.all(o_u == 0)
    u = s[:, :D] if not bf16 else oracle.round_bf16(s[:, :D])
    want = xu[:7] + u @ w2[:D]
    if bf16:
        want = oracle.round_bf16(want)
        assert np.max(np.abs(x_u - want)) <= 2.0 ** -7 * np.max(np.abs(want))
        assert np.mean(x_u == want) > 0.99
    else:
        assert rel(x_u, want) < 1e-14


# --------------------------------------------------------------------------- relative bias

@pytest.mark.parametrize("bf16", [False, True])
def test_relative_bias_single_history_token(bf16):
    """Pin (closed form): one history token with a relative bias table: its weight is
    SiLU(q.k) + rel[h, 0] (relative position 0), so O = (SiLU(q.k) + rel[h, 0]) v / max_len."""
    rng = np.random.default_rng(41)
    D, H, max_len = 8, 2, 10
    q, k, v = _qkv(rng, 1, D)
    table = rng.standard_normal((H, max_len)) * 0.3
    if bf16:
        q, k, v, table = (oracle.round_bf16(a) for a in (q, k, v, table))
    o_u, _ = oracle.attention_user(q, k, v, np.zeros((0, D)), np.zeros((0, D)), np.zeros((0, D)),
                                   m=0, heads=H, inv=1.0 / max_len, bf16=bf16, rel=table)
    for h in range(H):
        s = slice(h * 4, h * 4 + 4)
        dot = sum(q[0, t] * k[0, t] for t in range(h * 4, h * 4 + 4))
        a = dot / (1 + math.exp(-dot)) + table[h, 0]
        if bf16:
            a = brute.bf16_round(a)
            want = [brute.bf16_round(a * x / max_len) for x in v[0, s]]
        else:
            want = [a * x / max_len for x in v[0, s]]
        assert np.allclose(o_u[0, s], want, rtol=1e-15, atol=0)


def test_relative_bias_two_tokens_with_cache_and_candidate():
    """Pin (closed form): one cached key (position 0), two new rows (positions 1, 2) and one
    candidate (position 3): each weight picks rel[pos_query - pos_key]."""
    rng = np.random.default_rng(42)
    D, max_len = 4, 7
    q, k, v = _qkv(rng, 3, D)                # row 0 is the cached key/value, rows 1, 2 are new
    qc, kc, vc = _qkv(rng, 1, D)
    t = rng.standard_normal((1, max_len))
    o_u, o_c = oracle.attention_user(q[1:], k, v, qc, kc, vc, m=1, heads=1, inv=1.0 / max_len,
                                     bf16=False, rel=t)
    sl = lambda x: x / (1 + math.exp(-x))
    want1 = ((sl(q[1] @ k[0]) + t[0, 1]) * v[0] + (sl(q[1] @ k[1]) + t[0, 0]) * v[1]) / max_len
    want2 = ((sl(q[2] @ k[0]) + t[0, 2]) * v[0] + (sl(q[2] @ k[1]) + t[0, 1]) * v[1]
             + (sl(q[2] @ k[2]) + t[0, 0]) * v[2]) / max_len
    wantc = (sum((sl(qc[0] @ k[j]) + t[0, 3 - j]) * v[j] for j in range(3))
             + (sl(qc[0] @ kc[0]) + t[0, 0]) * vc[0]) / max_len
    assert np.allclose(o_u[0], want1, rtol=1e-14) and np.allclose(o_u[1], want2, rtol=1e-14)
    assert np.allclose(o_c[0], wantc, rtol=1e-14)


def test_relative_bias_zero_query_is_a_causal_convolution():
    """Pin (library routine): with q = 0 every SiLU term vanishes and history row i gets
    O_i = inv * sum_{j <= m+i} rel[m+i-j] v_j, a causal convolution of V with the table,
    computed here by numpy.convolve; a candidate gets inv * (sum_j rel[m+n-j] v_j + rel[0] v_c)."""
    rng = np.random.default_rng(43)
    D, H, m, n, c, max_len = 6, 2, 3, 9, 2, 20
    k_all = rng.standard_normal((m + n, D))
    v_all = rng.standard_normal((m + n, D))
    vc = rng.standard_normal((c, D))
    table = rng.standard_normal((H, max_len))
    o_u, o_c = oracle.attention_user(np.zeros((n, D)), k_all, v_all, np.zeros((c, D)),
                                     rng.standard_normal((c, D)), vc, m=m, heads=H, inv=0.25,
                                     bf16=False, rel=table)
    dh = D // H
    for h in range(H):
        for t in range(h * dh, (h + 1) * dh):
            conv = np.convolve(table[h], v_all[:, t])          # conv[p] = sum_j table[p - j] v_j
            assert np.allclose(o_u[:, t], 0.25 * conv[m:m + n], rtol=1e-13, atol=1e-13)
            cand_want = 0.25 * (conv[m + n] + table[h, 0] * vc[:, t])
            assert np.allclose(o_c[:, t], cand_want, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("position", ["relative", "both"])
@pytest.mark.parametrize("mode", ["f64", "bf16"])
def test_oracle_matches_brute_force_relative_bias(position, mode):
    """Pin: the stack with a relative bias (alone, and with the absolute table) re-derived
    with scalar loops, including cached history, an empty history and no candidates."""
    uih, cand, cached = [3, 0, 5], [2, 3, 0], [2, 3, 0]
    wl = workloads.make_custom(seed=44, dtype="bf16" if mode == "bf16" else "f32", layers=2, d_model=4,
                               heads=2, max_len=16, uih_lengths=uih, cand_lengths=cand,
                               cached_lengths=cached, position=position, rel_std=0.5)
    assert (wl.params[0].pos is None) == (position == "relative") and wl.params[0].rel is not None
    cache = random_cache(wl, 45, capacity=8, bf16=(mode == "bf16"))
    got_u, got_c, _ = run_oracle(wl, mode, cache=cache)
    ck = [[[list(map(float, cache.k[l, b, j])) for j in range(cached[b])] for b in range(3)]
          for l in range(wl.layers)]
    cv = [[[list(map(float, cache.v[l, b, j])) for j in range(cached[b])] for b in range(3)]
          for l in range(wl.layers)]
    tolist = lambda a: None if a is None else a.astype(np.float64).tolist()
    params = [(tolist(p.w1), tolist(p.w2), tolist(p.pos), tolist(p.rel)) for p in wl.params]
    bu, bc = brute.encode_brute(wl.uih.astype(np.float64).tolist(),
                                workloads.lengths_to_offsets(uih).tolist(),
                                wl.cand.astype(np.float64).tolist(),
                                workloads.lengths_to_offsets(cand).tolist(), params,
                                heads=wl.heads, max_len=wl.max_len, bf16=(mode == "bf16"),
                                cached_k=ck, cached_v=cv, cached_len=cached)
    assert rel(got_u, np.array(bu)) <= 1e-12
    assert rel(got_c, np.array(bc)) <= 1e-12


def test_relative_bias_history_independent_of_candidates():
    """Pin (invariant): with a relative bias the history outputs are still bit-identical
    for any candidate set (the bias depends on positions only)."""
    base = workloads.make_custom(seed=46, dtype="bf16", layers=2, d_model=16, heads=2, max_len=80,
                                 uih_lengths=[20, 33], cand_lengths=[6, 6], position="relative",
                                 rel_std=0.5)
    ref_u, _, _ = run_oracle(base, "bf16")
    for cl in ([0, 0], [6, 6], [3, 1]):
        cand = base.cand[:sum(cl)] if sum(cl) else np.zeros((0, 16), np.float32)
        got_u, _, _ = run_oracle(base, "bf16", cand=cand, cand_lengths=np.array(cl))
        assert np.array_equal(got_u, ref_u)


# --------------------------------------------------------------------------- invariants

def test_uih_outputs_bit_identical_for_any_candidate_set():
    """Pin (the history representation must not depend on the candidate being scored):
    history outputs are bit-identical for candidate sets {}, A, B and A permuted."""
    base = workloads.make_custom(seed=31, dtype="bf16", layers=2, d_model=16, heads=2, max_len=80,
                                 uih_lengths=[20, 33, 9], cand_lengths=[6, 6, 6])
    rng = np.random.default_rng(7)
    A = base.cand
    Bset = workloads.to_bf16_values(rng.standard_normal(A.shape).astype(np.float32))
    perm = np.concatenate([rng.permutation(6) + 6 * b for b in range(3)])
    outs = []
    for cand, cl in [(np.zeros((0, 16), np.float32), [0, 0, 0]), (A, [6, 6, 6]), (Bset, [6, 6, 6]),
                     (A[perm], [6, 6, 6])]:
        u, c, _ = run_oracle(base, "bf16", cand=cand, cand_lengths=np.array(cl))
        outs.append((u, c))
    for u, _ in outs[1:]:
        assert np.array_equal(u, outs[0][0])
    # permuting candidates permutes their outputs
    assert np.array_equal(outs[3][1], outs[1][1][perm])


def test_candidate_scored_alone_equals_within_set():
    base = workloads.make_custom(seed=32, dtype="bf16", layers=2, d_model=16, heads=2, max_len=80,
                                 uih_lengths=[25], cand_lengths=[7])
    _, c_all, _ = run_oracle(base, "bf16")
    for j in [0, 3, 6]:
        _, c_one, _ = run_oracle(base, "bf16", cand=base.cand[j:j + 1], cand_lengths=np.array([1]))
        assert np.array_equal(c_one[0], c_all[j])


def test_perturbation_locality():
    """Pin (mask): perturbing history token j changes only history rows at positions >= j and
    the candidates; perturbing a candidate changes only that candidate."""
    base = workloads.make_custom(seed=33, dtype="f32", layers=2, d_model=8, heads=2, max_len=40,
                                 uih_lengths=[12, 5], cand_lengths=[4, 2])
    u0, c0, _ = run_oracle(base, "f64")
    uih = base.uih.copy()
    uih[7] += 0.5                         # user 0, history row 7
    u1, c1, _ = run_oracle(base, "f64", uih=uih)
    changed = np.any(u1 != u0, axis=1)
    assert not changed[:7].any() and changed[7:12].all() and not changed[12:].any()
    assert np.any(c1[:4] != c0[:4], axis=1).all() and np.array_equal(c1[4:], c0[4:])
    cand = base.cand.copy()
    cand[2] -= 0.25
    u2, c2, _ = run_oracle(base, "f64", cand=cand)
    assert np.array_equal(u2, u0)
    ch = np.any(c2 != c0, axis=1)
    assert ch[2] and ch.sum() == 1


@pytest.mark.parametrize("mode", ["f64", "bf16"])
def test_streaming_equals_full_recompute(mode):
    """Pin (reusing a user's history key/value state across timestamps): encoding a prefix
    into the cache, then the new events plus candidates, equals encoding prefix + new events
    at once (exact causality of the history mask)."""
    wl = workloads.make_custom(seed=41, dtype="bf16" if mode == "bf16" else "f32", layers=3,
                               d_model=16, heads=2, max_len=64, uih_lengths=[9, 4, 0],
                               cand_lengths=[5, 3, 2], cached_lengths=[13, 20, 6])
    B, L, D, cap = 3, 3, 16, 40
    cache = OracleCache(np.zeros((L, B, cap, D)), np.zeros((L, B, cap, D)), np.array([2, 0, 1]),
                        np.zeros(B, dtype=np.int64))
    pre_off = workloads.lengths_to_offsets(wl.cached_lengths)
    # fill: the prefixes, no candidates
    _, _, filled = oracle.encode(wl.prefix, pre_off, np.zeros((0, D)), np.zeros(B + 1, np.int64),
                                 wl.params, heads=2, max_len=64, mode=mode, cache=cache)
    assert filled.cached_len.tolist() == [13, 20, 6]
    u_s, c_s, after = run_oracle(wl, mode, cache=filled)
    # full recompute: prefix + new history in one go
    full = np.concatenate([np.concatenate([wl.prefix[pre_off[b]:pre_off[b + 1]],
                                           wl.uih[sum(wl.uih_lengths[:b]):sum(wl.uih_lengths[:b + 1])]])
                           for b in range(B)])
    full_len = wl.cached_lengths + wl.uih_lengths
    fu, fc, _ = oracle.encode(full, workloads.lengths_to_offsets(full_len), wl.cand,
                              workloads.lengths_to_offsets(wl.cand_lengths), wl.params, heads=2,
                              max_len=64, mode=mode)
    foff = workloads.lengths_to_offsets(full_len)
    new_rows = np.concatenate([fu[foff[b] + wl.cached_lengths[b]:foff[b + 1]] for b in range(B)])
    tol = 1e-12 if mode == "f64" else 0.0
    assert rel(u_s, new_rows) <= tol and rel(c_s, fc) <= tol
    assert after.cached_len.tolist() == full_len.tolist()


# --------------------------------------------------------------------------- action/context packing

def test_pack_sum_closed_forms():
    """Pin (merging an event's two embeddings into one token): integer sums are exact; in
    bfloat16 the sum is rounded once, ties to even (1 + 2^-8 lies halfway between 1 and
    1 + 2^-7 and goes to 1; 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6 and goes to
    the even 1 + 2^-6)."""
    c = np.array([[1.0, -3.0, 2.0, 0.0], [1.0, 1.0, 5.0, -7.0]])
    a = np.array([[2.0, 3.0, -0.5, 0.0], [2.0 ** -8, 3 * 2.0 ** -8, 0.25, 7.0]])
    t, off = oracle.pack_uih(c, a, [0, 2], "sum")
    assert off.tolist() == [0, 2]
    assert t.tolist() == [[3.0, 0.0, 1.5, 0.0], [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 5.25, 0.0]]
    tb, _ = oracle.pack_uih(c, a, [0, 2], "sum", bf16=True)
    assert tb[1].tolist() == [1.0, 1.0 + 2.0 ** -6, 5.25, 0.0]


@pytest.mark.parametrize("mode", ["sum", "interleave"])
def test_pack_matches_brute_force(mode):
    """Pin: the packed tokens and offsets re-derived one user and one event at a time, with
    empty users at the front, middle and end."""
    rng = np.random.default_rng(91)
    lengths = [0, 3, 0, 1, 4, 0]
    E, D = sum(lengths), 8
    c = workloads.to_bf16_values(rng.standard_normal((E, D)).astype(np.float32)).astype(np.float64)
    a = workloads.to_bf16_values(rng.standard_normal((E, D)).astype(np.float32)).astype(np.float64)
    eo = workloads.lengths_to_offsets(lengths)
    for bf16 in (False, True):
        t, off = oracle.pack_uih(c, a, eo, mode, bf16=bf16)
        bt, boff = brute.pack_brute(c.tolist(), a.tolist(), eo.tolist(), mode, bf16=bf16)
        assert off.tolist() == boff
        assert t.shape == (len(bt), D) and t.tolist() == bt


def test_interleave_doubles_the_history():
    """Pin (interleaving doubles the effective sequence length): every user's token count
    is twice its event count, and its tokens alternate its own context and action rows."""
    lengths = [2, 0, 5]
    E, D = 7, 4
    c = np.arange(E * D, dtype=np.float64).reshape(E, D)
    a = -1.0 - c
    eo = workloads.lengths_to_offsets(lengths)
    t, off = oracle.pack_uih(c, a, eo, "interleave")
    assert off.tolist() == [0, 4, 4, 14]
    for b in range(3):
        for i in range(lengths[b]):
            e = eo[b] + i
            assert t[off[b] + 2 * i].tolist() == c[e].tolist()
            assert t[off[b] + 2 * i + 1].tolist() == a[e].tolist()


def _packed(wl, mode, *, prefix=False):
    """Tokens and token offsets of a packing workload's history (or of its cached prefix)."""
    lengths = wl.cached_lengths if prefix else wl.uih_lengths
    ctx, act = (wl.prefix, wl.prefix_action) if prefix else (wl.uih, wl.action)
    return oracle.pack_uih(ctx, act, workloads.lengths_to_offsets(lengths), wl.packing,
                           bf16=(mode == "bf16"))


def test_interleaved_stack_matches_brute_force():
    """Pin: interleaved tokens through the stack, re-derived end to end with scalar loops."""
    wl = workloads.make_custom(seed=93, dtype="bf16", layers=2, d_model=4, heads=2, max_len=16,
                               uih_lengths=[3, 0, 2], cand_lengths=[2, 1, 0], packing="interleave")
    tok, off = _packed(wl, "bf16")
    got_u, got_c, _ = oracle.encode(tok, off, wl.cand, workloads.lengths_to_offsets(wl.cand_lengths),
                                    wl.params, heads=2, max_len=16, mode="bf16")
    eo = workloads.lengths_to_offsets(wl.uih_lengths).tolist()
    btok, boff = brute.pack_brute(wl.uih.astype(np.float64).tolist(), wl.action.astype(np.float64).tolist(),
                                  eo, "interleave", bf16=True)
    params = [(p.w1.astype(np.float64).tolist(), p.w2.astype(np.float64).tolist(),
               p.pos.astype(np.float64).tolist()) for p in wl.params]
    bu, bc = brute.encode_brute(btok, boff, wl.cand.astype(np.float64).tolist(),
                                workloads.lengths_to_offsets(wl.cand_lengths).tolist(), params,
                                heads=2, max_len=16, bf16=True)
    assert rel(got_u, np.array(bu)) <= 1e-12 and rel(got_c, np.array(bc)) <= 1e-12


def test_interleaved_action_is_seen_only_after_its_context():
    """Pin (causal mask over the interleaved sequence): changing event i's action changes
    nothing at or before that event's context token, changes the action token and every
    later token of the same user and all of that user's candidates, and no other user."""
    wl = workloads.make_custom(seed=95, dtype="f32", layers=2, d_model=8, heads=2, max_len=40,
                               uih_lengths=[6, 4], cand_lengths=[3, 2], packing="interleave")
    co = workloads.lengths_to_offsets(wl.cand_lengths)
    run = lambda tok, off: oracle.encode(tok, off, wl.cand, co, wl.params, heads=2, max_len=40, mode="f64")
    tok, off = _packed(wl, "f64")
    u0, c0, _ = run(tok, off)
    wl.action[3] += 0.5                   # user 0, event 3: tokens 6 (context) and 7 (action)
    tok1, off1 = _packed(wl, "f64")
    u1, c1, _ = run(tok1, off1)
    changed = np.any(u1 != u0, axis=1)
    assert not changed[:7].any() and changed[7:12].all() and not changed[12:].any()
    assert np.any(c1[:3] != c0[:3], axis=1).all() and np.array_equal(c1[3:], c0[3:])


def test_sum_with_zero_actions_is_the_plain_stack():
    """Pin (special case): merging zero action embeddings leaves the tokens, and so the
    stack's outputs, exactly those of the context embeddings alone."""
    wl = workloads.make_custom(seed=97, dtype="bf16", layers=2, d_model=8, heads=2, max_len=32,
                               uih_lengths=[5, 0, 7], cand_lengths=[2, 3, 1], packing="sum")
    wl.action[:] = 0.0
    tok, off = _packed(wl, "bf16")
    assert np.array_equal(tok, wl.uih.astype(np.float64))
    got_u, got_c, _ = oracle.encode(tok, off, wl.cand, workloads.lengths_to_offsets(wl.cand_lengths),
                                    wl.params, heads=2, max_len=32, mode="bf16")
    ref_u, ref_c, _ = run_oracle(wl, "bf16")
    assert np.array_equal(got_u, ref_u) and np.array_equal(got_c, ref_c)


@pytest.mark.parametrize("packing", ["sum", "interleave"])
def test_packed_streaming_equals_one_shot(packing):
    """Pin: packing a cached prefix's events, then the new events, and encoding them with the
    cache gives the new tokens and candidates of packing and encoding all events at once."""
    wl = workloads.make_custom(seed=99, dtype="bf16", layers=2, d_model=16, heads=2, max_len=64,
                               uih_lengths=[4, 3], cand_lengths=[3, 2], cached_lengths=[5, 0],
                               packing=packing)
    B, L, D, cap = 2, 2, 16, 40
    f = 2 if packing == "interleave" else 1
    co = workloads.lengths_to_offsets(wl.cand_lengths)
    cache = OracleCache(np.zeros((L, B, cap, D)), np.zeros((L, B, cap, D)), np.array([1, 0]),
                        np.zeros(B, dtype=np.int64))
    ptok, poff = _packed(wl, "bf16", prefix=True)
    _, _, filled = oracle.encode(ptok, poff, np.zeros((0, D)), np.zeros(B + 1, np.int64), wl.params,
                                 heads=2, max_len=64, mode="bf16", cache=cache)
    assert filled.cached_len.tolist() == [5 * f, 0]
    tok, off = _packed(wl, "bf16")
    u_s, c_s, _ = oracle.encode(tok, off, wl.cand, co, wl.params, heads=2, max_len=64, mode="bf16",
                                cache=filled)
    eo_p = workloads.lengths_to_offsets(wl.cached_lengths)
    eo_n = workloads.lengths_to_offsets(wl.uih_lengths)
    ctx = np.concatenate([np.concatenate([wl.prefix[eo_p[b]:eo_p[b + 1]], wl.uih[eo_n[b]:eo_n[b + 1]]])
                          for b in range(B)])
    act = np.concatenate([np.concatenate([wl.prefix_action[eo_p[b]:eo_p[b + 1]],
                                          wl.action[eo_n[b]:eo_n[b + 1]]]) for b in range(B)])
    all_len = wl.cached_lengths + wl.uih_lengths
    ftok, foff = oracle.pack_uih(ctx, act, workloads.lengths_to_offsets(all_len), packing, bf16=True)
    fu, fc, _ = oracle.encode(ftok, foff, wl.cand, co, wl.params, heads=2, max_len=64, mode="bf16")
    new_rows = np.concatenate([fu[foff[b] + f * wl.cached_lengths[b]:foff[b + 1]] for b in range(B)])
    assert np.array_equal(u_s, new_rows) and np.array_equal(c_s, fc)


# --------------------------------------------------------------------------- scoring head

def test_sigmoid_closed_forms_and_library():
    """Pin: sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(z) + sigmoid(-z) = 1, the limits
    0 and 1 without overflow, and scipy's expit over a sweep."""
    from scipy.special import expit
    assert oracle.sigmoid(0.0) == 0.5
    assert abs(oracle.sigmoid(math.log(3.0)) - 0.75) <= 1e-15
    z = np.linspace(-40.0, 40.0, 2001)
    assert np.max(np.abs(oracle.sigmoid(z) + oracle.sigmoid(-z) - 1.0)) <= 1e-15
    assert np.max(np.abs(oracle.sigmoid(z) - expit(z))) <= 1e-15
    with np.errstate(over="raise", invalid="raise"):
        assert oracle.sigmoid(-1000.0) == 0.0 and oracle.sigmoid(1000.0) == 1.0


def test_score_head_single_layer_is_logistic_regression():
    """Pin (special case): one layer is a logistic regression, p = sigmoid(x . w + b); with w
    a unit vector the probability reads one feature."""
    x = np.array([[0.5, -2.0, 1.0], [0.0, 0.0, 0.0]])
    w = np.array([[0.0, 1.0, 0.0], [1.0, 1.0, 1.0]])
    b = np.array([0.0, math.log(3.0)])
    p = oracle.score_head(x, [(w, b)])
    assert abs(p[0, 0] - 1.0 / (1.0 + math.exp(2.0))) <= 1e-15
    assert abs(p[0, 1] - 1.0 / (1.0 + math.exp(-(-0.5 + math.log(3.0))))) <= 1e-15
    assert p[1, 0] == 0.5 and abs(p[1, 1] - 0.75) <= 1e-15


def test_score_head_relu_between_layers():
    """Pin (ReLU placement): a hidden unit with a negative pre-activation contributes nothing
    (the output is the sigmoid of the last bias alone); a positive one passes unchanged."""
    x = np.array([[1.0, 2.0]])
    hidden = (np.array([[-1.0, -1.0], [1.0, 0.0]]), np.array([0.0, 0.0]))   # pre-activations -3, 1
    last = (np.array([[5.0, 0.0]]), np.array([0.25]))
    assert oracle.score_head(x, [hidden, last])[0, 0] == oracle.sigmoid(0.25)
    last2 = (np.array([[0.0, 2.0]]), np.array([0.25]))
    assert oracle.score_head(x, [hidden, last2])[0, 0] == oracle.sigmoid(2.25)


@pytest.mark.parametrize("bf16", [False, True])
def test_score_head_matches_brute_force(bf16):
    """Pin: three layers (16 -> 8 -> 4 -> 3 outcomes) re-derived with scalar loops."""
    wl = workloads.make_custom(seed=101, dtype="bf16" if bf16 else "f32", layers=1, d_model=16, heads=2,
                               max_len=8, uih_lengths=[0], cand_lengths=[5], head=(8, 4, 3))
    got = oracle.score_head(wl.cand, wl.head, bf16=bf16)
    layers = [(w.astype(np.float64).tolist(), b.astype(np.float64).tolist()) for w, b in wl.head]
    want = brute.score_brute(wl.cand.astype(np.float64).tolist(), layers, bf16=bf16)
    assert got.shape == (5, 3)
    assert np.max(np.abs(got - np.array(want))) <= 1e-14


# --------------------------------------------------------------------------- FLOP counting

def test_counter_matches_closed_forms_and_page_formula():
    """Pin (the page's FLOP formula 2*layers*(n*n*D/2 + 4*n*D*D + 3*n*D*D)): the live counter's
    GEMM terms equal the formula's exactly; its causal q.k term exceeds n*n*D/2 by the diagonal's
    n*D/2; the candidates add their own terms."""
    D, H, L, max_len = 8, 2, 2, 64
    wl = workloads.make_custom(seed=51, dtype="f32", layers=L, d_model=D, heads=H, max_len=max_len,
                               uih_lengths=[10, 17], cand_lengths=[0, 0])
    cnt = oracle.MacCounter()
    run_oracle(wl, "f64", counter=cnt)
    ns = [10, 17]
    assert cnt.gemm_uvqk == L * sum(4 * n * D * D for n in ns)
    assert cnt.gemm_out == L * sum(3 * n * D * D for n in ns)
    assert cnt.attn_qk == L * sum(n * (n + 1) * D // 2 for n in ns)
    assert cnt.attn_qk == cnt.attn_pv and cnt.attn_self == 0
    formula = sum(2 * L * (n * n * D // 2 + n * D * D * 4 + n * D * D * 3) for n in ns)
    # the formula counts q.k of the strictly-causal pairs and both GEMMs
    assert formula == 2 * (cnt.gemm_uvqk + cnt.gemm_out + cnt.attn_qk) - 2 * L * sum(n * D // 2 for n in ns)


def test_counter_with_candidates_and_cache_matches_enumeration():
    wl = workloads.make_custom(seed=52, dtype="f32", layers=2, d_model=8, heads=2, max_len=64,
                               uih_lengths=[5, 0], cand_lengths=[3, 4], cached_lengths=[6, 2])
    cache = random_cache(wl, 1, capacity=16, bf16=False)
    cnt = oracle.MacCounter()
    run_oracle(wl, "f64", cache=cache, counter=cnt)
    want = {k: 0 for k in ["gemm_uvqk", "gemm_out", "attn_qk", "attn_pv", "attn_self"]}
    for n, c, m in [(5, 3, 6), (0, 4, 2)]:
        for k, v in count_macs(8, 2, n, c, m).items():
            want[k] += v
    assert {k: getattr(cnt, k) for k in want} == want


def test_streaming_saving_in_page_range():
    """Pin (page value): reusing the cached history state removes roughly 80-90% of the dense
    history-encoding compute in steady state. For 3000 cached + 300 new events at D=512 the
    incremental history work is 86.9% below a full re-encode of 3300 events."""
    D, L = 512, 8
    inc = count_macs(D, L, n=300, c=0, m=3000)
    full = count_macs(D, L, n=3300, c=0, m=0)
    saving = 1.0 - sum(inc.values()) / sum(full.values())
    assert abs(saving - 0.869) < 0.0005
    assert 0.80 <= saving <= 0.90
