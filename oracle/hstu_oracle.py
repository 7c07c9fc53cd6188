"""CPU oracle for the jagged HSTU encoder stack (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
module. It shares no code with the HIP path and must never be called by it.

What it computes is the plain definition of one DLRMv3/HSTU ranking-encoder stack,
as described on the page "DLRMv3: MLPerf Inference generative recommendation
benchmark" (section "Model selection"): per layer a D -> 4D projection, the
attention core Mask(SiLU(Q K^T)) V with an absolute position bias added to Q, K
and V, and a post-attention GEMM of 3*D*D multiply-adds per token; the user
interaction history (UIH) is encoded once and shared by every candidate, and a
user's UIH key/value state is reused across consecutive timestamps. Candidates
are target-aware ("Target-Aware Multi-Head Attention" on the page about Meta's
multi-stage sequence model): each candidate attends to the whole history and to
itself, never to another candidate, and the history's representation never
depends on the candidates. Jagged batches are concatenated values plus per-user
lengths (the KeyedJaggedTensor example of the TorchRec DLRM tutorial page,
section 2.1).

The same page's "Time/position encoding" paragraph (section "Model selection")
describes the form it replaced: the original HSTU attention Mask(SiLU(Q K^T) + bias) V
with a relative position bias. Layers may carry that bias too (``rel``, one value per
head and relative position pos_i - pos_j, added to each attention weight after the
SiLU, as the page writes it), and may omit the absolute table (``pos`` None).

The same section's action-embedding paragraph describes the input forms: the original
HSTU weaves each event's context features and its action into the sequence as two
tokens, doubling the sequence length, while DLRMv3 merges the two embeddings of an
event into one token. ``pack_uih`` builds either form from per-event embeddings.

``score_head`` turns candidate rows into probabilities: the same section keeps a
top-layer MLP for the final prediction, and the TorchRec tutorial page (section 1.1,
the combination and final output) takes the probability as the sigmoid of the top
MLP's output.

Readings adopted where the pages are silent (each listed in the design notes):
the 3*D*D GEMM consumes [U | O | U*O]; the residual is X + Z; each layer
normalises its input rows (zero mean, unit variance over D, eps 1e-6, no learned
scale or shift) before the projection, which keeps the stacked blocks stable (the
multi-stage page stresses stacking blocks with stable attention distributions;
without it the configured 8- and 16-layer stacks overflow); no GEMM biases; SiLU on all four projection slices; one [max_len, 3D]
position table per layer with column blocks V, Q, K, added after SiLU; every
candidate sits at position m+n (the next-event slot); the scale 1/max_len is
applied once to each attention output; the UIH mask is causal with the diagonal
included.

Arithmetic is float64 throughout. ``mode="f64"`` applies no intermediate
rounding. ``mode="bf16"`` mirrors a bfloat16 pipeline by rounding (to nearest,
ties to even) at exactly the values such a pipeline stores: U, V, Q, K after
bias; every attention weight (SiLU(q.k), plus the relative bias when present); every
attention output; the gate U*O;
and X + Z. The normalised layer input is not among them: the pipeline applies
the normalisation to the projection's float32 product and never stores
normalised rows.

Parity pins for every function here live in tests/test_oracle_pins.py (brute
force on tiny inputs, closed forms, invariants, the page's jagged example and
its FLOP formula).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = ["round_bf16", "silu", "normalize_rows", "NORM_EPS", "jagged_offsets", "MacCounter", "OracleCache",
           "encode", "layer_user", "attention_user", "user_positions", "count_macs", "pack_uih",
           "sigmoid", "score_head"]

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_BF16_MIN_QUANTUM_EXP = -133          # smallest bfloat16 subnormal is 2**-133
NORM_EPS = 1e-6


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits with float32's exponent range: a value of
    binade [2**(e-1), 2**e) is quantised to multiples of 2**(e-8), subnormals to
    multiples of 2**-133. Results beyond the largest finite bfloat16 become
    +-inf (IEEE overflow under round-to-nearest); signed zeros, inf and NaN pass
    through. Rounds once from float64 (no intermediate float32 step).
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, _BF16_MIN_QUANTUM_EXP)
    with np.errstate(invalid="ignore", over="ignore"):
        y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
        y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, x), y)
    return y


def silu(x) -> np.ndarray:
    """SiLU(x) = x / (1 + exp(-x)) in float64; tends to -0 as x -> -inf (no NaN)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def normalize_rows(x) -> np.ndarray:
    """Each row minus its mean, divided by sqrt(its variance + NORM_EPS) (population
    variance over the row's D features); no learned scale or shift."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = np.mean((x - mu) ** 2, axis=1, keepdims=True)
    return (x - mu) / np.sqrt(var + NORM_EPS)


def jagged_offsets(lengths) -> np.ndarray:
    """Offsets of a jagged batch: the exclusive running sum of the segment lengths,
    with one more entry than there are segments (values + lengths layout)."""
    out = [0]
    for n in lengths:
        if int(n) < 0:
            raise ValueError("negative segment length")
        out.append(out[-1] + int(n))
    return np.asarray(out, dtype=np.int64)


@dataclasses.dataclass
class MacCounter:
    """Multiply-accumulates counted while the oracle computes, by category.

    gemm_uvqk: the D -> 4D projection; gemm_out: the 3D -> D output GEMM;
    attn_qk / attn_pv: q.k and a*v over masked history keys (dh per pair and head,
    i.e. D per pair over all heads); attn_self: a candidate's q.k and a*v with itself.
    """
    gemm_uvqk: int = 0
    gemm_out: int = 0
    attn_qk: int = 0
    attn_pv: int = 0
    attn_self: int = 0

    def total_macs(self) -> int:
        return self.gemm_uvqk + self.gemm_out + self.attn_qk + self.attn_pv + self.attn_self

    def algorithmic_flops(self) -> int:
        return 2 * self.total_macs()


@dataclasses.dataclass
class OracleCache:
    """Per-layer, per-slot history keys and values (after bias), float64.

    k, v: [L, slots, capacity, D]; rows 0..cached_len[b]-1 of slot slot_of_user[b]
    hold the user's earlier history, in position order.
    """
    k: np.ndarray
    v: np.ndarray
    slot_of_user: np.ndarray
    cached_len: np.ndarray

    def copy(self) -> "OracleCache":
        return OracleCache(self.k.copy(), self.v.copy(), self.slot_of_user.copy(),
                           self.cached_len.copy())


def user_positions(m: int, n: int, c: int) -> Tuple[np.ndarray, np.ndarray]:
    """Absolute positions: new history row i sits at m+i; every candidate sits at m+n."""
    return np.arange(m, m + n, dtype=np.int64), np.full(c, m + n, dtype=np.int64)


def attention_user(q_u, k_all, v_all, q_c, k_c, v_c, *, m: int, heads: int, inv: float,
                   bf16: bool, counter: Optional[MacCounter] = None,
                   uih_rows: Optional[Sequence[int]] = None,
                   cand_rows: Optional[Sequence[int]] = None, block: int = 256, rel=None):
    """Target-aware causal SiLU attention for one user.

    q_u [n, D]: new history queries (row i at position m+i); k_all, v_all [m+n, D]:
    every history key/value, row j at position j; q_c, k_c, v_c [c, D]: candidates.
    History row i: O_i = inv * sum_{j <= m+i} a(i, j) v_j.
    Candidate r:   O_r = inv * (sum_{all j} a(r, j) v_j + a(r, r) v_r).
    The weight is a(i, j) = SiLU(q_i.k_j), plus rel[h, pos_i - pos_j] when a relative
    bias table rel [heads, >= m+n+1] is given (candidates sit at position m+n).
    Per head h the columns [h*dh, (h+1)*dh) are used. ``uih_rows`` / ``cand_rows``
    restrict the outputs to the listed rows (the results then have that many rows).
    Returns (O_u, O_c).
    """
    n, D = q_u.shape
    dh = D // heads
    rows = np.arange(n) if uih_rows is None else np.asarray(uih_rows, dtype=np.int64)
    if cand_rows is not None:
        sel = np.asarray(cand_rows, dtype=np.int64)
        q_c, k_c, v_c = q_c[sel], k_c[sel], v_c[sel]
    c = q_c.shape[0]
    R = round_bf16 if bf16 else (lambda a: a)
    o_u = np.zeros((rows.shape[0], D))
    o_c = np.zeros((c, D))
    nkeys = k_all.shape[0]
    key_pos = np.arange(nkeys)
    for h in range(heads):
        cols = slice(h * dh, (h + 1) * dh)
        kh, vh = k_all[:, cols], v_all[:, cols]
        for s in range(0, rows.shape[0], block):
            rb = rows[s:s + block]
            allowed = key_pos[None, :] <= (m + rb)[:, None]
            w = silu(q_u[rb][:, cols] @ kh.T)
            if rel is not None:
                w = w + rel[h][np.maximum((m + rb)[:, None] - key_pos[None, :], 0)]
            a = np.where(allowed, w, 0.0)
            a = R(a)
            o_u[s:s + block, cols] = R(inv * (a @ vh))
            if counter is not None:
                counter.attn_qk += int(allowed.sum()) * dh
                counter.attn_pv += int(allowed.sum()) * dh
        for s in range(0, c, block):
            qc = q_c[s:s + block, cols]
            w = silu(qc @ kh.T)
            w_self = silu(np.sum(qc * k_c[s:s + block, cols], axis=1))
            if rel is not None:
                w = w + rel[h][(m + n) - key_pos][None, :]
                w_self = w_self + rel[h][0]
            a = R(w)
            a_self = R(w_self)
            o_c[s:s + block, cols] = R(inv * (a @ vh + a_self[:, None] * v_c[s:s + block, cols]))
            if counter is not None:
                counter.attn_qk += qc.shape[0] * nkeys * dh
                counter.attn_pv += qc.shape[0] * nkeys * dh
                counter.attn_self += 2 * qc.shape[0] * dh
    return o_u, o_c


def _project(x, w1, pos_table, positions, bf16, counter):
    """S = SiLU(norm(X) W1) split into U, V, Q, K; position bias on V, Q, K (not U),
    none when pos_table is None. The normalised rows are never stored, so they take no
    rounding in either mode."""
    D = x.shape[1]
    R = round_bf16 if bf16 else (lambda a: a)
    s = silu(normalize_rows(x) @ w1)
    if counter is not None:
        counter.gemm_uvqk += x.shape[0] * D * 4 * D
    bias = pos_table[positions] if pos_table is not None else np.zeros((x.shape[0], 3 * D))
    u = R(s[:, 0:D])
    v = R(s[:, D:2 * D] + bias[:, 0:D])
    q = R(s[:, 2 * D:3 * D] + bias[:, D:2 * D])
    k = R(s[:, 3 * D:4 * D] + bias[:, 2 * D:3 * D])
    return u, v, q, k


def _output(x, u, o, w2, bf16, counter):
    """X' = X + [U | O | U*O] W2 (gate and sum rounded once each in bf16 mode)."""
    R = round_bf16 if bf16 else (lambda a: a)
    D = x.shape[1]
    gate = R(u * o)
    z = np.concatenate([u, o, gate], axis=1) @ w2
    if counter is not None:
        counter.gemm_out += x.shape[0] * 3 * D * D
    return R(x + z)


def layer_user(x_u, x_c, w1, w2, pos_table, *, k_cached, v_cached, heads: int, max_len: int,
               bf16: bool, counter: Optional[MacCounter] = None,
               uih_rows: Optional[Sequence[int]] = None,
               cand_rows: Optional[Sequence[int]] = None, rel=None):
    """One encoder layer for one user.

    x_u [n, D] new history tokens, x_c [c, D] candidates, k_cached/v_cached [m, D]
    the user's cached keys/values for this layer. History and candidate rows go
    through separate products, so history results never depend on the candidates.
    Returns (x_u', x_c', k_new, v_new); with ``uih_rows`` / ``cand_rows`` x_u' / x_c'
    hold only those rows (every history row is still projected: all are keys).
    """
    m = k_cached.shape[0]
    n, c = x_u.shape[0], x_c.shape[0]
    if m + n + 1 > max_len:
        raise ValueError("history plus candidate slot exceeds the position table")
    pos_u, pos_c = user_positions(m, n, c)
    u_u, v_u, q_u, k_u = _project(x_u, w1, pos_table, pos_u, bf16, counter)
    if cand_rows is not None:
        x_c = x_c[np.asarray(cand_rows, dtype=np.int64)]
        pos_c = pos_c[:x_c.shape[0]]
    u_c, v_c, q_c, k_c = _project(x_c, w1, pos_table, pos_c, bf16, counter)
    k_all = np.concatenate([k_cached, k_u], axis=0)
    v_all = np.concatenate([v_cached, v_u], axis=0)
    o_u, o_c = attention_user(q_u, k_all, v_all, q_c, k_c, v_c, m=m, heads=heads,
                              inv=1.0 / max_len, bf16=bf16, counter=counter, uih_rows=uih_rows, rel=rel)
    rows = np.arange(n) if uih_rows is None else np.asarray(uih_rows, dtype=np.int64)
    y_u = _output(x_u[rows], u_u[rows], o_u, w2, bf16, counter)
    y_c = _output(x_c, u_c, o_c, w2, bf16, counter)
    return y_u, y_c, k_u, v_u


def encode(uih, uih_offsets, cand, cand_offsets, params, *, heads: int, max_len: int,
           mode: str, cache: Optional[OracleCache] = None,
           counter: Optional[MacCounter] = None, users: Optional[Sequence[int]] = None):
    """The whole layer stack over a jagged batch.

    uih [Nu, D], cand [Nc, D]: tokens in jagged layout with int offsets [B+1].
    params: per layer (w1 [D,4D], w2 [3D,D], pos [max_len,3D] or None, and optionally
    rel [heads, max_len] or None) in math layout (objects with .w1/.w2/.pos[/.rel] or
    3- or 4-tuples). mode: "f64" or "bf16".
    cache: None (no earlier history) or an OracleCache; a copy is returned with
    every layer's new keys/values appended and cached_len advanced.
    users: optional subset of user indices to compute (the others' rows are NaN).
    Returns (uih_out [Nu, D], cand_out [Nc, D], new_cache).
    """
    if mode not in ("f64", "bf16"):
        raise ValueError(mode)
    bf16 = mode == "bf16"
    uih = np.asarray(uih, dtype=np.float64)
    cand = np.asarray(cand, dtype=np.float64)
    D = uih.shape[1]
    layers = [(p.w1, p.w2, p.pos, getattr(p, "rel", None)) if hasattr(p, "w1") else (tuple(p) + (None,))[:4]
              for p in params]
    layers = [tuple(None if a is None else np.asarray(a, dtype=np.float64) for a in lp) for lp in layers]
    B = len(uih_offsets) - 1
    new_cache = cache.copy() if cache is not None else None
    uih_out = np.full_like(uih, np.nan)
    cand_out = np.full_like(cand, np.nan)
    for b in (range(B) if users is None else users):
        xu = uih[uih_offsets[b]:uih_offsets[b + 1]]
        xc = cand[cand_offsets[b]:cand_offsets[b + 1]]
        n = xu.shape[0]
        if new_cache is not None:
            slot, m = int(new_cache.slot_of_user[b]), int(new_cache.cached_len[b])
            if m + n > new_cache.k.shape[2]:
                raise ValueError("cache capacity exceeded")
        else:
            slot, m = -1, 0
        for l, (w1, w2, pos, rel) in enumerate(layers):
            if new_cache is not None:
                kc, vc = new_cache.k[l, slot, :m], new_cache.v[l, slot, :m]
            else:
                kc, vc = np.zeros((0, D)), np.zeros((0, D))
            xu, xc, k_new, v_new = layer_user(xu, xc, w1, w2, pos, k_cached=kc, v_cached=vc,
                                              heads=heads, max_len=max_len, bf16=bf16,
                                              counter=counter, rel=rel)
            if new_cache is not None:
                new_cache.k[l, slot, m:m + n] = k_new
                new_cache.v[l, slot, m:m + n] = v_new
        if new_cache is not None:
            new_cache.cached_len[b] = m + n
        uih_out[uih_offsets[b]:uih_offsets[b + 1]] = xu
        cand_out[cand_offsets[b]:cand_offsets[b + 1]] = xc
    return uih_out, cand_out, new_cache


def pack_uih(context, action, event_offsets, mode: str, *, bf16: bool = False):
    """The encoder's history tokens from per-event context and action embeddings.

    The DLRMv3 page (section "Model selection", action-embedding preprocessing): the
    original HSTU interleaves context features and user actions in the input sequence,
    which doubles its length; DLRMv3 merges an event's action and context embeddings
    into one token instead. Readings: ``"interleave"`` gives user b the tokens
    c_0, a_0, c_1, a_1, ... (an event's context token, then its action token);
    ``"sum"`` merges by addition, c_i + a_i (rounded to bfloat16 when ``bf16``).

    context, action: [E, D] in the jagged order of ``event_offsets`` [B+1].
    Returns (tokens [rows, D] float64, token offsets [B+1] int64).
    """
    if mode not in ("sum", "interleave"):
        raise ValueError(mode)
    context = np.asarray(context, dtype=np.float64)
    action = np.asarray(action, dtype=np.float64)
    if context.shape != action.shape:
        raise ValueError("context and action shapes differ")
    D = context.shape[1]
    B = len(event_offsets) - 1
    parts, lengths = [], []
    for b in range(B):
        c = context[event_offsets[b]:event_offsets[b + 1]]
        a = action[event_offsets[b]:event_offsets[b + 1]]
        if mode == "sum":
            t = c + a
            if bf16:
                t = round_bf16(t)
        else:
            t = np.empty((2 * c.shape[0], D))
            t[0::2] = c
            t[1::2] = a
        parts.append(t)
        lengths.append(t.shape[0])
    tokens = np.concatenate(parts, axis=0) if parts else np.zeros((0, D))
    return tokens, jagged_offsets(lengths)


def sigmoid(z) -> np.ndarray:
    """The logistic function 1 / (1 + exp(-z)) in float64, evaluated as exp(z) / (1 + exp(z))
    for negative z so that neither branch overflows."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def score_head(x, layers, *, bf16: bool = False):
    """Probabilities of the predicted outcomes for each candidate row.

    x: [rows, D] candidate rows (the encoder's final outputs). layers: sequence of
    (weight [out, in], bias [out]). Readings where the pages are silent: every layer is
    affine, h W^T + b; a ReLU follows every layer but the last; the last layer's outputs
    are one logit per outcome and each probability is the sigmoid of its logit. In
    ``bf16`` mode the hidden activations are rounded to bfloat16 (a pipeline stores them);
    logits and probabilities are not.
    Returns [rows, outcomes] float64.
    """
    h = np.asarray(x, dtype=np.float64)
    for i, (w, b) in enumerate(layers):
        z = h @ np.asarray(w, dtype=np.float64).T + np.asarray(b, dtype=np.float64)
        if i == len(layers) - 1:
            return sigmoid(z)
        h = np.maximum(z, 0.0)
        if bf16:
            h = round_bf16(h)
    raise ValueError("the head needs at least one layer")


def count_macs(D: int, layers: int, n: int, c: int, m: int) -> Dict[str, int]:
    """Multiply-accumulates of ``layers`` layers for one user with m cached, n new and
    c candidate rows, enumerated query row by query row (history row i sees m+i+1 keys;
    each candidate sees the m+n history keys plus itself). Gives the counter's values
    at sizes where running the oracle itself would take too long."""
    pairs_u = sum(m + i + 1 for i in range(n))
    pairs_c = c * (m + n)
    per_layer = {
        "gemm_uvqk": (n + c) * D * 4 * D,
        "gemm_out": (n + c) * 3 * D * D,
        "attn_qk": (pairs_u + pairs_c) * D,
        "attn_pv": (pairs_u + pairs_c) * D,
        "attn_self": 2 * c * D,
    }
    return {k: v * layers for k, v in per_layer.items()}
