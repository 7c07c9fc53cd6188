"""Scalar brute force for tiny encoder problems (test infrastructure only).

Re-derives every output element of the layer stack with plain Python floats and
explicit index loops, straight from the definition (the attention core
Mask(SiLU(Q K^T)) V with absolute position bias on Q, K, V, from the DLRMv3
benchmark review's "Model selection" section, and the original form it replaced,
Mask(SiLU(Q K^T) + bias) V with a relative position bias; the target-aware candidate mask;
the per-row input normalisation, the D -> 4D projection and the 3D -> D output
GEMM). It shares nothing with
``hstu_oracle`` (no NumPy arithmetic, its own bfloat16 rounding and SiLU), so the
two pin each other: a dropped term, a wrong sign, a wrong index or a transposed
operand in either one shows up as a mismatch.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_EPS = 1e-6


def bf16_round(x: float) -> float:
    """Nearest bfloat16 value (8 significant bits, ties to even) by integer arithmetic."""
    if x != x or math.isinf(x) or x == 0.0:
        return x
    _, e = math.frexp(x)
    q = max(e - 8, -133)
    scaled = math.ldexp(x, -q)            # exact: a power-of-two rescale
    lo = math.floor(scaled)
    rem = scaled - lo                     # exact for |scaled| < 2**53
    if rem > 0.5 or (rem == 0.5 and lo % 2 == 1):
        lo += 1
    y = math.ldexp(float(lo), q)
    if abs(y) > _BF16_MAX:
        return math.copysign(math.inf, x)
    if y == 0.0:
        return math.copysign(0.0, x)
    return y


def silu_scalar(x: float) -> float:
    if x < -700.0:                        # exp(-x) overflows; the limit is -0
        return -0.0
    return x / (1.0 + math.exp(-x))


def _mat(rows: int, cols: int) -> List[List[float]]:
    return [[0.0] * cols for _ in range(rows)]


def encode_brute(uih, uih_offsets, cand, cand_offsets, params, *, heads: int, max_len: int,
                 bf16: bool, cached_k=None, cached_v=None, cached_len: Optional[Sequence[int]] = None):
    """uih/cand: lists of D-lists; params: list of (w1 [D][4D], w2 [3D][D], pos [max_len][3D]
    or None[, rel [heads][max_len] or None]) as nested lists; cached_k/cached_v: per layer,
    per user, list of D-lists (the user's earlier history keys/values), cached_len per
    user. Returns (uih_out, cand_out)."""
    rnd = bf16_round if bf16 else (lambda v: v)
    B = len(uih_offsets) - 1
    D = len(params[0][0])
    dh = D // heads
    inv = 1.0 / max_len
    uih_out = [None] * len(uih)
    cand_out = [None] * len(cand)
    for b in range(B):
        xs_u = [list(r) for r in uih[uih_offsets[b]:uih_offsets[b + 1]]]
        xs_c = [list(r) for r in cand[cand_offsets[b]:cand_offsets[b + 1]]]
        m = 0 if cached_len is None else cached_len[b]
        n, c = len(xs_u), len(xs_c)
        for l, lp in enumerate(params):
            w1, w2, pos = lp[0], lp[1], lp[2]
            rel = lp[3] if len(lp) > 3 else None
            # rows in one list: history rows first (positions m..m+n-1), then candidates (m+n)
            xs = xs_u + xs_c
            posn = [m + i for i in range(n)] + [m + n] * c
            U, V, Q, K = _mat(n + c, D), _mat(n + c, D), _mat(n + c, D), _mat(n + c, D)
            for r in range(n + c):
                mean = sum(xs[r]) / D
                var = sum((t - mean) * (t - mean) for t in xs[r]) / D
                xn = [(t - mean) / math.sqrt(var + _EPS) for t in xs[r]]   # never stored: no rounding
                for j in range(4 * D):
                    g = 0.0
                    for k in range(D):
                        g += xn[k] * w1[k][j]
                    s = silu_scalar(g)
                    blk, col = divmod(j, D)
                    if blk == 0:
                        U[r][col] = rnd(s)
                    elif blk == 1:
                        V[r][col] = rnd(s + (pos[posn[r]][col] if pos is not None else 0.0))
                    elif blk == 2:
                        Q[r][col] = rnd(s + (pos[posn[r]][D + col] if pos is not None else 0.0))
                    else:
                        K[r][col] = rnd(s + (pos[posn[r]][2 * D + col] if pos is not None else 0.0))
            keys_k = ([list(x) for x in cached_k[l][b]] if m else []) + K[:n]
            keys_v = ([list(x) for x in cached_v[l][b]] if m else []) + V[:n]
            O = _mat(n + c, D)
            for r in range(n + c):
                for h in range(heads):
                    acc = [0.0] * dh
                    # history keys j at position j; a history row sees j <= its own position
                    last = posn[r] if r < n else m + n - 1
                    for j in range(last + 1):
                        sc = 0.0
                        for t in range(dh):
                            sc += Q[r][h * dh + t] * keys_k[j][h * dh + t]
                        w = silu_scalar(sc)
                        if rel is not None:          # key j sits at position j
                            w += rel[h][posn[r] - j]
                        a = rnd(w)
                        for t in range(dh):
                            acc[t] += a * keys_v[j][h * dh + t]
                    if r >= n:                         # a candidate also sees itself
                        sc = 0.0
                        for t in range(dh):
                            sc += Q[r][h * dh + t] * K[r][h * dh + t]
                        w = silu_scalar(sc)
                        if rel is not None:          # relative position 0
                            w += rel[h][0]
                        a = rnd(w)
                        for t in range(dh):
                            acc[t] += a * V[r][h * dh + t]
                    for t in range(dh):
                        O[r][h * dh + t] = rnd(inv * acc[t])
            new_rows = []
            for r in range(n + c):
                feat = U[r] + O[r] + [rnd(U[r][t] * O[r][t]) for t in range(D)]
                out = []
                for j in range(D):
                    z = 0.0
                    for k in range(3 * D):
                        z += feat[k] * w2[k][j]
                    out.append(rnd(xs[r][j] + z))
                new_rows.append(out)
            if cached_k is not None:
                cached_k[l][b] = (list(cached_k[l][b]) if m else []) + K[:n]
                cached_v[l][b] = (list(cached_v[l][b]) if m else []) + V[:n]
            xs_u, xs_c = new_rows[:n], new_rows[n:]
        for i, r in enumerate(xs_u):
            uih_out[uih_offsets[b] + i] = r
        for i, r in enumerate(xs_c):
            cand_out[cand_offsets[b] + i] = r
    return uih_out, cand_out


def pack_brute(context, action, event_offsets, mode: str, *, bf16: bool):
    """History tokens from per-event context and action embeddings (lists of D-lists),
    one user and one event at a time: "interleave" emits the event's context token and
    then its action token; "sum" emits one token, their element-wise sum (rounded to
    bfloat16 when ``bf16``). Returns (tokens, token offsets)."""
    rnd = bf16_round if bf16 else (lambda v: v)
    tokens, offsets = [], [0]
    for b in range(len(event_offsets) - 1):
        for e in range(event_offsets[b], event_offsets[b + 1]):
            if mode == "interleave":
                tokens.append(list(context[e]))
                tokens.append(list(action[e]))
            elif mode == "sum":
                tokens.append([rnd(x + y) for x, y in zip(context[e], action[e])])
            else:
                raise ValueError(mode)
        offsets.append(len(tokens))
    return tokens, offsets


def score_brute(x, layers, *, bf16: bool):
    """Candidate probabilities with scalar loops: per row, each layer's outputs as explicit
    sums over its inputs plus the bias, ReLU between layers (hidden values rounded to
    bfloat16 when ``bf16``), and the logistic function of the last layer's outputs.
    x: list of rows; layers: list of (weight [out][in], bias [out]) nested lists."""
    rnd = bf16_round if bf16 else (lambda v: v)
    out = []
    for row in x:
        h = [float(v) for v in row]
        for li, (w, b) in enumerate(layers):
            z = []
            for o in range(len(w)):
                acc = 0.0
                for k in range(len(h)):
                    acc += h[k] * w[o][k]
                z.append(acc + b[o])
            if li == len(layers) - 1:
                h = [1.0 / (1.0 + math.exp(-v)) if v >= 0 else math.exp(v) / (1.0 + math.exp(v)) for v in z]
            else:
                h = [rnd(v if v > 0.0 else 0.0) for v in z]
        out.append(h)
    return out
