"""Seeded synthetic inputs for the jagged HSTU encoder.

This module only draws numbers: lengths, token embeddings and layer parameters.
It holds none of the encoder's arithmetic, and it is the one module that both the
CPU oracle (``oracle/``) and the HIP path's tests and benchmark import.

The DLRMv3 ranking benchmark reviewed on the page "DLRMv3: MLPerf Inference
generative recommendation benchmark" (section "Dataset selection") asks for
requests with thousands of history events over a huge hashed item set, replayed in
time order. That dataset is not available here; the workloads below stand in for it:

* token embeddings are drawn directly (the embedding-table lookup is upstream of
  the encoder), N(0, 1);
* per layer, the fused projection weight W1 [D, 4D] ~ N(0, var 1/D), the output
  weight W2 [3D, D] ~ N(0, var 1/D) and the absolute position-bias table
  P [max_len, 3D] ~ N(0, std 0.02); workloads in the original HSTU form (the page's
  "Time/position encoding" paragraph) draw instead, or as well, a relative bias
  table R [heads, max_len] ~ N(0, std 0.02 unless stated) over pos_i - pos_j;
* UIH lengths follow each workload's distribution; the streaming workload draws a
  cached prefix plus newly appended events per user;
* workloads with a packing step (the page's action-embedding paragraph, same
  section) draw per history event a context embedding and an action embedding,
  both N(0, 1); the encoder's tokens are made from them by that step.

Values are drawn in float32 from ``numpy.random.Generator(PCG64(seed))`` in a fixed
order (lengths; per user UIH (context) embeddings, action embeddings when packing,
then candidate embeddings; per layer W1, W2, then P and/or R; then, for a scoring head,
per head layer its weight [out, in] ~ N(0, var 1/in) and bias ~ N(0, std 0.1)).
For bfloat16 workloads every drawn value is then stored once as the nearest
bfloat16 (round to nearest even), so both sides consume identical bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = ["WORKLOADS", "Workload", "LayerParams", "make_workload", "make_custom",
           "to_bf16_values", "lengths_to_offsets", "ReplayStream", "make_replay"]


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    seed: int
    layers: int
    dtype: str            # "f32" or "bf16"
    users: int
    uih_dist: Tuple       # ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi) | ("fixed", n)
    cached: int           # cached prefix tokens per user (streaming), 0 otherwise
    cands: int            # candidates per user
    d_model: int
    heads: int
    max_len: int          # rows of the position-bias table = UIH bound + 1 candidate slot
    position: str = "absolute"   # "absolute" (P on V, Q, K), "relative" (R on the weights) or "both"
    packing: str = "none"        # "none": the history holds tokens; "sum" / "interleave": it holds
                                 # per-event context and action embeddings, merged into tokens by
                                 # the pack step (uih_dist and cached then count events)
    head: Tuple[int, ...] = ()   # scoring head: output widths of its layers (last = outcomes)


# The five workloads. The headline one is "d512_uih2k_c2k" (D=512, UIH ~2K, 2K candidates).
WORKLOADS: Dict[str, WorkloadSpec] = {
    s.name: s for s in [
        WorkloadSpec("tiny_f32", 1, 1, "f32", 4, ("uniform", 16, 64), 0, 8, 64, 2, 65),
        WorkloadSpec("d256_uih1k_c64", 2, 4, "bf16", 32, ("uniform", 256, 1024), 0, 64, 256, 4, 1025),
        WorkloadSpec("d512_uih2k_c2k", 3, 8, "bf16", 16, ("lognormal", 2000, 0.5, 512, 4096), 0, 2048,
                     512, 4, 4097),
        WorkloadSpec("stream_3000p300_c2k", 4, 8, "bf16", 64, ("fixed", 300), 3000, 2048, 512, 4, 3301),
        WorkloadSpec("long_uih16k_c2k", 5, 16, "bf16", 4, ("uniform", 8192, 16384), 0, 2048, 512, 8, 16385),
        # the headline workload (same seed: same lengths and tokens) in the original HSTU
        # form: relative position bias only
        WorkloadSpec("d512_uih2k_c2k_rel", 3, 8, "bf16", 16, ("lognormal", 2000, 0.5, 512, 4096), 0, 2048,
                     512, 4, 4097, "relative"),
        # the long-history workload (same seed: same lengths and tokens) in the original HSTU
        # form: relative position bias only, over histories of 8K-16K rows
        WorkloadSpec("long_uih16k_c2k_rel", 5, 16, "bf16", 4, ("uniform", 8192, 16384), 0, 2048, 512, 8, 16385,
                     "relative"),
        # the headline workload's users and event counts in the original HSTU input form:
        # each event's context and action embeddings interleaved, two tokens per event
        WorkloadSpec("d512_uih2k_c2k_interleaved", 3, 8, "bf16", 16, ("lognormal", 2000, 0.5, 512, 4096), 0,
                     2048, 512, 4, 8193, "absolute", "interleave"),
        # the headline workload followed by a candidate scoring head D -> 512 -> 256 -> 1
        WorkloadSpec("d512_uih2k_c2k_scored", 3, 8, "bf16", 16, ("lognormal", 2000, 0.5, 512, 4096), 0, 2048,
                     512, 4, 4097, head=(512, 256, 1)),
    ]
}


@dataclasses.dataclass
class LayerParams:
    """One layer's parameters in mathematical layout (float32 arrays).

    w1:  [D, 4D]; G = X @ w1; column blocks U, V, Q, K.
    w2:  [3D, D]; Z = [U | O | U*O] @ w2; row blocks U, O, U*O.
    pos: [max_len, 3D]; column blocks added to V, Q, K (None: no absolute bias).
    rel: [heads, max_len]; rel[h, d] added to head h's attention weights at relative
         position d = pos_i - pos_j (None: no relative bias).
    """
    w1: np.ndarray
    w2: np.ndarray
    pos: Optional[np.ndarray]
    rel: Optional[np.ndarray] = None


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    layers: int
    d_model: int
    heads: int
    max_len: int
    uih_lengths: np.ndarray      # [B] int64, new UIH tokens (events, if packing) per user
    cand_lengths: np.ndarray     # [B] int64
    cached_lengths: np.ndarray   # [B] int64, prefix tokens (events, if packing) to be cached first
    prefix: np.ndarray           # [sum cached, D] float32 prefix tokens or context embeddings
    uih: np.ndarray              # [sum uih_lengths, D] float32 tokens or context embeddings
    cand: np.ndarray             # [sum cand_lengths, D] float32
    params: List[LayerParams]
    packing: str = "none"        # "none", "sum" or "interleave" (see WorkloadSpec)
    prefix_action: Optional[np.ndarray] = None   # [sum cached, D] action embeddings (packing only)
    action: Optional[np.ndarray] = None          # [sum uih_lengths, D] action embeddings (packing only)
    head: List[Tuple[np.ndarray, np.ndarray]] = dataclasses.field(default_factory=list)
    # scoring head layers (weight [out, in], bias [out]); empty when there is none

    @property
    def users(self) -> int:
        return int(self.uih_lengths.shape[0])


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Storage conversion: float32 -> nearest bfloat16 (ties to even), kept as float32.

    Input preparation only. NaN is not produced by the generator, so it is not handled.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (rounded.astype(np.uint32) << 16).view(np.float32).reshape(x.shape)


def lengths_to_offsets(lengths) -> np.ndarray:
    """Exclusive scan of jagged lengths (values + lengths layout), as int32 [B+1]."""
    lengths = np.asarray(lengths, dtype=np.int64)
    out = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    np.cumsum(lengths, out=out[1:])
    return out.astype(np.int32)


def _draw_lengths(rng: np.random.Generator, spec: WorkloadSpec) -> np.ndarray:
    kind = spec.uih_dist[0]
    if kind == "uniform":
        lo, hi = spec.uih_dist[1], spec.uih_dist[2]
        return rng.integers(lo, hi, size=spec.users, endpoint=True).astype(np.int64)
    if kind == "lognormal":
        median, sigma, lo, hi = spec.uih_dist[1:]
        raw = rng.lognormal(mean=math.log(median), sigma=sigma, size=spec.users)
        return np.clip(np.rint(raw), lo, hi).astype(np.int64)
    if kind == "fixed":
        return np.full(spec.users, spec.uih_dist[1], dtype=np.int64)
    raise ValueError(kind)


def _normal(rng, shape, std) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)


def _finish(spec_dtype, arrays):
    if spec_dtype == "bf16":
        return [to_bf16_values(a) for a in arrays]
    return [np.ascontiguousarray(a, dtype=np.float32) for a in arrays]


def make_custom(*, seed: int, dtype: str, layers: int, d_model: int, heads: int, max_len: int,
                uih_lengths, cand_lengths, cached_lengths=None, name: str = "custom",
                position: str = "absolute", rel_std: float = 0.02, packing: str = "none",
                head: Tuple[int, ...] = ()) -> Workload:
    """A workload with explicit lengths (tests: ragged tails, empty users, tiny shapes)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    uih_lengths = np.asarray(uih_lengths, dtype=np.int64)
    cand_lengths = np.asarray(cand_lengths, dtype=np.int64)
    B = uih_lengths.shape[0]
    cached_lengths = (np.zeros(B, dtype=np.int64) if cached_lengths is None
                      else np.asarray(cached_lengths, dtype=np.int64))
    return _draw_rest(rng, name, dtype, layers, d_model, heads, max_len,
                      uih_lengths, cand_lengths, cached_lengths, position, rel_std, packing, head)


def _draw_rest(rng, name, dtype, layers, D, H, max_len, uih_lengths, cand_lengths, cached_lengths,
               position="absolute", rel_std=0.02, packing="none", head=()):
    if position not in ("absolute", "relative", "both"):
        raise ValueError(position)
    if packing not in ("none", "sum", "interleave"):
        raise ValueError(packing)
    prefix_parts, uih_parts, cand_parts, pact_parts, act_parts = [], [], [], [], []
    for b in range(uih_lengths.shape[0]):
        m, n, c = int(cached_lengths[b]), int(uih_lengths[b]), int(cand_lengths[b])
        hist = _normal(rng, (m + n, D), 1.0)        # the user's whole history, oldest first
        prefix_parts.append(hist[:m])
        uih_parts.append(hist[m:])
        if packing != "none":                       # one action embedding per history event
            act = _normal(rng, (m + n, D), 1.0)
            pact_parts.append(act[:m])
            act_parts.append(act[m:])
        cand_parts.append(_normal(rng, (c, D), 1.0))
    params = []
    for _ in range(layers):
        w1 = _normal(rng, (D, 4 * D), 1.0 / math.sqrt(D))
        w2 = _normal(rng, (3 * D, D), 1.0 / math.sqrt(D))
        w1, w2 = _finish(dtype, [w1, w2])
        pos = rel = None
        if position in ("absolute", "both"):
            pos = _finish(dtype, [_normal(rng, (max_len, 3 * D), 0.02)])[0]
        if position in ("relative", "both"):
            rel = _finish(dtype, [_normal(rng, (H, max_len), rel_std)])[0]
        params.append(LayerParams(w1, w2, pos, rel))
    cat = lambda parts: (np.concatenate(parts, axis=0) if parts else np.zeros((0, D), np.float32))
    prefix, uih, cand = _finish(dtype, [cat(prefix_parts), cat(uih_parts), cat(cand_parts)])
    head_params, fan_in = [], D
    for width in head:
        w = _normal(rng, (width, fan_in), 1.0 / math.sqrt(fan_in))
        b = _normal(rng, (width,), 0.1)
        head_params.append(tuple(_finish(dtype, [w, b])))
        fan_in = width
    prefix_action = action = None
    if packing != "none":
        prefix_action, action = _finish(dtype, [cat(pact_parts), cat(act_parts)])
    return Workload(name=name, dtype=dtype, layers=layers, d_model=D, heads=H, max_len=max_len,
                    uih_lengths=uih_lengths, cand_lengths=cand_lengths,
                    cached_lengths=cached_lengths, prefix=prefix, uih=uih, cand=cand, params=params,
                    packing=packing, prefix_action=prefix_action, action=action, head=head_params)


def make_workload(name: str, *, users: Optional[int] = None, layers: Optional[int] = None) -> Workload:
    """Draw one of the named workloads.

    ``users``/``layers`` truncate it for quick tests. The draw order is unchanged, so the
    first users' lengths and embeddings match the full draw, but the layer parameters
    (drawn after all users) do not: a truncated workload is a different problem."""
    spec = WORKLOADS[name]
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    lengths = _draw_lengths(rng, spec)
    B = spec.users if users is None else users
    L = spec.layers if layers is None else layers
    lengths = lengths[:B]
    cands = np.full(B, spec.cands, dtype=np.int64)
    cached = np.full(B, spec.cached, dtype=np.int64)
    return _draw_rest(rng, spec.name, spec.dtype, L, spec.d_model, spec.heads, spec.max_len,
                      lengths, cands, cached, spec.position, packing=spec.packing, head=spec.head)


@dataclasses.dataclass
class ReplayStream:
    """A time-ordered request stream over many users (streaming replay).

    history[u]: [events, D] the user's whole event history, oldest first; requests: list of
    (time, user, events known at that time, candidates), in time order. A request's
    candidate embeddings come from ``candidates(i)``, drawn on demand from their own seed.
    """
    model: Workload              # the encoder's parameters (its own users are empty)
    history: Dict[int, np.ndarray]
    requests: List[Tuple[int, int, int, int]]
    seed: int
    d_model: int

    def candidates(self, i: int) -> np.ndarray:
        c = self.requests[i][3]
        rng = np.random.Generator(np.random.PCG64([self.seed, i]))
        return to_bf16_values(_normal(rng, (c, self.d_model), 1.0))


def make_replay(*, seed: int = 11, users: int = 192, requests: int = 2048, layers: int = 8, d_model: int = 512,
                heads: int = 4, max_len: int = 4097, first=("lognormal", 2000, 0.5, 512, 3000),
                new_events=(16, 128), cands: int = 2048, mean_gap: float = 1.0) -> ReplayStream:
    """Users arrive with a lognormal history (as the benchmark workload) and come back with
    uniformly many new events; request times have exponential gaps (mean ``mean_gap``); users
    are drawn uniformly per request; each request has ``cands`` candidates, N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    model = make_custom(seed=seed + 1, dtype="bf16", layers=layers, d_model=d_model, heads=heads, max_len=max_len,
                        uih_lengths=[0], cand_lengths=[0])
    median, sigma, lo, hi = first[1:]
    start = np.clip(np.rint(rng.lognormal(math.log(median), sigma, size=users)), lo, hi).astype(np.int64)
    who = rng.integers(0, users, size=requests)
    gaps = rng.exponential(mean_gap, size=requests)
    seen = np.zeros(users, dtype=np.int64)
    plan = []
    t = 0.0
    for r in range(requests):
        u = int(who[r])
        t += float(gaps[r])
        seen[u] = start[u] if seen[u] == 0 else seen[u] + int(rng.integers(new_events[0], new_events[1] + 1))
        plan.append((int(t), u, int(seen[u]), cands))
    history = {u: to_bf16_values(_normal(rng, (int(seen[u]), d_model), 1.0)) for u in range(users) if seen[u] > 0}
    return ReplayStream(model, history, plan, seed, d_model)
