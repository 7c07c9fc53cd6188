"""Time-ordered request replay over the paged streaming key/value cache.

Each request brings a user's events since its previous request, and candidates to
encode. Requests are served in time order, in batches of distinct users. Per batch the
library's page pool (``KvPool``, hstu_pool_*) says, for each user, whether its cached
rows are extended (only the new events are sent) or its history is sent again (a user
seen for the first time, evicted, stale (older than the TTL), or out of room), and
which pages of the cache hold its rows; a user holds ceil(rows / 64) pages. A history
sent again is the user's latest ``window`` events.

This module is plumbing: it assembles each batch's history rows on the host (as a
serving front end receives them) and copies them to the device in one transfer,
gathers the candidates (host rows, or rows already on the device), calls ``encode``
(and ``score``, when a head is given) on the stream, and keeps the bookkeeping. Every
computation runs in the library's kernels. Histories are numpy arrays or CPU torch
tensors in the model's dtype (then the transfer moves the stored bytes as they are).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

from . import HSTU_OK, KvPool, Model, PagedKVCache, ScoringHead, encode, hstu_flops, score


@dataclasses.dataclass
class Request:
    time: int
    user: int
    events: int                  # events of the user's history known at this time (cumulative)
    cand: object                 # [c, D] candidate embeddings: numpy, or a device tensor


@dataclasses.dataclass
class Served:
    """What one request got: its rows as encoded, and where they sit in the user's history."""
    request: Request
    window_start: int            # history index of the user's cached row 0
    sent_from: int               # first history event sent with this request
    rebuild: bool
    uih_out: np.ndarray          # [events - sent_from, D] outputs of the rows sent
    cand_out: np.ndarray         # [c, D]
    prob: Optional[np.ndarray]   # [c, outcomes] when a head is given


class Replayer:
    """Serves requests against one model, one PagedKVCache and one KvPool of the cache's pages."""

    def __init__(self, model: Model, cache: PagedKVCache, pool: KvPool, history: Dict[int, np.ndarray], *,
                 window: int, head: Optional[ScoringHead] = None, device="cuda", keep_outputs: bool = True):
        if window < 1 or window > pool.max_rows:
            raise ValueError("window must be in [1, the pool's max_rows]")
        if (pool.max_rows > min(cache.pages_per_user * 64, model.max_len - 1) or pool.pages != cache.pages):
            raise ValueError("the pool must manage the cache's pages and allow at most min(pages_per_user * 64, "
                             "max_len - 1) rows per user")
        self.model, self.cache, self.pool, self.history = model, cache, pool, history
        self.window, self.head, self.device, self.keep_outputs = window, head, device, keep_outputs
        self.seen: Dict[int, int] = {}          # events of each user already in its cached rows
        self.start: Dict[int, int] = {}         # history index of each user's cached row 0
        self.rows_sent = 0
        self.batches = 0
        self.flops = 0              # algorithmic flops of the encodes served
        self.flops_no_cache = 0     # the same requests, each window encoded from scratch
        self.rows_no_cache = 0      # history rows those from-scratch encodes would send

    def batches_of(self, requests: Sequence[Request], max_users: int) -> List[List[Request]]:
        """Consecutive requests in time order, cut when a batch is full or a user repeats."""
        out, cur, users = [], [], set()
        for r in sorted(requests, key=lambda r: r.time):
            if len(cur) == max_users or r.user in users:
                out.append(cur)
                cur, users = [], set()
            cur.append(r)
            users.add(r.user)
        if cur:
            out.append(cur)
        return out

    def _to_device(self, parts):
        """Rows of several arrays as one device tensor in the model's dtype: host rows go in
        one pinned transfer, device rows are concatenated on the device."""
        import torch
        D = self.model.d_model
        if not parts:
            return torch.zeros((0, D), dtype=self.model.torch_dtype, device=self.device)
        if isinstance(parts[0], torch.Tensor):
            if parts[0].is_cuda:
                return torch.cat(parts)
            staged = torch.cat(parts).pin_memory()
        else:
            staged = torch.from_numpy(np.concatenate(parts).astype(np.float32)).pin_memory()
        return staged.to(device=self.device, dtype=self.model.torch_dtype, non_blocking=True)

    def serve(self, batch: Sequence[Request]) -> List[Served]:
        now = max(r.time for r in batch)
        users = [r.user for r in batch]
        if len(batch) > self.cache.max_users:
            raise ValueError("a batch has more users than the cache's page table")
        new = [r.events - self.seen.get(r.user, 0) for r in batch]
        window = [min(r.events, self.window) for r in batch]
        table, cached, rebuild = self.pool.assign(users, new, window, now, self.cache.pages_per_user)
        parts, lengths, sent_from = [], [], []
        for r, c, rb in zip(batch, cached, rebuild):
            lo = r.events - min(r.events, self.window) if rb else self.seen[r.user]
            if rb:
                self.start[r.user] = lo
            assert int(c) == (0 if rb else lo - self.start[r.user])
            parts.append(self.history[r.user][lo:r.events])
            lengths.append(r.events - lo)
            sent_from.append(lo)
        uih = self._to_device(parts)
        cand = self._to_device([r.cand for r in batch])
        uo = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        co = np.concatenate([[0], np.cumsum([int(r.cand.shape[0]) for r in batch])]).astype(np.int32)
        # the table is shared by the batches: the copy is ordered after the previous batch's
        # kernels on the stream they share
        self.cache.set_table(table)
        self.cache.cached_len = cached.astype(np.int32).copy()
        try:
            out_u, out_c = encode(self.model, uih, uo, cand, co, cache=self.cache)
        except Exception:
            self.pool.abort(users)
            for u in users:
                self.seen.pop(u, None)
                self.start.pop(u, None)
            raise
        total = [int(c) + n for c, n in zip(cached, lengths)]
        self.pool.commit(users, total, now)
        st, f, _ = hstu_flops(self.model.dims(), len(batch), uo, co, cached)
        st2, f0, _ = hstu_flops(self.model.dims(), len(batch), np.concatenate([[0], np.cumsum(total)]), co, None)
        if st == HSTU_OK and st2 == HSTU_OK:
            self.flops += f
            self.flops_no_cache += f0
        self.rows_no_cache += sum(total)
        for r in batch:
            self.seen[r.user] = r.events
        prob = score(self.model, self.head, out_c) if self.head is not None else None
        self.rows_sent += int(uo[-1])
        self.batches += 1
        if not self.keep_outputs:
            return []
        gu = out_u.float().cpu().numpy()
        gc = out_c.float().cpu().numpy()
        gp = prob.cpu().numpy() if prob is not None else None
        served = []
        for b, r in enumerate(batch):
            served.append(Served(r, self.start[r.user], sent_from[b], bool(rebuild[b]), gu[uo[b]:uo[b + 1]],
                                 gc[co[b]:co[b + 1]], None if gp is None else gp[co[b]:co[b + 1]]))
        return served
