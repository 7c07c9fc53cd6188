"""Host tests of the attention work planner (hstu_attention_plan, the plan hstu_encode
launches): every work item exactly once, a (user, head) group whole in one XCD bin, the
bins as an independent re-implementation of the documented rule fills them (groups
largest first onto the least loaded bin, items longest first inside a bin), and the
workgroup count. Nothing here touches a GPU."""
import numpy as np
import pytest

import hstu_silu_attention_amd as hsa
import workloads

XCDS = 8


def decode(codes):
    out = []
    for c in codes.tolist():
        if c < 0:
            out.append(None)
        else:
            user, code = c >> 32, c & 0xFFFFFFFF
            out.append((user, (code >> 1) & 0x7F, code & 1, code >> 8))   # user, head, candidate, block
    return out


def expected_bins(ul, cl, ml, heads, q):
    """The documented rule, written independently: per (user, head) its items with their
    costs (key blocks swept, plus a fixed 13 for a history item and 22 for a candidate
    item), groups largest first (ties in user-then-head order) onto the least loaded bin
    (the first such), items of a bin longest first (ties in the order they were added)."""
    groups = []
    for b in range(len(ul)):
        for h in range(heads):
            items = []
            for i, q0 in enumerate(range(0, ul[b], q)):
                nq = min(q, ul[b] - q0)
                items.append(((ml[b] + q0 + nq + 63) // 64 + 13, (b, h, 0, i)))
            for i, q0 in enumerate(range(0, cl[b], q)):
                items.append(((ml[b] + ul[b] + 63) // 64 + 22, (b, h, 1, i)))
            if items:
                items = [it for _, it in sorted(enumerate(items), key=lambda t: (-t[1][0], t[0]))]
                groups.append((sum(c for c, _ in items), items))
    order = sorted(range(len(groups)), key=lambda g: (-groups[g][0], g))
    load, bins = [0] * XCDS, [[] for _ in range(XCDS)]
    for g in order:
        x = load.index(min(load))
        load[x] += groups[g][0]
        bins[x] += groups[g][1]
    return [[it for _, it in sorted(enumerate(bn), key=lambda t: (-t[1][0], t[0]))] for bn in bins]


@pytest.mark.parametrize("seed,dtype,heads,dh", [(0, "bf16", 4, 128), (1, "bf16", 8, 128), (2, "f32", 2, 64),
                                                 (3, "bf16", 1, 128), (5, "bf16", 4, 64), (6, "bf16", 4, 32),
                                                 (4, "bf16", 127, 128)])   # the most heads an item code holds
def test_plan_matches_the_documented_rule(seed, dtype, heads, dh):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 24))
    ul = [int(x) for x in rng.integers(0, 1500, size=B)]
    cl = [int(x) for x in rng.integers(0, 700, size=B)]
    ml = [int(x) for x in rng.integers(0, 900, size=B)]
    ul[0], cl[0] = 0, 0                                 # an empty user
    D = dh * heads
    d = hsa.HstuDims(2, D, heads, 4000, hsa.HSTU_BF16 if dtype == "bf16" else hsa.HSTU_F32)
    st, codes = hsa.hstu_attention_plan(d, B, workloads.lengths_to_offsets(ul), workloads.lengths_to_offsets(cl), ml)
    assert st == 0
    q = 128 if dtype == "bf16" else 64
    bins = expected_bins(ul, cl, ml, heads, q)
    assert len(codes) == XCDS * max(len(bn) for bn in bins)
    got = decode(codes)
    for x in range(XCDS):
        mine = got[x::XCDS]                             # workgroup w runs on XCD w % 8
        want = [it for _, it in bins[x]]
        assert mine[:len(want)] == want and all(v is None for v in mine[len(want):])
    # every item exactly once; each (user, head) in one bin
    items = [g for g in got if g is not None]
    assert len(items) == len(set(items)) == sum(heads * (-(-ul[b] // q) + -(-cl[b] // q)) for b in range(B))
    where = {}
    for w, g in enumerate(got):
        if g is not None:
            assert where.setdefault(g[:2], w % XCDS) == w % XCDS


def test_plan_edge_cases():
    d = hsa.HstuDims(1, 256, 2, 100, hsa.HSTU_BF16)
    st, codes = hsa.hstu_attention_plan(d, 0, None, None)
    assert st == 0 and len(codes) == 0
    st, codes = hsa.hstu_attention_plan(d, 2, [0, 0, 0], [0, 0, 0])      # nothing to attend
    assert st == 0 and len(codes) == 0
    st, codes = hsa.hstu_attention_plan(d, 1, [0, 1], [0, 0])            # one row: two heads, two bins
    assert st == 0 and len(codes) == 8 and sorted(c for c in codes.tolist() if c >= 0) == [0 << 1, 1 << 1]
    assert hsa.hstu_attention_plan(d, 2, [0, 5, 3], [0, 0, 0])[0] == 3   # decreasing offsets
    assert hsa.hstu_attention_plan(d, 1, [0, 5], [0, 0], [-1])[0] == 4   # negative cached length
