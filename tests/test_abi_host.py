"""Host-side tests of the C ABI: the library loads and exports what include/hstu.h declares,
validation rejects bad arguments before anything touches a GPU, and the host FLOP counter
equals the oracle's live counter. Nothing here launches a kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

import hstu_silu_attention_amd as hsa
import oracle
from oracle.hstu_oracle import count_macs
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hstu.h")

OK, ERR_NULL, ERR_SHAPE, ERR_OFFSETS, ERR_CAPACITY, ERR_WORKSPACE, ERR_HIP, ERR_ALIGN, ERR_TOO_LARGE = range(9)


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:hstu_status|int32_t|const char\*|void)\s+(hstu_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = hsa.load_library()
    names = header_functions()
    assert {"hstu_abi_version", "hstu_status_string", "hstu_workspace_size", "hstu_flops", "hstu_encode",
            "hstu_pack_uih", "hstu_score", "hstu_pool_create", "hstu_pool_destroy", "hstu_pool_assign",
            "hstu_pool_commit", "hstu_pool_abort", "hstu_pool_stats", "hstu_pool_lookup", "hstu_timing_enable",
            "hstu_timing_select", "hstu_timing_read", "hstu_encode_static", "hstu_transpose_weights"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    version = int(re.search(r"#define HSTU_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert hsa.hstu_abi_version() == version


def test_status_strings():
    seen = set()
    for s in range(9):
        msg = hsa.hstu_status_string(s)
        assert msg and msg not in seen
        seen.add(msg)
    assert hsa.hstu_status_string(99) == "unknown status"


def dims(L=2, D=256, H=4, max_len=64, dtype=hsa.HSTU_BF16, weight_layout=hsa.HSTU_WEIGHTS_PREPARED):
    return hsa.HstuDims(L, D, H, max_len, dtype, weight_layout)


@pytest.mark.parametrize("d,want", [
    (dims(), OK),
    (dims(D=256, H=8), OK),                      # bf16, dh = 32
    (dims(D=256, H=16), ERR_SHAPE),              # dh = 16
    (dims(D=192, H=3), ERR_SHAPE),               # D % 128
    (dims(D=256, H=3), ERR_SHAPE),               # D % H
    (dims(dtype=2), ERR_SHAPE),
    (dims(L=0), ERR_SHAPE),
    (dims(max_len=0), ERR_SHAPE),
    (dims(D=512, max_len=1398101), OK),          # 3 * D * max_len = 2^31 - 512
    (dims(D=512, max_len=1398102), ERR_SHAPE),   # a position table of 2^31 elements
    (dims(D=64, H=2, dtype=hsa.HSTU_F32), OK),   # fp32, dh = 32
    (dims(D=96, H=3, dtype=hsa.HSTU_F32), ERR_SHAPE),
    (dims(D=512, H=2, dtype=hsa.HSTU_F32), ERR_SHAPE),   # dh = 256
    (dims(weight_layout=hsa.HSTU_WEIGHTS_MATH), OK),
    (dims(weight_layout=2), ERR_SHAPE),
    (dims(weight_layout=-1), ERR_SHAPE),
])
def test_workspace_size_dims(d, want):
    st, _ = hsa.hstu_workspace_size(d, 1, [0, 5], [0, 3])
    assert st == want


def test_workspace_size_offsets_and_growth():
    d = dims()
    assert hsa.hstu_workspace_size(d, 2, [1, 5, 6], [0, 0, 0])[0] == ERR_OFFSETS
    assert hsa.hstu_workspace_size(d, 2, [0, 5, 4], [0, 0, 0])[0] == ERR_OFFSETS
    assert hsa.hstu_workspace_size(d, 2, [0, 5, 6], [0, 2, 1])[0] == ERR_OFFSETS
    assert hsa.hstu_workspace_size(d, -1, None, None)[0] == ERR_SHAPE
    assert hsa.hstu_workspace_size(d, 0, None, None) == (OK, 0)
    assert hsa.hstu_workspace_size(d, 2, [0, 0, 0], [0, 0, 0]) == (OK, 0)
    _, small = hsa.hstu_workspace_size(d, 2, [0, 5, 6], [0, 2, 3])
    _, big = hsa.hstu_workspace_size(d, 2, [0, 500, 600], [0, 2, 3])
    assert 0 < small < big
    # at least the [T][4D] projection, [T][D] attention output and [T][D] layer buffer
    T = 603
    assert big >= T * 6 * 256 * 2


@pytest.mark.parametrize("dtype,D,L", [(hsa.HSTU_BF16, 256, 2), (hsa.HSTU_BF16, 512, 8), (hsa.HSTU_F32, 192, 3)])
def test_workspace_size_math_layout_adds_the_transposed_weights(dtype, D, L):
    """With weights in the math layout the workspace also holds every layer's W1 and W2
    transposed: 7 D^2 elements a layer (a multiple of the 256-byte alignment here)."""
    es = 2 if dtype == hsa.HSTU_BF16 else 4
    H = D // 64
    _, prep = hsa.hstu_workspace_size(dims(L, D, H, 64, dtype), 2, [0, 5, 9], [0, 3, 3])
    _, math = hsa.hstu_workspace_size(dims(L, D, H, 64, dtype, hsa.HSTU_WEIGHTS_MATH), 2, [0, 5, 9], [0, 3, 3])
    assert math - prep == L * 7 * D * D * es
    # nothing to encode: no workspace in either layout
    assert hsa.hstu_workspace_size(dims(L, D, H, 64, dtype, hsa.HSTU_WEIGHTS_MATH), 1, [0, 0], [0, 0]) == (OK, 0)


def test_binding_and_library_abi_versions_agree():
    assert hsa.hstu_abi_version() == hsa.ABI_VERSION


def test_workspace_size_page_offsets_example():
    """The jagged example's offsets (10 users, one of them empty) are a valid batch."""
    lengths = [1, 1, 1, 1, 1, 2, 3, 2, 2, 0]
    offs = oracle.jagged_offsets(lengths).tolist()
    st, nbytes = hsa.hstu_workspace_size(dims(), 10, offs, offs)
    assert st == OK and nbytes > 0


# ------------------------------------------------------------------------------ FLOP counter

@pytest.mark.parametrize("uih,cand,cached", [([10, 17], [0, 0], None), ([5, 0, 3], [3, 4, 0], [6, 2, 0])])
def test_flops_equal_oracle_counter(uih, cand, cached):
    D, H, L = 64, 2, 2
    wl = workloads.make_custom(seed=61, dtype="f32", layers=L, d_model=D, heads=H, max_len=64,
                               uih_lengths=uih, cand_lengths=cand, cached_lengths=cached)
    cache = None
    if cached is not None:
        cap = 16
        cache = oracle.OracleCache(np.zeros((L, len(uih), cap, D)), np.zeros((L, len(uih), cap, D)),
                                   np.arange(len(uih)), np.array(cached))
    cnt = oracle.MacCounter()
    oracle.encode(wl.uih, workloads.lengths_to_offsets(uih), wl.cand, workloads.lengths_to_offsets(cand),
                  wl.params, heads=H, max_len=64, mode="f64", cache=cache, counter=cnt)
    st, alg, form = hsa.hstu_flops(hsa.HstuDims(L, D, H, 64, hsa.HSTU_F32), len(uih),
                                   workloads.lengths_to_offsets(uih), workloads.lengths_to_offsets(cand),
                                   cached)
    assert st == OK
    assert alg == cnt.algorithmic_flops()
    ms = cached or [0] * len(uih)
    assert form == sum(2 * L * ((m + n) ** 2 * D // 2 + (m + n) * D * D * 7) for n, m in zip(uih, ms))


def test_flops_near_and_past_the_64_bit_limit():
    """Counts for batches far beyond any max_len: exact while they fit 64 bits (against
    Python's integers, the documented per-user formula), HSTU_ERR_SHAPE once either passes
    2^64 - 1, never a wrapped value."""
    def exact(L, D, users):
        alg = form = 0
        for n, c, m in users:
            pairs = n * m + n * (n + 1) // 2 + c * (m + n + 1)
            alg += L * (14 * (n + c) * D * D + 4 * D * pairs)
            form += 2 * L * ((m + n) ** 2 * D // 2 + (m + n) * D * D * 7)
        return alg, form

    D = 127 * 128                                                  # the widest model the checks allow
    cases = [
        (1, [(2 ** 20, 0, 0)]),                                    # about 2^55
        (16, [(2 ** 20, 3, 2 ** 20)]),                             # about 2^61
        (1024, [(2 ** 20, 3, 2 ** 20)]),                           # about 2^67
        (1, [(2 ** 30, 0, 0)]),                                    # 4 D n^2 / 2 is about 2^75
        (2 ** 31 - 1, [(1, 0, 0)] * 2),                            # about 2^63.8
        (2 ** 31 - 1, [(1, 0, 0)] * 3),                            # the third user passes 2^64
        (2 ** 31 - 1, [(2 ** 31 - 1, 2 ** 31 - 1, 2 ** 31 - 1)]),  # the largest user possible: about 2^111
    ]
    seen = set()
    for L, users in cases:
        uo, co = [0], [0]
        for n, c, _ in users:
            uo.append(uo[-1] + n)
            co.append(co[-1] + c)
        st, alg, form = hsa.hstu_flops(hsa.HstuDims(L, D, 127, 1, hsa.HSTU_BF16), len(users), uo, co,
                                       [m for _, _, m in users])
        want_alg, want_form = exact(L, D, users)
        fits = want_alg < 2 ** 64 and want_form < 2 ** 64
        seen.add(fits)
        if fits:
            assert st == OK and (alg, form) == (want_alg, want_form)
        else:
            assert st == ERR_SHAPE
    assert seen == {True, False}


@pytest.mark.parametrize("name", ["d256_uih1k_c64", "d512_uih2k_c2k", "stream_3000p300_c2k", "long_uih16k_c2k"])
def test_flops_of_workloads_equal_enumeration(name):
    spec = workloads.WORKLOADS[name]
    rng = np.random.default_rng(0)
    B = spec.users
    uih = rng.integers(1, 2000, B)
    cand = np.full(B, spec.cands)
    cached = np.full(B, spec.cached)
    st, alg, _ = hsa.hstu_flops(hsa.HstuDims(spec.layers, spec.d_model, spec.heads, spec.max_len,
                                             hsa.HSTU_BF16), B, workloads.lengths_to_offsets(uih),
                                workloads.lengths_to_offsets(cand), cached)
    want = sum(2 * sum(count_macs(spec.d_model, spec.layers, int(n), int(c), int(m)).values())
               for n, c, m in zip(uih, cand, cached))
    assert st == OK and alg == want


# ------------------------------------------------------------------------------ encode validation

class FakeArgs:
    """Arguments whose device pointers are never dereferenced: every case below must be rejected
    on the host before any HIP call (this container has no GPU)."""

    def __init__(self, L=2, D=256, H=4, max_len=64, uih=(5, 3), cand=(2, 0)):
        self.d = dims(L, D, H, max_len)
        self.B = len(uih)
        self.uo = workloads.lengths_to_offsets(uih)
        self.co = workloads.lengths_to_offsets(cand)
        self.w = [hsa.HstuLayerWeights(0x10000, 0x20000, 0x30000) for _ in range(L)]
        self.ptrs = dict(uih=0x40000, cand=0x50000, uih_out=0x60000, cand_out=0x70000, ws=0x100000)
        st, self.ws_bytes = hsa.hstu_workspace_size(self.d, self.B, self.uo, self.co)
        assert st == OK

    def call(self, kv=None, ws_bytes=None, **over):
        p = dict(self.ptrs, **over)
        return hsa.hstu_encode(self.d, self.B, self.uo, self.co, p["uih"], p["cand"], self.w, kv,
                               p["uih_out"], p["cand_out"], p["ws"],
                               self.ws_bytes if ws_bytes is None else ws_bytes, 0)


def fake_cache(cached, slots=4, capacity=32, slot_of_user=None):
    sl = np.ascontiguousarray(slot_of_user if slot_of_user is not None else np.arange(len(cached)),
                              dtype=np.int32)
    cl = np.ascontiguousarray(cached, dtype=np.int32)
    kv = hsa.HstuKvCache(0x200000, 0x300000, slots, capacity,
                         sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                         cl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    return kv, sl, cl


def test_encode_rejects_before_launch():
    a = FakeArgs()
    assert a.call(ws_bytes=a.ws_bytes - 1) == ERR_WORKSPACE
    assert a.call(ws=0) == ERR_WORKSPACE
    assert a.call(ws=0x100010) == ERR_ALIGN            # workspace must be 256-byte aligned
    assert a.call(uih=0) == ERR_NULL
    assert a.call(cand_out=0) == ERR_NULL
    assert a.call(uih=0x40008) == ERR_ALIGN
    a.w[1] = hsa.HstuLayerWeights(0x10000, 0, 0x30000)
    assert a.call() == ERR_NULL
    a.w[1] = hsa.HstuLayerWeights(0x10000, 0x20004, 0x30000)
    assert a.call() == ERR_ALIGN
    a.w[1] = hsa.HstuLayerWeights(0x10000, 0x20000, 0x30000, 0x38008)   # relative table misaligned
    assert a.call() == ERR_ALIGN


def test_encode_takes_relative_bias_at_any_max_len():
    """The attention streams the relative table through LDS a slice per key block, so a
    bfloat16 model with a relative bias takes any max_len: validation passes the table
    (and here stops at the workspace, before any launch)."""
    a = FakeArgs(max_len=65536)
    a.w = [hsa.HstuLayerWeights(0x10000, 0x20000, 0, 0x38000) for _ in range(2)]
    assert a.call(ws_bytes=a.ws_bytes - 1) == ERR_WORKSPACE


def test_encode_capacity_and_slots_leave_cached_len_unchanged():
    a = FakeArgs(max_len=64, uih=(5, 3), cand=(2, 0))
    # m + n + 1 must fit the position table: 58 + 5 + 1 = 64 fits, 59 does not
    kv, sl, cl = fake_cache([59, 0])
    assert a.call(kv=kv) == ERR_CAPACITY and cl.tolist() == [59, 0]
    kv, sl, cl = fake_cache([20, 30], capacity=32)          # 30 + 3 > capacity 32
    assert a.call(kv=kv) == ERR_CAPACITY and cl.tolist() == [20, 30]
    kv, sl, cl = fake_cache([1, 1], slot_of_user=[2, 2])    # one slot for two users
    assert a.call(kv=kv) == ERR_CAPACITY and cl.tolist() == [1, 1]
    kv, sl, cl = fake_cache([1, 1], slots=2, slot_of_user=[0, 2])
    assert a.call(kv=kv) == ERR_CAPACITY
    kv, sl, cl = fake_cache([-1, 1])
    assert a.call(kv=kv) == ERR_CAPACITY
    kv, sl, cl = fake_cache([0, 0])
    kv.k = 0
    assert a.call(kv=kv) == ERR_NULL
    # without a cache, n + 1 must fit max_len
    b = FakeArgs(max_len=6, uih=(5, 6), cand=(1, 1))
    assert b.call() == ERR_CAPACITY


def fake_paged(cached, pages=8, pages_per_user=2, page_rows=64, table=0x500000):
    cl = np.ascontiguousarray(cached, dtype=np.int32)
    kv = hsa.HstuKvCache(0x200000, 0x300000, 0, 0, None, cl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                         page_rows, pages, pages_per_user, table)
    return kv, cl


def test_encode_paged_cache_validation_leaves_cached_len_unchanged():
    """Paged layout (page_rows 64): each user's m + n rows must fit its pages_per_user pages,
    the page table must be given and 4-byte aligned, page_rows must be 64, and a layer's
    pool must span under 2 GiB. The device page table itself is not read on the host."""
    a = FakeArgs(max_len=200, uih=(5, 3), cand=(2, 0))
    kv, cl = fake_paged([124, 0])                       # 124 + 5 = 129 rows need three pages
    assert a.call(kv=kv) == ERR_CAPACITY and cl.tolist() == [124, 0]
    kv, cl = fake_paged([0, 0], page_rows=32)
    assert a.call(kv=kv) == ERR_CAPACITY
    kv, cl = fake_paged([0, 0], pages=0)
    assert a.call(kv=kv) == ERR_CAPACITY
    kv, cl = fake_paged([0, 0], pages_per_user=0)
    assert a.call(kv=kv) == ERR_CAPACITY
    kv, cl = fake_paged([0, 0], table=0)
    assert a.call(kv=kv) == ERR_NULL
    kv, cl = fake_paged([0, 0], table=0x500002)
    assert a.call(kv=kv) == ERR_ALIGN
    kv, cl = fake_paged([0, 0], pages=1 << 20)          # 2^20 pages x 64 rows x 256 x 2 B = 32 GiB
    assert a.call(kv=kv) == ERR_CAPACITY
    kv, cl = fake_paged([-1, 0])
    assert a.call(kv=kv) == ERR_CAPACITY and cl.tolist() == [-1, 0]


def test_encode_empty_batches_are_ok_without_device_work():
    d = dims()
    assert hsa.hstu_encode(d, 0, None, None, 0, 0, [hsa.HstuLayerWeights(1, 1, 1)] * 2, None,
                           0, 0, 0, 0, 0) == OK
    a = FakeArgs(uih=(0, 0), cand=(0, 0))
    kv, sl, cl = fake_cache([3, 4])
    assert a.call(kv=kv, ws=0, ws_bytes=0) == OK and cl.tolist() == [3, 4]
    a = FakeArgs()
    assert hsa.hstu_encode(a.d, a.B, [0, 5, 4], a.co, 1, 1, a.w, None, 1, 1, 1, 1, 0) == ERR_OFFSETS


# --------------------------------------------------------------------------- hstu_pack_uih

SUM, INTERLEAVE = 0, 1


@pytest.mark.parametrize("args,want", [
    ((None, 4, SUM, 16, 16, 16), ERR_NULL),                           # no dims
    ((dims(D=192, H=3), 4, SUM, 16, 16, 16), ERR_SHAPE),              # dims checked as for encode
    ((dims(), -1, SUM, 16, 16, 16), ERR_SHAPE),                       # negative event count
    ((dims(), 4, 2, 16, 16, 16), ERR_SHAPE),                          # unknown mode
    ((dims(), 0, SUM, None, None, None), OK),                         # nothing to pack: no launch
    ((dims(), 0, INTERLEAVE, None, None, None), OK),
    ((dims(), 4, SUM, None, 16, 16), ERR_NULL),
    ((dims(), 4, INTERLEAVE, 16, None, 16), ERR_NULL),
    ((dims(), 4, SUM, 16, 16, None), ERR_NULL),
    ((dims(), 4, SUM, 24, 16, 16), ERR_ALIGN),
    ((dims(), 4, INTERLEAVE, 16, 16, 8), ERR_ALIGN),
    # bf16, D = 256: 32 chunks per row; 2^26 events interleave to 2^27 rows = 2^32 chunks
    ((dims(), 1 << 26, INTERLEAVE, 16, 16, 16), ERR_SHAPE),
    ((dims(), (1 << 26) - 1, SUM, None, 16, 16), ERR_NULL),           # 2^31 - 32 chunks: size ok
    ((dims(), 1 << 26, SUM, None, 16, 16), ERR_SHAPE),                # 2^31 chunks
    ((dims(), 1 << 25, INTERLEAVE, None, 16, 16), ERR_SHAPE),         # 2^26 rows = 2^31 chunks
])
def test_pack_validation(args, want):
    """Every rejected case returns before anything is enqueued (no GPU here)."""
    d, events, mode, c, a, o = args
    lib = hsa.load_library()
    st = lib.hstu_pack_uih(ctypes.byref(d) if d is not None else None, events, mode, c, a, o, None)
    assert st == want


# --------------------------------------------------------------------------- hstu_transpose_weights

BIG = 1 << 40   # device-looking addresses far apart (never dereferenced: every case is rejected)


@pytest.mark.parametrize("dtype,rows,cols,src,dst,want", [
    (2, 4, 4, BIG, 2 * BIG, ERR_SHAPE),                           # unknown dtype
    (hsa.HSTU_BF16, -1, 4, BIG, 2 * BIG, ERR_SHAPE),
    (hsa.HSTU_BF16, 4, -1, BIG, 2 * BIG, ERR_SHAPE),
    (hsa.HSTU_BF16, 1 << 16, 1 << 15, BIG, 2 * BIG, ERR_SHAPE),  # 2^31 elements
    (hsa.HSTU_BF16, 4, 4, None, 2 * BIG, ERR_NULL),
    (hsa.HSTU_F32, 4, 4, BIG, None, ERR_NULL),
    (hsa.HSTU_BF16, 4, 4, BIG + 1, 2 * BIG, ERR_ALIGN),         # bfloat16 elements are 2-byte aligned
    (hsa.HSTU_F32, 4, 4, BIG, 2 * BIG + 2, ERR_ALIGN),           # float32 elements 4-byte aligned
    (hsa.HSTU_F32, 4, 4, BIG, BIG + 60, ERR_SHAPE),              # the matrices overlap (64 bytes each)
    (hsa.HSTU_BF16, 0, 5, None, None, OK),                       # empty: nothing to do, pointers unused
    (hsa.HSTU_F32, 7, 0, None, None, OK),
])
def test_transpose_weights_validation(dtype, rows, cols, src, dst, want):
    """Every rejected case returns before anything is enqueued (no GPU here)."""
    assert hsa.hstu_transpose_weights(dtype, rows, cols, src, dst, None) == want


# --------------------------------------------------------------------------- hstu_score

def _head(widths, ptr=16):
    arr = (hsa.HstuHeadLayer * max(len(widths), 1))()
    for i, w in enumerate(widths):
        arr[i] = hsa.HstuHeadLayer(ptr, ptr, w)
    return arr


@pytest.mark.parametrize("d,rows,widths,x,prob,want", [
    (None, 4, [1], 16, 16, ERR_NULL),
    (dims(D=192, H=3), 4, [1], 16, 16, ERR_SHAPE),                 # dims checked as for encode
    (dims(D=640, H=5), 4, [1], 16, 16, ERR_SHAPE),                 # input wider than 512
    (dims(), -1, [1], 16, 16, ERR_SHAPE),
    (dims(), 4, [], 16, 16, ERR_SHAPE),                            # no layer
    (dims(), 4, [128] * 8 + [1], 16, 16, ERR_SHAPE),               # more than 8 layers
    (dims(), 4, [100, 1], 16, 16, ERR_SHAPE),                      # hidden width not a multiple of 128
    (dims(), 4, [640, 1], 16, 16, ERR_SHAPE),                      # hidden width above 512
    (dims(), 4, [512, 0], 16, 16, ERR_SHAPE),                      # no outcome
    (dims(), 4, [512, 17], 16, 16, ERR_SHAPE),                     # more than 16 outcomes
    (dims(), 0, [512, 256, 1], None, None, OK),                    # nothing to score: no launch
    (dims(), 4, [512, 256, 1], None, 16, ERR_NULL),
    (dims(), 4, [512, 256, 1], 16, None, ERR_NULL),
    (dims(), 4, [512, 256, 1], 8, 16, ERR_ALIGN),
    (dims(), 4, [512, 256, 1], 16, 4, ERR_ALIGN),
])
def test_score_validation(d, rows, widths, x, prob, want):
    """Every rejected case returns before anything is enqueued (no GPU here)."""
    lib = hsa.load_library()
    head = _head(widths)
    st = lib.hstu_score(ctypes.byref(d) if d is not None else None, rows, x, head, len(widths), prob, None)
    assert st == want


def test_score_validation_layer_pointers():
    lib = hsa.load_library()
    head = _head([512, 1])
    head[1] = hsa.HstuHeadLayer(16, None, 1)
    assert lib.hstu_score(ctypes.byref(dims()), 4, 16, head, 2, 16, None) == ERR_NULL
    head[1] = hsa.HstuHeadLayer(24, 16, 1)
    assert lib.hstu_score(ctypes.byref(dims()), 4, 16, head, 2, 16, None) == ERR_ALIGN
    assert lib.hstu_score(ctypes.byref(dims()), 4, 16, None, 2, 16, None) == ERR_NULL


def test_missing_library_fails_loudly(tmp_path):
    """No fallback: with the shared library absent every entry point raises instead of
    computing anything some other way (run in a child process so this one keeps its
    loaded library)."""
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import hstu_silu_attention_amd as hsa\n"
        "hsa.library_path = lambda: %r\n"
        "try:\n"
        "    hsa.hstu_abi_version()\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "    sys.exit(0)\n"
        "sys.exit(3)\n" % (ROOT, str(tmp_path / "absent" / "libhstu.so")))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "build the HIP library" in r.stdout


def test_static_entry_rejects_batches_beyond_its_scratch():
    """hstu_encode_static (no workspace argument, a fixed device scratch) refuses, before
    touching the GPU, batches whose workspace exceeds its 64 MiB or whose plan exceeds its
    fixed host arrays (1024 users, 16384 attention work items); validation errors come
    first, as in hstu_encode."""
    fake = 1 << 20                      # never dereferenced: the call returns before any launch
    d = dims(L=1, D=512, H=4, max_len=20000)
    w = (hsa.HstuLayerWeights * 1)(hsa.HstuLayerWeights(fake, fake, None, None))

    def call(uo, co, d=d):
        return hsa.hstu_encode_static(d, len(uo) - 1, uo, co, fake, fake, w, None, fake, fake, 0)

    assert call([0, 16000], [0, 2048]) == ERR_TOO_LARGE                   # 18K rows at D = 512
    many = list(range(0, 1026))                                           # 1025 users of one row
    assert call(many, [0] * 1026, d=dims(L=1, D=128, H=2, max_len=20000)) == ERR_TOO_LARGE
    assert call([3, 5], [0, 2]) == ERR_OFFSETS
    assert hsa.hstu_encode_static(d, 0, None, None, None, None, w, None, None, None, 0) == OK
