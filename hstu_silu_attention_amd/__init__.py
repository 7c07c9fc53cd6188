"""Python binding of libhstu.so, the gfx950 jagged HSTU encoder (C ABI in include/hstu.h).

Argument marshalling only: PyTorch supplies device memory and the current stream,
and every step of the encoder runs in the library's HIP kernels. There is no
fallback: if the library is missing or fails to load, every call raises.

Low-level functions carry the C names (``hstu_encode``, ``hstu_pack_uih``,
``hstu_score``, ``hstu_workspace_size``, ``hstu_flops``, ``hstu_abi_version``,
``hstu_status_string``). ``Model``, ``KVCache`` (slot layout), ``PagedKVCache``,
``ScoringHead``, ``encode``, ``encode_static``, ``pack_uih`` and ``score`` wrap them for
torch tensors; ``KvPool`` wraps the host-side page manager (hstu_pool_*).
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = ["HSTU_F32", "HSTU_BF16", "HSTU_WEIGHTS_PREPARED", "HSTU_WEIGHTS_MATH", "ABI_VERSION", "HstuError", "load_library", "library_path",
           "hstu_abi_version", "hstu_status_string", "hstu_workspace_size", "hstu_flops", "hstu_attention_plan",
           "hstu_encode", "hstu_encode_static", "encode_static", "HSTU_ERR_TOO_LARGE", "hstu_pack_uih",
           "hstu_transpose_weights", "transpose_weights", "hstu_timing_enable", "hstu_timing_select",
           "hstu_timing_read", "KERNEL_KINDS", "PACK_MODES", "Model", "KVCache", "ScoringHead", "encode", "pack_uih",
           "score", "hstu_score", "HstuDims", "HstuLayerWeights", "HstuKvCache", "HstuHeadLayer", "KvPool",
           "PagedKVCache", "POOL_STATS", "PAGE_ROWS"]

HSTU_F32, HSTU_BF16 = 0, 1
HSTU_WEIGHTS_PREPARED, HSTU_WEIGHTS_MATH = 0, 1
ABI_VERSION = 9          # the HSTU_ABI_VERSION these structures follow
HSTU_OK = 0
HSTU_ERR_TOO_LARGE = 8
KERNEL_KINDS = ("plan", "uvqk", "attention", "out", "norm", "pack", "score")
PACK_MODES = {"sum": 0, "interleave": 1}
POOL_STATS = ("hits", "rebuild_new", "rebuild_stale", "rebuild_full", "evictions", "pages_in_use", "pages_peak")
PAGE_ROWS = 64


class HstuDims(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("max_len", ctypes.c_int32), ("dtype", ctypes.c_int32), ("weight_layout", ctypes.c_int32)]


class HstuLayerWeights(ctypes.Structure):
    _fields_ = [("w_uvqk", ctypes.c_void_p), ("w_out", ctypes.c_void_p), ("pos_bias", ctypes.c_void_p),
                ("rel_bias", ctypes.c_void_p)]


class HstuKvCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("slots", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("slot_of_user", ctypes.POINTER(ctypes.c_int32)),
                ("cached_len", ctypes.POINTER(ctypes.c_int32)), ("page_rows", ctypes.c_int32),
                ("pages", ctypes.c_int32), ("pages_per_user", ctypes.c_int32), ("page_table", ctypes.c_void_p)]


class HstuHeadLayer(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("out_features", ctypes.c_int32)]


class HstuError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({hstu_status_string(status)})")


def library_path() -> str:
    """The in-tree libhstu.so, or the library named by $HSTU_LIBRARY (e.g. the sanitizer
    build, libhstu_asan.so)."""
    return os.environ.get("HSTU_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhstu.so")


_lib: Optional[ctypes.CDLL] = None


def load_library() -> ctypes.CDLL:
    """Load libhstu.so (built in-tree by ``__graft_entry__.build()``). Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first (__graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    i32p = P(ctypes.c_int32)
    lib.hstu_abi_version.restype = ctypes.c_int32
    lib.hstu_abi_version.argtypes = []
    if lib.hstu_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {lib.hstu_abi_version()}, this binding follows {ABI_VERSION}: "
                           "rebuild the library (__graft_entry__.build())")
    lib.hstu_status_string.restype = ctypes.c_char_p
    lib.hstu_status_string.argtypes = [ctypes.c_int32]
    lib.hstu_workspace_size.restype = ctypes.c_int32
    lib.hstu_workspace_size.argtypes = [P(HstuDims), ctypes.c_int32, i32p, i32p, P(ctypes.c_size_t)]
    lib.hstu_flops.restype = ctypes.c_int32
    lib.hstu_flops.argtypes = [P(HstuDims), ctypes.c_int32, i32p, i32p, i32p, P(ctypes.c_uint64),
                               P(ctypes.c_uint64)]
    lib.hstu_attention_plan.restype = ctypes.c_int32
    lib.hstu_attention_plan.argtypes = [P(HstuDims), ctypes.c_int32, i32p, i32p, i32p, i32p, P(ctypes.c_int64),
                                        ctypes.c_int64]
    lib.hstu_timing_enable.restype = ctypes.c_int32
    lib.hstu_timing_enable.argtypes = [ctypes.c_int32]
    lib.hstu_timing_select.restype = ctypes.c_int32
    lib.hstu_timing_select.argtypes = [ctypes.c_uint32]
    lib.hstu_timing_read.restype = ctypes.c_int32
    lib.hstu_timing_read.argtypes = [P(ctypes.c_double), P(ctypes.c_int64), ctypes.c_int32]
    lib.hstu_encode.restype = ctypes.c_int32
    lib.hstu_encode.argtypes = [P(HstuDims), ctypes.c_int32, i32p, i32p, ctypes.c_void_p, ctypes.c_void_p,
                                P(HstuLayerWeights), P(HstuKvCache), ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.hstu_encode_static.restype = ctypes.c_int32
    lib.hstu_encode_static.argtypes = [P(HstuDims), ctypes.c_int32, i32p, i32p, ctypes.c_void_p, ctypes.c_void_p,
                                       P(HstuLayerWeights), P(HstuKvCache), ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
    i64p = P(ctypes.c_int64)
    lib.hstu_pool_create.restype = ctypes.c_int32
    lib.hstu_pool_create.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, P(ctypes.c_void_p)]
    lib.hstu_pool_destroy.restype = None
    lib.hstu_pool_destroy.argtypes = [ctypes.c_void_p]
    lib.hstu_pool_assign.restype = ctypes.c_int32
    lib.hstu_pool_assign.argtypes = [ctypes.c_void_p, ctypes.c_int32, i64p, i32p, i32p, ctypes.c_int64, ctypes.c_int32,
                                     i32p, i32p, i32p]
    lib.hstu_pool_commit.restype = ctypes.c_int32
    lib.hstu_pool_commit.argtypes = [ctypes.c_void_p, ctypes.c_int32, i64p, i32p, ctypes.c_int64]
    lib.hstu_pool_abort.restype = ctypes.c_int32
    lib.hstu_pool_abort.argtypes = [ctypes.c_void_p, ctypes.c_int32, i64p]
    lib.hstu_pool_stats.restype = ctypes.c_int32
    lib.hstu_pool_stats.argtypes = [ctypes.c_void_p, i64p, ctypes.c_int32]
    lib.hstu_pool_lookup.restype = ctypes.c_int32
    lib.hstu_pool_lookup.argtypes = [ctypes.c_void_p, ctypes.c_int64, i32p, i32p]
    lib.hstu_score.restype = ctypes.c_int32
    lib.hstu_score.argtypes = [P(HstuDims), ctypes.c_int32, ctypes.c_void_p, P(HstuHeadLayer), ctypes.c_int32,
                               ctypes.c_void_p, ctypes.c_void_p]
    lib.hstu_pack_uih.restype = ctypes.c_int32
    lib.hstu_pack_uih.argtypes = [P(HstuDims), ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.hstu_transpose_weights.restype = ctypes.c_int32
    lib.hstu_transpose_weights.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]
    _lib = lib
    return lib


def _i32(a) -> Tuple[np.ndarray, ctypes.POINTER(ctypes.c_int32)]:
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _dims(layers, d_model, heads, max_len, dtype, weight_layout=HSTU_WEIGHTS_PREPARED) -> HstuDims:
    return HstuDims(layers, d_model, heads, max_len, dtype, weight_layout)


def hstu_abi_version() -> int:
    return int(load_library().hstu_abi_version())


def hstu_status_string(status: int) -> str:
    return load_library().hstu_status_string(int(status)).decode()


def hstu_workspace_size(dims: HstuDims, B: int, uih_offsets, cand_offsets) -> Tuple[int, int]:
    """Returns (status, bytes)."""
    _, uo = _i32(uih_offsets)
    _, co = _i32(cand_offsets)
    out = ctypes.c_size_t(0)
    st = load_library().hstu_workspace_size(ctypes.byref(dims), B, uo, co, ctypes.byref(out))
    return int(st), int(out.value)


def hstu_flops(dims: HstuDims, B: int, uih_offsets, cand_offsets, cached_len=None) -> Tuple[int, int, int]:
    """Returns (status, algorithmic_flops, formula_flops)."""
    _, uo = _i32(uih_offsets)
    _, co = _i32(cand_offsets)
    _, cl = _i32(cached_len)
    alg, form = ctypes.c_uint64(0), ctypes.c_uint64(0)
    st = load_library().hstu_flops(ctypes.byref(dims), B, uo, co, cl, ctypes.byref(alg), ctypes.byref(form))
    return int(st), int(alg.value), int(form.value)


def hstu_attention_plan(dims: HstuDims, B: int, uih_offsets, cand_offsets, cached_len=None):
    """Returns (status, codes): the attention's work item of every workgroup, as int64
    (user << 32) | (query block << 8) | (head << 1) | is_candidate, -1 for none."""
    _, uo = _i32(uih_offsets)
    _, co = _i32(cand_offsets)
    _, cl = _i32(cached_len)
    lib = load_library()
    grid = ctypes.c_int32(0)
    st = int(lib.hstu_attention_plan(ctypes.byref(dims), B, uo, co, cl, ctypes.byref(grid), None, 0))
    if st != HSTU_OK:
        return st, None
    codes = np.empty(max(grid.value, 1), dtype=np.int64)
    st = int(lib.hstu_attention_plan(ctypes.byref(dims), B, uo, co, cl, ctypes.byref(grid),
                                     codes.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), codes.shape[0]))
    return st, codes[:grid.value]


def hstu_encode(dims: HstuDims, B: int, uih_offsets, cand_offsets, uih_ptr: int, cand_ptr: int,
                weights: Sequence[HstuLayerWeights], kv: Optional[HstuKvCache], uih_out_ptr: int,
                cand_out_ptr: int, workspace_ptr: int, workspace_bytes: int, stream: int) -> int:
    """Raw call with integer device pointers. Returns the status."""
    _, uo = _i32(uih_offsets)
    _, co = _i32(cand_offsets)
    warr = (HstuLayerWeights * max(len(weights), 1))(*weights)
    return int(load_library().hstu_encode(ctypes.byref(dims), B, uo, co, uih_ptr, cand_ptr, warr,
                                          ctypes.byref(kv) if kv is not None else None,
                                          uih_out_ptr, cand_out_ptr, workspace_ptr, workspace_bytes, stream))


def hstu_encode_static(dims: HstuDims, B: int, uih_offsets, cand_offsets, uih_ptr: int, cand_ptr: int,
                       weights: Sequence[HstuLayerWeights], kv: Optional[HstuKvCache], uih_out_ptr: int,
                       cand_out_ptr: int, stream: int) -> int:
    """Raw call of the entry point that allocates nothing (its workspace is the library's fixed
    device array). Returns the status."""
    _, uo = _i32(uih_offsets)
    _, co = _i32(cand_offsets)
    warr = (HstuLayerWeights * max(len(weights), 1))(*weights)
    return int(load_library().hstu_encode_static(ctypes.byref(dims), B, uo, co, uih_ptr, cand_ptr, warr,
                                                 ctypes.byref(kv) if kv is not None else None,
                                                 uih_out_ptr, cand_out_ptr, stream))


def hstu_pack_uih(dims: HstuDims, events: int, mode: int, context_ptr: int, action_ptr: int,
                  uih_ptr: int, stream: int) -> int:
    """Raw call with integer device pointers. Returns the status."""
    return int(load_library().hstu_pack_uih(ctypes.byref(dims), events, mode, context_ptr, action_ptr,
                                            uih_ptr, stream))


def hstu_transpose_weights(dtype: int, rows: int, cols: int, src_ptr: int, dst_ptr: int, stream: int) -> int:
    """Raw call with integer device pointers. Returns the status."""
    return int(load_library().hstu_transpose_weights(dtype, rows, cols, src_ptr, dst_ptr, stream))


def hstu_score(dims: HstuDims, rows: int, x_ptr: int, head: Sequence[HstuHeadLayer], prob_ptr: int,
               stream: int) -> int:
    """Raw call with integer device pointers. Returns the status."""
    harr = (HstuHeadLayer * max(len(head), 1))(*head)
    return int(load_library().hstu_score(ctypes.byref(dims), rows, x_ptr, harr, len(head), prob_ptr, stream))


def hstu_timing_enable(enable: bool) -> int:
    return int(load_library().hstu_timing_enable(1 if enable else 0))


def hstu_timing_select(kinds=None) -> int:
    """Time only the given kernel kinds (names from KERNEL_KINDS); None: all of them."""
    mask = 0xFFFFFFFF if kinds is None else sum(1 << KERNEL_KINDS.index(k) for k in kinds)
    return int(load_library().hstu_timing_select(mask))


def hstu_timing_read():
    """Returns (status, {kind: (total_ms, launches)}) for the kinds in KERNEL_KINDS."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    st = int(load_library().hstu_timing_read(ms, cnt, n))
    return st, {k: (float(ms[i]), int(cnt[i])) for i, k in enumerate(KERNEL_KINDS)}


# ---------------------------------------------------------------------------- torch helpers

def _torch():
    import torch
    return torch


class Model:
    """Device-resident parameters of an encoder stack in the ABI's layout.

    ``params``: per layer objects with ``w1`` [D,4D], ``w2`` [3D,D], ``pos`` [max_len,3D] or
    None and optionally ``rel`` [heads,max_len] or None (math layout, float32 numpy
    arrays). ``weight_layout`` "prepared" stores the weights transposed as [out][in], the
    layout the GEMMs read; "math" stores W1 and W2 as given, and every encode call then
    transposes them into its workspace (HSTU_WEIGHTS_MATH).
    """

    def __init__(self, params, *, d_model: int, heads: int, max_len: int, dtype: str, device="cuda",
                 weight_layout: str = "prepared"):
        torch = _torch()
        self.d_model, self.heads, self.max_len = d_model, heads, max_len
        self.dtype_code = HSTU_BF16 if dtype == "bf16" else HSTU_F32
        if weight_layout not in ("prepared", "math"):
            raise ValueError(f"weight_layout must be 'prepared' or 'math', not {weight_layout!r}")
        self.weight_layout = HSTU_WEIGHTS_MATH if weight_layout == "math" else HSTU_WEIGHTS_PREPARED
        math = self.weight_layout == HSTU_WEIGHTS_MATH
        self.torch_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.layers: List[Tuple] = []
        dev = lambda a: (None if a is None else
                         torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=self.torch_dtype).contiguous())
        ptr = lambda t: None if t is None else t.data_ptr()
        for p in params:
            self.layers.append((dev(p.w1 if math else p.w1.T), dev(p.w2 if math else p.w2.T), dev(p.pos),
                                dev(getattr(p, "rel", None))))
        self.weights = [HstuLayerWeights(ptr(a), ptr(b), ptr(c), ptr(r)) for a, b, c, r in self.layers]

    def dims(self, layers: Optional[int] = None) -> HstuDims:
        return _dims(len(self.layers) if layers is None else layers, self.d_model, self.heads,
                     self.max_len, self.dtype_code, self.weight_layout)


class KVCache:
    """Caller-owned streaming cache: k, v [layers][slots][capacity][D] on the device plus
    host int32 ``cached_len`` and ``slot_of_user`` (per user of the next call)."""

    def __init__(self, model: Model, slots: int, capacity: int, device="cuda"):
        torch = _torch()
        L, D = len(model.layers), model.d_model
        self.k = torch.zeros((L, slots, capacity, D), dtype=model.torch_dtype, device=device)
        self.v = torch.zeros((L, slots, capacity, D), dtype=model.torch_dtype, device=device)
        self.slots, self.capacity = slots, capacity
        self.slot_of_user = np.arange(slots, dtype=np.int32)
        self.cached_len = np.zeros(slots, dtype=np.int32)

    def struct(self) -> HstuKvCache:
        self.slot_of_user = np.ascontiguousarray(self.slot_of_user, dtype=np.int32)
        self.cached_len = np.ascontiguousarray(self.cached_len, dtype=np.int32)
        return HstuKvCache(self.k.data_ptr(), self.v.data_ptr(), self.slots, self.capacity,
                           self.slot_of_user.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                           self.cached_len.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 0, 0, 0, None)


class PagedKVCache:
    """Caller-owned paged cache: k, v [layers][pages][64][D] on the device, the device page
    table [max_users][pages_per_user] int32 (row b: user b of the next call) and host int32
    ``cached_len`` per user of the next call. ``set_table`` queues a copy of host rows into
    the device table on the current stream (ordered after the kernels queued before it)."""

    def __init__(self, model: Model, pages: int, pages_per_user: int, max_users: int, device="cuda"):
        torch = _torch()
        L, D = len(model.layers), model.d_model
        self.k = torch.zeros((L, pages, PAGE_ROWS, D), dtype=model.torch_dtype, device=device)
        self.v = torch.zeros((L, pages, PAGE_ROWS, D), dtype=model.torch_dtype, device=device)
        self.pages, self.pages_per_user, self.max_users = pages, pages_per_user, max_users
        self.table = torch.full((max_users, pages_per_user), -1, dtype=torch.int32, device=device)
        self.cached_len = np.zeros(max_users, dtype=np.int32)

    def set_table(self, rows) -> None:
        """Rows 0..B-1 of the device page table from a host int array [B][pages_per_user]."""
        torch = _torch()
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        if rows.ndim != 2 or rows.shape[1] != self.pages_per_user or rows.shape[0] > self.max_users:
            raise ValueError("page table rows must be [B <= max_users][pages_per_user]")
        # staged in pinned memory: the copy is queued on the stream without waiting for the
        # host, after the kernels queued before it (torch keeps the staging block until then)
        self.table[:rows.shape[0]].copy_(torch.from_numpy(rows).pin_memory(), non_blocking=True)

    def struct(self) -> HstuKvCache:
        self.cached_len = np.ascontiguousarray(self.cached_len, dtype=np.int32)
        return HstuKvCache(self.k.data_ptr(), self.v.data_ptr(), 0, 0, None,
                           self.cached_len.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), PAGE_ROWS,
                           self.pages, self.pages_per_user, self.table.data_ptr())


def workspace_bytes(model: Model, uih_offsets, cand_offsets) -> int:
    B = len(uih_offsets) - 1
    st, nbytes = hstu_workspace_size(model.dims(), B, uih_offsets, cand_offsets)
    if st != HSTU_OK:
        raise HstuError(st, "hstu_workspace_size")
    return nbytes


def encode(model: Model, uih, uih_offsets, cand, cand_offsets, *, cache: Optional[KVCache] = None,
           out: Optional[Tuple] = None, workspace=None, stream=None):
    """Run hstu_encode on the current (or given) stream; returns (uih_out, cand_out).

    uih/cand: device tensors [rows, D] in the model's dtype; offsets: host int sequences.
    The cache's ``cached_len`` advances on success.
    """
    torch = _torch()
    B = len(uih_offsets) - 1
    if out is None:
        out = (torch.empty_like(uih), torch.empty_like(cand))
    nbytes = workspace_bytes(model, uih_offsets, cand_offsets)
    own_workspace = workspace is None or workspace.numel() < nbytes
    if own_workspace:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=uih.device)
    if stream is None:
        stream = torch.cuda.current_stream(uih.device).cuda_stream
    elif own_workspace and stream != torch.cuda.current_stream(uih.device).cuda_stream:
        # the workspace was allocated on the current stream but is used on `stream`: keep
        # the caching allocator from handing it out again before that stream's work ends
        workspace.record_stream(torch.cuda.ExternalStream(stream, device=uih.device))
    kv = cache.struct() if cache is not None else None
    st = hstu_encode(model.dims(), B, uih_offsets, cand_offsets, uih.data_ptr(), cand.data_ptr(),
                     model.weights, kv, out[0].data_ptr(), out[1].data_ptr(), workspace.data_ptr(),
                     workspace.numel(), stream)
    if st != HSTU_OK:
        raise HstuError(st, "hstu_encode")
    return out


def encode_static(model: Model, uih, uih_offsets, cand, cand_offsets, *, cache: Optional[KVCache] = None,
                  out: Optional[Tuple] = None, stream=None):
    """Run hstu_encode_static (no workspace: the library's fixed device scratch, for callers that
    cannot allocate) on the current (or given) stream; returns (uih_out, cand_out). Outputs are
    allocated here unless ``out`` is given. Calls that overlap on one GPU race (one scratch)."""
    torch = _torch()
    B = len(uih_offsets) - 1
    if out is None:
        out = (torch.empty_like(uih), torch.empty_like(cand))
    if stream is None:
        stream = torch.cuda.current_stream(uih.device).cuda_stream
    kv = cache.struct() if cache is not None else None
    st = hstu_encode_static(model.dims(), B, uih_offsets, cand_offsets, uih.data_ptr(), cand.data_ptr(),
                            model.weights, kv, out[0].data_ptr(), out[1].data_ptr(), stream)
    if st != HSTU_OK:
        raise HstuError(st, "hstu_encode_static")
    return out


def transpose_weights(w, *, out=None, stream=None):
    """Run hstu_transpose_weights on the current (or given) stream: a device matrix [rows][cols]
    (bfloat16 or float32) in the layout the method writes it (W1 [D][4D], W2 [3D][D]) to the
    layout hstu_encode reads (w_uvqk [4D][D], w_out [D][3D]). Returns out [cols][rows]."""
    torch = _torch()
    dtypes = {torch.bfloat16: HSTU_BF16, torch.float32: HSTU_F32}
    if w.dim() != 2 or w.dtype not in dtypes:
        raise ValueError("a 2-D bfloat16 or float32 device matrix")
    w = w.contiguous()
    rows, cols = int(w.shape[0]), int(w.shape[1])
    if out is None:
        out = torch.empty((cols, rows), dtype=w.dtype, device=w.device)
    if stream is None:
        stream = torch.cuda.current_stream(w.device).cuda_stream
    ptr = lambda t: t.data_ptr() if t.numel() else None
    st = hstu_transpose_weights(dtypes[w.dtype], rows, cols, ptr(w), ptr(out), stream)
    if st != HSTU_OK:
        raise HstuError(st, "hstu_transpose_weights")
    return out


def pack_uih(model: Model, context, action, event_offsets, mode: str, *, out=None, stream=None):
    """Run hstu_pack_uih on the current (or given) stream.

    context/action: device tensors [E, D] in the model's dtype, every user's events in the
    order of ``event_offsets`` (host [B+1]). Returns (tokens, token offsets): tokens is a
    device tensor [E, D] ("sum") or [2E, D] ("interleave"), and the token offsets (host
    int32 [B+1]) are the event offsets, doubled for "interleave".
    """
    torch = _torch()
    if mode not in PACK_MODES:
        raise ValueError(mode)
    E = int(context.shape[0])
    f = 2 if mode == "interleave" else 1
    if out is None:
        out = torch.empty((f * E, model.d_model), dtype=context.dtype, device=context.device)
    if stream is None:
        stream = torch.cuda.current_stream(context.device).cuda_stream
    ptr = lambda t: t.data_ptr() if t.numel() else None
    st = hstu_pack_uih(model.dims(), E, PACK_MODES[mode], ptr(context), ptr(action), ptr(out), stream)
    if st != HSTU_OK:
        raise HstuError(st, "hstu_pack_uih")
    offsets = np.asarray(event_offsets, dtype=np.int64) * f
    return out, offsets.astype(np.int32)


class ScoringHead:
    """Device-resident candidate scoring head: per layer (weight [out, in], bias [out]) as
    float32 numpy arrays, stored in the model's dtype."""

    def __init__(self, layers, *, dtype: str, device="cuda"):
        torch = _torch()
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device=device, dtype=tdt)
        self.tensors = [(dev(w), dev(b)) for w, b in layers]
        self.layers = [HstuHeadLayer(w.data_ptr(), b.data_ptr(), int(w.shape[0])) for w, b in self.tensors]
        self.outcomes = int(self.tensors[-1][0].shape[0]) if self.tensors else 0


def score(model: Model, head: ScoringHead, x, *, out=None, stream=None):
    """Run hstu_score on candidate rows x (device [rows, D] in the model's dtype) on the current
    (or given) stream; returns the float32 probabilities [rows, outcomes]."""
    torch = _torch()
    rows = int(x.shape[0])
    if out is None:
        out = torch.empty((rows, head.outcomes), dtype=torch.float32, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    ptr = lambda t: t.data_ptr() if t.numel() else None
    st = hstu_score(model.dims(), rows, ptr(x), head.layers, ptr(out), stream)
    if st != HSTU_OK:
        raise HstuError(st, "hstu_score")
    return out


class KvPool:
    """The library's host-side page manager of a paged cache (hstu_pool_*): per request whether
    a user's cached rows are extended or its history is sent again, and which pages hold the
    user's rows."""

    def __init__(self, pages: int, max_rows: int, ttl: int):
        self._lib = load_library()
        self._h = ctypes.c_void_p()
        st = int(self._lib.hstu_pool_create(pages, max_rows, ttl, ctypes.byref(self._h)))
        if st != HSTU_OK:
            raise HstuError(st, "hstu_pool_create")
        self.pages, self.max_rows, self.ttl = pages, max_rows, ttl

    def __del__(self):
        if getattr(self, "_h", None) and self._h.value:
            self._lib.hstu_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    @staticmethod
    def _i64(a):
        arr = np.ascontiguousarray(np.asarray(a, dtype=np.int64))
        return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))

    def assign_raw(self, users, new_events, window, now: int, pages_per_user: int):
        """Returns (status, page_table [B][pages_per_user], cached_len, rebuild) as int32 arrays."""
        B = len(users)
        ua, up = self._i64(users)
        na, np_ = _i32(new_events)
        wa, wp = _i32(window)
        table = np.full((B, max(pages_per_user, 1)), -7, dtype=np.int32)
        outs = [np.full(B, -7, dtype=np.int32) for _ in range(2)]
        ptr = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        st = int(self._lib.hstu_pool_assign(self._h, B, up if B else None, np_ if B else None, wp if B else None,
                                            int(now), int(pages_per_user), ptr(table), ptr(outs[0]),
                                            ptr(outs[1])))
        return (st, table, *outs)

    def assign(self, users, new_events, window, now: int, pages_per_user: int):
        st, table, cached, rebuild = self.assign_raw(users, new_events, window, now, pages_per_user)
        if st != HSTU_OK:
            raise HstuError(st, "hstu_pool_assign")
        return table, cached, rebuild

    def commit_raw(self, users, total_len, now: int) -> int:
        ua, up = self._i64(users)
        ta, tp = _i32(total_len)
        return int(self._lib.hstu_pool_commit(self._h, len(users), up, tp, int(now)))

    def commit(self, users, total_len, now: int):
        st = self.commit_raw(users, total_len, now)
        if st != HSTU_OK:
            raise HstuError(st, "hstu_pool_commit")

    def abort(self, users):
        ua, up = self._i64(users)
        st = int(self._lib.hstu_pool_abort(self._h, len(users), up))
        if st != HSTU_OK:
            raise HstuError(st, "hstu_pool_abort")

    def stats(self) -> dict:
        out = (ctypes.c_int64 * len(POOL_STATS))()
        st = int(self._lib.hstu_pool_stats(self._h, out, len(POOL_STATS)))
        if st != HSTU_OK:
            raise HstuError(st, "hstu_pool_stats")
        return {k: int(out[i]) for i, k in enumerate(POOL_STATS)}

    def lookup(self, user: int):
        """(committed rows, pages held) of a user; (0, 0) if absent."""
        n, pages = ctypes.c_int32(0), ctypes.c_int32(0)
        st = int(self._lib.hstu_pool_lookup(self._h, int(user), ctypes.byref(n), ctypes.byref(pages)))
        if st != HSTU_OK:
            raise HstuError(st, "hstu_pool_lookup")
        return int(n.value), int(pages.value)
