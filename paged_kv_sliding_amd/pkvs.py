"""ctypes binding of libpkvs (include/pkvs.h): argument marshalling only.

Every function below has the name of the C entry point it calls and does
nothing but convert arguments (torch tensors -> device pointers, host int32
arrays, the current HIP stream) and turn a negative status into ``PkvsError``.
All attention arithmetic runs in the library's HIP kernels; there is no
fallback: importing this module raises when ``libpkvs.so`` has not been built.

``BatchAttention`` is a small convenience holder (plan handle + workspaces
allocated with torch) for callers that want the FlashInfer-style
plan()/run() object.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKVS_LIBRARY names another build of the same C ABI (the tests load a
# sanitizer-instrumented host-only build this way); default: the in-tree one
LIB_PATH = os.environ.get("PKVS_LIBRARY") or os.path.join(_HERE, "libpkvs.so")

PKVS_OK = 0
PKVS_ERR_INVALID_ARG = -1
PKVS_ERR_UNSUPPORTED = -2
PKVS_ERR_WORKSPACE = -3
PKVS_ERR_CAPACITY = -4
PKVS_ERR_PLAN_MISMATCH = -5
PKVS_ERR_HIP = -6
PKVS_ERR_NOT_PLANNED = -7

PKVS_BF16 = 0
PKVS_FP32 = 1
PKVS_FP16 = 2
PKVS_KV_SAME = 0
PKVS_KV_FP8_E4M3 = 1
PKVS_KV_FP8_E5M2 = 2
_KV_FORMATS = {None: PKVS_KV_SAME, torch.float8_e4m3fn: PKVS_KV_FP8_E4M3,
               torch.float8_e5m2: PKVS_KV_FP8_E5M2}
PKVS_PREFILL = 0
PKVS_DECODE = 1
PKVS_CASCADE = 2

_DTYPES = {torch.bfloat16: PKVS_BF16, torch.float32: PKVS_FP32, torch.float16: PKVS_FP16}
_TORCH_DTYPES = {v: k for k, v in _DTYPES.items()}

# Every symbol include/pkvs.h declares.
EXPORTED = [
    "pkvs_plan_create", "pkvs_workspace_size", "pkvs_prefill_plan", "pkvs_prefill_run",
    "pkvs_decode_plan", "pkvs_decode_run", "pkvs_cascade_plan", "pkvs_cascade_run",
    "pkvs_merge_state", "pkvs_append_kv", "pkvs_build_kv_indices", "pkvs_plan_get_info",
    "pkvs_plan_copy_items", "pkvs_plan_destroy", "pkvs_strerror", "pkvs_last_error",
    "pkvs_workspace_bytes", "pkvs_last_error_message", "pkvs_decode_noalloc",
]

# bytes of the library's per-device scratch array (PKVS_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


class pkvs_desc(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("num_qo_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("window_left", ctypes.c_int32), ("fixed_split_size", ctypes.c_int32),
        ("disable_split_kv", ctypes.c_int32), ("batch_capacity", ctypes.c_int32),
        ("prefill_variant", ctypes.c_int32), ("qo_capacity", ctypes.c_int64),
        ("kv_capacity", ctypes.c_int64), ("logits_soft_cap", ctypes.c_float),
        ("kv_format", ctypes.c_int32), ("decode_waves", ctypes.c_int32),
    ]


class pkvs_plan_info(ctypes.Structure):
    _fields_ = [
        ("num_items", ctypes.c_int64), ("num_merges", ctypes.c_int64),
        ("float_ws_bytes", ctypes.c_int64), ("int_ws_bytes", ctypes.c_int64),
        ("grid_blocks", ctypes.c_int32), ("block_threads", ctypes.c_int32),
        ("split_size", ctypes.c_int32), ("item_words", ctypes.c_int32),
        ("query_tile", ctypes.c_int32), ("num_cus", ctypes.c_int32),
        ("prefill_variant", ctypes.c_int32), ("decode_waves", ctypes.c_int32),
        ("cascade_passes", ctypes.c_int32), ("key_chunks", ctypes.c_int32),
    ]


class PkvsError(RuntimeError):
    def __init__(self, code: int, func: str, detail: str):
        self.code = code
        super().__init__(f"{func}: {strerror(code)} ({code}): {detail}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libpkvs.so not built at {LIB_PATH}; run "
                          "`python -m paged_kv_sliding_amd.build` (there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    sz = ctypes.c_size_t
    sig = {
        "pkvs_plan_create": (ctypes.c_int, [ctypes.POINTER(P), ctypes.POINTER(pkvs_desc)]),
        "pkvs_workspace_size": (ctypes.c_int, [P, ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "pkvs_prefill_plan": (ctypes.c_int, [P, P, P, P, i32, P, sz, P, sz, P]),
        "pkvs_prefill_run": (ctypes.c_int, [P, P, P, P, i64, P, P, P, f32, i32, i32, f32, f32,
                                            P]),
        "pkvs_decode_plan": (ctypes.c_int, [P, P, P, i32, P, sz, P, sz, P]),
        "pkvs_decode_run": (ctypes.c_int, [P, P, P, P, i64, P, P, P, f32, i32, f32, f32, P]),
        "pkvs_cascade_plan": (ctypes.c_int, [P, P, P, P, i32, P, sz, P, sz, P]),
        "pkvs_cascade_run": (ctypes.c_int, [P, P, P, P, P, P, i64, P, P, P, f32, i32, f32, f32,
                                            P]),
        "pkvs_merge_state": (ctypes.c_int, [P, P, P, P, P, P, i64, i32, i32, i32, P]),
        "pkvs_append_kv": (ctypes.c_int, [P, P, P, i64, P, P, i64, i32, i32, i32, i32, f32, f32,
                                          P, P]),
        "pkvs_build_kv_indices": (ctypes.c_int, [P, i64, i64, P, P, P, i32, P, P, i64, P, P]),
        "pkvs_plan_get_info": (ctypes.c_int, [P, ctypes.POINTER(pkvs_plan_info)]),
        "pkvs_plan_copy_items": (ctypes.c_int, [P, P, i64, ctypes.POINTER(i64)]),
        "pkvs_plan_destroy": (None, [P]),
        "pkvs_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "pkvs_last_error": (ctypes.c_char_p, []),
        "pkvs_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(pkvs_desc), i32, i64,
                                                ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "pkvs_last_error_message": (ctypes.c_char_p, []),
        "pkvs_decode_noalloc": (ctypes.c_int, [P, P, P, i32, P, P, P, i64, P, P, P, f32, i32,
                                               f32, f32, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def strerror(code: int) -> str:
    return _lib.pkvs_strerror(code).decode()


def last_error() -> str:
    return _lib.pkvs_last_error().decode()


def _check(rc: int, func: str) -> None:
    if rc != PKVS_OK:
        raise PkvsError(rc, func, last_error())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("pkvs: tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _host_i32(t) -> Tuple[object, torch.Tensor]:
    t = torch.as_tensor(t, dtype=torch.int32).cpu().contiguous()
    return ctypes.c_void_p(t.data_ptr()), t


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("pkvs: run() tensors must live on the GPU")


def make_desc(kind: int, *, num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
              dtype: torch.dtype, window_left: int, causal: bool = True,
              fixed_split_size: int = -1, disable_split_kv: bool = False,
              batch_capacity: int, qo_capacity: int = 0, kv_capacity: int,
              prefill_variant: int = 0, logits_soft_cap: float = 0.0,
              kv_dtype: Optional[torch.dtype] = None, decode_waves: int = 0) -> pkvs_desc:
    """``kv_dtype``: None (caches in ``dtype``) or torch.float8_e4m3fn /
    torch.float8_e5m2.  ``decode_waves``: 0 (planner's choice), 1 or 4."""
    return pkvs_desc(kind, num_qo_heads, num_kv_heads, head_dim, page_size, _DTYPES[dtype],
                     int(bool(causal)), window_left, fixed_split_size, int(bool(disable_split_kv)),
                     batch_capacity, prefill_variant, qo_capacity, kv_capacity,
                     float(logits_soft_cap), _KV_FORMATS[kv_dtype], decode_waves)


def pkvs_plan_create(desc: pkvs_desc) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(_lib.pkvs_plan_create(ctypes.byref(h), ctypes.byref(desc)), "pkvs_plan_create")
    return h


def pkvs_workspace_size(plan) -> Tuple[int, int]:
    f, i = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.pkvs_workspace_size(plan, ctypes.byref(f), ctypes.byref(i)),
           "pkvs_workspace_size")
    return f.value, i.value


def pkvs_workspace_bytes(desc: pkvs_desc, is_decode: bool, max_kv_len: int = 0) -> Tuple[int, int]:
    f, i = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.pkvs_workspace_bytes(ctypes.byref(desc), int(bool(is_decode)), int(max_kv_len),
                                     ctypes.byref(f), ctypes.byref(i)), "pkvs_workspace_bytes")
    return f.value, i.value


def pkvs_last_error_message() -> str:
    return _lib.pkvs_last_error_message().decode()


def pkvs_prefill_plan(plan, qo_indptr_h, kv_indptr_h, kv_last_page_len_h, batch_size: int,
                      float_ws: Optional[torch.Tensor], int_ws: Optional[torch.Tensor],
                      stream=None) -> None:
    qp, _q = _host_i32(qo_indptr_h)
    kp, _k = _host_i32(kv_indptr_h)
    lp, _l = _host_i32(kv_last_page_len_h)
    fb = float_ws.numel() * float_ws.element_size() if float_ws is not None else 0
    ib = int_ws.numel() * int_ws.element_size() if int_ws is not None else 0
    st = _stream(stream) if int_ws is not None else None
    _check(_lib.pkvs_prefill_plan(plan, qp, kp, lp, batch_size, _ptr(float_ws), fb, _ptr(int_ws),
                                  ib, st), "pkvs_prefill_plan")


def pkvs_decode_plan(plan, kv_indptr_h, kv_last_page_len_h, batch_size: int,
                     float_ws: Optional[torch.Tensor], int_ws: Optional[torch.Tensor],
                     stream=None) -> None:
    kp, _k = _host_i32(kv_indptr_h)
    lp, _l = _host_i32(kv_last_page_len_h)
    fb = float_ws.numel() * float_ws.element_size() if float_ws is not None else 0
    ib = int_ws.numel() * int_ws.element_size() if int_ws is not None else 0
    st = _stream(stream) if int_ws is not None else None
    _check(_lib.pkvs_decode_plan(plan, kp, lp, batch_size, _ptr(float_ws), fb, _ptr(int_ws), ib,
                                 st), "pkvs_decode_plan")


def pkvs_cascade_plan(plan, qo_indptr_h, kv_indptr_h, kv_last_page_len_h, batch_size: int,
                      float_ws: Optional[torch.Tensor], int_ws: Optional[torch.Tensor],
                      stream=None) -> None:
    qp, _q = _host_i32(qo_indptr_h)
    kp, _k = _host_i32(kv_indptr_h)
    lp, _l = _host_i32(kv_last_page_len_h)
    fb = float_ws.numel() * float_ws.element_size() if float_ws is not None else 0
    ib = int_ws.numel() * int_ws.element_size() if int_ws is not None else 0
    st = _stream(stream) if int_ws is not None else None
    _check(_lib.pkvs_cascade_plan(plan, qp, kp, lp, batch_size, _ptr(float_ws), fb, _ptr(int_ws),
                                  ib, st), "pkvs_cascade_plan")


def pkvs_cascade_run(plan, q, k_extend, v_extend, k_cache, v_cache, kv_indices, o, lse,
                     sm_scale: float, window_left: int, k_scale: float = 1.0,
                     v_scale: float = 1.0, stream=None) -> None:
    _need_device(q, k_extend, v_extend, k_cache, v_cache, kv_indices, o, lse)
    _check(_lib.pkvs_cascade_run(plan, _ptr(q), _ptr(k_extend), _ptr(v_extend), _ptr(k_cache),
                                 _ptr(v_cache), k_cache.shape[0], _ptr(kv_indices), _ptr(o),
                                 _ptr(lse), float(sm_scale), window_left, float(k_scale),
                                 float(v_scale), _stream(stream)), "pkvs_cascade_run")


def pkvs_prefill_run(plan, q, k_cache, v_cache, kv_indices, o, lse, sm_scale: float,
                     window_left: int, causal: bool = True, k_scale: float = 1.0,
                     v_scale: float = 1.0, stream=None) -> None:
    _need_device(q, k_cache, v_cache, kv_indices, o, lse)
    _check(_lib.pkvs_prefill_run(plan, _ptr(q), _ptr(k_cache), _ptr(v_cache), k_cache.shape[0],
                                 _ptr(kv_indices), _ptr(o), _ptr(lse), float(sm_scale),
                                 window_left, int(bool(causal)), float(k_scale), float(v_scale),
                                 _stream(stream)), "pkvs_prefill_run")


def pkvs_decode_run(plan, q, k_cache, v_cache, kv_indices, o, lse, sm_scale: float,
                    window_left: int, k_scale: float = 1.0, v_scale: float = 1.0,
                    stream=None) -> None:
    _need_device(q, k_cache, v_cache, kv_indices, o, lse)
    _check(_lib.pkvs_decode_run(plan, _ptr(q), _ptr(k_cache), _ptr(v_cache), k_cache.shape[0],
                                _ptr(kv_indices), _ptr(o), _ptr(lse), float(sm_scale),
                                window_left, float(k_scale), float(v_scale), _stream(stream)),
           "pkvs_decode_run")


def pkvs_decode_noalloc(plan, kv_indptr_h, kv_last_page_len_h, batch_size: int, q, k_cache,
                        v_cache, kv_indices, o, lse, sm_scale: float, window_left: int,
                        k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    kp, _k = _host_i32(kv_indptr_h)
    lp, _l = _host_i32(kv_last_page_len_h)
    _need_device(q, k_cache, v_cache, kv_indices, o, lse)
    _check(_lib.pkvs_decode_noalloc(plan, kp, lp, batch_size, _ptr(q), _ptr(k_cache),
                                    _ptr(v_cache), k_cache.shape[0], _ptr(kv_indices), _ptr(o),
                                    _ptr(lse), float(sm_scale), window_left, float(k_scale),
                                    float(v_scale), _stream(stream)), "pkvs_decode_noalloc")


def pkvs_merge_state(v_a, s_a, v_b, s_b, v_out=None, s_out=None, stream=None):
    """(v, s) = merge of two partials; allocates the outputs when not given."""
    _need_device(v_a, s_a, v_b, s_b)
    n, h, d = v_a.shape
    if v_out is None:
        v_out = torch.empty_like(v_a)
    if s_out is None:
        s_out = torch.empty_like(s_a)
    _check(_lib.pkvs_merge_state(_ptr(v_a), _ptr(s_a), _ptr(v_b), _ptr(s_b), _ptr(v_out),
                                 _ptr(s_out), n, h, d, _DTYPES[v_a.dtype], _stream(stream)),
           "pkvs_merge_state")
    return v_out, s_out


def pkvs_append_kv(k_new, v_new, loc, k_cache, v_cache, status=None, stream=None,
                   k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """k_cache.view(-1, H_kv, D)[loc[i]] = k_new[i] (same for v) on the GPU;
    an 8-bit cache (torch.float8_e4m3fn / e5m2) receives k_new / k_scale and
    v_new / v_scale rounded to its type.  ``loc`` int64 device slots;
    ``status`` optional int32 device counter."""
    _need_device(k_new, v_new, loc, k_cache, v_cache, status)
    n, h, d = k_new.shape
    if v_new.shape != k_new.shape or k_cache.shape != v_cache.shape:
        raise ValueError("pkvs_append_kv: k/v shapes differ")
    kv_format = _KV_FORMATS.get(k_cache.dtype, PKVS_KV_SAME)
    if v_new.dtype != k_new.dtype or v_cache.dtype != k_cache.dtype or (
            kv_format == PKVS_KV_SAME and k_cache.dtype != k_new.dtype):
        raise ValueError("pkvs_append_kv: one dtype for new rows, and the caches in it or 8-bit")
    if tuple(k_cache.shape[-2:]) != (h, d):
        raise ValueError("pkvs_append_kv: cache rows must be [.., num_kv_heads, head_dim]")
    if loc.dtype != torch.int64 or loc.numel() < n:
        raise ValueError("pkvs_append_kv: loc must be int64 with one slot per row")
    num_slots = k_cache.numel() // (h * d)
    _check(_lib.pkvs_append_kv(_ptr(k_new), _ptr(v_new), _ptr(loc), n, _ptr(k_cache),
                               _ptr(v_cache), num_slots, h, d, _DTYPES[k_new.dtype], kv_format,
                               float(k_scale), float(v_scale), _ptr(status), _stream(stream)),
           "pkvs_append_kv")


def pkvs_build_kv_indices(page_map, slot, length, start=None, kv_indptr=None, kv_indices=None,
                          capacity: Optional[int] = None, status=None, stream=None):
    """Device page table from a request-to-page map (all int32 device
    tensors); allocates kv_indptr / kv_indices when not given."""
    _need_device(page_map, slot, length, start, kv_indptr, kv_indices, status)
    for t in (page_map, slot, length, start):
        if t is not None and t.dtype != torch.int32:
            raise ValueError("pkvs_build_kv_indices: int32 arrays")
    if page_map.dim() != 2:
        raise ValueError("pkvs_build_kv_indices: the map is [rows, cols]")
    B = slot.numel()
    if kv_indptr is None:
        kv_indptr = torch.empty(B + 1, dtype=torch.int32, device=slot.device)
    if kv_indices is None:
        kv_indices = torch.empty(max(capacity or 0, 1), dtype=torch.int32, device=slot.device)
    if capacity is None:
        capacity = kv_indices.numel()
    if capacity > kv_indices.numel() or kv_indptr.numel() < B + 1:
        raise ValueError("pkvs_build_kv_indices: output arrays too small")
    _check(_lib.pkvs_build_kv_indices(_ptr(page_map), page_map.shape[0], page_map.shape[1],
                                      _ptr(slot), _ptr(start), _ptr(length), B, _ptr(kv_indptr),
                                      _ptr(kv_indices), capacity, _ptr(status), _stream(stream)),
           "pkvs_build_kv_indices")
    return kv_indptr, kv_indices


def pkvs_plan_get_info(plan) -> pkvs_plan_info:
    info = pkvs_plan_info()
    _check(_lib.pkvs_plan_get_info(plan, ctypes.byref(info)), "pkvs_plan_get_info")
    return info


def pkvs_plan_copy_items(plan) -> torch.Tensor:
    info = pkvs_plan_get_info(plan)
    n = ctypes.c_int64()
    out = torch.zeros(max(info.num_items, 1) * info.item_words, dtype=torch.int32)
    _check(_lib.pkvs_plan_copy_items(plan, ctypes.c_void_p(out.data_ptr()), info.num_items,
                                     ctypes.byref(n)), "pkvs_plan_copy_items")
    return out[: n.value * info.item_words].view(n.value, info.item_words)


def pkvs_plan_destroy(plan) -> None:
    _lib.pkvs_plan_destroy(plan)


class BatchAttention:
    """Plan handle plus caller-owned workspaces (torch device tensors).

    ``kind`` is PKVS_PREFILL or PKVS_DECODE; the remaining keywords are the
    fields of ``pkvs_desc``.  ``plan()`` takes host CSR arrays, ``run()`` the
    device tensors, on torch's current stream.
    """

    def __init__(self, kind: int, device="cuda", **desc_kw):
        self.kind = kind
        self.desc = make_desc(kind, **desc_kw)
        self.handle = pkvs_plan_create(self.desc)
        fb, ib = pkvs_workspace_size(self.handle)
        self.float_ws = torch.empty(max(fb, 4), dtype=torch.uint8, device=device)
        self.int_ws = torch.empty(ib, dtype=torch.uint8, device=device)

    def plan(self, *, qo_indptr=None, kv_indptr, kv_last_page_len, stream=None):
        batch = len(kv_last_page_len)
        kv_indptr = torch.as_tensor(kv_indptr, dtype=torch.int32).cpu()
        self._nnz_pages = int(kv_indptr[-1])
        self._nnz_qo = int(torch.as_tensor(qo_indptr)[-1]) if self.kind == PKVS_PREFILL else batch
        if self.kind == PKVS_PREFILL:
            pkvs_prefill_plan(self.handle, qo_indptr, kv_indptr, kv_last_page_len, batch,
                              self.float_ws, self.int_ws, stream)
        else:
            pkvs_decode_plan(self.handle, kv_indptr, kv_last_page_len, batch, self.float_ws,
                             self.int_ws, stream)

    def _check_shapes(self, q, k_cache, v_cache, kv_indices, out, lse):
        d = self.desc
        dt = _TORCH_DTYPES[d.dtype]
        # rows past the planned batch (capacity-sized buffers, e.g. under a
        # captured graph) are neither read nor written
        exp_q = (max(self._nnz_qo, q.shape[0] if q.dim() == 3 else 0), d.num_qo_heads, d.head_dim)
        if tuple(q.shape) != exp_q or q.dtype != dt:
            raise ValueError(f"q must be {dt} [>= {self._nnz_qo}, {d.num_qo_heads}, "
                             f"{d.head_dim}], got {q.dtype} {tuple(q.shape)}")
        if out.shape != q.shape or out.dtype != dt:
            raise ValueError("out must match q")
        kv_shape = (d.page_size, d.num_kv_heads, d.head_dim)
        kv_dt = {v: k for k, v in _KV_FORMATS.items()}[d.kv_format] or dt
        for c in (k_cache, v_cache):
            if c.dim() != 4 or tuple(c.shape[1:]) != kv_shape or c.dtype != kv_dt:
                raise ValueError(f"caches must be {kv_dt} [num_pages, {kv_shape}]")
        if k_cache.shape[0] != v_cache.shape[0]:
            raise ValueError("k_cache and v_cache page counts differ")
        if kv_indices.dtype != torch.int32 or kv_indices.numel() < self._nnz_pages:
            raise ValueError(f"kv_indices must be int32 with >= {self._nnz_pages} entries")
        if lse is not None and (tuple(lse.shape) != exp_q[:2] or lse.dtype != torch.float32):
            raise ValueError(f"lse must be float32 {exp_q[:2]}")

    def run(self, q, k_cache, v_cache, kv_indices, *, sm_scale: float, window_left: int,
            causal: bool = True, return_lse: bool = True, out=None, lse=None, stream=None,
            k_scale: float = 1.0, v_scale: float = 1.0):
        if out is None:
            out = torch.empty_like(q)
        if return_lse and lse is None:
            lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
        self._check_shapes(q, k_cache, v_cache, kv_indices, out, lse)
        if self.kind == PKVS_PREFILL:
            pkvs_prefill_run(self.handle, q, k_cache, v_cache, kv_indices, out, lse, sm_scale,
                             window_left, causal, k_scale, v_scale, stream)
        else:
            pkvs_decode_run(self.handle, q, k_cache, v_cache, kv_indices, out, lse, sm_scale,
                            window_left, k_scale, v_scale, stream)
        return (out, lse) if return_lse else out

    def info(self) -> pkvs_plan_info:
        return pkvs_plan_get_info(self.handle)

    def close(self):
        if self.handle is not None:
            pkvs_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class CascadeAttention:
    """Cascade prefill holder: new tokens' K/V in a contiguous array, cached
    prefix in the paged cache (``pkvs_cascade_plan`` / ``pkvs_cascade_run``).

    Keywords are the fields of ``pkvs_desc`` (kind is PKVS_CASCADE);
    ``kv_capacity`` bounds the cached keys of one request's page table.
    """

    def __init__(self, device="cuda", **desc_kw):
        self.desc = make_desc(PKVS_CASCADE, **desc_kw)
        self.handle = pkvs_plan_create(self.desc)
        fb, ib = pkvs_workspace_size(self.handle)
        self.float_ws = torch.empty(max(fb, 4), dtype=torch.uint8, device=device)
        self.int_ws = torch.empty(ib, dtype=torch.uint8, device=device)

    def plan(self, *, qo_indptr, kv_indptr, kv_last_page_len, stream=None):
        batch = len(kv_last_page_len)
        self._nnz_pages = int(torch.as_tensor(kv_indptr)[-1])
        self._nnz_qo = int(torch.as_tensor(qo_indptr)[-1])
        pkvs_cascade_plan(self.handle, qo_indptr, kv_indptr, kv_last_page_len, batch,
                          self.float_ws, self.int_ws, stream)

    def _check_shapes(self, q, k_extend, v_extend, k_cache, v_cache, kv_indices, out, lse):
        d = self.desc
        dt = _TORCH_DTYPES[d.dtype]
        rows = max(self._nnz_qo, q.shape[0] if q.dim() == 3 else 0)
        if tuple(q.shape) != (rows, d.num_qo_heads, d.head_dim) or q.dtype != dt:
            raise ValueError(f"q must be {dt} [>= {self._nnz_qo}, {d.num_qo_heads}, "
                             f"{d.head_dim}], got {q.dtype} {tuple(q.shape)}")
        if out.shape != q.shape or out.dtype != dt:
            raise ValueError("out must match q")
        for t in (k_extend, v_extend):
            if (t.dim() != 3 or t.shape[0] < self._nnz_qo
                    or tuple(t.shape[1:]) != (d.num_kv_heads, d.head_dim) or t.dtype != dt):
                raise ValueError(f"k_extend / v_extend must be {dt} [>= {self._nnz_qo}, "
                                 f"{d.num_kv_heads}, {d.head_dim}]")
        kv_shape = (d.page_size, d.num_kv_heads, d.head_dim)
        kv_dt = {v: k for k, v in _KV_FORMATS.items()}[d.kv_format] or dt
        for c in (k_cache, v_cache):
            if c.dim() != 4 or tuple(c.shape[1:]) != kv_shape or c.dtype != kv_dt:
                raise ValueError(f"caches must be {kv_dt} [num_pages, {kv_shape}]")
        if k_cache.shape[0] != v_cache.shape[0]:
            raise ValueError("k_cache and v_cache page counts differ")
        if kv_indices.dtype != torch.int32 or kv_indices.numel() < self._nnz_pages:
            raise ValueError(f"kv_indices must be int32 with >= {self._nnz_pages} entries")
        if lse is not None and (tuple(lse.shape) != (rows, d.num_qo_heads)
                                or lse.dtype != torch.float32):
            raise ValueError(f"lse must be float32 {(rows, d.num_qo_heads)}")

    def run(self, q, k_extend, v_extend, k_cache, v_cache, kv_indices, *, sm_scale: float,
            window_left: int, return_lse: bool = True, out=None, lse=None, stream=None,
            k_scale: float = 1.0, v_scale: float = 1.0):
        if out is None:
            out = torch.empty_like(q)
        if return_lse and lse is None:
            lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
        self._check_shapes(q, k_extend, v_extend, k_cache, v_cache, kv_indices, out, lse)
        pkvs_cascade_run(self.handle, q, k_extend, v_extend, k_cache, v_cache, kv_indices, out,
                         lse, sm_scale, window_left, k_scale, v_scale, stream)
        return (out, lse) if return_lse else out

    def info(self) -> pkvs_plan_info:
        return pkvs_plan_get_info(self.handle)

    def close(self):
        if self.handle is not None:
            pkvs_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
