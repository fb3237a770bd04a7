"""CPU oracle for paged sliding-window attention and the LSE merge.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the product package.  The numerics
live in ``oracle.c`` (plain C, IEEE double); this module only compiles it with
gcc, marshals arrays and calls it.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (closed forms, special cases that reduce to a
library routine, invariants and brute force on tiny inputs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16 = 0
FP32 = 1
FP16 = 2
FP8_E4M3 = 3
FP8_E5M2 = 4


def compile_source(src: str, out: str) -> str:
    """gcc -O2 a copy of the oracle source into a shared library at ``out``."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.run(["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread",
                    "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it (gcc, -O2)."""
    stale = (not os.path.exists(_LIB_PATH)
             or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))
    if force or stale:
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


class OracleLib:
    """ctypes handle on one compiled copy of ``oracle.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oracle_paged_attention.restype = ctypes.c_int
        lib.oracle_paged_attention.argtypes = [
            i32, P, P, P, P, i32, i32, i32, i32, i32, i32, f64, f64, i32, P, i32, f64, f64, P, P,
            P, i64, i64, i64, P, P, i32,
        ]
        lib.oracle_merge_state.restype = None
        lib.oracle_merge_state.argtypes = [i64, i32, i32, P, P, P, P, P, P]
        lib.oracle_widen.restype = None
        lib.oracle_widen.argtypes = [i32, P, i64, P]
        lib.oracle_append_kv.restype = i64
        lib.oracle_append_kv.argtypes = [i64, P, i64, P, P, i64, P, P]
        lib.oracle_quantize.restype = ctypes.c_uint8
        lib.oracle_quantize.argtypes = [i32, f64, ctypes.c_float, i32]
        lib.oracle_quantize_many.restype = None
        lib.oracle_quantize_many.argtypes = [i32, P, i64, ctypes.c_float, i32, P]
        lib.oracle_append_kv_quant.restype = i64
        lib.oracle_append_kv_quant.argtypes = [i64, P, i64, i32, P, P, i64, i32, ctypes.c_float,
                                               ctypes.c_float, P, P]
        lib.oracle_build_kv_indices.restype = i64
        lib.oracle_build_kv_indices.argtypes = [i32, P, i64, i64, P, P, P, P, P, i64]
        self.lib = lib
        self.path = path


def _load():
    global _lib
    if _lib is None:
        _lib = OracleLib(build())
    return _lib


def default_threads() -> int:
    """Threads the oracle uses unless told otherwise: ORACLE_THREADS, else the
    host's cores, at most 16 (the CPU share of one GPU on a shared host)."""
    env = os.environ.get("ORACLE_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_stored(t) -> tuple:
    """(contiguous numpy array of the stored bits, dtype code)."""
    import torch

    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy(), BF16
    if t.dtype == torch.float16:
        return t.view(torch.int16).numpy(), FP16
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy(), FP8_E4M3
    if t.dtype == torch.float8_e5m2:
        return t.view(torch.uint8).numpy(), FP8_E5M2
    if t.dtype == torch.float32:
        return t.numpy(), FP32
    raise TypeError(f"oracle: unsupported input dtype {t.dtype}")


def _i32(t) -> np.ndarray:
    import torch

    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(t, dtype=np.int32))


def paged_attention(q, k_cache, v_cache, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, *,
                    num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
                    causal: bool, window_left: int, sm_scale: float, soft_cap: float = 0.0,
                    k_scale: float = 1.0, v_scale: float = 1.0,
                    rows: Optional[Sequence[int]] = None, key_lo: int = 0,
                    key_hi: int = np.iinfo(np.int64).max, impl: Optional[OracleLib] = None,
                    threads: Optional[int] = None):
    """Reference (O, LSE) in float64.

    ``q``/``k_cache``/``v_cache`` are torch tensors (bf16 or fp32, any device;
    they are copied to the host).  Returns ``o`` ``[nnz_qo, H_q, D]`` and ``lse``
    ``[nnz_qo, H_q]``; with ``rows`` (global query-token indices) the outputs
    are compact: ``[len(rows), H_q, D]`` and ``[len(rows), H_q]``.  Rows are
    spread over ``threads`` POSIX threads (default ``default_threads()``); each
    row is computed by one thread with unchanged arithmetic, so the result does
    not depend on the thread count.
    """
    lib = (impl or _load()).lib
    qa, qd = _as_stored(q)
    ka, kd = _as_stored(k_cache)
    va, vd = _as_stored(v_cache)
    if kd != vd:
        raise TypeError("oracle: k and v caches must share one stored dtype")
    qo = _i32(qo_indptr)
    kvp = _i32(kv_indptr)
    kvi = _i32(kv_indices)
    last = _i32(kv_last_page_len)
    batch = len(kvp) - 1
    nnz_qo = int(qo[-1])
    n_out = nnz_qo if rows is None else len(rows)
    o = np.full((n_out, num_qo_heads, head_dim), np.nan, dtype=np.float64)
    lse = np.full((n_out, num_qo_heads), np.nan, dtype=np.float64)
    if rows is not None:
        rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        rp, nr = _ptr(rows_a), len(rows_a)
    else:
        rows_a, rp, nr = None, None, 0
    rc = lib.oracle_paged_attention(
        batch, _ptr(qo), _ptr(kvp), _ptr(kvi), _ptr(last), page_size, num_qo_heads,
        num_kv_heads, head_dim, int(bool(causal)), window_left, float(sm_scale),
        float(soft_cap), qd, _ptr(qa), kd, float(k_scale), float(v_scale),
        _ptr(ka), _ptr(va), rp, nr, int(key_lo), int(key_hi), _ptr(o), _ptr(lse),
        int(default_threads() if threads is None else threads))
    if rc != 0:
        raise ValueError(f"oracle_paged_attention: malformed layout (rc={rc})")
    return o, lse


def case_attention(case, rows=None, window_left: Optional[int] = None, **kw):
    """``paged_attention`` on a ``paged_kv_sliding_amd.synth.Case``."""
    return paged_attention(
        case.q, case.k_cache, case.v_cache, case.qo_indptr, case.kv_indptr, case.kv_indices,
        case.kv_last_page_len, num_qo_heads=case.num_qo_heads, num_kv_heads=case.num_kv_heads,
        head_dim=case.head_dim, page_size=case.page_size, causal=case.causal,
        window_left=case.window_left if window_left is None else window_left,
        sm_scale=case.sm_scale, soft_cap=case.logits_soft_cap, k_scale=case.k_scale,
        v_scale=case.v_scale, rows=rows, **kw)


def merge_state(v_a, s_a, v_b, s_b, impl: Optional[OracleLib] = None):
    """Pairwise merge of two (v [N,H,D], s [N,H]) partials, float64 in and out."""
    lib = (impl or _load()).lib
    v_a = np.ascontiguousarray(v_a, dtype=np.float64)
    v_b = np.ascontiguousarray(v_b, dtype=np.float64)
    s_a = np.ascontiguousarray(s_a, dtype=np.float64)
    s_b = np.ascontiguousarray(s_b, dtype=np.float64)
    n, h, d = v_a.shape
    if v_b.shape != v_a.shape or s_a.shape != (n, h) or s_b.shape != (n, h):
        raise ValueError("merge_state: shape mismatch")
    v = np.empty_like(v_a)
    s = np.empty_like(s_a)
    lib.oracle_merge_state(n, h, d, _ptr(v_a), _ptr(s_a), _ptr(v_b), _ptr(s_b), _ptr(v), _ptr(s))
    return v, s


def merge_many(parts, impl: Optional[OracleLib] = None):
    """Left fold of ``merge_state`` over a list of (v, s) partials."""
    v, s = parts[0]
    for vb, sb in parts[1:]:
        v, s = merge_state(v, s, vb, sb, impl=impl)
    return v, s


def append_kv(k_new, v_new, loc, k_cache, v_cache, impl: Optional[OracleLib] = None):
    """Host copies of the caches after writing row i of k_new / v_new to slot
    loc[i] (slot = page * page_size + position in the page); returns
    (k_cache, v_cache, skipped rows).  Inputs are torch tensors of one dtype."""
    import torch

    lib = (impl or _load()).lib
    kc = k_cache.detach().cpu().contiguous().clone()
    vc = v_cache.detach().cpu().contiguous().clone()
    kn = k_new.detach().cpu().contiguous()
    vn = v_new.detach().cpu().contiguous()
    if not (kc.dtype == vc.dtype == kn.dtype == vn.dtype):
        raise TypeError("append_kv: one dtype for caches and new rows")
    row = kn[0].numel() * kn.element_size() if kn.shape[0] else 0
    num_slots = kc.numel() * kc.element_size() // row if row else 0
    lo = np.ascontiguousarray(torch.as_tensor(loc).cpu().numpy().astype(np.int64))
    u8 = lambda t: t.view(torch.uint8).numpy()
    kb, vb = u8(kc.view(-1)), u8(vc.view(-1))
    skipped = lib.oracle_append_kv(kn.shape[0], _ptr(lo), row, _ptr(u8(kn.view(-1))),
                                   _ptr(u8(vn.view(-1))), num_slots, _ptr(kb), _ptr(vb))
    return kc, vc, int(skipped)


def build_kv_indices(page_map, slot, length, start=None, capacity=None,
                     impl: Optional[OracleLib] = None):
    """(kv_indptr [B+1], kv_indices [capacity], errors) gathered from the
    request-to-page map ``page_map`` [rows, cols] int32.  Unwritten entries of
    kv_indices hold the sentinel 0x7fffffff."""
    lib = (impl or _load()).lib
    m = _i32(page_map)
    if m.ndim != 2:
        raise ValueError("build_kv_indices: the map is 2-D")
    sl, ln = _i32(slot), _i32(length)
    st = _i32(start) if start is not None else None
    B = len(sl)
    if capacity is None:
        capacity = int(np.maximum(ln, 0).sum())
    indptr = np.zeros(B + 1, dtype=np.int32)
    idx = np.full(max(capacity, 1), 0x7FFFFFFF, dtype=np.int32)
    err = lib.oracle_build_kv_indices(B, _ptr(m), m.shape[0], m.shape[1], _ptr(sl),
                                      _ptr(st) if st is not None else None, _ptr(ln),
                                      _ptr(indptr), _ptr(idx), capacity)
    return indptr, idx[:capacity], int(err)


def widen(t, impl: Optional[OracleLib] = None) -> np.ndarray:
    """The oracle's exact float64 reading of a tensor's stored elements."""
    lib = (impl or _load()).lib
    a, code = _as_stored(t)
    a = np.ascontiguousarray(a).reshape(-1)
    out = np.empty(a.size, dtype=np.float64)
    lib.oracle_widen(code, _ptr(a), a.size, _ptr(out))
    return out


def quantize(x, scale: float, kv_dtype, impl: Optional[OracleLib] = None):
    """uint8 codes of the elements of tensor ``x`` divided by ``scale`` and
    rounded to the 8-bit type ``kv_dtype`` (torch.float8_e4m3fn / e5m2), the
    way an 8-bit cache write does it."""
    import torch

    lib = (impl or _load()).lib
    a, code = _as_stored(x)
    a = np.ascontiguousarray(a).reshape(-1)
    kd = FP8_E4M3 if kv_dtype == torch.float8_e4m3fn else FP8_E5M2
    out = np.empty(a.size, dtype=np.uint8)
    lib.oracle_quantize_many(code, _ptr(a), a.size, float(scale), kd, _ptr(out))
    return out


def append_kv_quant(k_new, v_new, loc, k_cache, v_cache, k_scale: float, v_scale: float,
                    impl: Optional[OracleLib] = None):
    """Host copies of 8-bit caches after writing row i of k_new / v_new (16 or
    32-bit), divided by the scales and rounded, to slot loc[i]; returns
    (k_cache, v_cache, skipped rows)."""
    import torch

    lib = (impl or _load()).lib
    kc = k_cache.detach().cpu().contiguous().clone()
    vc = v_cache.detach().cpu().contiguous().clone()
    ka, code = _as_stored(k_new)
    va, code2 = _as_stored(v_new)
    assert code == code2
    _, kd = _as_stored(kc)
    n = k_new.shape[0]
    elems = k_new[0].numel() if n else 0
    num_slots = kc.numel() // elems if elems else 0
    lo = np.ascontiguousarray(torch.as_tensor(loc).cpu().numpy().astype(np.int64))
    kb, vb = kc.view(torch.uint8).numpy(), vc.view(torch.uint8).numpy()
    skipped = lib.oracle_append_kv_quant(n, _ptr(lo), elems, code, _ptr(np.ascontiguousarray(ka)),
                                         _ptr(np.ascontiguousarray(va)), num_slots, kd,
                                         float(k_scale), float(v_scale), _ptr(kb), _ptr(vb))
    return kc, vc, int(skipped)

