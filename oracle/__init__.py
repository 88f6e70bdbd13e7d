"""fp64 CPU oracle for hybrid paged GQA attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library never uses it, and this
package imports nothing from the library.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP over
(query, head)); this wrapper only builds it with gcc and marshals numpy arrays.
Citations for what is computed are in ``oracle.c``'s header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")
# A prebuilt oracle library to load instead of building liboracle.so (the sanitizer tests point this
# at an AddressSanitizer / UndefinedBehaviorSanitizer build of the same oracle.c).
_LIB_OVERRIDE = os.environ.get("GATTN_ORACLE_LIB")
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]
_lock = threading.Lock()
_lib = None

OK, BAD_ARG, MISSING_KEYS, NO_MEM = 0, -1, -2, -3


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, -O2, OpenMP)."""
    stale = (not os.path.exists(_LIB) or
             os.path.getmtime(_LIB) < max(os.path.getmtime(_SRC), os.path.getmtime(_HDR)))
    if force or stale:
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """Compile oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer into ``path`` (loaded
    through GATTN_ORACLE_LIB by a process that preloads the sanitizer runtime)."""
    subprocess.check_call(["gcc", *SANITIZE_FLAGS, "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", path, _SRC,
                           "-lm"])
    return path


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if _LIB_OVERRIDE:
                lib = ctypes.CDLL(_LIB_OVERRIDE)
            else:
                build()
                lib = ctypes.CDLL(_LIB)
            i32p = ctypes.POINTER(ctypes.c_int32)
            u16p = ctypes.POINTER(ctypes.c_uint16)
            f64p = ctypes.POINTER(ctypes.c_double)
            c_int, c_double = ctypes.c_int, ctypes.c_double
            lib.oracle_attend.restype = c_int
            lib.oracle_attend.argtypes = [c_int, c_int, c_int, c_int, c_int, c_double, c_int,
                                          i32p, i32p, i32p, u16p, u16p, u16p, f64p, f64p]
            lib.oracle_decode_split.restype = c_int
            lib.oracle_decode_split.argtypes = [c_int, c_int, c_int, c_int, c_int, c_double, c_int,
                                                i32p, i32p, u16p, u16p, u16p, c_int, f64p, f64p]
            lib.oracle_merge.restype = c_int
            lib.oracle_merge.argtypes = [ctypes.c_int64, c_int, c_int, f64p, f64p, f64p, f64p]
            lib.oracle_layer_is_global.restype = c_int
            lib.oracle_layer_is_global.argtypes = [c_int, c_int]
            lib.oracle_threads.restype = c_int
            lib.oracle_threads.argtypes = []
            lib.oracle_kv_append.restype = ctypes.c_int64
            lib.oracle_kv_append.argtypes = [c_int, c_int, c_int, c_int, i32p, i32p, i32p, c_int, ctypes.c_int64,
                                             c_int, u16p, u16p, u16p, u16p]
            u8p = ctypes.POINTER(ctypes.c_uint8)
            lib.oracle_attend_fp8kv.restype = c_int
            lib.oracle_attend_fp8kv.argtypes = [c_int, c_int, c_int, c_int, c_int, c_double, c_int,
                                                i32p, i32p, i32p, u16p, u8p, u8p, c_double, c_double, f64p, f64p]
            lib.oracle_e4m3_value.restype = c_double
            lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
            lib.oracle_e4m3_encode.restype = ctypes.c_uint8
            lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
            lib.oracle_e4m3_encode_n.restype = None
            lib.oracle_e4m3_encode_n.argtypes = [ctypes.c_int64, ctypes.POINTER(ctypes.c_float), u8p]
            lib.oracle_kv_append_fp8.restype = ctypes.c_int64
            lib.oracle_kv_append_fp8.argtypes = [c_int, c_int, c_int, c_int, i32p, i32p, i32p, c_int, ctypes.c_int64,
                                                 c_int, u16p, u16p, ctypes.c_float, ctypes.c_float, u8p, u8p]
            _lib = lib
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype)) if a is not None else None


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _u16(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.uint16)


class OracleError(RuntimeError):
    pass


def attend(is_global: bool, num_q_heads: int, num_kv_heads: int, head_dim: int, window: int,
           scale: float, q_lens, ctx_lens, k_starts, q, k, v=None):
    """Exact-definition attention in fp64. Returns (out [T][Hq][hd], lse [T][Hq])."""
    lib = _load()
    q_lens, ctx_lens = _i32(q_lens), _i32(ctx_lens)
    k_starts = None if k_starts is None else _i32(k_starts)
    q, k, v = _u16(q), _u16(k), _u16(v)
    T = int(q_lens.sum())
    out = np.empty((T, num_q_heads, head_dim), dtype=np.float64)
    lse = np.empty((T, num_q_heads), dtype=np.float64)
    rc = lib.oracle_attend(int(bool(is_global)), num_q_heads, num_kv_heads, head_dim, int(window),
                           float(scale), int(q_lens.shape[0]), _ptr(q_lens, ctypes.c_int32),
                           _ptr(ctx_lens, ctypes.c_int32), _ptr(k_starts, ctypes.c_int32),
                           _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
                           _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if rc != OK:
        raise OracleError(f"oracle_attend failed: {rc}")
    return out, lse


def decode_split(is_global: bool, num_q_heads: int, num_kv_heads: int, head_dim: int, window: int,
                 scale: float, ctx_lens, k_starts, q, k, v, split_tokens: int):
    """Split-KV decode merged by logsumexp, in fp64. Returns (out [B][Hq][hd], lse [B][Hq])."""
    lib = _load()
    ctx_lens = _i32(ctx_lens)
    k_starts = None if k_starts is None else _i32(k_starts)
    q, k, v = _u16(q), _u16(k), _u16(v)
    B = int(ctx_lens.shape[0])
    out = np.empty((B, num_q_heads, head_dim), dtype=np.float64)
    lse = np.empty((B, num_q_heads), dtype=np.float64)
    rc = lib.oracle_decode_split(int(bool(is_global)), num_q_heads, num_kv_heads, head_dim, int(window),
                                 float(scale), B, _ptr(ctx_lens, ctypes.c_int32),
                                 _ptr(k_starts, ctypes.c_int32), _ptr(q, ctypes.c_uint16),
                                 _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16), int(split_tokens),
                                 _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if rc != OK:
        raise OracleError(f"oracle_decode_split failed: {rc}")
    return out, lse


def merge(lse_parts, o_parts):
    """Logsumexp merge in fp64. lse_parts [..., n]; o_parts [..., n, hd] -> (out [..., hd], lse [...])."""
    lib = _load()
    lp = np.ascontiguousarray(lse_parts, dtype=np.float64)
    op = np.ascontiguousarray(o_parts, dtype=np.float64)
    lead, n, hd = lp.shape[:-1], lp.shape[-1], op.shape[-1]
    rows = int(np.prod(lead)) if lead else 1
    out = np.empty(lead + (hd,), dtype=np.float64)
    lse = np.empty(lead, dtype=np.float64)
    rc = lib.oracle_merge(rows, n, hd, _ptr(lp, ctypes.c_double), _ptr(op, ctypes.c_double),
                          _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if rc != OK:
        raise OracleError(f"oracle_merge failed: {rc}")
    return out, lse


def kv_append(num_kv_heads: int, head_dim: int, page_size: int, cu_new, ctx_lens, page_table, num_pages: int,
              k_new, v_new, k_pool, v_pool, max_new=None):
    """Paged KV append (``oracle_kv_append``): returns (k_pool', v_pool', skipped tokens) with the
    new tokens copied into copies of the given pools. ``max_new`` is the call's declared bound on a
    row's new tokens (None: no bound); a row above it writes nothing."""
    lib = _load()
    cu_new, ctx_lens = _i32(cu_new), _i32(ctx_lens)
    pt = _i32(page_table)
    k_new = _u16(k_new)
    v_new = None if v_new is None else _u16(v_new)
    kp = np.array(k_pool, dtype=np.uint16, copy=True, order="C")
    vp = None if v_pool is None else np.array(v_pool, dtype=np.uint16, copy=True, order="C")
    B = int(ctx_lens.shape[0])
    n = lib.oracle_kv_append(num_kv_heads, head_dim, page_size, B, _ptr(cu_new, ctypes.c_int32),
                             _ptr(ctx_lens, ctypes.c_int32), _ptr(pt, ctypes.c_int32), int(pt.shape[1]),
                             int(num_pages), -1 if max_new is None else int(max_new), _ptr(k_new, ctypes.c_uint16),
                             _ptr(v_new, ctypes.c_uint16), _ptr(kp, ctypes.c_uint16), _ptr(vp, ctypes.c_uint16))
    if n < 0:
        raise OracleError(f"oracle_kv_append failed: {n}")
    return kp, vp, int(n)


def _u8(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.uint8)


def attend_fp8kv(is_global: bool, num_q_heads: int, num_kv_heads: int, head_dim: int, window: int,
                 scale: float, q_lens, ctx_lens, k_starts, q, k8, v8, k_scale: float, v_scale: float):
    """``attend`` over an E4M3 K/V (codes standing for code_value * k_scale / v_scale), in fp64."""
    lib = _load()
    q_lens, ctx_lens = _i32(q_lens), _i32(ctx_lens)
    k_starts = None if k_starts is None else _i32(k_starts)
    q, k8, v8 = _u16(q), _u8(k8), _u8(v8)
    T = int(q_lens.sum())
    out = np.empty((T, num_q_heads, head_dim), dtype=np.float64)
    lse = np.empty((T, num_q_heads), dtype=np.float64)
    rc = lib.oracle_attend_fp8kv(int(bool(is_global)), num_q_heads, num_kv_heads, head_dim, int(window),
                                 float(scale), int(q_lens.shape[0]), _ptr(q_lens, ctypes.c_int32),
                                 _ptr(ctx_lens, ctypes.c_int32), _ptr(k_starts, ctypes.c_int32),
                                 _ptr(q, ctypes.c_uint16), _ptr(k8, ctypes.c_uint8), _ptr(v8, ctypes.c_uint8),
                                 float(k_scale), float(v_scale), _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if rc != OK:
        raise OracleError(f"oracle_attend_fp8kv failed: {rc}")
    return out, lse


def e4m3_value(codes):
    """fp64 values of E4M3 codes (any shape)."""
    lib = _load()
    table = np.array([lib.oracle_e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x):
    """E4M3 codes of float32 values (nearest, ties to even, saturating at 448, NaN kept)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib.oracle_e4m3_encode_n(int(x.size), _ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint8))
    return out


def kv_append_fp8(num_kv_heads: int, head_dim: int, page_size: int, cu_new, ctx_lens, page_table, num_pages: int,
                  k_new, v_new, k_scale: float, v_scale: float, k_pool8, v_pool8, max_new=None):
    """``kv_append`` into E4M3 pools (``oracle_kv_append_fp8``): returns (k_pool', v_pool', skipped)."""
    lib = _load()
    cu_new, ctx_lens = _i32(cu_new), _i32(ctx_lens)
    pt = _i32(page_table)
    k_new = _u16(k_new)
    v_new = None if v_new is None else _u16(v_new)
    kp = np.array(k_pool8, dtype=np.uint8, copy=True, order="C")
    vp = None if v_pool8 is None else np.array(v_pool8, dtype=np.uint8, copy=True, order="C")
    B = int(ctx_lens.shape[0])
    n = lib.oracle_kv_append_fp8(num_kv_heads, head_dim, page_size, B, _ptr(cu_new, ctypes.c_int32),
                                 _ptr(ctx_lens, ctypes.c_int32), _ptr(pt, ctypes.c_int32), int(pt.shape[1]),
                                 int(num_pages), -1 if max_new is None else int(max_new),
                                 _ptr(k_new, ctypes.c_uint16), _ptr(v_new, ctypes.c_uint16), float(k_scale),
                                 float(v_scale), _ptr(kp, ctypes.c_uint8), _ptr(vp, ctypes.c_uint8))
    if n < 0:
        raise OracleError(f"oracle_kv_append_fp8 failed: {n}")
    return kp, vp, int(n)


def layer_is_global(layer: int, n_layers: int) -> int:
    return _load().oracle_layer_is_global(int(layer), int(n_layers))


def threads() -> int:
    return _load().oracle_threads()


def attend_batch(batch, rows=None):
    """Run ``attend`` on a ``workloads.Batch`` (all rows, or a subset). Contiguous side only; a batch
    carrying an FP8 KV copy (``batch.fp8``) is attended over that copy."""
    b = batch if rows is None else batch.subset(rows)
    s = b.spec
    f = getattr(b, "fp8", None)
    if f is not None:
        return attend_fp8kv(s.is_global, s.num_q_heads, s.num_kv_heads, s.head_dim, s.window, s.softmax_scale,
                            b.q_lens, b.ctx_lens, b.k_starts, b.q, f.k, f.v, f.k_scale, f.v_scale)
    return attend(s.is_global, s.num_q_heads, s.num_kv_heads, s.head_dim, s.window,
                  s.softmax_scale, b.q_lens, b.ctx_lens, b.k_starts, b.q, b.k, b.v)
