"""ctypes binding of libgattn.so: the C ABI of include/gattn.h under the same names.

Argument marshalling only: pointers may be torch tensors (their data_ptr()),
numpy arrays (host pointers, for gattn_kv_offset), raw integer addresses or
None. Every computation happens in the library's HIP kernels. A nonzero status
raises GattnError carrying the status code.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# GATTN_LIBRARY names another build of the library to load (the CPU sanitizer tests load a host-only
# build whose kernel launches all fail); by default the in-tree gfx950 build.
LIB_PATH = os.environ.get("GATTN_LIBRARY") or os.path.join(_HERE, "libgattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build the gfx950 library first "
                      "(python -c 'import __graft_entry__ as g; g.build()')")
# torch ships its own HIP runtime (soname libamdhip64.so.7). Loading torch first makes the
# library's libamdhip64.so.7 dependency resolve to that same runtime; loaded the other way
# round, the process holds two runtimes and torch's streams are not valid handles in the one
# the library launches on (every launch then fails).
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

LOCAL, GLOBAL = 0, 1
OK, ERR_NULL_PTR, ERR_BAD_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_BAD_SPLIT, ERR_HIP = range(7)
PAGE_SIZE = 16
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # GATTN_NOALLOC_SCRATCH_BYTES

c_int, c_i64, c_size, c_vp, c_float = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float


class Layer(ctypes.Structure):
    """struct gattn_layer."""
    _fields_ = [("family", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("kv_shared", ctypes.c_int32), ("scale", ctypes.c_float)]


def make_layer(family, num_q_heads, num_kv_heads, head_dim, window=0, kv_shared=False, scale=None,
               page_size=PAGE_SIZE):
    fam = family if isinstance(family, int) else (GLOBAL if family == "global" else LOCAL)
    if scale is None:
        scale = head_dim ** -0.5
    return Layer(fam, num_q_heads, num_kv_heads, head_dim, window, page_size, int(bool(kv_shared)), scale)


class GattnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {gattn_status_str(status)} (status {status})")


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None


_lib.gattn_abi_version.restype = c_int
_lib.gattn_abi_version.argtypes = []
_lib.gattn_status_str.restype = ctypes.c_char_p
_lib.gattn_status_str.argtypes = [c_int]
_lib.gattn_layer_family.restype = c_int
_lib.gattn_layer_family.argtypes = [c_int, c_int]
_lib.gattn_kv_offset.restype = c_i64
_lib.gattn_kv_offset.argtypes = [ctypes.POINTER(Layer), c_vp, c_int, c_int, c_int, c_int, c_int, c_i64]
_lib.gattn_decode_workspace_bytes.restype = c_size
_lib.gattn_decode_workspace_bytes.argtypes = [ctypes.POINTER(Layer), c_int, c_int, c_int]
_lib.gattn_decode.restype = c_int
_lib.gattn_decode.argtypes = [ctypes.POINTER(Layer), c_vp, c_vp, c_vp, c_i64, c_vp, c_int, c_vp, c_int, c_int,
                              c_int, c_vp, c_size, c_vp, c_vp, c_vp]
_lib.gattn_decode_noalloc.restype = c_int
_lib.gattn_decode_noalloc.argtypes = [ctypes.POINTER(Layer), c_vp, c_vp, c_vp, c_i64, c_vp, c_int, c_vp, c_int, c_int,
                                      c_int, c_vp, c_vp, c_vp]
_lib.gattn_decode_fp8kv.restype = c_int
_lib.gattn_decode_fp8kv.argtypes = [ctypes.POINTER(Layer), c_vp, c_vp, c_vp, c_float, c_float, c_i64, c_vp, c_int,
                                    c_vp, c_int, c_int, c_int, c_vp, c_size, c_vp, c_vp, c_vp]
_lib.gattn_prefill.restype = c_int
_lib.gattn_prefill.argtypes = [ctypes.POINTER(Layer), c_vp, c_vp, c_vp, c_i64, c_vp, c_int, c_vp, c_vp, c_int,
                               c_int, c_vp, c_vp, c_vp]
_lib.gattn_kv_append.restype = c_int
_lib.gattn_kv_append.argtypes = [ctypes.POINTER(Layer), c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_int, c_vp, c_vp,
                                 c_int, c_int, c_vp, c_vp]
_lib.gattn_kv_append_fp8.restype = c_int
_lib.gattn_kv_append_fp8.argtypes = [ctypes.POINTER(Layer), c_vp, c_vp, c_vp, c_vp, c_float, c_float, c_i64, c_vp,
                                     c_int, c_vp, c_vp, c_int, c_int, c_vp, c_vp]
_lib.gattn_combine.restype = c_int
_lib.gattn_combine.argtypes = [c_int, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp]
_lib.gattn_decode_graphs_create.restype = c_int
_lib.gattn_decode_graphs_create.argtypes = [ctypes.POINTER(Layer), c_vp, c_vp, c_vp, c_i64, c_vp, c_int, c_vp, c_int,
                                            c_int, c_vp, c_size, c_vp, c_vp, c_vp, c_int, ctypes.POINTER(c_vp)]
_lib.gattn_decode_graphs_bucket.restype = c_int
_lib.gattn_decode_graphs_bucket.argtypes = [c_vp, c_int]
_lib.gattn_decode_graphs_launch.restype = c_int
_lib.gattn_decode_graphs_launch.argtypes = [c_vp, c_int, c_vp]
_lib.gattn_decode_graphs_destroy.restype = None
_lib.gattn_decode_graphs_destroy.argtypes = [c_vp]


def _check(rc, where):
    if rc != OK:
        raise GattnError(rc, where)


def gattn_abi_version():
    return _lib.gattn_abi_version()


def gattn_status_str(status):
    return _lib.gattn_status_str(int(status)).decode()


def gattn_layer_family(layer, n_layers):
    return _lib.gattn_layer_family(int(layer), int(n_layers))


def gattn_kv_offset(layer, page_table_host, rows, pt_stride, row, token, kv_head, num_pages):
    return _lib.gattn_kv_offset(ctypes.byref(layer), _addr(page_table_host), rows, pt_stride, row, token,
                                kv_head, num_pages)


def gattn_decode_workspace_bytes(layer, batch, max_ctx, split_tokens):
    return _lib.gattn_decode_workspace_bytes(ctypes.byref(layer), batch, max_ctx, split_tokens)


def gattn_decode(layer, q, k_pool, v_pool, num_pages, page_table, pt_stride, ctx_lens, batch, max_ctx,
                 split_tokens, workspace, workspace_bytes, out, lse, stream=None):
    rc = _lib.gattn_decode(ctypes.byref(layer), _addr(q), _addr(k_pool), _addr(v_pool), int(num_pages),
                           _addr(page_table), int(pt_stride), _addr(ctx_lens), int(batch), int(max_ctx),
                           int(split_tokens), _addr(workspace), int(workspace_bytes), _addr(out), _addr(lse),
                           _stream(stream))
    _check(rc, "gattn_decode")


def gattn_decode_noalloc(layer, q, k_pool, v_pool, num_pages, page_table, pt_stride, ctx_lens, batch, max_ctx,
                         split_tokens, out, lse, stream=None):
    rc = _lib.gattn_decode_noalloc(ctypes.byref(layer), _addr(q), _addr(k_pool), _addr(v_pool), int(num_pages),
                                   _addr(page_table), int(pt_stride), _addr(ctx_lens), int(batch), int(max_ctx),
                                   int(split_tokens), _addr(out), _addr(lse), _stream(stream))
    _check(rc, "gattn_decode_noalloc")


def gattn_decode_fp8kv(layer, q, k_pool, v_pool, k_scale, v_scale, num_pages, page_table, pt_stride, ctx_lens,
                       batch, max_ctx, split_tokens, workspace, workspace_bytes, out, lse, stream=None):
    rc = _lib.gattn_decode_fp8kv(ctypes.byref(layer), _addr(q), _addr(k_pool), _addr(v_pool), float(k_scale),
                                 float(v_scale), int(num_pages), _addr(page_table), int(pt_stride), _addr(ctx_lens),
                                 int(batch), int(max_ctx), int(split_tokens), _addr(workspace), int(workspace_bytes),
                                 _addr(out), _addr(lse), _stream(stream))
    _check(rc, "gattn_decode_fp8kv")


def gattn_prefill(layer, q, k_pool, v_pool, num_pages, page_table, pt_stride, cu_q, ctx_lens, batch, max_q,
                  out, lse, stream=None):
    rc = _lib.gattn_prefill(ctypes.byref(layer), _addr(q), _addr(k_pool), _addr(v_pool), int(num_pages),
                            _addr(page_table), int(pt_stride), _addr(cu_q), _addr(ctx_lens), int(batch),
                            int(max_q), _addr(out), _addr(lse), _stream(stream))
    _check(rc, "gattn_prefill")


def gattn_kv_append(layer, k_new, v_new, k_pool, v_pool, num_pages, page_table, pt_stride, cu_new, ctx_lens, batch,
                    max_new, status=None, stream=None):
    rc = _lib.gattn_kv_append(ctypes.byref(layer), _addr(k_new), _addr(v_new), _addr(k_pool), _addr(v_pool),
                              int(num_pages), _addr(page_table), int(pt_stride), _addr(cu_new), _addr(ctx_lens),
                              int(batch), int(max_new), _addr(status), _stream(stream))
    _check(rc, "gattn_kv_append")


def gattn_kv_append_fp8(layer, k_new, v_new, k_pool, v_pool, k_scale, v_scale, num_pages, page_table, pt_stride,
                        cu_new, ctx_lens, batch, max_new, status=None, stream=None):
    rc = _lib.gattn_kv_append_fp8(ctypes.byref(layer), _addr(k_new), _addr(v_new), _addr(k_pool), _addr(v_pool),
                                  float(k_scale), float(v_scale), int(num_pages), _addr(page_table), int(pt_stride),
                                  _addr(cu_new), _addr(ctx_lens), int(batch), int(max_new), _addr(status),
                                  _stream(stream))
    _check(rc, "gattn_kv_append_fp8")


def gattn_combine(batch, num_q_heads, head_dim, num_splits, o_part, lse_part, out, lse, stream=None):
    rc = _lib.gattn_combine(int(batch), int(num_q_heads), int(head_dim), int(num_splits), _addr(o_part),
                            _addr(lse_part), _addr(out), _addr(lse), _stream(stream))
    _check(rc, "gattn_combine")


def gattn_decode_graphs_create(layer, q, k_pool, v_pool, num_pages, page_table, pt_stride, ctx_lens, max_ctx,
                               split_tokens, workspace, workspace_bytes, out, lse, buckets):
    """Returns the handle (an int) of the captured set; ``buckets`` is a sequence of batch sizes."""
    arr = (ctypes.c_int32 * len(buckets))(*[int(b) for b in buckets])
    handle = c_vp()
    rc = _lib.gattn_decode_graphs_create(ctypes.byref(layer), _addr(q), _addr(k_pool), _addr(v_pool), int(num_pages),
                                         _addr(page_table), int(pt_stride), _addr(ctx_lens), int(max_ctx),
                                         int(split_tokens), _addr(workspace), int(workspace_bytes), _addr(out),
                                         _addr(lse), arr, len(buckets), ctypes.byref(handle))
    _check(rc, "gattn_decode_graphs_create")
    return handle.value


def gattn_decode_graphs_bucket(graphs, batch):
    return _lib.gattn_decode_graphs_bucket(graphs, int(batch))


def gattn_decode_graphs_launch(graphs, batch, stream=None):
    rc = _lib.gattn_decode_graphs_launch(graphs, int(batch), _stream(stream))
    _check(rc, "gattn_decode_graphs_launch")


def gattn_decode_graphs_destroy(graphs):
    _lib.gattn_decode_graphs_destroy(graphs)


def exported_symbols():
    """Names the shared library exports (for the ABI check)."""
    return sorted(n for n in ("gattn_abi_version", "gattn_status_str", "gattn_layer_family", "gattn_kv_offset",
                              "gattn_decode_workspace_bytes", "gattn_decode", "gattn_decode_noalloc",
                              "gattn_decode_fp8kv", "gattn_prefill",
                              "gattn_combine", "gattn_kv_append", "gattn_kv_append_fp8",
                              "gattn_decode_graphs_create", "gattn_decode_graphs_bucket",
                              "gattn_decode_graphs_launch", "gattn_decode_graphs_destroy")
                  if hasattr(_lib, n))
