"""Python binding of libcke_xattn.so (ctypes, argument marshalling only).

Every computation runs in the HIP kernels behind the C ABI declared in
include/cke_xattn.h; this module turns torch tensors into device pointers,
picks the current HIP stream and turns non-OK status codes into exceptions.
PyTorch serves only as the device-memory and stream provider. There is no
fallback: if the shared library is missing, importing this package fails.

Function names mirror the C entry points:
  cke_xattn_populate(cache, E, WK, WV)         prefill the projection cache
  cke_xattn_decode(q, cache, layer, scale, out) cross-attention at one layer
  cke_selfattn_decode_append(q, k_new, v_new, kv, pos, scale, out)
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# CKE_XATTN_LIB selects another build of the same library (e.g. a variant
# compiled with different launch-shape macros); default: the in-tree build.
LIB_PATH = os.environ.get("CKE_XATTN_LIB") or os.path.join(_PKG, "libcke_xattn.so")

CKE_OK, CKE_EINVAL, CKE_ENOTREADY, CKE_ERANGE, CKE_EDEVICE = 0, -1, -2, -3, -4
CKE_F32, CKE_BF16, CKE_FP8 = 0, 1, 2
# fp8 (E4M3, OCP "fn" variant: no infinities, largest finite 448) is a
# projection-cache type only, populated from bf16 E and weights
_DTYPES = {torch.float32: CKE_F32, torch.bfloat16: CKE_BF16, torch.float8_e4m3fn: CKE_FP8}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libcke_xattn.so is not built (%s); run projection_cache_amd/_build.py "
        "or __graft_entry__.build() first" % LIB_PATH)


class cke_xattn_geom(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_streams", ctypes.c_int32),
                ("mem_len", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_q", ctypes.c_int32), ("cache_dtype", ctypes.c_int32)]


class cke_kv_layer(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("n_seqs", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_pos", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class cke_decoder_layer(ctypes.Structure):
    _fields_ = [("wq_self", ctypes.c_void_p), ("wk_self", ctypes.c_void_p),
                ("wv_self", ctypes.c_void_p), ("wo_self", ctypes.c_void_p),
                ("wq_cross", ctypes.c_void_p), ("wo_cross", ctypes.c_void_p),
                ("dtype", ctypes.c_int32)]


_P, _I, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_lib = ctypes.CDLL(LIB_PATH)
_lib.cke_last_error.restype = ctypes.c_char_p
_lib.cke_version.restype = ctypes.c_char_p
_lib.cke_xattn_region_bytes.restype = _SZ
_lib.cke_xattn_region_bytes.argtypes = [ctypes.POINTER(cke_xattn_geom)]
_lib.cke_xattn_layer_offset_bytes.restype = _SZ
_lib.cke_xattn_layer_offset_bytes.argtypes = [ctypes.POINTER(cke_xattn_geom), _I]
_lib.cke_xattn_workspace_bytes.restype = _SZ
_lib.cke_xattn_workspace_bytes.argtypes = [ctypes.POINTER(cke_xattn_geom)]
_lib.cke_xattn_num_splits.restype = _I
_lib.cke_xattn_num_splits.argtypes = [ctypes.POINTER(cke_xattn_geom)]
_lib.cke_xattn_whole_pairs.restype = _I
_lib.cke_xattn_whole_pairs.argtypes = [ctypes.POINTER(cke_xattn_geom)]
_lib.cke_xattn_cache_create.restype = _I
_lib.cke_xattn_cache_create.argtypes = [ctypes.POINTER(cke_xattn_geom), _P, _P, _P,
                                        ctypes.POINTER(_P)]
_lib.cke_xattn_cache_destroy.restype = None
_lib.cke_xattn_cache_destroy.argtypes = [_P]
_lib.cke_xattn_invalidate.restype = _I
_lib.cke_xattn_invalidate.argtypes = [_P]
_lib.cke_xattn_is_ready.restype = _I
_lib.cke_xattn_is_ready.argtypes = [_P]
_lib.cke_xattn_set_merge_mode.restype = _I
_lib.cke_xattn_set_merge_mode.argtypes = [_I]
_lib.cke_xattn_merges_in_launch.restype = _I
_lib.cke_xattn_merges_in_launch.argtypes = [_P, _I]
_lib.cke_xattn_populate.restype = _I
_lib.cke_xattn_populate.argtypes = [_P, _P, _I, ctypes.POINTER(_P), ctypes.POINTER(_P), _I, _P]
_lib.cke_xattn_populate_workspace_bytes.restype = _SZ
_lib.cke_xattn_populate_workspace_bytes.argtypes = [ctypes.POINTER(cke_xattn_geom), _I, _I]
_lib.cke_xattn_populate_ws.restype = _I
_lib.cke_xattn_populate_ws.argtypes = [_P, _P, _I, ctypes.POINTER(_P), ctypes.POINTER(_P), _I, _P,
                                       _SZ, _P]
_lib.cke_memory_lift_workspace_bytes.restype = _SZ
_lib.cke_memory_lift_workspace_bytes.argtypes = [_I, _I, _I]
_lib.cke_memory_lift_gelu_ws.restype = _I
_lib.cke_memory_lift_gelu_ws.argtypes = [_P, _I, _I, _P, _I, _P, _I, _P, _P, _SZ, _P]
_lib.cke_xattn_decode.restype = _I
_lib.cke_xattn_decode.argtypes = [_P, _I, _P, _I, _F, _P, _P]
_lib.cke_selfattn_decode_append.restype = _I
_lib.cke_selfattn_decode_append.argtypes = [_P, _P, _P, ctypes.POINTER(cke_kv_layer), _I, _F,
                                            _P, _P]
_lib.cke_xattn_decode_weights.restype = _I
_lib.cke_xattn_decode_weights.argtypes = [_P, _I, _P, _I, _F, ctypes.POINTER(ctypes.c_int32), _I,
                                          _P, _P, _P]
_lib.cke_selfattn_prefill_append.restype = _I
_lib.cke_selfattn_prefill_append.argtypes = [_P, _P, _P, ctypes.POINTER(cke_kv_layer), _I, _I, _I,
                                             _F, _P, _P]
_lib.cke_decoder_step_workspace_bytes.restype = _SZ
_lib.cke_decoder_step_workspace_bytes.argtypes = [ctypes.POINTER(cke_xattn_geom), _I]
_lib.cke_decoder_layer_step.restype = _I
_lib.cke_decoder_layer_step.argtypes = [_P, ctypes.POINTER(cke_decoder_layer),
                                        ctypes.POINTER(cke_kv_layer), _I, _P, _I, _F, _P, _P]
_lib.cke_decoder_step_scratch_bytes.restype = _SZ
_lib.cke_decoder_step_scratch_bytes.argtypes = []
_lib.cke_decoder_layer_step_noalloc.restype = _I
_lib.cke_decoder_layer_step_noalloc.argtypes = [_P, ctypes.POINTER(cke_decoder_layer),
                                                ctypes.POINTER(cke_kv_layer), _I, _P, _I, _F, _P]
_lib.cke_memory_lift_gelu.restype = _I
_lib.cke_memory_lift_gelu.argtypes = [_P, _I, _I, _P, _I, _P, _I, _P, _P]
_lib.cke_weight_planes_bytes.restype = _SZ
_lib.cke_weight_planes_bytes.argtypes = [_I, _I, _I]
_lib.cke_weight_planes.restype = _I
_lib.cke_weight_planes.argtypes = [ctypes.POINTER(_P), _I, _I, _I, _P, _SZ, _P]
_lib.cke_row_planes_bytes.restype = _SZ
_lib.cke_row_planes_bytes.argtypes = [_I, _I]
_lib.cke_xattn_populate_planes.restype = _I
_lib.cke_xattn_populate_planes.argtypes = [_P, _P, _P, _SZ, _P, _SZ, _P]
_lib.cke_memory_lift_planes_workspace_bytes.restype = _SZ
_lib.cke_memory_lift_planes_workspace_bytes.argtypes = [_I, _I, _I]
_lib.cke_memory_lift_gelu_planes.restype = _I
_lib.cke_memory_lift_gelu_planes.argtypes = [_P, _I, _I, _P, _SZ, _I, _P, _I, _P, _P, _SZ, _P]

EXPORTED = ["cke_xattn_region_bytes", "cke_xattn_layer_offset_bytes",
            "cke_xattn_workspace_bytes", "cke_xattn_num_splits", "cke_xattn_whole_pairs",
            "cke_xattn_cache_create",
            "cke_xattn_cache_destroy", "cke_xattn_invalidate", "cke_xattn_is_ready",
            "cke_xattn_populate", "cke_xattn_populate_workspace_bytes", "cke_xattn_populate_ws",
            "cke_memory_lift_workspace_bytes", "cke_memory_lift_gelu_ws",
            "cke_xattn_decode", "cke_selfattn_decode_append",
            "cke_selfattn_prefill_append", "cke_xattn_decode_weights",
            "cke_decoder_step_workspace_bytes", "cke_decoder_layer_step",
            "cke_decoder_step_scratch_bytes", "cke_decoder_layer_step_noalloc",
            "cke_memory_lift_gelu", "cke_weight_planes_bytes", "cke_weight_planes",
            "cke_row_planes_bytes", "cke_xattn_populate_planes", "cke_memory_lift_gelu_planes",
            "cke_memory_lift_planes_workspace_bytes", "cke_xattn_set_merge_mode",
            "cke_xattn_merges_in_launch",
            "cke_last_error", "cke_version"]


class CkeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (status %d)" % (msg, code))
        self.code = code


def lib():
    return _lib


def cke_last_error() -> str:
    return _lib.cke_last_error().decode()


def cke_version() -> str:
    return _lib.cke_version().decode()


def _check(rc: int) -> None:
    if rc != CKE_OK:
        raise CkeError(rc, cke_last_error())


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        if x.numel() and not x.is_contiguous():
            raise ValueError("tensor must be contiguous")
        return x.data_ptr()
    return int(x)


def _meta(name, t, shape=None, dtypes=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor (got %s)" % (name, type(t).__name__))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError("%s must be of dtype %s (got %s)"
                         % (name, " or ".join(str(d) for d in dtypes), t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _devs(*specs):
    """Check (name, tensor, shape, dtypes) specs: every shape, dtype and
    contiguity first, then that each tensor lives on the GPU, before the
    addresses are handed to a kernel (a host address or a short buffer would
    be read or written out of bounds on the GPU). Returns the addresses."""
    for spec in specs:
        _meta(*spec)
    for spec in specs:
        if spec[1].device.type != "cuda":
            raise ValueError("%s must be a device tensor (got device %s)" % (spec[0], spec[1].device))
    return [spec[1].data_ptr() for spec in specs]


def _dev(name, t, shape=None, dtypes=None):
    return _devs((name, t, shape, dtypes))[0]


_F32 = (torch.float32,)
_IN_DTYPES = {CKE_F32: torch.float32, CKE_BF16: torch.bfloat16, CKE_FP8: torch.float8_e4m3fn}


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def make_geom(n_layers, n_streams, mem_len, d_model, n_heads, head_dim, max_q=1,
              cache_dtype=CKE_F32) -> cke_xattn_geom:
    return cke_xattn_geom(n_layers, n_streams, mem_len, d_model, n_heads, head_dim, max_q,
                          cache_dtype)


def cke_xattn_region_bytes(g: cke_xattn_geom) -> int:
    return int(_lib.cke_xattn_region_bytes(ctypes.byref(g)))


def cke_xattn_layer_offset_bytes(g: cke_xattn_geom, layer: int) -> int:
    r = int(_lib.cke_xattn_layer_offset_bytes(ctypes.byref(g), layer))
    if r == ctypes.c_size_t(-1).value:
        raise CkeError(CKE_ERANGE, cke_last_error())
    return r


def cke_xattn_workspace_bytes(g: cke_xattn_geom) -> int:
    return int(_lib.cke_xattn_workspace_bytes(ctypes.byref(g)))


def cke_xattn_num_splits(g: cke_xattn_geom) -> int:
    return int(_lib.cke_xattn_num_splits(ctypes.byref(g)))


def cke_xattn_whole_pairs(g: cke_xattn_geom) -> int:
    return int(_lib.cke_xattn_whole_pairs(ctypes.byref(g)))


def cke_xattn_cache_create(g: cke_xattn_geom, k_dev, v_dev, ws_dev) -> int:
    h = _P()
    _check(_lib.cke_xattn_cache_create(ctypes.byref(g), _ptr(k_dev), _ptr(v_dev), _ptr(ws_dev),
                                       ctypes.byref(h)))
    return h.value


def cke_xattn_cache_destroy(handle) -> None:
    _lib.cke_xattn_cache_destroy(handle)


def cke_xattn_invalidate(handle) -> None:
    _check(_lib.cke_xattn_invalidate(handle))


def cke_xattn_is_ready(handle) -> bool:
    return bool(_lib.cke_xattn_is_ready(handle))


def cke_xattn_set_merge_mode(mode: int) -> int:
    """1: split decodes merge in their own launch where the device allows;
    0: always in a second kernel. Returns the previous mode."""
    rc = _lib.cke_xattn_set_merge_mode(int(mode))
    if rc < 0:
        raise CkeError(rc, cke_last_error())
    return rc


def cke_xattn_merges_in_launch(cache, n_q: int) -> bool:
    return bool(_lib.cke_xattn_merges_in_launch(_handle(cache), int(n_q)))


def _handle(cache):
    return cache.handle if isinstance(cache, XattnCache) else cache


def _geom(cache) -> cke_xattn_geom:
    """Geometry of an XattnCache; the tensor-level wrappers need it to check
    the shapes they hand to the library (raw handles go through lib())."""
    if not isinstance(cache, XattnCache):
        raise TypeError("cache must be an XattnCache (raw handles: call lib() directly)")
    if not cache.handle:
        raise ValueError("cache has been closed")
    return cache.geom


def cke_xattn_populate_workspace_bytes(g: cke_xattn_geom, e_dtype=CKE_F32, w_dtype=CKE_F32) -> int:
    return int(_lib.cke_xattn_populate_workspace_bytes(ctypes.byref(g), int(e_dtype), int(w_dtype)))


def cke_memory_lift_workspace_bytes(rows: int, k_in: int, n: int) -> int:
    return int(_lib.cke_memory_lift_workspace_bytes(int(rows), int(k_in), int(n)))


def cke_weight_planes_bytes(n_mat: int, k: int, n: int) -> int:
    return int(_lib.cke_weight_planes_bytes(int(n_mat), int(k), int(n)))


def cke_row_planes_bytes(rows: int, k: int) -> int:
    return int(_lib.cke_row_planes_bytes(int(rows), int(k)))


def cke_memory_lift_planes_workspace_bytes(rows: int, k_in: int, n: int) -> int:
    return int(_lib.cke_memory_lift_planes_workspace_bytes(int(rows), int(k_in), int(n)))


def _planes(name, t):
    """(address, bytes) of a planes or workspace tensor (device, any dtype)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a device tensor" % name)
    return _dev(name, t), t.numel() * t.element_size()


def cke_weight_planes(W, planes, stream=None) -> None:
    """Split fp32 weights W (a sequence of n_mat device tensors [k][n]) into
    bf16 hi/lo planes in `planes` (a device tensor of at least
    cke_weight_planes_bytes(n_mat, k, n) bytes)."""
    if len(W) < 1:
        raise ValueError("W must hold at least one weight")
    k, n = W[0].shape
    ptrs = _devs(*[("W[%d]" % i, w, (k, n), _F32) for i, w in enumerate(W)])
    p_ptr, p_bytes = _planes("planes", planes)
    arr = (_P * len(W))(*ptrs)
    _check(_lib.cke_weight_planes(arr, len(W), int(k), int(n), p_ptr, p_bytes, _stream(stream)))


def weight_planes(W, stream=None):
    """A new device tensor holding the planes of the fp32 weights W."""
    k, n = W[0].shape
    nbytes = cke_weight_planes_bytes(len(W), k, n)
    if nbytes == 0:
        raise CkeError(CKE_EINVAL, "weights of shape %s x %d take no planes" % ((k, n), len(W)))
    planes = torch.empty(nbytes // 2, dtype=torch.int16, device=W[0].device)
    cke_weight_planes(W, planes, stream)
    return planes


def cke_xattn_populate_planes(cache, E, w_planes, ws, stream=None) -> None:
    """Populate every layer from fp32 E [B][T][d_model] and the prepared
    planes of WK_0..WK_{L-1}, WV_0..WV_{L-1} (cke_weight_planes); E's planes
    go to `ws` (at least cke_row_planes_bytes(B*T, d_model) bytes)."""
    g = _geom(cache)
    e_ptr = _dev("E", E, (g.n_streams, g.mem_len, g.d_model), _F32)
    w_ptr, w_bytes = _planes("w_planes", w_planes)
    ws_ptr, ws_bytes = _planes("ws", ws)
    _check(_lib.cke_xattn_populate_planes(_handle(cache), e_ptr, w_ptr, w_bytes, ws_ptr, ws_bytes,
                                          _stream(stream)))


def cke_memory_lift_gelu_planes(x, w_planes, n, out, ws, pos=None, stream=None) -> None:
    """cke_memory_lift_gelu with the lift weight [k_in][n] prepared by
    cke_weight_planes; x's planes (and the partial sums of a lift split over
    k_in) go to `ws` (at least cke_memory_lift_planes_workspace_bytes(rows,
    k_in, n) bytes)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-d tensor [rows][k_in]")
    rows, k_in = x.shape
    if out.numel() != rows * n:
        raise ValueError("out must hold rows x n = %d elements (got %d)" % (rows * n, out.numel()))
    specs = [("x", x, (rows, k_in), _F32), ("out", out, None, _F32)]
    pos_rows = 0
    if pos is not None:
        if pos.dim() != 2:
            raise ValueError("pos must be a 2-d tensor [pos_rows][n]")
        pos_rows = pos.shape[0]
        specs.append(("pos", pos, (pos_rows, n), _F32))
    ptrs = _devs(*specs)
    w_ptr, w_bytes = _planes("w_planes", w_planes)
    ws_ptr, ws_bytes = _planes("ws", ws)
    _check(_lib.cke_memory_lift_gelu_planes(ptrs[0], int(rows), int(k_in), w_ptr, w_bytes, int(n),
                                            ptrs[2] if pos is not None else None, int(pos_rows),
                                            ptrs[1], ws_ptr, ws_bytes, _stream(stream)))


def _ws(ws):
    """(address, bytes) of an optional workspace tensor."""
    if ws is None:
        return None, 0
    return _dev("ws", ws), ws.numel() * ws.element_size()


def cke_xattn_populate(cache, E, WK, WV, stream=None, e_dtype=None, w_dtype=None, ws=None) -> None:
    """Prefill every layer's K/V slab from encoder memory E [B][T][d_model];
    WK and WV are sequences of L weight tensors [d_model][H*D], one per layer
    of the cache (an XattnCache). With `ws` (a device tensor of at least
    cke_xattn_populate_workspace_bytes bytes) the fp32 path splits its
    operands once into bf16 planes there (cke_xattn_populate_ws)."""
    g = _geom(cache)
    if len(WK) != g.n_layers or len(WV) != g.n_layers:
        raise ValueError("WK and WV must hold one weight per layer: %d each (got %d and %d)"
                         % (g.n_layers, len(WK), len(WV)))
    if e_dtype is None:
        e_dtype = _DTYPES[E.dtype]
    if w_dtype is None:
        w_dtype = _DTYPES[WK[0].dtype]
    wshape, wdt = (g.d_model, g.n_heads * g.head_dim), (_IN_DTYPES[w_dtype],)
    ptrs = _devs(("E", E, (g.n_streams, g.mem_len, g.d_model), (_IN_DTYPES[e_dtype],)),
                 *[("WK[%d]" % i, w, wshape, wdt) for i, w in enumerate(WK)],
                 *[("WV[%d]" % i, w, wshape, wdt) for i, w in enumerate(WV)])
    e_ptr = ptrs[0]
    arr = _P * g.n_layers
    wk = arr(*ptrs[1:1 + g.n_layers])
    wv = arr(*ptrs[1 + g.n_layers:])
    if ws is None:
        _check(_lib.cke_xattn_populate(_handle(cache), e_ptr, e_dtype, wk, wv, w_dtype,
                                       _stream(stream)))
    else:
        ws_ptr, ws_bytes = _ws(ws)
        _check(_lib.cke_xattn_populate_ws(_handle(cache), e_ptr, e_dtype, wk, wv, w_dtype, ws_ptr,
                                          ws_bytes, _stream(stream)))


def _qshape(g, q):
    """(B, n_q, H, D) of a query tensor for the cache geometry g."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-d tensor [B][n_q][H][D]")
    return (g.n_streams, q.shape[1], g.n_heads, g.head_dim)


def cke_xattn_decode(q, cache, layer: int, scale: float, out, n_q=None, stream=None) -> None:
    """Cross-attention of q [B][n_q][H][D] (fp32) against layer `layer` of the
    projection cache (an XattnCache), into out (same shape)."""
    g = _geom(cache)
    shape = _qshape(g, q)
    if n_q is None:
        n_q = shape[1]
    elif int(n_q) > shape[1]:
        raise ValueError("n_q %d exceeds the %d queries q holds" % (n_q, shape[1]))
    q_ptr, out_ptr = _devs(("q", q, shape, _F32), ("out", out, shape, _F32))
    _check(_lib.cke_xattn_decode(q_ptr, int(n_q), _handle(cache), int(layer), float(scale),
                                 out_ptr, _stream(stream)))


def cke_xattn_decode_weights(q, cache, layer: int, scale: float, heads, out, weights,
                             stream=None) -> None:
    """Cross decode plus the softmax weights of the listed heads averaged over
    them: weights [B][n_q][T] fp32. cache is an XattnCache."""
    g = _geom(cache)
    shape = _qshape(g, q)
    q_ptr, out_ptr, w_ptr = _devs(("q", q, shape, _F32), ("out", out, shape, _F32),
                                  ("weights", weights, (g.n_streams, shape[1], g.mem_len), _F32))
    hs = (ctypes.c_int32 * len(heads))(*[int(h) for h in heads])
    _check(_lib.cke_xattn_decode_weights(q_ptr, shape[1], cache.handle, int(layer), float(scale),
                                         hs, len(heads), out_ptr, w_ptr, _stream(stream)))


def _kv(kv):
    if not isinstance(kv, KVLayer):
        raise TypeError("kv must be a KVLayer")
    return kv


def cke_selfattn_prefill_append(q, k_new, v_new, kv, pos: int, n_new: int, n_q_heads: int,
                                scale: float, out, stream=None) -> None:
    """Write rows pos..pos+n_new-1 of kv from k_new/v_new [S][n_new][Hkv][D] and
    attend causally for q [S][n_new][n_q_heads][D] (grouped kv heads)."""
    kv = _kv(kv)
    d = kv.desc
    qshape = (d.n_seqs, int(n_new), int(n_q_heads), d.head_dim)
    kshape = (d.n_seqs, int(n_new), d.n_heads, d.head_dim)
    *ptrs, out_ptr = _devs(("q", q, qshape, _F32), ("k_new", k_new, kshape, _F32),
                           ("v_new", v_new, kshape, _F32), ("out", out, qshape, _F32))
    _check(_lib.cke_selfattn_prefill_append(*ptrs, ctypes.byref(d), int(pos), int(n_new),
                                            int(n_q_heads), float(scale), out_ptr,
                                            _stream(stream)))


def cke_selfattn_decode_append(q, k_new, v_new, kv, pos: int, scale: float, out,
                               stream=None) -> None:
    """Scatter k_new/v_new [S][H][D] into row pos of kv (a KVLayer) and attend
    over rows 0..pos."""
    kv = _kv(kv)
    d = kv.desc
    shape = (d.n_seqs, d.n_heads, d.head_dim)
    *ptrs, out_ptr = _devs(*[(n, t, shape, _F32) for n, t in (("q", q), ("k_new", k_new),
                                                               ("v_new", v_new), ("out", out))])
    _check(_lib.cke_selfattn_decode_append(*ptrs, ctypes.byref(d), int(pos), float(scale),
                                           out_ptr, _stream(stream)))


def cke_decoder_step_workspace_bytes(g: cke_xattn_geom, n_seqs: int) -> int:
    return int(_lib.cke_decoder_step_workspace_bytes(ctypes.byref(g), int(n_seqs)))


def decoder_layer_desc(WQs, WKs, WVs, WOs, WQ, WO) -> cke_decoder_layer:
    """Descriptor of one layer's six [d_model][d_model] device weights, stored
    output-major (row j = output j's input weights, as nn.Linear.weight), one
    dtype, fp32 or bf16. The tensors must outlive every call that uses it."""
    ws = (WQs, WKs, WVs, WOs, WQ, WO)
    dt = {w.dtype for w in ws}
    if len(dt) != 1:
        raise ValueError("decoder weights must share one dtype")
    dt = dt.pop()
    if dt not in (torch.float32, torch.bfloat16):
        raise ValueError("decoder weights must be fp32 or bf16 (got %s)" % dt)
    dm = WQs.shape[0] if WQs.dim() == 2 else -1
    names = ("WQs", "WKs", "WVs", "WOs", "WQ", "WO")
    desc = cke_decoder_layer(*_devs(*[(n, w, (dm, dm)) for n, w in zip(names, ws)]), _DTYPES[dt])
    desc.d_model = dm
    return desc


def cke_decoder_layer_step(x, w, kv, pos: int, cache, layer: int, scale: float, ws,
                           stream=None) -> None:
    """One decoder layer for one token per sequence: x [S][d_model] fp32 is
    updated in place (self-attention residual, then cross-attention residual
    over `cache` slab `layer`); w is a cke_decoder_layer from
    decoder_layer_desc, kv a KVLayer, ws a workspace of
    cke_decoder_step_workspace_bytes bytes."""
    g = _geom(cache)
    d = _kv(kv).desc
    if getattr(w, "d_model", None) != g.d_model:
        raise ValueError("decoder weights must come from decoder_layer_desc with d_model %d"
                         % g.d_model)
    need = cke_decoder_step_workspace_bytes(g, d.n_seqs)
    if isinstance(ws, torch.Tensor) and ws.numel() * ws.element_size() < need:
        raise ValueError("ws holds %d bytes; the step needs %d"
                         % (ws.numel() * ws.element_size(), need))
    x_ptr, ws_ptr = _devs(("x", x, (d.n_seqs, g.d_model), _F32), ("ws", ws, None, None))
    _check(_lib.cke_decoder_layer_step(x_ptr, ctypes.byref(w), ctypes.byref(d), int(pos),
                                       _handle(cache), int(layer), float(scale), ws_ptr,
                                       _stream(stream)))


def cke_decoder_step_scratch_bytes() -> int:
    return int(_lib.cke_decoder_step_scratch_bytes())


def cke_decoder_layer_step_noalloc(x, w, kv, pos: int, cache, layer: int, scale: float,
                                   stream=None) -> None:
    """cke_decoder_layer_step with the step buffers in the library's own
    per-GPU scratch array: no workspace argument, nothing allocated."""
    g = _geom(cache)
    d = _kv(kv).desc
    if getattr(w, "d_model", None) != g.d_model:
        raise ValueError("decoder weights must come from decoder_layer_desc with d_model %d"
                         % g.d_model)
    x_ptr = _dev("x", x, (d.n_seqs, g.d_model), _F32)
    _check(_lib.cke_decoder_layer_step_noalloc(x_ptr, ctypes.byref(w), ctypes.byref(d), int(pos),
                                               _handle(cache), int(layer), float(scale),
                                               _stream(stream)))


def cke_memory_lift_gelu(x, w, out, pos=None, stream=None, ws=None) -> None:
    """out [rows][n] = gelu(x [rows][k_in] . w [k_in][n]) + pos[r % pos_rows]
    (exact GELU; pos [pos_rows][n] or None), all fp32 device tensors (out may
    be any contiguous view of rows x n elements, such as an encoder memory
    [B][T][n]). With `ws` (at least cke_memory_lift_workspace_bytes bytes)
    the operands are split once into bf16 planes there
    (cke_memory_lift_gelu_ws)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or w.dim() != 2:
        raise ValueError("x and w must be 2-d tensors [rows][k_in] and [k_in][n]")
    rows, k_in = x.shape
    n = w.shape[1]
    if out.numel() != rows * n:
        raise ValueError("out must hold rows x n = %d elements (got %d)" % (rows * n, out.numel()))
    specs = [("x", x, (rows, k_in), _F32), ("w", w, (k_in, n), _F32), ("out", out, None, _F32)]
    pos_rows = 0
    if pos is not None:
        if pos.dim() != 2:
            raise ValueError("pos must be a 2-d tensor [pos_rows][n]")
        pos_rows = pos.shape[0]
        specs.append(("pos", pos, (pos_rows, n), _F32))
    ptrs = _devs(*specs)
    x_ptr, w_ptr, out_ptr = ptrs[:3]
    pos_ptr = ptrs[3] if pos is not None else None
    if ws is None:
        _check(_lib.cke_memory_lift_gelu(x_ptr, int(rows), int(k_in), w_ptr, int(n), pos_ptr,
                                         int(pos_rows), out_ptr, _stream(stream)))
    else:
        ws_ptr, ws_bytes = _ws(ws)
        _check(_lib.cke_memory_lift_gelu_ws(x_ptr, int(rows), int(k_in), w_ptr, int(n), pos_ptr,
                                            int(pos_rows), out_ptr, ws_ptr, ws_bytes,
                                            _stream(stream)))


class XattnCache:
    """A projection cache whose K, V and workspace are torch device tensors.

    The tensors are plain device memory handed to the library by pointer; the
    handle holds the geometry and the ready flag."""

    def __init__(self, n_layers, n_streams, mem_len, d_model, n_heads, head_dim, max_q=1,
                 dtype=torch.float32, device="cuda"):
        self.geom = make_geom(n_layers, n_streams, mem_len, d_model, n_heads, head_dim, max_q,
                              _DTYPES[dtype])
        nbytes = cke_xattn_region_bytes(self.geom)
        if nbytes == 0:
            raise CkeError(CKE_EINVAL, cke_last_error())
        shape = (n_layers, n_streams, n_heads, mem_len, head_dim)
        self.k = torch.empty(shape, dtype=dtype, device=device)
        self.v = torch.empty(shape, dtype=dtype, device=device)
        ws_bytes = cke_xattn_workspace_bytes(self.geom)
        self.ws = torch.zeros((ws_bytes + 255) // 256 * 64, dtype=torch.float32, device=device)
        self.handle = cke_xattn_cache_create(self.geom, self.k, self.v, self.ws)
        self.n_splits = cke_xattn_num_splits(self.geom)

    def populate(self, E, WK, WV, stream=None, ws=None):
        cke_xattn_populate(self, E, WK, WV, stream, ws=ws)

    def weight_planes(self, WK, WV, stream=None):
        """The prepared planes of this geometry's fp32 weights (one device
        tensor; call once per set of weights)."""
        return weight_planes(list(WK) + list(WV), stream)

    def populate_planes(self, E, w_planes, ws, stream=None):
        cke_xattn_populate_planes(self, E, w_planes, ws, stream)

    def row_planes_workspace(self, device="cuda"):
        """A device workspace for populate_planes (E's planes)."""
        n = cke_row_planes_bytes(self.geom.n_streams * self.geom.mem_len, self.geom.d_model)
        if n == 0:
            raise CkeError(CKE_EINVAL, "this geometry takes no planes")
        return torch.empty((n + 3) // 4, dtype=torch.float32, device=device)

    def populate_workspace(self, device="cuda"):
        """A device workspace for populate(..., ws=) of fp32 inputs, or None
        when the geometry takes none."""
        n = cke_xattn_populate_workspace_bytes(self.geom)
        return torch.empty((n + 3) // 4, dtype=torch.float32, device=device) if n else None

    def decode(self, q, layer, scale, out=None, stream=None):
        if out is None:
            out = torch.empty_like(q)
        cke_xattn_decode(q, self, layer, scale, out, stream=stream)
        return out

    def decode_weights(self, q, layer, scale, heads, out=None, weights=None, stream=None):
        """(out, weights): decode output and the listed heads' mean attention
        weights [B][n_q][T]."""
        if out is None:
            out = torch.empty_like(q)
        if weights is None:
            weights = torch.empty(q.shape[0], q.shape[1], self.geom.mem_len, dtype=torch.float32,
                                  device=q.device)
        cke_xattn_decode_weights(q, self, layer, scale, heads, out, weights, stream)
        return out, weights

    def invalidate(self):
        cke_xattn_invalidate(self.handle)

    @property
    def ready(self) -> bool:
        return cke_xattn_is_ready(self.handle)

    def close(self):
        if getattr(self, "handle", None):
            cke_xattn_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class KVLayer:
    """One layer's self-attention cache [S][H][max_pos][D] as torch tensors.

    With k and v given, their shape and dtype describe the cache (they must
    agree with each other and with any explicit arguments)."""

    def __init__(self, n_seqs=None, n_heads=None, head_dim=None, max_pos=None, dtype=None,
                 device="cuda", k=None, v=None):
        if (k is None) != (v is None):
            raise ValueError("give both k and v, or neither")
        if k is None:
            dtype = torch.float32 if dtype is None else dtype
            shape = (n_seqs, n_heads, max_pos, head_dim)
            self.k = torch.zeros(shape, dtype=dtype, device=device)
            self.v = torch.zeros(shape, dtype=dtype, device=device)
        else:
            if k.dim() != 4 or k.shape != v.shape or k.dtype != v.dtype:
                raise ValueError("k and v must be 4-d tensors [S][H][max_pos][D] of one shape "
                                 "and dtype")
            want = (n_seqs, n_heads, max_pos, head_dim)
            for name, a, b in zip(("n_seqs", "n_heads", "max_pos", "head_dim"), want, k.shape):
                if a is not None and a != b:
                    raise ValueError("%s %d disagrees with k's shape %s" % (name, a, tuple(k.shape)))
            if dtype is not None and dtype != k.dtype:
                raise ValueError("dtype %s disagrees with k's dtype %s" % (dtype, k.dtype))
            _devs(("k", k, None, (torch.float32, torch.bfloat16)),
                  ("v", v, None, (torch.float32, torch.bfloat16)))
            self.k, self.v = k, v
        n_seqs, n_heads, max_pos, head_dim = self.k.shape
        self.desc = cke_kv_layer(self.k.data_ptr(), self.v.data_ptr(), n_seqs, n_heads, head_dim,
                                 max_pos, _DTYPES[self.k.dtype])

    def append_attend(self, q, k_new, v_new, pos, scale, out=None, stream=None):
        if out is None:
            out = torch.empty_like(q)
        cke_selfattn_decode_append(q, k_new, v_new, self, pos, scale, out, stream)
        return out

    def prefill_attend(self, q, k_new, v_new, pos, scale, out=None, stream=None):
        """q [S][n][Hq][D], k_new/v_new [S][n][H][D]; Hq a multiple of H."""
        if out is None:
            out = torch.empty_like(q)
        cke_selfattn_prefill_append(q, k_new, v_new, self, pos, q.shape[1], q.shape[2], scale, out,
                                    stream)
        return out
