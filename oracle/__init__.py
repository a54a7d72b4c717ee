"""Plain CPU oracle (fp64, naive loops) for the cross-attention projection cache.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers. The product library never
imports this package, and this package never imports the product library.

The arithmetic lives in ``oracle.c`` (built with gcc, -ffp-contract=off, no
fast-math). This module builds it and marshals numpy arrays; it computes
nothing itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "liborc.so")

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-Wall", "-Wextra", "-Werror"]

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into oracle/_build/liborc.so (always, when force)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    os.makedirs(_BUILD, exist_ok=True)
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_D = ctypes.c_double
_I = ctypes.c_int
_P = ctypes.c_void_p
_SZ = ctypes.c_size_t


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_round_bf16.restype = _D
        L.orc_round_bf16.argtypes = [_D]
        L.orc_round_bf16_array.argtypes = [_P, _P, _SZ]
        L.orc_round_fp8.restype = _D
        L.orc_round_fp8.argtypes = [_D]
        L.orc_round_fp8_array.argtypes = [_P, _P, _SZ]
        L.orc_project_head.argtypes = [_I, _I, _I, _P, _P, _I, _I, _I, _P]
        L.orc_populate.argtypes = [_I] * 6 + [_P, _P, _P, _I, _P, _P]
        L.orc_layer_offset_bytes.restype = _SZ
        L.orc_layer_offset_bytes.argtypes = [_I] * 6
        L.orc_attend.argtypes = [_I, _I, _D, _P, _P, _P, _P]
        L.orc_cross_decode.argtypes = [_I] * 5 + [_D, _P, _P, _P, _P]
        L.orc_self_append_attend.argtypes = [_I] * 5 + [_D, _I] + [_P] * 6
        L.orc_kv_blend_update.argtypes = [_I] * 5 + [_P, _P]
        L.orc_self_prefill_append.argtypes = [_I] * 7 + [_D, _I] + [_P] * 6
        L.orc_cross_decode_weights.argtypes = [_I] * 5 + [_D, _P, _P, _P, _P, _I, _P, _P]
        L.orc_matvec.argtypes = [_I, _I, _P, _P, _P]
        L.orc_rms_feedback.argtypes = [_I, _P, _P]
        L.orc_lift_gelu.argtypes = [_I, _I, _I, _P, _P, _P, _I, _P]
        L.orc_gelu.restype = _D
        L.orc_gelu.argtypes = [_D]
        L.orc_decoder_layer_step.restype = _I
        L.orc_decoder_layer_step.argtypes = [_I] * 8 + [_D, _I] + [_P] * 17
        L.orc_decoder_run.restype = _I
        L.orc_decoder_run.argtypes = ([_I] * 10 + [_D, _I] + [_P] * 10 +
                                      [_P] * 7 + [_P] * 4)
        L.orc_set_threads.argtypes = [_I]
        L.orc_get_threads.restype = _I
        _lib = L
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


def round_bf16(x) -> np.ndarray:
    """Round every element to the nearest bfloat16 value (ties to even)."""
    a = _f64(x)
    y = np.empty_like(a)
    lib().orc_round_bf16_array(_ptr(a), _ptr(y), a.size)
    return y


def round_fp8(x) -> np.ndarray:
    """Clamp to [-448, 448], then round to the nearest fp8 e4m3 value (ties
    to even)."""
    a = _f64(x)
    y = np.empty_like(a)
    lib().orc_round_fp8_array(_ptr(a), _ptr(y), a.size)
    return y


def _round_mode(round_bf16: bool, round_fp8: bool) -> int:
    assert not (round_bf16 and round_fp8)
    return 1 if round_bf16 else (2 if round_fp8 else 0)


def project_head(E_b, W, col0: int, D: int, round_bf16: bool = False,
                 round_fp8: bool = False) -> np.ndarray:
    """One head's projection slab [T][D] of E_b [T][dm] by W [dm][ldw]."""
    E_b, W = _f64(E_b), _f64(W)
    T, dm = E_b.shape
    out = np.empty((T, D), dtype=np.float64)
    lib().orc_project_head(T, dm, D, _ptr(E_b), _ptr(W), W.shape[1], col0,
                           _round_mode(round_bf16, round_fp8), _ptr(out))
    return out


def populate(E, WK, WV, H: int, D: int, round_bf16: bool = False, round_fp8: bool = False):
    """Projection caches (Kc, Vc), each [L][B][H][T][D], from E [B][T][dm]
    and per-layer weights WK, WV (sequences of [dm][H*D]); stored values
    rounded to bfloat16 or to fp8 e4m3 when asked."""
    E = _f64(E)
    WK = _f64(np.stack(list(WK)))
    WV = _f64(np.stack(list(WV)))
    B, T, dm = E.shape
    L = WK.shape[0]
    Kc = np.empty((L, B, H, T, D), dtype=np.float64)
    Vc = np.empty_like(Kc)
    lib().orc_populate(L, B, T, dm, H, D, _ptr(E), _ptr(WK), _ptr(WV),
                       _round_mode(round_bf16, round_fp8), _ptr(Kc), _ptr(Vc))
    return Kc, Vc


def layer_offset_bytes(layer, B, H, T, D, elem_bytes) -> int:
    return int(lib().orc_layer_offset_bytes(layer, B, H, T, D, elem_bytes))


def attend(q, K, V, scale: float) -> np.ndarray:
    """Softmax attention of one query q [D] over rows K, V [n][D]."""
    q, K, V = _f64(q), _f64(K), _f64(V)
    n, D = K.shape
    out = np.empty(D, dtype=np.float64)
    lib().orc_attend(n, D, float(scale), _ptr(q), _ptr(K), _ptr(V), _ptr(out))
    return out


def cross_decode(q, Kc_l, Vc_l, scale: float) -> np.ndarray:
    """q [B][nq][H][D] against one layer's slab Kc_l, Vc_l [B][H][T][D]."""
    q, Kc_l, Vc_l = _f64(q), _f64(Kc_l), _f64(Vc_l)
    B, nq, H, D = q.shape
    T = Kc_l.shape[2]
    out = np.empty_like(q)
    lib().orc_cross_decode(B, nq, H, T, D, float(scale), _ptr(q), _ptr(Kc_l),
                           _ptr(Vc_l), _ptr(out))
    return out


def cross_decode_weights(q, Kc_l, Vc_l, scale: float, heads):
    """cross_decode plus the softmax weights of the heads listed in ``heads``,
    averaged over them: returns (out [B][nq][H][D], weights [B][nq][T])."""
    q, Kc_l, Vc_l = _f64(q), _f64(Kc_l), _f64(Vc_l)
    B, nq, H, D = q.shape
    T = Kc_l.shape[2]
    hs = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    assert hs.ndim == 1 and len(hs) >= 1 and (hs >= 0).all() and (hs < H).all()
    out = np.empty_like(q)
    w = np.empty((B, nq, T), dtype=np.float64)
    lib().orc_cross_decode_weights(B, nq, H, T, D, float(scale), _ptr(q), _ptr(Kc_l),
                                   _ptr(Vc_l), hs.ctypes.data_as(ctypes.c_void_p), len(hs),
                                   _ptr(out), _ptr(w))
    return out, w


def self_append_attend(q, k_new, v_new, Ks, Vs, pos: int, scale: float,
                       round_bf16: bool = False) -> np.ndarray:
    """Scatter row ``pos`` of Ks, Vs [S][H][max_pos][D] (float64 arrays,
    updated in place) and attend over rows 0..pos. q, k_new, v_new: [S][H][D]."""
    q, k_new, v_new = _f64(q), _f64(k_new), _f64(v_new)
    assert Ks.dtype == np.float64 and Ks.flags.c_contiguous
    assert Vs.dtype == np.float64 and Vs.flags.c_contiguous
    S, H, max_pos, D = Ks.shape
    out = np.empty_like(q)
    lib().orc_self_append_attend(S, H, D, max_pos, int(pos), float(scale),
                                 int(round_bf16), _ptr(q), _ptr(k_new),
                                 _ptr(v_new), _ptr(Ks), _ptr(Vs), _ptr(out))
    return out


def self_prefill_append(q, k_new, v_new, Ks, Vs, pos: int, scale: float,
                        round_bf16: bool = False) -> np.ndarray:
    """Write rows pos .. pos+n-1 of Ks, Vs [S][Hkv][max_pos][D] (float64,
    updated in place) and attend causally. q [S][n][Hq][D], k_new and v_new
    [S][n][Hkv][D]; Hq a multiple of Hkv (grouped heads). Returns [S][n][Hq][D]."""
    q, k_new, v_new = _f64(q), _f64(k_new), _f64(v_new)
    assert Ks.dtype == np.float64 and Ks.flags.c_contiguous
    assert Vs.dtype == np.float64 and Vs.flags.c_contiguous
    S, Hkv, max_pos, D = Ks.shape
    n, Hq = q.shape[1], q.shape[2]
    assert q.shape == (S, n, Hq, D) and k_new.shape == (S, n, Hkv, D) == v_new.shape
    assert Hq % Hkv == 0 and 0 <= pos and pos + n <= max_pos
    out = np.empty_like(q)
    lib().orc_self_prefill_append(S, n, Hq, Hkv, D, max_pos, int(pos), float(scale),
                                  int(round_bf16), _ptr(q), _ptr(k_new), _ptr(v_new),
                                  _ptr(Ks), _ptr(Vs), _ptr(out))
    return out


def kv_blend_update(cache, cur, pos: int) -> None:
    """One-hot masked blend of cur [S][H][D] into cache [S][H][max_pos][D]."""
    cur = _f64(cur)
    assert cache.dtype == np.float64 and cache.flags.c_contiguous
    S, H, max_pos, D = cache.shape
    lib().orc_kv_blend_update(S, H, D, max_pos, int(pos), _ptr(cur), _ptr(cache))


def matvec(x, W) -> np.ndarray:
    x, W = _f64(x), _f64(W)
    y = np.empty(W.shape[1], dtype=np.float64)
    lib().orc_matvec(W.shape[0], W.shape[1], _ptr(x), _ptr(W), _ptr(y))
    return y


def lift_gelu(x, W, pos=None) -> np.ndarray:
    """Projector memory: gelu(x . W) (exact erf GELU) plus the window positions
    pos [pos_rows][n] broadcast over blocks of pos_rows rows; x [rows][k_in],
    W [k_in][n]."""
    x, W = _f64(x), _f64(W)
    rows, k_in = x.shape
    n = W.shape[1]
    out = np.empty((rows, n), dtype=np.float64)
    if pos is None:
        lib().orc_lift_gelu(rows, k_in, n, _ptr(x), _ptr(W), None, 1, _ptr(out))
    else:
        pos = _f64(pos)
        lib().orc_lift_gelu(rows, k_in, n, _ptr(x), _ptr(W), _ptr(pos), pos.shape[0], _ptr(out))
    return out


def gelu(v: float) -> float:
    return float(lib().orc_gelu(float(v)))


def decoder_layer_step(x, W: dict, Kc, Vc, Ks, Vs, pos: int, *, n_q: int, scale: float,
                       round_bf16: bool = False, records: bool = False):
    """One harness-decoder layer for one token of each of S sequences.

    x [S][dm] (returned updated, the input is not modified); W holds this
    layer's [dm][dm] weights under WQs, WKs, WVs, WOs, WQ, WO; Kc, Vc are the
    layer's projection-cache slab [B][H][T][D] (sequence s reads stream
    s // n_q); Ks, Vs [S][H][max_pos][D] are this layer's self caches,
    updated in place (row pos written, rounded to bf16 if asked). With
    records, also returns the per-call values (qs, kn, vn, so, qc, co).
    """
    x = _f64(x).copy()
    S, dm = x.shape
    Kc, Vc = _f64(Kc), _f64(Vc)
    B, H, T, D = Kc.shape
    assert Ks.dtype == np.float64 and Ks.flags.c_contiguous and Vs.flags.c_contiguous
    max_pos = Ks.shape[2]
    Ws = [_f64(W[k]) for k in ("WQs", "WKs", "WVs", "WOs", "WQ", "WO")]
    rec = {k: np.zeros((S, dm)) for k in ("qs", "kn", "vn", "so", "qc", "co")}
    rc = lib().orc_decoder_layer_step(S, n_q, T, dm, H, D, max_pos, int(pos), float(scale),
                                      int(round_bf16), _ptr(x), *[_ptr(w) for w in Ws],
                                      _ptr(Kc), _ptr(Vc), _ptr(Ks), _ptr(Vs),
                                      *[_ptr(rec[k]) for k in ("qs", "kn", "vn", "so", "qc", "co")])
    if rc != 0:
        raise ValueError("orc_decoder_layer_step rejected its geometry")
    return (x, rec) if records else x


def decoder_run(mode: str, E, W: dict, x0, *, n_heads: int, head_dim: int,
                n_q: int, max_pos: int, n_steps: int, scale: float,
                round_bf16: bool = False) -> dict:
    """Run the harness decoder for n_steps. mode is "incremental" (projection
    cache + appended self cache) or "full" (whole-window recompute each step).

    W holds lists of L [dm][dm] arrays under WK, WV, WQ, WO, WQs, WKs, WVs, WOs.
    Returns per-call records [n_steps][L][S][dm], the token inputs
    x [n_steps+1][S][dm] and the caches.
    """
    E = _f64(E)
    B, T, dm = E.shape
    Ws = {k: _f64(np.stack(list(W[k]))) for k in
          ("WK", "WV", "WQ", "WO", "WQs", "WKs", "WVs", "WOs")}
    L = Ws["WK"].shape[0]
    S = B * n_q
    H, D = n_heads, head_dim
    x0 = _f64(x0).reshape(S, dm)
    rec = {k: np.zeros((n_steps, L, S, dm)) for k in
           ("qs", "kn", "vn", "so", "qc", "co")}
    x_seq = np.zeros((n_steps + 1, S, dm))
    Kc = np.zeros((L, B, H, T, D))
    Vc = np.zeros_like(Kc)
    Ks = np.zeros((L, S, H, max_pos, D))
    Vs = np.zeros_like(Ks)
    rc = lib().orc_decoder_run(
        0 if mode == "incremental" else 1, L, B, n_q, T, dm, H, D, max_pos,
        n_steps, float(scale), int(round_bf16), _ptr(E),
        *[_ptr(Ws[k]) for k in ("WK", "WV", "WQ", "WO", "WQs", "WKs", "WVs", "WOs")],
        _ptr(x0), *[_ptr(rec[k]) for k in ("qs", "kn", "vn", "so", "qc", "co")],
        _ptr(x_seq), _ptr(Kc), _ptr(Vc), _ptr(Ks), _ptr(Vs))
    if rc != 0:
        raise ValueError("orc_decoder_run rejected its geometry")
    return {"rec": rec, "x": x_seq, "Kc": Kc, "Vc": Vc, "Ks": Ks, "Vs": Vs}
