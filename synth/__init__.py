"""Seeded synthetic inputs for the cross-attention projection-cache workloads.

This module only draws random numbers and describes workload geometry. It holds
none of the method's arithmetic (no projection, no attention, no softmax): both
the oracle tests and the HIP path take their inputs from here, and nothing else
is shared between them.

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence(key))`` where
``key = [config_seed, tensor_id, *indices]``. Values are drawn as float64
standard normals, multiplied by the tensor's standard deviation and rounded to
float32 (round-to-nearest-even, numpy's cast). Tensors that a workload stores in
bfloat16 are rounded once more, float32 -> bfloat16, round-to-nearest-even, and
handed out as the raw 16-bit patterns (``uint16``) together with their exact
float32 value.

Geometry follows the pages:
  * C-Kernel-Engine, "Whisper: Trace One Encoder Tensor into Every Decoder
    Layer", section "The concept": encoder memory E is [1500, 512] fp32 for
    Whisper Base and every one of the 6 decoder layers owns WK/WV.
  * same page, "View 2": 8 heads, head_dim 64, 1500 key tokens, scale 0.125.
  * WhisperKit case study, section 4: self-attention cache capacity 448.
  * transcribe.cpp granite_nar forward map, "Projector": 2 layers, 32 heads x 64,
    blocks of 15 frames, 3 queries per block; the memory comes from a 4096 -> 2048
    lift of the encoder concat (X_lift, W_lift) plus window positions (pos).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Geometry", "CONFIGS", "get", "normal", "to_bf16_bits", "bf16_bits_to_f32",
    "workload_tensors", "decode_call_inputs", "q_std",
]


@dataclasses.dataclass(frozen=True)
class Geometry:
    name: str
    n_streams: int      # B: independent encoder memories / cross caches
    n_q: int            # queries per stream in one cross-attention call
    n_seqs: int         # S: self-attention sequences (0 = no self-attention)
    n_layers: int       # L
    mem_len: int        # T: encoder memory rows per stream
    d_model: int
    n_heads: int        # H
    head_dim: int       # D
    scale: float
    dtype: str          # cache storage type: "f32", "bf16" or "fp8" (E/W are bf16 for
                        # both of the latter, fp32 for "f32")
    steps: int          # decode steps in one window
    max_pos: int        # self-attention cache capacity
    seed: int
    e_std: float = 1.0
    w_std: float = 0.02
    lift_in: int = 0    # projector memory lift input width (0: E is drawn directly)

    @property
    def hd(self) -> int:
        return self.n_heads * self.head_dim


CONFIGS = {
    "tiny": Geometry("tiny", 1, 1, 1, 1, 64, 64, 2, 32, 1.0 / math.sqrt(32.0),
                     "f32", 8, 8, 0),
    "base": Geometry("base", 1, 1, 1, 6, 1500, 512, 8, 64, 0.125,
                     "f32", 224, 448, 1),
    "beam": Geometry("beam", 1, 5, 5, 6, 1500, 512, 8, 64, 0.125,
                     "f32", 448, 448, 2),
    "large": Geometry("large", 16, 1, 16, 32, 1500, 1280, 20, 64, 0.125,
                      "bf16", 128, 448, 3),
    "qformer": Geometry("qformer", 100, 3, 0, 2, 15, 2048, 32, 64, 0.125,
                        "f32", 1, 0, 4, lift_in=4096),
    # the Large workload over an 8-bit (E4M3) projection cache, same inputs
    "large_fp8": Geometry("large_fp8", 16, 1, 16, 32, 1500, 1280, 20, 64, 0.125,
                          "fp8", 128, 448, 3),
}

# Fixed enumeration of tensor kinds; part of every seed key.
TENSOR_IDS = {
    "E": 0, "WK": 1, "WV": 2, "WQ": 3, "WO": 4,
    "WQs": 5, "WKs": 6, "WVs": 7, "WOs": 8, "x0": 9,
    "q_cross": 10, "q_self": 11, "k_new": 12, "v_new": 13,
    "X_lift": 14, "W_lift": 15, "pos": 16,
    "custom": 99,
}


def get(name: str) -> Geometry:
    return CONFIGS[name]


def _rng(key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def normal(key, shape, std: float = 1.0) -> np.ndarray:
    """float32 array of N(0, std^2) draws for the integer seed ``key``."""
    x = _rng(key).standard_normal(size=shape, dtype=np.float64)
    if std != 1.0:
        x *= std
    return x.astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    Input preparation only (finite values); returns uint16.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def q_std(g: Geometry) -> float:
    """Spread of a projected query/key row: x has unit RMS and W entries have
    std w_std, so each output entry has std w_std * sqrt(d_model)."""
    return g.w_std * math.sqrt(g.d_model)


def workload_tensors(g: Geometry, which=("E", "WK", "WV")) -> dict:
    """Encoder memory and per-layer weights of a workload.

    Returns float32 arrays (exact values) and, for bf16 and fp8 workloads
    (bf16 inputs), the bf16 bit patterns under the key ``name + "_bits"``. E
    is [B][T][d_model]; each weight is a list of L arrays [d_model][H*D]
    (y = x . W orientation). For those workloads the float32 arrays hold the
    bf16-rounded values.
    """
    out = {}
    seed = g.seed
    for name in which:
        tid = TENSOR_IDS[name]
        if name == "E":
            a = normal([seed, tid], (g.n_streams, g.mem_len, g.d_model), g.e_std)
            out[name] = a
        elif name == "x0":
            n = max(g.n_seqs, 1)
            out[name] = normal([seed, tid], (n, g.d_model), 1.0)
            continue
        elif name == "X_lift":   # stands in for the normalised 4-way encoder concat
            out[name] = normal([seed, tid], (g.n_streams * g.mem_len, g.lift_in), 1.0)
            continue
        elif name == "W_lift":
            out[name] = normal([seed, tid], (g.lift_in, g.d_model), g.w_std)
            continue
        elif name == "pos":      # window position embedding, one row per frame of a block
            out[name] = normal([seed, tid], (g.mem_len, g.d_model), 0.02)
            continue
        else:
            out[name] = [normal([seed, tid, l], (g.d_model, g.hd), g.w_std)
                         for l in range(g.n_layers)]
        if g.dtype in ("bf16", "fp8"):
            if name == "E":
                bits = to_bf16_bits(out[name])
                out[name + "_bits"] = bits
                out[name] = bf16_bits_to_f32(bits)
            else:
                bits = [to_bf16_bits(w) for w in out[name]]
                out[name + "_bits"] = bits
                out[name] = [bf16_bits_to_f32(b) for b in bits]
    return out


def decode_call_inputs(g: Geometry, step: int, layer: int) -> dict:
    """Per-call inputs of one decode step at one layer, drawn independently.

    q_cross is [B][n_q][H][D]; q_self, k_new, v_new are [S][H][D]. All float32
    with the spread of a projected unit-RMS row (q_std).
    """
    s = q_std(g)
    seed = g.seed
    out = {"q_cross": normal([seed, TENSOR_IDS["q_cross"], step, layer],
                             (g.n_streams, g.n_q, g.n_heads, g.head_dim), s)}
    if g.n_seqs > 0:
        for name in ("q_self", "k_new", "v_new"):
            out[name] = normal([seed, TENSOR_IDS[name], step, layer],
                               (g.n_seqs, g.n_heads, g.head_dim), s)
    return out
