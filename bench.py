#!/usr/bin/env python3
"""Benchmark: cross-attention projection cache on one MI355X.

One step = one decode window of the workload, i.e. one pass of the whole hot
path over one batch of synthetic input:
  populate the projection cache of every decoder layer from E, then
  for every decode token, for every layer in order:
      fused self-attention append + attend (cke_selfattn_decode_append)
      cross-attention over the layer's cache slab (cke_xattn_decode)
The per-call inputs (queries, new K/V rows) are seeded synthetic tensors,
resident in device memory before timing starts.

value = decode tokens per second over the timed windows (tokens of all
sequences, populate included in the time), each window replayed as one HIP
graph. Per-call durations come from three more graphs captured from the same
window, each holding only one kind of call (all populate, all self-attention
or all cross-attention calls of the window, same inputs, same order, same
stream; a window with fewer than 32 calls of a kind is repeated up to 32),
timed with HIP events around their replay: graph-dispatched kernels run back
to back, so replay time / calls is the kernels' own duration (rocprofv3
kernel durations agree to a few percent).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "decode tokens/s (cross+self attn, all layers) + populate TFLOP/s, % roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}

WORKLOAD_TEXT = {
    "base": "whisper-base cross+self decode: E[1500,512] fp32, 6 layers, 8 heads x 64, "
            "batch 1, populate + 224 decode steps, self cache capacity 448",
    "beam": "whisper-base 5-beam decode: shared E[1500,512] fp32 cache, 5 self caches, "
            "6 layers, 8 heads x 64, populate + 448 decode steps",
    "large": "large: 16 streams x E[1500,1280] bf16, 32 layers, 20 heads x 64, "
             "populate + 128 decode steps, bf16 caches, fp32 accumulate",
    "large_fp8": "large over an fp8 cache: 16 streams x E[1500,1280] bf16, 32 layers, "
                 "20 heads x 64, populate + 128 decode steps, fp8 E4M3 projection cache, "
                 "bf16 self caches, fp32 accumulate",
    "qformer": "q-former projector cross-attn: 1500 x 4096 encoder concat lifted to 2048 "
               "(exact GELU, window positions), 100 blocks x 15 frames, 2 layers, 32 heads x 64, "
               "3 queries per block, one pass",
    "tiny": "tiny: E[64,64] fp32, 1 layer, 2 heads x 32, 8 decode steps",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="base", choices=sorted(synth.CONFIGS))
    ap.add_argument("--mode", default="graph", choices=["graph", "eager"])
    ap.add_argument("--also", default="large,beam,qformer",
                    help="comma-separated workloads measured after the headline one and "
                         "reported under 'also' (their windows and rooflines, no extras); "
                         "'none' for none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the headline workload's other entry points (attention weights, decoder "
                         "step, prefill, MALL-cold decode, launch floor): a kernel trace of such a run "
                         "holds only the timed windows and the per-kind graphs")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    ap.add_argument("--counters", action="store_true",
                    help="only run --steps windows with eager launches and no graph capture "
                         "(the mode hardware-counter passes use)")
    ap.add_argument("--counter-tokens", type=int, default=None,
                    help="with --counters: stop each window after this many decode steps "
                         "(every call of a kind moves the same bytes, so a few suffice)")
    return ap.parse_args()


class Workload:
    """Device-resident inputs, caches and outputs of one workload."""

    def __init__(self, name, torch, pc):
        self.torch, self.pc = torch, pc
        g = self.g = synth.get(name)
        dev = "cuda:0"
        self.bf16 = g.dtype in ("bf16", "fp8")      # bf16 E, W and self caches
        self.cache_elem = {"f32": 4, "bf16": 2, "fp8": 1}[g.dtype]
        wt = synth.workload_tensors(g)

        def dev_f32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

        def dev_bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
                torch.bfloat16).to(dev)

        if self.bf16:
            self.E = dev_bf16(wt["E_bits"])
            self.WK = [dev_bf16(b) for b in wt["WK_bits"]]
            self.WV = [dev_bf16(b) for b in wt["WV_bits"]]
        else:
            self.E = dev_f32(wt["E"])
            self.WK = [dev_f32(w) for w in wt["WK"]]
            self.WV = [dev_f32(w) for w in wt["WV"]]
        del wt
        # a projector memory (Q-Former): E is produced in the window by the
        # lift gelu(X_lift . W_lift) + window positions, then populated
        self.lift = None
        if g.lift_in:
            lt = synth.workload_tensors(g, ("X_lift", "W_lift", "pos"))
            self.lift = {k: dev_f32(v) for k, v in lt.items()}
            del lt
        cdt = {"f32": torch.float32, "bf16": torch.bfloat16,
               "fp8": torch.float8_e4m3fn}[g.dtype]
        sdt = torch.bfloat16 if self.bf16 else torch.float32
        self.cache = pc.XattnCache(g.n_layers, g.n_streams, g.mem_len, g.d_model, g.n_heads,
                                   g.head_dim, max_q=g.n_q, dtype=cdt)
        self.kv = [pc.KVLayer(g.n_seqs, g.n_heads, g.head_dim, g.max_pos, dtype=sdt)
                   for _ in range(g.n_layers)] if g.n_seqs else []
        # fp32 inputs: workspace in which populate (and the lift) split their
        # operands into bf16 planes once per call (allocated here, outside
        # the timed windows; None where the library takes none)
        self.pop_ws = self.cache.populate_workspace()
        self.lift_ws = None
        if self.lift is not None:
            n = pc.cke_memory_lift_workspace_bytes(g.n_streams * g.mem_len, g.lift_in, g.d_model)
            self.lift_ws = torch.empty((n + 3) // 4, device=dev) if n else None
        # the weights are the same for every window: where the planes path
        # applies they are split once here, as a deployment does after
        # loading them, and each window splits only its own E (and lift
        # input). The per-call split is measured beside it.
        self.w_planes = self.e_ws = self.lift_planes = self.lift_rws = None
        if self.pop_ws is not None:
            self.w_planes = self.cache.weight_planes(self.WK, self.WV)
            self.e_ws = self.cache.row_planes_workspace()
        if self.lift_ws is not None:
            self.lift_planes = pc.weight_planes([self.lift["W_lift"]])
            n = pc.cke_memory_lift_planes_workspace_bytes(g.n_streams * g.mem_len, g.lift_in,
                                                         g.d_model)
            self.lift_rws = torch.empty((n + 3) // 4, device=dev)
        # per-call inputs [steps][L][...]
        steps, L = g.steps, g.n_layers
        qc = np.empty((steps, L, g.n_streams, g.n_q, g.n_heads, g.head_dim), np.float32)
        if g.n_seqs:
            qs = np.empty((steps, L, g.n_seqs, g.n_heads, g.head_dim), np.float32)
            kn, vn = np.empty_like(qs), np.empty_like(qs)
        for t in range(steps):
            for l in range(L):
                d = synth.decode_call_inputs(g, t, l)
                qc[t, l] = d["q_cross"]
                if g.n_seqs:
                    qs[t, l], kn[t, l], vn[t, l] = d["q_self"], d["k_new"], d["v_new"]
        self.qc = dev_f32(qc)
        self.out_c = torch.empty_like(self.qc)
        if g.n_seqs:
            self.qs, self.kn, self.vn = dev_f32(qs), dev_f32(kn), dev_f32(vn)
            self.out_s = torch.empty_like(self.qs)
        torch.cuda.synchronize()

    @property
    def tokens_per_window(self):
        g = self.g
        return g.steps * (g.n_seqs if g.n_seqs else g.n_streams * g.n_q)

    def window(self, stream, kinds=("populate", "selfattn", "xattn_decode"), tokens=None):
        """Enqueue one decode window on `stream`, or only the calls of the
        given kinds (in window order); `tokens` cuts it after that many decode
        steps (counter runs only)."""
        g, pc = self.g, self.pc
        if "populate" in kinds:
            if self.lift_planes is not None:
                pc.cke_memory_lift_gelu_planes(self.lift["X_lift"], self.lift_planes, g.d_model,
                                               self.E.view(-1, g.d_model), self.lift_rws,
                                               pos=self.lift["pos"], stream=stream)
            elif self.lift is not None:
                pc.cke_memory_lift_gelu(self.lift["X_lift"], self.lift["W_lift"],
                                        self.E.view(-1, g.d_model), self.lift["pos"],
                                        stream=stream, ws=self.lift_ws)
            if self.w_planes is not None:
                pc.cke_xattn_populate_planes(self.cache, self.E, self.w_planes, self.e_ws,
                                             stream=stream)
            else:
                pc.cke_xattn_populate(self.cache, self.E, self.WK, self.WV, stream=stream,
                                      ws=self.pop_ws)
        if "populate_split_weights" in kinds:
            # the same populate with the weights split inside every call
            if self.lift is not None:
                pc.cke_memory_lift_gelu(self.lift["X_lift"], self.lift["W_lift"],
                                        self.E.view(-1, g.d_model), self.lift["pos"],
                                        stream=stream, ws=self.lift_ws)
            pc.cke_xattn_populate(self.cache, self.E, self.WK, self.WV, stream=stream,
                                  ws=self.pop_ws)
        for t in range(g.steps if tokens is None else min(tokens, g.steps)):
            for l in range(g.n_layers):
                if g.n_seqs and "selfattn" in kinds:
                    pc.cke_selfattn_decode_append(self.qs[t, l], self.kn[t, l], self.vn[t, l],
                                                  self.kv[l], t, g.scale, self.out_s[t, l],
                                                  stream=stream)
                if "xattn_decode" in kinds:
                    pc.cke_xattn_decode(self.qc[t, l], self.cache, l, g.scale, self.out_c[t, l],
                                        stream=stream)

    def calls(self, kind):
        g = self.g
        if kind in ("populate", "populate_split_weights"):
            return 1
        if kind == "selfattn":
            return g.steps * g.n_layers if g.n_seqs else 0
        return g.steps * g.n_layers

    # algorithmic work -------------------------------------------------------
    def elem(self):
        """Bytes per self-attention cache element."""
        return 2 if self.bf16 else 4

    def cross_bytes_per_call(self):
        g = self.g
        kv = 2 * g.n_streams * g.n_heads * g.mem_len * g.head_dim * self.cache_elem
        qo = 2 * g.n_streams * g.n_q * g.n_heads * g.head_dim * 4
        return kv + qo

    def self_bytes_per_call(self, pos):
        g = self.g
        rows = 2 * g.n_seqs * g.n_heads * pos * g.head_dim * self.elem()       # read 0..pos-1
        new = 2 * g.n_seqs * g.n_heads * g.head_dim * (4 + self.elem())        # k/v in + row out
        qo = 2 * g.n_seqs * g.n_heads * g.head_dim * 4
        return rows + new + qo

    def populate_flops(self):
        """K/V projections of every layer, plus the memory lift when there is one."""
        g = self.g
        f = 2.0 * g.n_streams * g.mem_len * (2 * g.n_layers * g.d_model) * g.d_model
        if g.lift_in:
            f += 2.0 * g.n_streams * g.mem_len * g.lift_in * g.d_model
        return f


def cpu_baseline(name, budget_s, threads=None):
    """The oracle as it stands, on the host's cores (or `threads` of them), on
    a bounded sample: populate, then decode tokens until the budget is used;
    the window time is populate + steps x the mean token time. For the Large
    workloads (16 streams x 32 layers) the sample is one stream's first
    `LARGE_POP_ROWS` memory rows for populate (scaled to all 16 x 1500 rows)
    and one stream of the sixteen for decode (scaled x16): extrapolated."""
    import oracle

    g = synth.get(name)
    saved = oracle.get_threads()
    if threads:
        oracle.set_threads(threads)
    threads = oracle.get_threads()
    wt = synth.workload_tensors(g)
    one = name in ("large", "large_fp8")   # one stream of the sixteen
    t0 = time.perf_counter()
    if one:
        rows = LARGE_POP_ROWS
        oracle.populate(wt["E"][:1, :rows], wt["WK"], wt["WV"], g.n_heads, g.head_dim,
                        round_bf16=(g.dtype == "bf16"), round_fp8=(g.dtype == "fp8"))
        t_pop = (time.perf_counter() - t0) * (g.n_streams * g.mem_len / rows)
        # decode reads the projection of the whole memory: the oracle's own
        # projection of one stream is too slow to run here, and attention
        # time does not depend on the values, so the rows are drawn
        shp = (g.n_layers, 1, g.n_heads, g.mem_len, g.head_dim)
        Kc = synth.normal([g.seed, 97, 0], shp, synth.q_std(g))
        Vc = synth.normal([g.seed, 97, 1], shp, synth.q_std(g))
    else:
        E = wt["E"]
        if g.lift_in:   # the projector memory is lifted first, as on the GPU
            lt = synth.workload_tensors(g, ("X_lift", "W_lift", "pos"))
            E = oracle.lift_gelu(lt["X_lift"], lt["W_lift"], lt["pos"]).reshape(
                g.n_streams, g.mem_len, -1)
        Kc, Vc = oracle.populate(E, wt["WK"], wt["WV"], g.n_heads, g.head_dim,
                                 round_bf16=(g.dtype == "bf16"))
        t_pop = time.perf_counter() - t0
    del wt
    S = g.n_seqs if not one else 1
    self_bf16 = g.dtype in ("bf16", "fp8")
    Ks = [np.zeros((S, g.n_heads, g.max_pos, g.head_dim)) for _ in range(g.n_layers)] if S else []
    Vs = [np.zeros_like(k) for k in Ks]
    t1 = time.perf_counter()
    n_tok = 0
    for t in range(g.steps):
        for l in range(g.n_layers):
            d = synth.decode_call_inputs(g, t, l)
            if S:
                oracle.self_append_attend(d["q_self"][:S], d["k_new"][:S], d["v_new"][:S], Ks[l],
                                          Vs[l], t, g.scale, round_bf16=self_bf16)
            q = d["q_cross"][:1] if one else d["q_cross"]
            oracle.cross_decode(q, Kc[l], Vc[l], g.scale)
        n_tok += 1
        if time.perf_counter() - t1 > max(1.0, budget_s - (time.perf_counter() - t0)):
            break
    t_tok = (time.perf_counter() - t1) / n_tok
    if one:
        t_tok *= g.n_streams
    per_window = t_pop + g.steps * t_tok
    tokens = g.steps * (g.n_seqs if g.n_seqs else g.n_streams * g.n_q)
    if one:
        sample = ("extrapolated: oracle populate of %d of 1500 memory rows of 1 of 16 streams "
                  "(x%d), then %d of %d decode steps of 1 of 16 streams (x16, all layers, self + "
                  "cross); window time = populate + %d x mean step time"
                  % (LARGE_POP_ROWS, g.n_streams * g.mem_len // LARGE_POP_ROWS, n_tok, g.steps,
                     g.steps))
    else:
        sample = ("oracle populate of the %s cache, then %d of %d decode steps (all layers, "
                  "self + cross); window time = populate + %d x mean step time"
                  % (name, n_tok, g.steps, g.steps))
    oracle.set_threads(saved)
    return {"value": tokens / per_window, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": sample, "populate_s": t_pop, "step_s": t_tok,
            "host_cpu": _host_cpu()}


# memory rows of one stream the Large oracle baseline populates (of 1500)
LARGE_POP_ROWS = 64


# HBM bandwidth x loaded latency (8 TB/s x ~2 us): a call that moves fewer bytes
# than this cannot keep enough requests in flight to approach the peak, so its
# time is set by latency and launch cost, not by bandwidth.
LATENCY_BOUND_BYTES = 16e6


def roofline_regime(bytes_per_call):
    """Which limit a decode call of this size runs into (reported beside frac)."""
    if bytes_per_call < LATENCY_BOUND_BYTES:
        return ("latency: %.1f MB per call is below the ~16 MB HBM bandwidth x latency product"
                % (bytes_per_call / 1e6))
    return "bandwidth"


# the sources of the decode kernels and of their launch plan (split counts,
# the in-launch merge): counters taken before any of them changed no longer
# describe the kernels that run
DECODE_SOURCES = ("attn_kernels.h", "attn_decode.hip", "attn_f32.hip", "attn_bf16.hip",
                  "attn_fp8.hip", "cke_device.h", "cke_internal.h", "cke_api.hip")


def graph_kernel_nodes(graph):
    """Kernel launches in a captured window graph (hipGraphGetNodes on its raw
    handle, kernel nodes only), or None where the runtime does not expose it."""
    import ctypes
    try:
        raw = graph.raw_cuda_graph()
        hip = ctypes.CDLL("libamdhip64.so")
        n = ctypes.c_size_t(0)
        if hip.hipGraphGetNodes(ctypes.c_void_p(raw), None, ctypes.byref(n)) != 0:
            return None
        nodes = (ctypes.c_void_p * n.value)()
        if hip.hipGraphGetNodes(ctypes.c_void_p(raw), nodes, ctypes.byref(n)) != 0:
            return None
        kinds = ctypes.c_int(-1)
        count = 0
        for i in range(n.value):
            if hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(kinds)) != 0:
                return None
            count += kinds.value == 0   # hipGraphNodeTypeKernel
        return count
    except (AttributeError, OSError, RuntimeError):
        return None


def measured_traffic(config):
    """HBM bytes per cross-attention decode call (split + merge kernels) from the
    committed rocprofv3 counter summary, scaled by its copy calibration; None if
    the decode kernel sources changed since the counters were taken or the
    workload was not counted."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        t = json.load(open(path))
    except (OSError, ValueError):
        return None
    for f in DECODE_SOURCES:
        src = os.path.join(ROOT, "projection_cache_amd", "csrc", f)
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != t["sources_sha256"].get(f):
            return None
    per = t["per_dispatch_KiB"].get(config)
    if not per:
        return None
    cal = t["calibration"]
    read = write = 0.0
    found = False
    for k, v in per.items():
        if any(n in k for n in ("xattn_partial_kernel", "xattn_merge_kernel", "xattn_short_kernel")):
            if "FETCH_SIZE" not in v or "WRITE_SIZE" not in v:
                return None
            found = True
            read += v["FETCH_SIZE"] * 1024 / cal["read_factor"]
            write += v["WRITE_SIZE"] * 1024 / cal["write_factor"]
    if not found:
        return None
    return {"bytes": read + write, "read": read, "write": write}


def measure_split_weights(torch, pc, w, stream, capture):
    """The populate with the weights split inside every call (the workspace
    calls), and the one-time split of the weights into planes that the
    window's populate reads instead."""
    def best_of(fn, reps):
        best = float("inf")
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3 / reps)
        return best
    gk = capture(("populate_split_weights",), 8)

    def replay():
        with torch.cuda.stream(stream):
            gk.replay()
    per_call = best_of(replay, 8)
    del gk
    mats = list(w.WK) + list(w.WV)

    def prepare():
        with torch.cuda.stream(stream):
            pc.cke_weight_planes(mats, w.w_planes, stream=stream)
            if w.lift_planes is not None:
                pc.cke_weight_planes([w.lift["W_lift"]], w.lift_planes, stream=stream)
    prepare()
    torch.cuda.synchronize()
    once = best_of(prepare, 1)
    return {"avg_us": per_call * 1e6,
            "tflops": w.populate_flops() / per_call / 1e12,
            "weight_planes_prepare_us": once * 1e6,
            "note": "populate with every weight split into bf16 planes inside the call; the "
                    "window instead reads planes split once when the weights are loaded "
                    "(weight_planes_prepare_us, eager launches, outside the window)"}


def measure_prefill(torch, pc, g, stream):
    """Time cke_selfattn_prefill_append at the workload's self-attention shape:
    3 rows from an empty cache (a ContextPrefill start) and a 64-row chunk at
    position 64. Each is one HIP graph of 16 identical calls (each call rewrites
    the same rows), replayed and timed with events. Bytes per call are the
    rows read once (0 .. pos+n-1 of K and V), the rows written and the fp32
    q, k_new, v_new and out."""
    if not g.n_seqs:
        return None
    self_bf16 = g.dtype in ("bf16", "fp8")   # self caches of fp8 workloads are bf16
    dt = torch.bfloat16 if self_bf16 else torch.float32
    elem = 2 if self_bf16 else 4
    S, H, D = g.n_seqs, g.n_heads, g.head_dim
    kv = pc.KVLayer(S, H, D, g.max_pos, dtype=dt)
    kv.k.normal_(0, 0.45)
    kv.v.normal_(0, 0.45)
    res = []
    for n, pos in ((3, 0), (64, 64)):
        q = torch.randn(S, n, H, D, device="cuda") * 0.45
        kn = torch.randn(S, n, H, D, device="cuda") * 0.45
        vn = torch.randn(S, n, H, D, device="cuda") * 0.45
        out = torch.empty_like(q)

        def calls():
            for _ in range(16):
                pc.cke_selfattn_prefill_append(q, kn, vn, kv, pos, n, H, g.scale, out,
                                               stream=torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            calls()
        stream.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            calls()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            with torch.cuda.stream(stream):
                gr.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3 / 16)
        nbytes = S * H * D * (2 * (pos + n) * elem + 2 * n * elem + 4 * n * 4)
        res.append({"n_new": n, "pos": pos, "seqs": S, "heads": H, "kv_heads": H,
                    "avg_us": best * 1e6, "bytes_per_call": nbytes, "GB_s": nbytes / best / 1e9})
        del gr
    return res


def measure_weights(torch, pc, w, stream):
    """Time cke_xattn_decode_weights against cke_xattn_decode on the workload's
    cache: one HIP graph per call kind holding one call per layer (the same
    queries), with every other head selected."""
    g = w.g
    heads = list(range(0, g.n_heads, 2))[:32]
    q = w.qc[0, 0]
    out = torch.empty_like(q)
    wts = torch.empty(g.n_streams, g.n_q, g.mem_len, device="cuda")

    def timed(fn):
        with torch.cuda.stream(stream):
            fn()
        stream.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            with torch.cuda.stream(stream):
                gr.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3 / g.n_layers)
        return best

    cs = torch.cuda.current_stream
    t_w = timed(lambda: [pc.cke_xattn_decode_weights(q, w.cache, l, g.scale, heads, out, wts,
                                                     stream=cs()) for l in range(g.n_layers)])
    t_d = timed(lambda: [pc.cke_xattn_decode(q, w.cache, l, g.scale, out, stream=cs())
                         for l in range(g.n_layers)])
    return {"heads": len(heads), "avg_us": t_w * 1e6, "decode_only_us": t_d * 1e6,
            "extra_us": (t_w - t_d) * 1e6}


def measure_decoder_step(torch, pc, w, stream, tokens=4):
    """Time cke_decoder_layer_step at the workload's shape: a HIP graph of
    `tokens` decode tokens x all layers (one call per layer, positions
    0..tokens-1) over the workload's populated cache, with random weights of
    the layer shape (fp32 or bf16 as the workload's inputs). For fp32 weights
    the same layer is also timed as the composition of separate calls (torch
    matmuls for the six products, the library's self and cross calls, torch
    residual adds), for comparison. Weights are output-major, as the step
    takes them."""
    g = w.g
    S = g.n_streams * g.n_q
    if not g.n_seqs or g.n_seqs != S:
        return None
    L, dm = g.n_layers, g.d_model
    wdt = torch.bfloat16 if w.bf16 else torch.float32
    gen = torch.Generator(device="cuda").manual_seed(11)
    Wd = [[(torch.randn(dm, dm, device="cuda", generator=gen) * 0.02).to(wdt) for _ in range(6)]
          for _ in range(L)]
    descs = [pc.decoder_layer_desc(*Wl) for Wl in Wd]
    kvs = [pc.KVLayer(S, g.n_heads, g.head_dim, g.max_pos, dtype=wdt) for _ in range(L)]
    ws = torch.empty(pc.cke_decoder_step_workspace_bytes(w.cache.geom, S) // 4, device="cuda")
    x = torch.randn(S, dm, device="cuda", generator=gen)

    def graph_time(fn):
        with torch.cuda.stream(stream):
            fn()
        stream.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            with torch.cuda.stream(stream):
                gr.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3)
        return best

    cs = torch.cuda.current_stream

    def fused():
        for t in range(tokens):
            for l in range(L):
                pc.cke_decoder_layer_step(x, descs[l], kvs[l], t, w.cache, l, g.scale, ws,
                                          stream=cs())
    t_f = graph_time(fused) / (tokens * L)
    welem = 2 if w.bf16 else 4
    slab = 2 * g.n_streams * g.n_heads * g.mem_len * g.head_dim * w.cache_elem
    self_rows = 2 * S * g.n_heads * ((tokens + 1) / 2) * g.head_dim * welem
    by = 6 * dm * dm * welem + slab + self_rows + 12 * S * dm * 4
    res = {"seqs": S, "layers": L, "tokens": tokens, "avg_us_per_layer": t_f * 1e6,
           "tokens_per_s": S / (t_f * L), "bytes_per_layer": by, "GB_s": by / t_f / 1e9,
           # a split cross call adds a merge launch unless it merges in its own
           "launches_per_layer": 6 if (w.cache.n_splits == 1 or
                                       pc.cke_xattn_merges_in_launch(w.cache, max(g.n_q, 1))) else 7}
    if not w.bf16:
        H, D = g.n_heads, g.head_dim
        q, k, v, so, x1, qc, co = (torch.empty(S, dm, device="cuda") for _ in range(7))

        def composed():
            for t in range(tokens):
                for l in range(L):
                    WQs, WKs, WVs, WOs, WQ, WO = Wd[l]   # output-major, as nn.Linear
                    torch.mm(x, WQs.t(), out=q)
                    torch.mm(x, WKs.t(), out=k)
                    torch.mm(x, WVs.t(), out=v)
                    pc.cke_selfattn_decode_append(q.view(S, H, D), k.view(S, H, D),
                                                  v.view(S, H, D), kvs[l], t, g.scale,
                                                  so.view(S, H, D), stream=cs())
                    torch.addmm(x, so, WOs.t(), out=x1)
                    torch.mm(x1, WQ.t(), out=qc)
                    pc.cke_xattn_decode(qc.view(g.n_streams, g.n_q, H, D), w.cache, l, g.scale,
                                        co.view(g.n_streams, g.n_q, H, D), stream=cs())
                    torch.addmm(x1, co, WO.t(), out=x)
        t_c = graph_time(composed) / (tokens * L)
        res["composed_us_per_layer"] = t_c * 1e6
        res["speedup_vs_composed"] = t_c / t_f
    return res


def measure_launch_floor(torch, stream, launches=256):
    """Time per launch of a chain of dependent one-element kernels (torch's
    in-place add on a single float) replayed as one HIP graph: the floor
    that every call of a window pays whatever its work, against which the
    latency-bound per-call times are read."""
    x = torch.zeros(1, device="cuda")
    with torch.cuda.stream(stream):
        for _ in range(8):
            x.add_(1.0)
    stream.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=stream):
        for _ in range(launches):
            x.add_(1.0)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        with torch.cuda.stream(stream):
            gr.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3 / launches)
    return {"launches": launches, "us_per_launch": best * 1e6,
            "kernel": "one-element in-place add (torch), dependent chain in one HIP graph"}


def measure_cold_decode(torch, pc, w, stream, calls=24):
    """Cross-decode time with the 256 MB MALL cold: each call follows a fill of
    a 512 MB buffer (which evicts the cache). One HIP graph holds `calls` of
    (fill, decode) pairs, another the fills alone; the difference per call is
    the cold decode time. Only for workloads whose whole cross cache (K + V,
    all layers) would otherwise stay resident."""
    g = w.g
    whole = 2 * g.n_layers * g.n_streams * g.n_heads * g.mem_len * g.head_dim * w.cache_elem
    if whole > (256 << 20):
        return None
    flush = torch.empty(128 << 20, device="cuda")   # 512 MB
    out = torch.empty_like(w.qc[0, 0])
    cs = torch.cuda.current_stream

    def timed(fn):
        with torch.cuda.stream(stream):
            fn()
        stream.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            with torch.cuda.stream(stream):
                gr.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3)
        return best

    def pairs():
        for i in range(calls):
            flush.fill_(float(i + 1))
            pc.cke_xattn_decode(w.qc[0, i % g.n_layers], w.cache, i % g.n_layers, g.scale, out,
                                stream=cs())

    def fills():
        for i in range(calls):
            flush.fill_(float(i + 1))

    t = (timed(pairs) - timed(fills)) / calls
    b = w.cross_bytes_per_call()
    return {"avg_us": t * 1e6, "bytes_per_call": b, "GB_s": b / t / 1e9,
            "frac_of_hbm_peak": b / t / 1e9 / HBM_PEAK_GBS}


def populate_report(w, tflops, pop_dt):
    """Populate TFLOP/s against the MFMA peak of the instruction it issues.
    fp32 products of a width that is a multiple of 128 run as three bf16 MFMA
    products (operands split into two bf16 terms): `frac` is their issued
    rate (3x the algorithmic FLOP) against the bf16 peak; the algorithmic
    rate against the fp32 peak is reported beside it."""
    g = w.g
    x3 = not w.bf16 and g.d_model % 128 == 0
    r = {"tflops": tflops}
    if w.bf16:
        r.update(mfma="v_mfma_f32_32x32x16_bf16", peak_tflops=MFMA_PEAK_TFLOPS["bf16"],
                 frac=tflops / MFMA_PEAK_TFLOPS["bf16"])
    elif x3:
        r.update(mfma="v_mfma_f32_32x32x16_bf16, three products of fp32 operands split into "
                      "bf16 planes: the weights once when loaded, E (and the lift input) in "
                      "every window (that split included in the time)"
                 if w.w_planes is not None else
                 "v_mfma_f32_32x32x16_bf16, three products of bf16-split fp32 operands",
                 issued_tflops=3 * tflops, peak_tflops=MFMA_PEAK_TFLOPS["bf16"],
                 frac=3 * tflops / MFMA_PEAK_TFLOPS["bf16"],
                 algorithmic_frac_vs_f32_peak=tflops / MFMA_PEAK_TFLOPS["f32"])
    else:
        r.update(mfma="v_mfma_f32_32x32x2_f32", peak_tflops=MFMA_PEAK_TFLOPS["f32"],
                 frac=tflops / MFMA_PEAK_TFLOPS["f32"])
    if g.lift_in:
        # the library runs the lift as three bf16 products when its input is at least 1024 wide
        lift_mfma = "three bf16 products" if g.lift_in >= 1024 else "v_mfma_f32_32x32x2_f32"
        r["includes"] = "memory lift (%s) + K/V projections" % lift_mfma
    r["target_frac"] = 0.5
    r["target_met"] = r["frac"] >= 0.5
    return r


def library_info(pc):
    """Which build of the library this process loaded: its path, whether the
    path came from the override variable, the SHA-256 of the file and of the
    sources it is built from (csrc/ and the public header)."""
    import hashlib

    def sha(paths):
        h = hashlib.sha256()
        for path in paths:
            h.update(os.path.relpath(path, ROOT).encode())
            h.update(open(path, "rb").read())
        return h.hexdigest()

    csrc = os.path.join(ROOT, "projection_cache_amd", "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc))
    srcs.append(os.path.join(ROOT, "include", "cke_xattn.h"))
    return {"path": pc.LIB_PATH, "override": bool(os.environ.get("CKE_XATTN_LIB")),
            "sha256": sha([pc.LIB_PATH]), "sources_sha256": sha(srcs)}


def _progress(msg):
    """One line per finished phase on stderr (stdout carries only the JSON
    line), so that a long default run is never silent for minutes."""
    print("bench: " + msg, file=sys.stderr, flush=True)


def _host_cpu():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _git_sha():
    try:
        return subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT,
                              capture_output=True, text=True, timeout=5).stdout.strip() or None
    except Exception:
        return None


# Environment variables rocprofv3 exports to the profiled process when it
# collects hardware counters (--pmc or a counter input file).
COUNTER_ENV = ("ROCPROF_COUNTER_COLLECTION", "ROCPROF_COUNTERS")


def counter_collection_active(environ=None) -> bool:
    environ = os.environ if environ is None else environ
    return any(environ.get(k) not in (None, "", "0") for k in COUNTER_ENV)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if counter_collection_active() and not (args.counters or args.calibrate_copy):
        # a process that captures HIP graphs while rocprofv3 collects
        # counters has crashed inside the profiler: refuse before any GPU work
        print("bench.py: hardware-counter collection is active; the default run captures HIP "
              "graphs, which is not supported under counter collection. Run the eager counter "
              "mode instead: bench.py --counters [--counter-tokens N]", file=sys.stderr)
        sys.exit(3)

    import torch

    import projection_cache_amd as pc

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        # plain copy kernel of known size: HBM counters per dispatch are read
        # against its 256 MiB read + 256 MiB write
        n = 64 << 20
        src = torch.empty(n, device="cuda").normal_()
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4,
                          "dispatches": 5}))
        return
    stream = torch.cuda.Stream()
    if args.counters:
        w = Workload(args.config, torch, pc)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            w.window(stream, tokens=args.counter_tokens)
        torch.cuda.synchronize()
        print(json.dumps({"counters_windows": args.steps, "config": args.config,
                          "xattn_bytes_per_call": w.cross_bytes_per_call(),
                          "xattn_calls_per_window": w.calls("xattn_decode")}))
        return

    # wall-clock seconds of each phase: the GPU measurements and the host-only
    # oracle baselines, so that a sampled GPU-busy figure can be read against them
    phases = {}
    t_start = time.perf_counter()
    head = measure(args.config, args, torch, pc, stream, extras=not args.no_extras)
    phases[args.config + "_gpu"] = time.perf_counter() - t_start
    _progress("%s measured" % args.config)
    result = {
        "metric": METRIC,
        "value": head.pop("value"),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.pop("dtype"),
        "data": "synthetic",
        "config": head.pop("config"),
        "roofline": head.pop("roofline"),
    }
    result.update(head)
    result["gpu"] = torch.cuda.get_device_name(0)
    result["git"] = _git_sha()
    result["library"] = library_info(pc)
    also = [c for c in args.also.split(",") if c and c != "none" and c != args.config]
    if also:
        result["also"] = {}
        for name in also:
            t0 = time.perf_counter()
            blk = measure(name, args, torch, pc, stream, extras=False)
            phases[name + "_gpu"] = time.perf_counter() - t0
            _progress("%s measured" % name)
            if not args.no_cpu_baseline:
                t0 = time.perf_counter()
                blk["cpu_baseline"] = cpu_baseline(name, args.cpu_seconds)
                phases[name + "_cpu_baseline"] = time.perf_counter() - t0
                _progress("%s oracle baseline timed" % name)
            result["also"][name] = blk
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        result["cpu_baseline"] = cpu_baseline(args.config, args.cpu_seconds)
        if args.config in ("tiny", "base", "beam"):
            result["cpu_baseline_1thread"] = cpu_baseline(args.config, args.cpu_seconds,
                                                          threads=1)
        phases[args.config + "_cpu_baseline"] = time.perf_counter() - t0
        _progress("%s oracle baseline timed" % args.config)
    phases["total"] = time.perf_counter() - t_start
    result["phases_s"] = phases
    print(json.dumps(result))


def measure(name, args, torch, pc, stream, extras):
    """Time one workload: `args.steps` whole windows replayed as one HIP graph
    each (value, ms_per_step), then the per-call durations from one graph per
    call kind, the roofline of the cross-attention call and of the window, and
    (extras) the other entry points at the workload's shape. Frees the
    workload's device memory before returning."""
    w = Workload(name, torch, pc)
    g = w.g
    torch.cuda.synchronize()

    def capture(kinds, reps=1, keep=False):
        with torch.cuda.stream(stream):
            w.window(stream, kinds)    # warm the kernels once outside capture
        stream.synchronize()
        # keep_graph: the captured graph stays inspectable (for counting its launches)
        graph = torch.cuda.CUDAGraph(keep_graph=True) if keep else torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for _ in range(reps):
                w.window(torch.cuda.current_stream(), kinds)
        torch.cuda.synchronize()
        return graph

    window_launches = None
    if args.mode == "graph":
        graph = capture(("populate", "selfattn", "xattn_decode"))
        try:   # a second capture of the same window, kept to count its kernel launches
            counted = capture(("populate", "selfattn", "xattn_decode"), keep=True)
            window_launches = graph_kernel_nodes(counted)
            del counted
        except (TypeError, RuntimeError):
            window_launches = None

        def run():
            with torch.cuda.stream(stream):
                graph.replay()
    else:
        def run():
            w.window(stream)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    tok_s = w.tokens_per_window * args.steps / elapsed
    if args.mode == "graph":
        del graph
    _progress("%s: %d windows timed, %.2f ms each" % (name, args.steps, ms_per_step))

    # per-call durations: one graph per call kind, replayed, timed with events
    avg, total = {}, {}
    for kind in ("populate", "selfattn", "xattn_decode"):
        n = w.calls(kind)
        if n == 0:
            continue
        # a window with few calls of a kind (Q-Former: 2 cross calls, one
        # populate everywhere) is repeated so that the graph's own launch
        # cost is spread over >= 32 calls (populate: >= 8)
        reps = 8 if kind == "populate" else -(-32 // n)
        gk = capture((kind,), reps)
        best = float("inf")
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            with torch.cuda.stream(stream):
                gk.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3)
        avg[kind] = best / (n * reps)
        total[kind] = best / reps
        del gk
    dur = {k: [avg[k]] * w.calls(k) for k in avg}

    cross_b = w.cross_bytes_per_call()
    cross_gbs = cross_b / avg["xattn_decode"] / 1e9
    fused_merge = pc.cke_xattn_merges_in_launch(w.cache, max(g.n_q, 1))
    # memories of at most 64 rows take the one-wave-per-head kernel
    cross_kernel = "xattn_short_kernel" if g.mem_len <= 64 else "xattn_partial_kernel"
    merge_text = ("" if w.cache.n_splits == 1 else
                  ", split partials merged in the same launch" if fused_merge else " + xattn_merge_kernel")
    traffic = measured_traffic(name)
    kernels = {
        "xattn_decode": {"avg_us": avg["xattn_decode"] * 1e6, "calls_per_step": len(dur["xattn_decode"]),
                         "bytes_per_call": cross_b, "GB_s": cross_gbs},
        "populate": {"avg_us": avg["populate"] * 1e6,
                     "tflops": w.populate_flops() / avg["populate"] / 1e12},
    }
    self_bytes = 0.0
    if "selfattn" in dur:
        sb = [w.self_bytes_per_call(t) for t in range(g.steps) for _ in range(g.n_layers)]
        self_bytes = float(np.sum(sb))
        kernels["selfattn"] = {"avg_us": avg["selfattn"] * 1e6,
                               "calls_per_step": len(dur["selfattn"]),
                               "bytes_per_call_mean": float(np.mean(sb)),
                               "GB_s": float(self_bytes / np.sum(dur["selfattn"]) / 1e9)}
    share = {k: float(np.sum(v)) for k, v in dur.items()}
    dominant = max(share, key=share.get)
    pop_dt = "bf16" if w.bf16 else "f32"        # the MFMA input type
    # the whole window against HBM: the decode calls' algorithmic bytes (K/V
    # rows read, new rows, queries and outputs) over the measured window time
    decode_bytes = cross_b * w.calls("xattn_decode") + self_bytes
    window_gbs = decode_bytes / (ms_per_step * 1e-3) / 1e9
    tok_at_peak = w.tokens_per_window / (decode_bytes / (HBM_PEAK_GBS * 1e9))
    blk = {
        "value": tok_s,
        "ms_per_step": ms_per_step,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8"}[g.dtype],
        "config": {"workload": WORKLOAD_TEXT[name], "name": name,
                   "tokens_per_step": w.tokens_per_window, "decode_steps": g.steps,
                   "layers": g.n_layers, "mode": args.mode},
        "roofline": {"bound": "hbm",
                     "kernel": "cke_xattn_decode (%s%s)" % (cross_kernel, merge_text),
                     "achieved": cross_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": cross_gbs / HBM_PEAK_GBS,
                     "traffic": traffic["bytes"] if traffic else None,
                     "traffic_read_write": [traffic["read"], traffic["write"]] if traffic else None,
                     "bytes_per_launch": cross_b, "avg_launch_us": avg["xattn_decode"] * 1e6,
                     "regime": roofline_regime(cross_b)},
        "window_roofline": {"bound": "hbm", "decode_bytes_per_step": decode_bytes,
                            "achieved": window_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": window_gbs / HBM_PEAK_GBS,
                            "tokens_per_s_at_peak": tok_at_peak,
                            "target_tokens_per_s": 0.6 * tok_at_peak,
                            "target_met": tok_s >= 0.6 * tok_at_peak},
        "populate": populate_report(w, kernels["populate"]["tflops"], pop_dt),
        "kernels": kernels,
        "time_share": {k: v / sum(share.values()) for k, v in share.items()},
        "kernel_sum_ms_per_step": sum(total.values()) * 1e3,
        "dominant_kernel": dominant,
    }
    if w.w_planes is not None:
        blk["populate"]["weights_split_per_call"] = measure_split_weights(torch, pc, w, stream, capture)
    if extras:
        blk["xattn_decode_weights"] = measure_weights(torch, pc, w, stream)
        step = measure_decoder_step(torch, pc, w, stream)
        if step:
            blk["decoder_layer_step"] = step
        prefill = measure_prefill(torch, pc, g, stream)
        if prefill:
            blk["selfattn_prefill"] = prefill
        cold = measure_cold_decode(torch, pc, w, stream)
        if cold:
            blk["xattn_decode_mall_cold"] = cold
        floor = measure_launch_floor(torch, stream)
        launches = window_launches
        if launches is None:   # estimate: one populate launch, the decode calls' kernels
            per_cross = 2 if (w.cache.n_splits > 1 and not fused_merge) else 1
            launches = 1 + w.calls("selfattn") + w.calls("xattn_decode") * per_cross
        floor["launches_per_step"] = launches
        floor["launches_counted"] = window_launches is not None
        floor["floor_tokens_per_s"] = w.tokens_per_window / (launches * floor["us_per_launch"] * 1e-6)
        blk["launch_floor"] = floor
    del w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return blk


if __name__ == "__main__":
    main()
