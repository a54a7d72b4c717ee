"""Host-side checks of bench.py that need no GPU: the one-GPU refusal and the
helpers that label its roofline figure."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_roofline_regime_separates_latency_and_bandwidth_bound_calls():
    # Whisper Base: one layer slab of K and V in fp32 is 6,144,000 bytes (+ q/out)
    assert bench.roofline_regime(6148096).startswith("latency: 6.1 MB")
    # Large: one bf16 layer slab over 16 streams is 122,880,000 bytes (+ q/out)
    assert bench.roofline_regime(123043840) == "bandwidth"
    assert bench.roofline_regime(bench.LATENCY_BOUND_BYTES) == "bandwidth"


def test_graph_modes_refuse_to_run_under_counter_collection():
    """Counter passes must use the eager --counters mode: with rocprofv3's
    counter-collection variables set, the default (graph-capturing) run exits
    with a message before touching the GPU."""
    env = dict(os.environ, ROCPROF_COUNTER_COLLECTION="1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny"],
                       capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 3
    assert "--counters" in r.stderr and r.stdout == ""
    assert bench.counter_collection_active({"ROCPROF_COUNTERS": "pmc: FETCH_SIZE"})
    assert not bench.counter_collection_active({"ROCPROF_COUNTER_COLLECTION": "0"})
    assert not bench.counter_collection_active({})


class _W:
    """Stand-in for bench.Workload with just what populate_report reads."""
    def __init__(self, name, bf16, planes):
        self.g = bench.synth.get(name)
        self.bf16 = bf16
        self.w_planes = object() if planes else None
        self.pop_ws = object() if planes else None


def test_populate_report_scores_the_issued_instruction_rate():
    """fp32 products run as three bf16 MFMA products: `frac` is their issued
    rate (3x the algorithmic FLOP) against the bf16 peak, with the algorithmic
    rate against the fp32 peak beside it; bf16 populates use the bf16 peak."""
    r = bench.populate_report(_W("base", False, True), 200.0, "f32")
    assert abs(r["issued_tflops"] - 600.0) < 1e-9
    assert abs(r["frac"] - 600.0 / bench.MFMA_PEAK_TFLOPS["bf16"]) < 1e-12
    assert abs(r["algorithmic_frac_vs_f32_peak"] - 200.0 / bench.MFMA_PEAK_TFLOPS["f32"]) < 1e-12
    assert "once when loaded" in r["mfma"] and r["target_met"] is False
    r = bench.populate_report(_W("large", True, False), 1300.0, "bf16")
    assert abs(r["frac"] - 1300.0 / bench.MFMA_PEAK_TFLOPS["bf16"]) < 1e-12
    assert r["target_met"] is True
    q = bench.populate_report(_W("qformer", False, True), 250.0, "f32")
    assert "memory lift" in q["includes"]


def test_phases_and_extras_flags_are_parsed():
    old = sys.argv
    try:
        sys.argv = ["bench.py", "--no-extras", "--also", "none"]
        a = bench.parse()
    finally:
        sys.argv = old
    assert a.no_extras and a.also == "none"
    sys.argv = ["bench.py"]
    try:
        d = bench.parse()
    finally:
        sys.argv = old
    assert d.also == "large,beam,qformer" and not d.no_extras and d.gpus == 1


def test_counter_traffic_of_the_decode_call_is_near_its_algorithmic_bytes():
    """The committed HBM counters (profiles/hbm_traffic.json), where they still
    describe the decode kernels' sources, put each workload's cross-attention
    call within a few percent above its algorithmic bytes: K and V of one layer
    slab once, queries and outputs, plus the split partials where a second
    kernel merges them (Beam); the one-wave-per-head kernel of the Q-Former's
    15-row memories is counted too. Configurations without counters give None,
    never 0."""
    algorithmic = {"base": 6148096, "beam": 6164480, "large": 123043840, "large_fp8": 61603840,
                   "qformer": 29491200}
    for name, want in algorithmic.items():
        t = bench.measured_traffic(name)
        if t is None:        # sources changed since the counters were taken
            continue
        assert 0.99 * want <= t["bytes"] <= 1.2 * want, (name, t["bytes"], want)
        assert t["bytes"] == t["read"] + t["write"]
    assert bench.measured_traffic("no such workload") is None
