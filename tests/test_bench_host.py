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
