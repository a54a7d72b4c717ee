"""The allocation-free decoder-layer step (its step buffers in the library's
own per-GPU scratch array) against the step that takes a caller workspace:
same kernels, so the hidden state and the self-cache rows must agree bit for
bit. Two runs in a row, the second at a smaller shape, so the scratch array is
reused with less of it written; and a shape too large for the array is
refused before anything is launched."""
import math

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("WQs", "WKs", "WVs", "WOs", "WQ", "WO")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global pc
    import projection_cache_amd as pc  # noqa: F401  (fails loudly if not built)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _setup(g, bf):
    """Populated cache, output-major layer weights and two sets of self
    caches (one per entry point) for the geometry g."""
    wt = synth.workload_tensors(g, ("E", "WK", "WV") + NAMES + ("x0",))
    dt = torch.bfloat16 if bf else torch.float32

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt).to(DEV)

    cache = pc.XattnCache(g.n_layers, g.n_streams, g.mem_len, g.d_model, g.n_heads, g.head_dim,
                          max_q=g.n_q, dtype=dt)
    cache.populate(dev(wt["E"]), [dev(w) for w in wt["WK"]], [dev(w) for w in wt["WV"]])
    descs = []
    keep = []
    for l in range(g.n_layers):
        ws = [dev(wt[k][l].T) for k in NAMES]
        keep.append(ws)
        descs.append(pc.decoder_layer_desc(*ws))
    S = g.n_streams * g.n_q
    kvs = [[pc.KVLayer(S, g.n_heads, g.head_dim, g.max_pos, dtype=dt) for _ in range(g.n_layers)]
           for _ in range(2)]
    x0 = torch.from_numpy(wt["x0"][:S].astype(np.float32)).to(DEV)
    return cache, descs, keep, kvs, x0, S


def _run_both(g, bf, steps=3):
    cache, descs, keep, kvs, x0, S = _setup(g, bf)
    ws = torch.empty(pc.cke_decoder_step_workspace_bytes(cache.geom, S) // 4, device=DEV)
    xa, xb = x0.clone(), x0.clone()
    for t in range(steps):
        for l in range(g.n_layers):
            pc.cke_decoder_layer_step(xa, descs[l], kvs[0][l], t, cache, l, g.scale, ws)
            pc.cke_decoder_layer_step_noalloc(xb, descs[l], kvs[1][l], t, cache, l, g.scale)
            torch.cuda.synchronize()
            assert torch.equal(xa, xb), (g.d_model, t, l)
            assert bool(torch.isfinite(xb).all())
    for a, b in zip(kvs[0], kvs[1]):
        assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    del keep


def _geom(**kw):
    d = dict(name="custom", n_seqs=0, steps=4, max_pos=8, seed=61, dtype="f32")
    d.update(kw)
    d["scale"] = 1.0 / math.sqrt(d["head_dim"])
    d["n_seqs"] = d["n_streams"] * d["n_q"]
    return synth.Geometry(**d)


def test_noalloc_step_matches_the_workspace_step_then_a_smaller_one():
    # first: 16 sequences over 16 streams at the Large width, bf16 weights and caches
    big = _geom(n_streams=16, n_q=1, n_layers=2, mem_len=300, d_model=1280, n_heads=20,
                head_dim=64, dtype="bf16")
    assert 7 * 16 * 1280 * 4 <= pc.cke_decoder_step_scratch_bytes()
    _run_both(big, bf=True)
    # then: one sequence at the Whisper Base width, fp32, split cross decode
    small = _geom(n_streams=1, n_q=1, n_layers=2, mem_len=1500, d_model=512, n_heads=8,
                  head_dim=64)
    _run_both(small, bf=False)


def test_noalloc_step_refuses_shapes_beyond_its_scratch():
    g = _geom(n_streams=16, n_q=8, n_layers=1, mem_len=16, d_model=1280, n_heads=20,
              head_dim=64, dtype="bf16")
    cache, descs, keep, kvs, x0, S = _setup(g, bf=True)
    assert 7 * S * g.d_model * 4 > pc.cke_decoder_step_scratch_bytes()
    x = x0.clone()
    with pytest.raises(pc.CkeError) as e:
        pc.cke_decoder_layer_step_noalloc(x, descs[0], kvs[1][0], 0, cache, 0, g.scale)
    assert e.value.code == pc.CKE_EINVAL and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(x, x0)
    assert float(kvs[1][0].k.abs().max()) == 0.0      # nothing was launched
    del keep
