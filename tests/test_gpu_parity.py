"""Parity of the HIP library (through its C ABI) with the CPU oracle.

Inputs are seeded and synthetic (synth/); the oracle computes in float64 from
the same values. Floating-point outputs must agree within max-abs 1e-4 where
the cache is fp32 and 2e-2 where it is bf16. Stored cache rows written by the
self-attention append are compared bit for bit (a copy, or a round-to-nearest
bf16 conversion of an fp32 value, has exactly one correct result).

fp8 (E4M3) projection caches: a stored value is a rounding decision, taken
from the kernel's fp32 accumulation, so each stored element must lie between
the fp8 roundings of (exact - e) and (exact + e), e the fp32 accumulation
error bound; attention over an fp8 cache is checked on the oracle's own fp8
cache, uploaded in place of the kernel's, to the fp32 bar of 1e-4.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global pc
    import projection_cache_amd as pc  # noqa: F401  (fails loudly if not built)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


DEV = "cuda:0"


def t32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def tbf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).to(DEV)


def to_np(t):
    return t.detach().cpu().float().numpy().astype(np.float64)


def tfp8(a):
    """float64 values that are exact fp8 E4M3 numbers -> device fp8 tensor
    (the conversion of a representable value is exact)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(
        torch.float8_e4m3fn).to(DEV)


CACHE_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


def geometry(name=None, **kw):
    if name is not None:
        g = synth.get(name)
        if not kw:
            return g
        d = {f: getattr(g, f) for f in g.__dataclass_fields__}
    else:
        d = dict(name="custom", n_streams=1, n_q=1, n_seqs=1, n_layers=1, mem_len=64,
                 d_model=64, n_heads=2, head_dim=32, scale=1 / math.sqrt(32), dtype="f32",
                 steps=4, max_pos=8, seed=77)
    d.update(kw)
    return synth.Geometry(**d)


def make_cache(g, inputs=None):
    """GPU cache populated from the workload's seeded E/WK/WV."""
    wt = inputs or synth.workload_tensors(g)
    cache = pc.XattnCache(g.n_layers, g.n_streams, g.mem_len, g.d_model, g.n_heads, g.head_dim,
                          max_q=max(g.n_q, 1), dtype=CACHE_DT[g.dtype])
    if g.dtype in ("bf16", "fp8"):
        E = tbf16(wt["E_bits"])
        WK = [tbf16(b) for b in wt["WK_bits"]]
        WV = [tbf16(b) for b in wt["WV_bits"]]
    else:
        E = t32(wt["E"])
        WK = [t32(w) for w in wt["WK"]]
        WV = [t32(w) for w in wt["WV"]]
    cache.populate(E, WK, WV)
    torch.cuda.synchronize()
    return cache, wt, (E, WK, WV)


_ORACLE_CACHE = {}


def oracle_caches(g, wt):
    """Oracle projection caches of a named workload, computed once per module."""
    key = (g.name, g.seed, g.n_layers, g.n_streams, g.mem_len, g.d_model, g.dtype)
    if g.name == "custom" or key not in _ORACLE_CACHE:
        r = oracle.populate(wt["E"], wt["WK"], wt["WV"], g.n_heads, g.head_dim,
                            round_bf16=(g.dtype == "bf16"), round_fp8=(g.dtype == "fp8"))
        if g.name == "custom":
            return r
        _ORACLE_CACHE[key] = r
    return _ORACLE_CACHE[key]


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


# ------------------------------------------------------------------ populate
POP_CASES = [
    ("tiny", {}),
    ("base", {}),
    (None, dict(n_layers=2, n_streams=3, mem_len=77, d_model=256, n_heads=4, head_dim=64)),
    (None, dict(n_layers=2, n_streams=3, mem_len=77, d_model=256, n_heads=4, head_dim=64,
                dtype="bf16")),
    (None, dict(n_layers=3, n_streams=2, mem_len=1, d_model=96, n_heads=3, head_dim=32)),
    (None, dict(n_layers=1, n_streams=1, mem_len=200, d_model=256, n_heads=2, head_dim=128,
                dtype="bf16")),
    (None, dict(n_layers=2, n_streams=2, mem_len=130, d_model=384, n_heads=3, head_dim=128)),
    # bf16, 256-wide column tiles: memories shorter than a row tile (several
    # streams per tile) and longer than one (a tile straddling two streams)
    (None, dict(n_layers=2, n_streams=3, mem_len=100, d_model=256, n_heads=8, head_dim=32,
                dtype="bf16")),
    (None, dict(n_layers=1, n_streams=2, mem_len=300, d_model=512, n_heads=8, head_dim=64,
                dtype="bf16")),
    # bf16 widths that are not a multiple of 256 (128-wide tiles) or of 128
    (None, dict(n_layers=2, n_streams=2, mem_len=130, d_model=384, n_heads=3, head_dim=128,
                dtype="bf16")),
    (None, dict(n_layers=3, n_streams=2, mem_len=33, d_model=96, n_heads=3, head_dim=32,
                dtype="bf16")),
]


@pytest.mark.parametrize("name,kw", POP_CASES, ids=lambda x: str(x))
def test_populate_matches_oracle(name, kw):
    g = geometry(name, **kw)
    cache, wt, _ = make_cache(g)
    Kc, Vc = oracle_caches(g, wt)
    tol = TOL[g.dtype]
    assert max_abs(to_np(cache.k), Kc) <= tol
    assert max_abs(to_np(cache.v), Vc) <= tol
    assert cache.ready


def _random_geometries(n, seed=2026):
    """Seeded random shapes for populate + decode: every head_dim, fp32 and
    bf16, ragged memory lengths, 1-3 layers and streams, 1-8 queries; every
    other bf16 shape has H*D a multiple of 256 (the 256-wide tile kernel)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([32, 64, 128]))
        dtype = ("f32", "bf16")[i % 2]
        if i % 4 == 1:
            H = 256 * int(rng.integers(1, 4)) // D
        else:
            H = int(rng.integers(1, 9))
        out.append(dict(n_layers=int(rng.integers(1, 4)), n_streams=int(rng.integers(1, 4)),
                        n_q=int(rng.integers(1, 9)), mem_len=int(rng.integers(1, 601)),
                        d_model=H * D, n_heads=H, head_dim=D, dtype=dtype,
                        scale=1 / math.sqrt(D), seed=1000 + i))
    return out


@pytest.mark.parametrize("kw", _random_geometries(16),
                         ids=lambda k: "L%d-B%d-q%d-T%d-H%dx%d-%s" % (
                             k["n_layers"], k["n_streams"], k["n_q"], k["mem_len"], k["n_heads"],
                             k["head_dim"], k["dtype"]))
def test_random_geometry_populate_then_decode(kw):
    g = geometry(None, **kw)
    cache, wt, _ = make_cache(g)
    Kc, Vc = oracle_caches(g, wt)
    tol = TOL[g.dtype]
    assert max_abs(to_np(cache.k), Kc) <= tol
    assert max_abs(to_np(cache.v), Vc) <= tol
    for layer in range(g.n_layers):
        q = synth.decode_call_inputs(g, 0, layer)["q_cross"]
        out = cache.decode(t32(q), layer, g.scale)
        torch.cuda.synchronize()
        err = max_abs(to_np(out), oracle.cross_decode(q, Kc[layer], Vc[layer], g.scale))
        assert err <= tol, (layer, err)


# ------------------------------------------ populate from split bf16 planes
PLANES_CASES = [
    ("base", {}),
    (None, dict(n_layers=2, n_streams=3, mem_len=77, d_model=256, n_heads=4, head_dim=64)),
    (None, dict(n_layers=3, n_streams=2, mem_len=130, d_model=384, n_heads=3, head_dim=128)),
    (None, dict(n_layers=1, n_streams=5, mem_len=1, d_model=128, n_heads=4, head_dim=32)),
    (None, dict(n_layers=2, n_streams=1, mem_len=300, d_model=640, n_heads=10, head_dim=64)),
]


@pytest.mark.parametrize("name,kw", PLANES_CASES, ids=lambda x: str(x))
def test_populate_from_split_planes_matches_oracle(name, kw):
    """The workspace populate (operands split once into bf16 planes, then
    three bf16 products per k step) within 1e-4 of the oracle on every
    element, and bit-identical to the populate that splits every tile as it
    loads it (the same products in the same order); the workspace starts as
    NaN, so nothing may be read from it before it is written."""
    g = geometry(name, **kw)
    cache, wt, (E, WK, WV) = make_cache(g)
    ref_k, ref_v = cache.k.clone(), cache.v.clone()
    ws = cache.populate_workspace()
    assert ws is not None and ws.numel() * 4 == pc.cke_xattn_populate_workspace_bytes(cache.geom)
    ws.fill_(float("nan"))
    cache.k.fill_(float("nan"))
    cache.v.fill_(float("nan"))
    cache.populate(E, WK, WV, ws=ws)
    torch.cuda.synchronize()
    Kc, Vc = oracle_caches(g, wt)
    assert max_abs(to_np(cache.k), Kc) <= TOL["f32"]
    assert max_abs(to_np(cache.v), Vc) <= TOL["f32"]
    assert torch.equal(cache.k, ref_k) and torch.equal(cache.v, ref_v)
    assert cache.ready


@pytest.mark.parametrize("name,kw", PLANES_CASES, ids=lambda x: str(x))
def test_populate_from_prepared_weight_planes(name, kw):
    """Weight planes prepared once (cke_weight_planes) and reused by two
    populates of different encoder memories: each is bit-identical to the
    workspace populate that splits the weights itself (the oracle pins that
    one). Planes, workspace and caches start as NaN."""
    g = geometry(name, **kw)
    cache, wt, (E, WK, WV) = make_cache(g)
    nan = float("nan")
    ws = cache.populate_workspace()
    E2 = (E * -0.5 + 0.25).contiguous()
    refs = []
    for e_in in (E, E2):
        cache.populate(e_in, WK, WV, ws=ws)
        refs.append((cache.k.clone(), cache.v.clone()))
    HD = g.n_heads * g.head_dim
    nbytes = pc.cke_weight_planes_bytes(2 * g.n_layers, g.d_model, HD)
    assert nbytes == 2 * g.n_layers * 2 * HD * g.d_model * 2
    planes = torch.full((nbytes // 4,), -1, dtype=torch.int32, device=DEV)   # NaN bit patterns
    pc.cke_weight_planes(list(WK) + list(WV), planes)
    rws = torch.full((pc.cke_row_planes_bytes(g.n_streams * g.mem_len, g.d_model) // 4,), nan,
                     device=DEV)
    for e_in, (rk, rv) in zip((E, E2), refs):
        cache.k.fill_(nan)
        cache.v.fill_(nan)
        cache.populate_planes(e_in, planes, rws)
        torch.cuda.synchronize()
        assert torch.equal(cache.k, rk) and torch.equal(cache.v, rv)
        assert cache.ready
    # the planes of a subset of the weights, made by the same call, are the
    # matching slice of the whole
    part = torch.full((pc.cke_weight_planes_bytes(1, g.d_model, HD) // 4,), -1, dtype=torch.int32,
                      device=DEV)
    pc.cke_weight_planes([WV[-1]], part)
    torch.cuda.synchronize()
    assert torch.equal(part, planes[-part.numel():])


def test_populate_from_prepared_planes_refuses_short_buffers():
    g = geometry("base")
    cache, wt, (E, WK, WV) = make_cache(g)
    planes = cache.weight_planes(WK, WV)
    rws = cache.row_planes_workspace()
    cache.k.fill_(0.0)
    torch.cuda.synchronize()
    for p_, w_ in ((planes[:-128], rws), (planes, rws[:-64])):
        with pytest.raises(pc.CkeError) as e:
            cache.populate_planes(E, p_, w_)
        assert e.value.code == pc.CKE_EINVAL
    torch.cuda.synchronize()
    assert float(cache.k.abs().max()) == 0.0      # nothing was launched
    assert cache.ready                            # refused before the flag was touched


def test_populate_workspace_is_refused_when_too_small():
    g = geometry("base")
    cache, wt, (E, WK, WV) = make_cache(g)
    need = pc.cke_xattn_populate_workspace_bytes(cache.geom)
    small = torch.empty((need - 256) // 4, device=DEV)
    cache.k.fill_(0.0)
    with pytest.raises(pc.CkeError) as e:
        cache.populate(E, WK, WV, ws=small)
    assert e.value.code == pc.CKE_EINVAL
    torch.cuda.synchronize()
    assert float(cache.k.abs().max()) == 0.0      # nothing was launched


# -------------------------------------------------------------- cross decode
DEC_CASES = [
    ("tiny", {}),
    ("base", {}),
    ("beam", {}),
    (None, dict(n_layers=2, n_streams=3, n_q=8, mem_len=77, d_model=256, n_heads=4,
                head_dim=64)),
    (None, dict(n_layers=2, n_streams=3, n_q=3, mem_len=77, d_model=256, n_heads=4,
                head_dim=64, dtype="bf16")),
    (None, dict(n_layers=3, n_streams=2, mem_len=1, d_model=96, n_heads=3, head_dim=32)),
    (None, dict(n_layers=1, n_streams=1, n_q=2, mem_len=200, d_model=256, n_heads=2,
                head_dim=128, dtype="bf16")),
    (None, dict(n_layers=1, n_streams=1, n_q=5, mem_len=3001, d_model=128, n_heads=2,
                head_dim=64)),
    # either side of the short-memory path (one wave per head, no split)
    (None, dict(n_layers=1, n_streams=2, n_q=3, mem_len=64, d_model=128, n_heads=2, head_dim=64)),
    (None, dict(n_layers=1, n_streams=2, n_q=3, mem_len=65, d_model=128, n_heads=2, head_dim=64)),
    (None, dict(n_layers=1, n_streams=5, n_q=2, mem_len=15, d_model=256, n_heads=2, head_dim=128,
                dtype="bf16")),
    # a long memory: the split count reaches its cap (64) and the merge runs 4 batches
    (None, dict(n_layers=1, n_streams=1, n_q=2, mem_len=20000, d_model=128, n_heads=2,
                head_dim=64)),
    # Whisper Base geometry with the largest query count (8) on the split path
    (None, dict(n_layers=1, n_streams=1, n_q=8, mem_len=1500, d_model=512, n_heads=8,
                head_dim=64)),
    # more (stream, head) pairs than compute units (264, 300): split in 3 only to even out the
    # workgroups per unit, merged in launch (fp32 with 2 queries; bf16, 300 pairs, not a
    # multiple of 8)
    (None, dict(n_layers=1, n_streams=33, n_q=2, mem_len=800, d_model=256, n_heads=8,
                head_dim=32)),
    (None, dict(n_layers=1, n_streams=75, mem_len=800, d_model=128, n_heads=4, head_dim=32,
                dtype="bf16")),
    # 320 pairs = 256 whole + 64 in 8 pieces, two per unit (bf16, one query)
    (None, dict(n_layers=1, n_streams=40, mem_len=1536, d_model=256, n_heads=8, head_dim=32,
                dtype="bf16")),
    # 320 pairs = 256 whole (one workgroup each) + 64 split in 4: the whole-pairs plan (fp32,
    # and bf16 with 2 queries)
    (None, dict(n_layers=1, n_streams=40, mem_len=1024, d_model=256, n_heads=8, head_dim=32)),
    (None, dict(n_layers=1, n_streams=40, n_q=2, mem_len=1100, d_model=256, n_heads=8, head_dim=32,
                dtype="bf16")),
]


@pytest.mark.parametrize("name,kw", DEC_CASES, ids=lambda x: str(x))
def test_cross_decode_matches_oracle(name, kw):
    g = geometry(name, **kw)
    cache, wt, _ = make_cache(g)
    Kc, Vc = oracle_caches(g, wt)
    tol = TOL[g.dtype]
    for step in (0, 1):
        for layer in range(g.n_layers):
            q = synth.decode_call_inputs(g, step, layer)["q_cross"]
            out = cache.decode(t32(q), layer, g.scale)
            torch.cuda.synchronize()
            want = oracle.cross_decode(q, Kc[layer], Vc[layer], g.scale)
            err = max_abs(to_np(out), want)
            assert err <= tol, (step, layer, err)


WEIGHT_CASES = [
    ("base", {}, [0, 3, 5]),                                   # split over workgroups + merge
    (None, dict(n_layers=1, n_streams=16, mem_len=100, d_model=1280, n_heads=20, head_dim=64,
                dtype="bf16"), [2, 19, 7, 2]),                 # unsplit (one workgroup per head)
    (None, dict(n_layers=2, n_streams=5, n_q=3, mem_len=15, d_model=256, n_heads=4,
                head_dim=64), [1, 2]),                         # short memory, several queries
    (None, dict(n_layers=1, n_streams=2, n_q=2, mem_len=300, d_model=256, n_heads=2,
                head_dim=128, dtype="bf16"), [1]),
    (None, dict(n_layers=1, n_streams=3, mem_len=77, d_model=96, n_heads=3, head_dim=32), [0, 1, 2]),
    # streams 0-31 whole, streams 32-39 split in 4 (the whole-pairs plan)
    (None, dict(n_layers=1, n_streams=40, mem_len=1024, d_model=256, n_heads=8, head_dim=32),
     [0, 5, 7]),
]


@pytest.mark.parametrize("name,kw,heads", WEIGHT_CASES, ids=lambda x: str(x))
def test_cross_decode_weights_match_oracle(name, kw, heads):
    """Mean attention weights of the selected heads within the cache dtype's
    tolerance of the oracle, rows summing to 1, and the decode output of the
    same call unchanged."""
    g = geometry(name, **kw)
    cache, wt, _ = make_cache(g)
    Kc, Vc = oracle_caches(g, wt)
    tol = TOL[g.dtype]
    layer = g.n_layers - 1
    q = synth.decode_call_inputs(g, 1, layer)["q_cross"]
    out, w = cache.decode_weights(t32(q), layer, g.scale, heads)
    plain = cache.decode(t32(q), layer, g.scale)
    torch.cuda.synchronize()
    want_out, want_w = oracle.cross_decode_weights(q, Kc[layer], Vc[layer], g.scale, heads)
    assert max_abs(to_np(out), want_out) <= tol
    assert max_abs(to_np(w), want_w) <= tol
    np.testing.assert_allclose(to_np(w).sum(axis=-1), 1.0, atol=1e-4)
    np.testing.assert_array_equal(to_np(out), to_np(plain))


def test_cross_decode_peaked_softmax_and_shift_invariance():
    """A large scale concentrates the softmax (online max tracking across
    splits matters); adding one constant vector to every key of a head leaves
    the output unchanged (WhisperKit case study, section 2: a key bias is
    redundant under softmax)."""
    g = geometry("base")
    cache, wt, _ = make_cache(g)
    Kc, Vc = oracle_caches(g, wt)
    q = synth.decode_call_inputs(g, 5, 2)["q_cross"]
    out = cache.decode(t32(q), 2, 4.0)
    want = oracle.cross_decode(q, Kc[2], Vc[2], 4.0)
    assert max_abs(to_np(out), want) <= 1e-4
    base_out = to_np(cache.decode(t32(q), 3, g.scale))
    # bias per head chosen so that q . b = +40 for this query
    qv = q[0, 0]
    bias = qv / np.sum(qv * qv, axis=1, keepdims=True) * (40.0 / g.scale)
    cache.k[3, 0] += t32(bias)[:, None, :]
    shifted = to_np(cache.decode(t32(q), 3, g.scale))
    assert max_abs(shifted, base_out) <= 1e-4


def test_cross_decode_is_deterministic_and_nq_zero_is_noop():
    g = geometry("beam")
    cache, _, _ = make_cache(g)
    q = t32(synth.decode_call_inputs(g, 0, 0)["q_cross"])
    a = cache.decode(q, 1, g.scale).clone()
    b = cache.decode(q, 1, g.scale).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    out = torch.full_like(q, 7.0)
    pc.cke_xattn_decode(q, cache, 1, g.scale, out, n_q=0)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))


# Split geometries for the in-launch merge, with whether it applies (one pass
# of the split kernel's 256 threads must cover n_q * D * lanes, lanes = 1, 2,
# 4 or 8 for up to 8, 16, 32 or 64 splits): Whisper Base; B*H not a multiple
# of 8 (12 and 15 heads); 2, 13, 16 and 63 splits (odd split counts leave
# some lanes fewer splits); D = 32, 64 and 128; fp32, bf16 and fp8 rows;
# several queries. Beam's 5 queries, Base with 8, a 63-split head with 2
# queries and 3 queries of 128 dims take the second kernel (several
# workgroups per head).
MERGE_CASES = [
    ("base", {}, True),
    ("beam", {}, False),
    (None, dict(n_layers=2, n_streams=3, n_q=1, mem_len=777, d_model=256, n_heads=4, head_dim=64,
                dtype="bf16"), True),
    (None, dict(n_layers=1, n_streams=5, n_q=2, mem_len=300, d_model=96, n_heads=3, head_dim=32),
     True),
    (None, dict(n_layers=1, n_streams=8, n_q=1, mem_len=1000, d_model=256, n_heads=2, head_dim=128,
                dtype="fp8"), True),
    (None, dict(n_layers=1, n_streams=1, n_q=1, mem_len=20000, d_model=64, n_heads=2, head_dim=32),
     True),
    (None, dict(n_layers=1, n_streams=4, n_q=4, mem_len=500, d_model=128, n_heads=4, head_dim=32),
     True),
    (None, dict(n_layers=1, n_streams=32, n_q=1, mem_len=300, d_model=256, n_heads=4, head_dim=64),
     True),
    (None, dict(n_layers=1, n_streams=1, n_q=8, mem_len=1500, d_model=512, n_heads=8, head_dim=64),
     False),
    (None, dict(n_layers=1, n_streams=1, n_q=2, mem_len=20000, d_model=128, n_heads=2,
                head_dim=64), False),
    (None, dict(n_layers=1, n_streams=8, n_q=3, mem_len=900, d_model=256, n_heads=2, head_dim=128,
                dtype="bf16"), False),
    # 256 whole pairs + 64 split in 4 (only the split pairs merge)
    (None, dict(n_layers=1, n_streams=40, mem_len=1024, d_model=256, n_heads=8, head_dim=32),
     True),
]


def _ticket_words(cache):
    """The per-head arrival counters of a split cache's workspace (the layout
    cke_xattn_workspace_bytes documents): one 32-bit word every 128 bytes."""
    g = cache.geom
    ns = pc.cke_xattn_num_splits(g)
    al = lambda x: (x + 255) // 256 * 256
    stats_off = al(g.n_streams * g.max_q * g.n_heads * ns * (g.head_dim + 2) * 4)
    off = al(stats_off + g.n_streams * g.max_q * g.n_heads * 2 * 4)
    n = g.n_streams * g.n_heads
    words = cache.ws.view(torch.int32)[off // 4: off // 4 + 32 * n]
    return words.view(n, 32)[:, 0]


@pytest.mark.parametrize("name,kw,fused", MERGE_CASES, ids=lambda x: str(x))
def test_in_launch_merge_matches_the_merge_kernel_bit_for_bit(name, kw, fused):
    """The last-arriving workgroup of each head merges in the split kernel's
    own launch (mode 1) with the same bits as the second merge kernel (mode
    0), over consecutive calls (every call leaves the arrival counters at
    zero), with and without attention weights; and it is what runs by default
    on this device wherever it applies."""
    g = geometry(name, **kw)
    cache, wt, _ = make_cache(g)
    assert pc.cke_xattn_num_splits(cache.geom) > 1
    prev = pc.cke_xattn_set_merge_mode(1)
    try:
        assert pc.cke_xattn_merges_in_launch(cache, g.n_q) == fused, "placement probe failed?"
        runs = []
        for mode in (1, 0, 1):
            assert pc.cke_xattn_set_merge_mode(mode) in (0, 1)
            assert pc.cke_xattn_merges_in_launch(cache, g.n_q) == (fused and bool(mode))
            res = []
            for step in range(3):
                for layer in range(g.n_layers):
                    q = t32(synth.decode_call_inputs(g, step, layer)["q_cross"])
                    res.append(cache.decode(q, layer, g.scale).clone())
            q = t32(synth.decode_call_inputs(g, 3, 0)["q_cross"])
            out, w = cache.decode_weights(q, 0, g.scale, [0, g.n_heads - 1])
            res += [out.clone(), w.clone()]
            torch.cuda.synchronize()
            assert int(_ticket_words(cache).abs().sum()) == 0, mode
            runs.append(res)
        for a, b in zip(runs[0], runs[1]):
            assert torch.equal(a, b)
        for a, b in zip(runs[0], runs[2]):
            assert torch.equal(a, b)
        if g.dtype != "fp8":   # fp8: parity on the oracle's own fp8 values, test_fp8_cross_decode_*
            Kc, Vc = oracle_caches(g, wt)
            q = synth.decode_call_inputs(g, 0, 0)["q_cross"]
            want = oracle.cross_decode(q, Kc[0], Vc[0], g.scale)
            assert max_abs(to_np(runs[0][0]), want) <= TOL[g.dtype]
    finally:
        pc.cke_xattn_set_merge_mode(prev)


def test_populate_clears_the_arrival_counters():
    """Counters left non-zero (here: overwritten) are zeroed by the next
    populate, so the first decode after it merges every head."""
    g = geometry("base")
    cache, wt, (E, WK, WV) = make_cache(g)
    Kc, Vc = oracle_caches(g, wt)
    q = synth.decode_call_inputs(g, 0, 1)["q_cross"]
    good = cache.decode(t32(q), 1, g.scale).clone()
    words = _ticket_words(cache)
    words.fill_(5)
    cache.populate(E, WK, WV)
    out = torch.full_like(good, float("nan"))
    cache.decode(t32(q), 1, g.scale, out=out)
    torch.cuda.synchronize()
    assert int(_ticket_words(cache).abs().sum()) == 0
    assert torch.equal(out, good)
    assert max_abs(to_np(out), oracle.cross_decode(q, Kc[1], Vc[1], g.scale)) <= 1e-4


def test_ready_flag_on_gpu():
    """C-Kernel-Engine 'View 3': new encoder memory invalidates the cache and
    decode refuses (-2) until populate has run again."""
    g = geometry("tiny")
    cache, wt, (E, WK, WV) = make_cache(g)
    q = t32(synth.decode_call_inputs(g, 0, 0)["q_cross"])
    cache.decode(q, 0, g.scale)
    cache.invalidate()
    with pytest.raises(pc.CkeError) as e:
        cache.decode(q, 0, g.scale)
    assert e.value.code == -2
    # install new encoder memory, repopulate, and decode reads the new projection
    E2 = E * 2.0
    cache.populate(E2, WK, WV)
    out = cache.decode(q, 0, g.scale)
    Kc, Vc = oracle.populate(2.0 * wt["E"].astype(np.float64), wt["WK"], wt["WV"], g.n_heads,
                             g.head_dim)
    want = oracle.cross_decode(to_np(q), Kc[0], Vc[0], g.scale)
    assert max_abs(to_np(out), want) <= 1e-4


# ----------------------------------------------------- self append + attend
SELF_CASES = [
    dict(S=1, H=2, D=32, P=8, dtype="f32"),          # Tiny
    dict(S=1, H=8, D=64, P=448, dtype="f32"),        # Whisper Base, full capacity
    dict(S=5, H=8, D=64, P=40, dtype="f32"),         # beams
    dict(S=3, H=4, D=64, P=70, dtype="bf16"),
    dict(S=2, H=2, D=128, P=33, dtype="f32"),
    dict(S=2, H=3, D=128, P=33, dtype="bf16"),
    dict(S=2, H=2, D=64, P=200, dtype="bf16"),       # bf16 rows past 4 load tiles
    dict(S=2, H=2, D=32, P=1, dtype="f32"),          # capacity 1: only the new row, never a cache row
    dict(S=7, H=3, D=64, P=17, dtype="bf16"),        # odd sequence and head counts
]


@pytest.mark.parametrize("c", SELF_CASES, ids=lambda c: "S%d-H%d-D%d-P%d-%s" % tuple(c.values()))
def test_self_append_attend_matches_oracle(c):
    S, H, D, P = c["S"], c["H"], c["D"], c["P"]
    bf = c["dtype"] == "bf16"
    dt = torch.bfloat16 if bf else torch.float32
    kv = pc.KVLayer(S, H, D, P, dtype=dt)
    Ks = np.zeros((S, H, P, D))
    Vs = np.zeros((S, H, P, D))
    scale = 1 / math.sqrt(D)
    std = 0.02 * math.sqrt(H * D)
    worst = 0.0
    # every position: the wave that owns row pos changes with pos, and so do
    # the waves per workgroup the launcher picks
    for pos in range(P):
        key = [31, S, H, D, P, pos]
        q = synth.normal(key + [0], (S, H, D), std)
        kn = synth.normal(key + [1], (S, H, D), std)
        vn = synth.normal(key + [2], (S, H, D), std)
        out = kv.append_attend(t32(q), t32(kn), t32(vn), pos, scale)
        want = oracle.self_append_attend(q, kn, vn, Ks, Vs, pos, scale, round_bf16=bf)
        torch.cuda.synchronize()
        worst = max(worst, max_abs(to_np(out), want))
    torch.cuda.synchronize()
    assert worst <= 1e-4
    # the stored rows are exactly the scattered (rounded) inputs
    np.testing.assert_array_equal(to_np(kv.k), Ks)
    np.testing.assert_array_equal(to_np(kv.v), Vs)


PREFILL_CASES = [
    dict(S=1, n=3, Hq=8, Hkv=8, D=64, P=448, pos=0, dtype="f32"),     # Whisper Base ContextPrefill
    dict(S=2, n=5, Hq=6, Hkv=2, D=64, P=40, pos=7, dtype="bf16"),     # grouped kv heads
    dict(S=3, n=16, Hq=4, Hkv=1, D=128, P=64, pos=20, dtype="f32"),   # one kv head, D 128
    dict(S=2, n=1, Hq=8, Hkv=2, D=32, P=16, pos=15, dtype="f32"),     # one row, last position
    dict(S=4, n=33, Hq=20, Hkv=20, D=64, P=448, pos=100, dtype="bf16"),  # Large heads, 33-row chunk
    dict(S=1, n=448, Hq=8, Hkv=8, D=64, P=448, pos=0, dtype="f32"),   # the whole capacity at once
    dict(S=2, n=2, Hq=8, Hkv=2, D=128, P=24, pos=9, dtype="bf16"),    # 8 queries per kv head
    dict(S=1, n=12, Hq=2, Hkv=1, D=32, P=30, pos=3, dtype="bf16"),    # ragged last token group
]


def _random_prefill_cases(n, seed=2027):
    """Seeded random prefill shapes: 1-4 sequences and kv heads, 1-8 query
    heads per kv head, every head_dim, capacities up to 200, chunks up to 64
    rows anywhere in the cache."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        P = int(rng.integers(1, 201))
        rows = int(rng.integers(1, min(P, 64) + 1))
        Hkv = int(rng.integers(1, 5))
        out.append(dict(S=int(rng.integers(1, 5)), n=rows, Hq=Hkv * int(rng.choice([1, 2, 3, 4, 8])),
                        Hkv=Hkv, D=int(rng.choice([32, 64, 128])), P=P,
                        pos=int(rng.integers(0, P - rows + 1)), dtype=("f32", "bf16")[i % 2]))
    return out


PREFILL_CASES += _random_prefill_cases(12)


@pytest.mark.parametrize("c", PREFILL_CASES,
                         ids=lambda c: "S%d-n%d-Hq%d-Hkv%d-D%d-P%d-pos%d-%s" % tuple(c.values()))
def test_prefill_matches_oracle(c):
    """Several rows per sequence at once, grouped kv heads: output within the
    cache dtype's tolerance of the oracle, stored rows bit-exact, and the rows
    past the new ones (poisoned with NaN) neither read nor written."""
    S, n, Hq, Hkv, D, P, pos = (c[k] for k in ("S", "n", "Hq", "Hkv", "D", "P", "pos"))
    bf = c["dtype"] == "bf16"
    dt = torch.bfloat16 if bf else torch.float32
    r = np.random.default_rng([43, S, n, Hq, Hkv, D, P, pos])
    q = (r.standard_normal((S, n, Hq, D)) * 0.45).astype(np.float32)
    kn = (r.standard_normal((S, n, Hkv, D)) * 0.45).astype(np.float32)
    vn = (r.standard_normal((S, n, Hkv, D)) * 0.45).astype(np.float32)
    old = (r.standard_normal((S, Hkv, P, D)) * 0.45).astype(np.float32)
    old[:, :, pos + n:] = np.nan
    kv = pc.KVLayer(S, Hkv, D, P, dtype=dt)
    kv.k.copy_(torch.from_numpy(old).to(dt))
    kv.v.copy_(torch.from_numpy(-old).to(dt))
    Ks = kv.k.double().cpu().numpy().copy()
    Vs = kv.v.double().cpu().numpy().copy()
    scale = 1.0 / math.sqrt(D)
    out = kv.prefill_attend(t32(q), t32(kn), t32(vn), pos, scale)
    torch.cuda.synchronize()
    want = oracle.self_prefill_append(q, kn, vn, Ks, Vs, pos, scale, round_bf16=bf)
    assert max_abs(to_np(out), want) <= TOL[c["dtype"]]
    got_k = kv.k.double().cpu().numpy()
    got_v = kv.v.double().cpu().numpy()
    np.testing.assert_array_equal(got_k[:, :, :pos + n], Ks[:, :, :pos + n])
    np.testing.assert_array_equal(got_v[:, :, :pos + n], Vs[:, :, :pos + n])
    assert np.isnan(got_k[:, :, pos + n:]).all() and np.isnan(got_v[:, :, pos + n:]).all()


def test_self_rows_past_pos_are_never_read_or_written():
    """Poison every row past pos with NaN: the output equals the clean run bit
    for bit and the poisoned rows are untouched."""
    S, H, D, P = 2, 8, 64, 64
    for dt in (torch.float32, torch.bfloat16):
        clean = pc.KVLayer(S, H, D, P, dtype=dt)
        dirty = pc.KVLayer(S, H, D, P, dtype=dt)
        g = torch.Generator().manual_seed(5)
        for pos in range(0, 40):
            q, kn, vn = (torch.randn(S, H, D, generator=g).to(DEV) * 0.45 for _ in range(3))
            dirty.k[:, :, pos + 1:] = float("nan")
            dirty.v[:, :, pos + 1:] = float("nan")
            a = clean.append_attend(q, kn, vn, pos, 0.125)
            b = dirty.append_attend(q, kn, vn, pos, 0.125)
            torch.cuda.synchronize()
            assert torch.equal(a, b), pos
            assert bool(torch.isnan(dirty.k[:, :, pos + 1:]).all())
            assert torch.equal(clean.k[:, :, :pos + 1], dirty.k[:, :, :pos + 1])


# ------------------------------------------------- teacher-forced decode run
@pytest.mark.parametrize("name", ["tiny", "beam_tiny"])
def test_teacher_forced_decoder_run_matches_oracle(name):
    """Whole decode window in the order of the decoder body (self-attention,
    then cross-attention, per layer, per step): the oracle's harness decoder
    records every call's inputs and outputs; the GPU replays each call from
    the recorded inputs (teacher forcing) and must reproduce each output."""
    if name == "tiny":
        g = synth.get("tiny")
    else:
        g = geometry(None, n_layers=2, n_streams=1, n_q=3, n_seqs=3, mem_len=100, d_model=128,
                     n_heads=2, head_dim=64, steps=12, max_pos=12, scale=0.125, seed=9)
    names = ("E", "WK", "WV", "WQ", "WO", "WQs", "WKs", "WVs", "WOs", "x0")
    wt = synth.workload_tensors(g, names)
    W = {k: wt[k] for k in names[1:-1]}
    run = oracle.decoder_run("incremental", wt["E"], W, wt["x0"], n_heads=g.n_heads,
                             head_dim=g.head_dim, n_q=g.n_q, max_pos=g.max_pos, n_steps=g.steps,
                             scale=g.scale)
    cache, _, _ = make_cache(g, wt)
    kvs = [pc.KVLayer(g.n_seqs, g.n_heads, g.head_dim, g.max_pos) for _ in range(g.n_layers)]
    rec = run["rec"]
    shp_s = (g.n_seqs, g.n_heads, g.head_dim)
    shp_c = (g.n_streams, g.n_q, g.n_heads, g.head_dim)
    worst = 0.0
    for t in range(g.steps):
        for l in range(g.n_layers):
            so = kvs[l].append_attend(t32(rec["qs"][t, l].reshape(shp_s)),
                                      t32(rec["kn"][t, l].reshape(shp_s)),
                                      t32(rec["vn"][t, l].reshape(shp_s)), t, g.scale)
            co = cache.decode(t32(rec["qc"][t, l].reshape(shp_c)), l, g.scale)
            torch.cuda.synchronize()
            worst = max(worst, max_abs(to_np(so).reshape(g.n_seqs, -1), rec["so"][t, l]),
                        max_abs(to_np(co).reshape(g.n_seqs, -1), rec["co"][t, l]))
    assert worst <= 1e-4
    for l in range(g.n_layers):
        assert max_abs(to_np(kvs[l].k), run["Ks"][l].astype(np.float32)) == 0.0


# --------------------------------------------------------- decoder step
STEP_NAMES = ("WQs", "WKs", "WVs", "WOs", "WQ", "WO")


def _step_setup(g):
    """Populated GPU cache, the layer weights on the GPU and as float64, GPU
    self caches, the oracle's projection cache and empty oracle self caches."""
    wt = synth.workload_tensors(g, ("E", "WK", "WV") + STEP_NAMES + ("x0",))
    cache, _, _ = make_cache(g, wt)
    bf = g.dtype in ("bf16", "fp8")
    # the step takes output-major weights: the transpose of the oracle's y = x.W matrices
    dev_w = {k: ([tbf16(b.T) for b in wt[k + "_bits"]] if bf else [t32(w.T) for w in wt[k]])
             for k in STEP_NAMES}
    descs = [pc.decoder_layer_desc(*[dev_w[k][l] for k in STEP_NAMES]) for l in range(g.n_layers)]
    S = g.n_streams * g.n_q
    sdt = torch.bfloat16 if bf else torch.float32
    kvs = [pc.KVLayer(S, g.n_heads, g.head_dim, g.max_pos, dtype=sdt) for _ in range(g.n_layers)]
    ws = torch.empty(pc.cke_decoder_step_workspace_bytes(cache.geom, S) // 4, device=DEV)
    Kc, Vc = oracle_caches(g, wt)
    Ks = np.zeros((g.n_layers, S, g.n_heads, g.max_pos, g.head_dim))
    Vs = np.zeros_like(Ks)
    return dict(wt=wt, cache=cache, dev_w=dev_w, descs=descs, kvs=kvs, ws=ws, Kc=Kc, Vc=Vc,
                Ks=Ks, Vs=Vs, S=S, bf=bf)


STEP_CASES = [
    ("tiny", {}),
    (None, dict(n_layers=2, n_streams=1, n_q=1, mem_len=1500, d_model=512, n_heads=8,
                head_dim=64, max_pos=16)),
    (None, dict(n_layers=2, n_streams=1, n_q=5, mem_len=300, d_model=512, n_heads=8,
                head_dim=64, max_pos=16)),                     # 5 beams over one cache
    (None, dict(n_layers=2, n_streams=2, n_q=2, mem_len=77, d_model=256, n_heads=8,
                head_dim=32, max_pos=16)),                     # 2 streams x 2 queries
    (None, dict(n_layers=2, n_streams=3, n_q=1, mem_len=200, d_model=640, n_heads=5,
                head_dim=128, max_pos=16, dtype="bf16")),      # bf16 weights and caches
    (None, dict(n_layers=1, n_streams=2, n_q=8, mem_len=100, d_model=384, n_heads=6,
                head_dim=64, max_pos=16, dtype="bf16")),       # 16 sequences, one pass
    (None, dict(n_layers=1, n_streams=2, n_q=1, mem_len=1, d_model=256, n_heads=8,
                head_dim=32, max_pos=16)),                     # one memory row
    (None, dict(n_layers=1, n_streams=1, n_q=1, mem_len=300, d_model=512, n_heads=8,
                head_dim=64, max_pos=16, dtype="fp8")),        # over an fp8 cache
    (None, dict(n_layers=2, n_streams=1, n_q=1, mem_len=500, d_model=256, n_heads=8,
                head_dim=32, max_pos=16)),                     # split cross merged by the product
]


def _random_step_cases(n, seed=2030):
    """Seeded random decoder-layer steps: fp32, bf16 and fp8 caches in turn,
    every head_dim, 1-3 streams x 1-8 queries, ragged memories."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ("f32", "bf16", "fp8")[i % 3]
        D = int(rng.choice([32, 64, 128]))
        H = 256 * int(rng.integers(1, 3)) // D if dtype == "fp8" else int(rng.integers(1, 9))
        out.append((None, dict(n_layers=int(rng.integers(1, 3)), n_streams=int(rng.integers(1, 4)),
                               n_q=int(rng.integers(1, 9)), mem_len=int(rng.integers(1, 400)),
                               d_model=H * D, n_heads=H, head_dim=D, scale=1 / math.sqrt(D),
                               max_pos=8, dtype=dtype, seed=4000 + i)))
    return out


STEP_CASES += _random_step_cases(6)


@pytest.mark.parametrize("name,kw", STEP_CASES, ids=lambda x: str(x))
def test_decoder_layer_step_matches_oracle(name, kw):
    """Teacher-forced: every call gets the oracle's input hidden state; its
    output and the self-cache row it wrote are compared with the oracle's
    layer step, for several tokens and every layer."""
    g = geometry(name, **kw)
    g = dataclasses.replace(g, n_seqs=g.n_streams * g.n_q)
    st = _step_setup(g)
    tol = TOL["bf16" if st["bf"] else "f32"]
    W = [{k: st["wt"][k][l] for k in STEP_NAMES} for l in range(g.n_layers)]
    x = st["wt"]["x0"][:st["S"]].astype(np.float64)
    xd = torch.empty(st["S"], g.d_model, device=DEV)
    for t in range(3):
        for l in range(g.n_layers):
            xd.copy_(t32(x))
            pc.cke_decoder_layer_step(xd, st["descs"][l], st["kvs"][l], t, st["cache"], l, g.scale,
                                      st["ws"])
            x = oracle.decoder_layer_step(x, W[l], st["Kc"][l], st["Vc"][l], st["Ks"][l],
                                          st["Vs"][l], t, n_q=g.n_q, scale=g.scale,
                                          round_bf16=st["bf"])
            torch.cuda.synchronize()
            assert max_abs(to_np(xd), x) <= tol, (t, l, max_abs(to_np(xd), x))
            assert max_abs(to_np(st["kvs"][l].k[:, :, t]), st["Ks"][l][:, :, t]) <= tol
            assert max_abs(to_np(st["kvs"][l].v[:, :, t]), st["Vs"][l][:, :, t]) <= tol
        x = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True))
    # rows past the last position were never written
    assert float(np.abs(to_np(st["kvs"][0].k[:, :, 3:])).max(initial=0.0)) == 0.0


def test_decoder_layer_step_rejects_bad_pairings_on_a_ready_cache():
    g = geometry(None, n_layers=1, n_streams=2, n_q=2, n_seqs=4, mem_len=40, d_model=256,
                 n_heads=8, head_dim=32, max_pos=8)
    st = _step_setup(g)
    x = torch.zeros(st["S"], g.d_model, device=DEV)
    kv3 = pc.KVLayer(3, g.n_heads, g.head_dim, g.max_pos)      # 3 sequences over 2 streams
    kv6 = pc.KVLayer(6, g.n_heads, g.head_dim, g.max_pos)      # n_q = 3 > max_q = 2
    kvh = pc.KVLayer(4, 4, 64, g.max_pos)                      # other head split
    wsb = torch.zeros(pc.cke_decoder_step_workspace_bytes(st["cache"].geom, 6) // 4, device=DEV)
    for kv, code in ((kv3, pc.CKE_ERANGE), (kv6, pc.CKE_ERANGE), (kvh, pc.CKE_EINVAL)):
        xs = torch.zeros(kv.desc.n_seqs, g.d_model, device=DEV)
        with pytest.raises(pc.CkeError) as e:
            pc.cke_decoder_layer_step(xs, st["descs"][0], kv, 0, st["cache"], 0, g.scale, wsb)
        assert e.value.code == code
        assert float(xs.abs().max()) == 0.0
    with pytest.raises(pc.CkeError) as e:
        pc.cke_decoder_layer_step(x, st["descs"][0], st["kvs"][0], 8, st["cache"], 0, g.scale,
                                  st["ws"])
    assert e.value.code == pc.CKE_ERANGE
    torch.cuda.synchronize()
    assert float(x.abs().max()) == 0.0     # nothing was launched


# ------------------------------------------------------ projector memory lift
LIFT_CASES = [
    dict(rows=45, k_in=64, n=128, pos_rows=15),     # ragged row tile, three blocks of positions
    dict(rows=200, k_in=256, n=192, pos_rows=0),    # no positions
    dict(rows=64, k_in=4096, n=64, pos_rows=15),    # the Q-Former's input width
]


LIFT_CASES += [
    dict(rows=200, k_in=256, n=256, pos_rows=15),   # the split-planes path: k_in % 64, n % 128
    dict(rows=130, k_in=1024, n=384, pos_rows=0),
    dict(rows=200, k_in=1024, n=256, pos_rows=15),  # too few 192 x 256 tiles: 4 k slices
    dict(rows=45, k_in=2048, n=512, pos_rows=0),    # 4 k slices over a ragged row tile
    dict(rows=1500, k_in=1024, n=2560, pos_rows=15),  # 80 tiles: 2 k slices
]


@pytest.mark.parametrize("ws", [False, True], ids=["tile-split", "planes"])
@pytest.mark.parametrize("c", LIFT_CASES, ids=lambda c: "r%d-k%d-n%d-p%d" % tuple(c.values()))
def test_memory_lift_matches_oracle(c, ws):
    x = synth.normal([90, 0, c["rows"]], (c["rows"], c["k_in"]))
    W = synth.normal([90, 1, c["rows"]], (c["k_in"], c["n"]), 0.02)
    pos = synth.normal([90, 2, c["rows"]], (c["pos_rows"], c["n"]), 0.02) if c["pos_rows"] else None
    out = torch.full((c["rows"], c["n"]), float("nan"), device=DEV)
    wsb = None
    if ws:
        need = pc.cke_memory_lift_workspace_bytes(c["rows"], c["k_in"], c["n"])
        if need == 0:
            assert c["k_in"] % 64 or c["n"] % 128
        wsb = torch.full((max(need, 256) // 4,), float("nan"), device=DEV)
    pc.cke_memory_lift_gelu(t32(x), t32(W), out, None if pos is None else t32(pos), ws=wsb)
    torch.cuda.synchronize()
    want = oracle.lift_gelu(x, W, pos)
    assert max_abs(to_np(out), want) <= TOL["f32"]


@pytest.mark.parametrize("c", [c for c in LIFT_CASES if c["k_in"] % 64 == 0 and c["n"] % 128 == 0],
                         ids=lambda c: "r%d-k%d-n%d-p%d" % tuple(c.values()))
def test_memory_lift_from_prepared_weight_planes(c):
    """The lift from a weight split once by cke_weight_planes is
    bit-identical to the workspace lift that splits it per call."""
    x = synth.normal([90, 0, c["rows"]], (c["rows"], c["k_in"]))
    W = synth.normal([90, 1, c["rows"]], (c["k_in"], c["n"]), 0.02)
    pos = synth.normal([90, 2, c["rows"]], (c["pos_rows"], c["n"]), 0.02) if c["pos_rows"] else None
    pos_t = None if pos is None else t32(pos)
    need = pc.cke_memory_lift_workspace_bytes(c["rows"], c["k_in"], c["n"])
    ref = torch.empty((c["rows"], c["n"]), device=DEV)
    pc.cke_memory_lift_gelu(t32(x), t32(W), ref, pos_t, ws=torch.empty(need // 4, device=DEV))
    planes = pc.weight_planes([t32(W)])
    rws = torch.full((pc.cke_memory_lift_planes_workspace_bytes(c["rows"], c["k_in"], c["n"]) // 4,), float("nan"), device=DEV)
    out = torch.full((c["rows"], c["n"]), float("nan"), device=DEV)
    pc.cke_memory_lift_gelu_planes(t32(x), planes, c["n"], out, rws, pos=pos_t)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert max_abs(to_np(out), oracle.lift_gelu(x, W, pos)) <= TOL["f32"]
    again = torch.full_like(out, float("nan"))      # k slices are added in a fixed order
    pc.cke_memory_lift_gelu_planes(t32(x), planes, c["n"], again, rws, pos=pos_t)
    torch.cuda.synchronize()
    assert torch.equal(again, out)


def fp8_bracket(exact, absdot, dm):
    """Lowest and highest fp8 values a correct populate may store for the
    exact products `exact`. The kernel sums dm products of bf16 values, each
    exact in fp32, in fp32: in any order the sum errs by at most
    dm * 2^-24 * sum|e w| to first order (doubled here to cover the second);
    rounding is monotone, so the stored value lies between the roundings of
    the two ends of that interval."""
    bound = 2.0 * dm * 2.0 ** -24 * absdot
    return oracle.round_fp8(exact - bound), oracle.round_fp8(exact + bound)


def _abs_products(E, W, H, D):
    """sum_k |E[b,t,k]| |W[k,n]| as [B][H][T][D]."""
    B, T, _ = E.shape
    a = np.abs(np.asarray(E, np.float64)) @ np.abs(np.asarray(W, np.float64))
    return a.reshape(B, T, H, D).transpose(0, 2, 1, 3)


def _random_fp8_geometries(n, seed=2028):
    """Seeded random fp8-cache shapes (H*D a multiple of 256, as its populate
    requires): every head_dim, 1-2 layers, 1-3 streams, 1-8 queries, ragged
    memories."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([32, 64, 128]))
        H = 256 * int(rng.integers(1, 4)) // D
        out.append(dict(n_layers=int(rng.integers(1, 3)), n_streams=int(rng.integers(1, 4)),
                        n_q=int(rng.integers(1, 9)), mem_len=int(rng.integers(1, 700)),
                        d_model=H * D, n_heads=H, head_dim=D, scale=1 / math.sqrt(D),
                        seed=3000 + i))
    return out



FP8_POP_CASES = [
    dict(n_layers=2, n_streams=3, mem_len=100, d_model=256, n_heads=8, head_dim=32),
    dict(n_layers=1, n_streams=2, mem_len=300, d_model=512, n_heads=8, head_dim=64),
    dict(n_layers=1, n_streams=1, mem_len=257, d_model=256, n_heads=2, head_dim=128),
    # values past the largest finite fp8 (448) are clamped to it
    dict(n_layers=1, n_streams=1, mem_len=64, d_model=256, n_heads=4, head_dim=64, e_std=1000.0),
    # values in the subnormal range (below 2^-6)
    dict(n_layers=1, n_streams=2, mem_len=40, d_model=256, n_heads=4, head_dim=64, e_std=0.02),
]
FP8_POP_CASES += _random_fp8_geometries(6, seed=2029)


@pytest.mark.parametrize("kw", FP8_POP_CASES, ids=lambda x: str(x))
def test_fp8_populate_rounds_the_exact_products(kw):
    g = geometry(None, dtype="fp8", **kw)
    cache, wt, _ = make_cache(g)
    Kx, Vx = oracle.populate(wt["E"], wt["WK"], wt["WV"], g.n_heads, g.head_dim)
    flips = 0
    for l in range(g.n_layers):
        for got, exact, W in ((cache.k[l], Kx[l], wt["WK"][l]), (cache.v[l], Vx[l], wt["WV"][l])):
            lo, hi = fp8_bracket(exact, _abs_products(wt["E"], W, g.n_heads, g.head_dim), g.d_model)
            got = to_np(got)
            assert np.all(got >= lo) and np.all(got <= hi)
            flips += int(np.count_nonzero(got != oracle.round_fp8(exact)))
    # a stored value other than the rounding of the exact product needs the
    # exact value within the accumulation error of a rounding boundary: rare
    assert flips <= max(2, 1e-3 * 2 * Kx.size)
    if kw.get("e_std", 1.0) > 100:
        assert float(to_np(cache.k).max()) == 448.0 and float(to_np(cache.k).min()) == -448.0
    assert cache.ready


FP8_DEC_CASES = [
    dict(n_layers=2, n_streams=3, mem_len=1500, d_model=512, n_heads=8, head_dim=64),
    dict(n_layers=2, n_streams=3, n_q=3, mem_len=77, d_model=256, n_heads=4, head_dim=64),
    dict(n_layers=1, n_streams=5, n_q=2, mem_len=15, d_model=256, n_heads=2, head_dim=128),
    dict(n_layers=1, n_streams=2, n_q=8, mem_len=300, d_model=256, n_heads=8, head_dim=32),
    dict(n_layers=1, n_streams=1, n_q=5, mem_len=3001, d_model=256, n_heads=2, head_dim=128),
    dict(n_layers=2, n_streams=3, n_q=2, mem_len=1, d_model=256, n_heads=4, head_dim=64),
]

FP8_DEC_CASES += _random_fp8_geometries(6)


def _fp8_cache_with_oracle_values(g):
    """A populated (ready) GPU fp8 cache whose contents are then replaced by
    the oracle's fp8 cache, so that kernel and oracle attend over identical
    values."""
    cache, wt, _ = make_cache(g)
    Kc, Vc = oracle.populate(wt["E"], wt["WK"], wt["WV"], g.n_heads, g.head_dim, round_fp8=True)
    cache.k.copy_(tfp8(Kc))
    cache.v.copy_(tfp8(Vc))
    torch.cuda.synchronize()
    return cache, Kc, Vc


@pytest.mark.parametrize("kw", FP8_DEC_CASES, ids=lambda x: str(x))
def test_fp8_cross_decode_matches_oracle(kw):
    g = geometry(None, dtype="fp8", **kw)
    cache, Kc, Vc = _fp8_cache_with_oracle_values(g)
    assert cache.ready
    for layer in range(g.n_layers):
        q = synth.decode_call_inputs(g, 1, layer)["q_cross"]
        out = cache.decode(t32(q), layer, g.scale)
        torch.cuda.synchronize()
        want = oracle.cross_decode(q, Kc[layer], Vc[layer], g.scale)
        assert max_abs(to_np(out), want) <= TOL["f32"], layer


@pytest.mark.parametrize("kw,heads", [
    (dict(n_layers=1, n_streams=2, mem_len=1500, d_model=512, n_heads=8, head_dim=64), [0, 5, 7]),
    (dict(n_layers=1, n_streams=5, n_q=3, mem_len=15, d_model=256, n_heads=4, head_dim=64), [3]),
    (dict(n_layers=1, n_streams=2, n_q=2, mem_len=300, d_model=256, n_heads=8, head_dim=32), [1, 1, 6]),
], ids=lambda x: str(x))
def test_fp8_cross_decode_weights_match_oracle(kw, heads):
    g = geometry(None, dtype="fp8", **kw)
    cache, Kc, Vc = _fp8_cache_with_oracle_values(g)
    q = synth.decode_call_inputs(g, 2, 0)["q_cross"]
    out, w = cache.decode_weights(t32(q), 0, g.scale, heads)
    torch.cuda.synchronize()
    want_out, want_w = oracle.cross_decode_weights(q, Kc[0], Vc[0], g.scale, heads)
    assert max_abs(to_np(out), want_out) <= TOL["f32"]
    assert max_abs(to_np(w), want_w) <= TOL["f32"]


# ---------------------------------------------------- full-size workloads
# The workloads at their full sizes, in the launch configuration the benchmark
# times. What the oracle can compute one element at a time is compared
# element by element; the rest is covered by properties that hold at any size:
#   - every output element is written (outputs and caches start as NaN);
#   - populate: every 256 x 256 output tile of the grouped product (rows of
#     the B*T memory rows, all columns of every layer) is compared on its
#     first, last and one random row, against the oracle's projection of
#     just those rows; and every (layer, stream, head) slab satisfies a
#     random-sign projection identity, K.r = E.(W_h r), within the rounding
#     bound of the cache type (Freivalds' check: a wrong row, column block or
#     tile anywhere breaks it);
#   - decode: every (stream, query, head) output at the first and the last
#     layer, over seeded slabs written into the cache, against the oracle on
#     the same slabs.
def _nan_fill(t):
    if t.dtype == torch.float8_e4m3fn:
        t.view(torch.uint8).fill_(0x7F)      # E4M3 NaN
    else:
        t.fill_(float("nan"))


def _finite_per_layer(t):
    return all(bool(torch.isfinite(t[l].float()).all()) for l in range(t.shape[0]))


def _tile_rows(M, tile, rng):
    """First, last and one random row of every `tile`-row block of M rows."""
    rows = set()
    for r0 in range(0, M, tile):
        r1 = min(M, r0 + tile) - 1
        rows.update((r0, r1, int(rng.integers(r0, r1 + 1))))
    return np.array(sorted(rows))


def _round_bracket(exact, absdot, dm, dtype):
    """Lowest and highest values a correct populate may store: the roundings
    (bf16 or fp8, both monotone) of exact -/+ the fp32 accumulation bound
    (products of bf16 values are exact in fp32; a dm-term fp32 sum errs by at
    most dm * 2^-24 * sum|e w| to first order, doubled for the second)."""
    bound = 2.0 * dm * 2.0 ** -24 * absdot
    rnd = oracle.round_fp8 if dtype == "fp8" else oracle.round_bf16
    return rnd(exact - bound), rnd(exact + bound)


# per stored element: largest rounding error relative to the value (half an
# ulp: 2^-9 for bf16, 2^-4 for E4M3, with a factor 2-4 of margin for the fp32
# accumulation) and the absolute floor (E4M3 subnormal spacing 2^-9)
_FREIVALDS = {"bf16": (2.0 ** -7, 1e-3), "fp8": (2.0 ** -3, 64 * 2.0 ** -10 + 1e-3)}


@pytest.mark.parametrize("name", ["large", "large_fp8"])
def test_full_size_populate_every_tile(name):
    g = synth.get(name)
    wt = synth.workload_tensors(g)
    cache = pc.XattnCache(g.n_layers, g.n_streams, g.mem_len, g.d_model, g.n_heads, g.head_dim,
                          max_q=g.n_q, dtype=CACHE_DT[g.dtype])
    _nan_fill(cache.k)
    _nan_fill(cache.v)
    E = tbf16(wt["E_bits"])
    WK = [tbf16(b) for b in wt["WK_bits"]]
    WV = [tbf16(b) for b in wt["WV_bits"]]
    cache.populate(E, WK, WV)
    torch.cuda.synchronize()
    assert cache.ready
    assert _finite_per_layer(cache.k) and _finite_per_layer(cache.v)
    B, T, H, D, L, dm = g.n_streams, g.mem_len, g.n_heads, g.head_dim, g.n_layers, g.d_model
    # every 256 x 256 tile: its first, last and one random row, all columns
    rows = _tile_rows(B * T, 256, np.random.default_rng(77))
    worst = 0.0
    for b in range(B):
        rb = rows[(rows // T) == b] % T
        if len(rb) == 0:
            continue
        Kx, Vx = oracle.populate(wt["E"][b:b + 1, rb], wt["WK"], wt["WV"], H, D)
        idx = torch.from_numpy(rb).to(DEV)
        absE = np.abs(wt["E"][b, rb].astype(np.float64))
        for got_all, exact_all, Ws in ((cache.k, Kx, wt["WK"]), (cache.v, Vx, wt["WV"])):
            got = to_np(got_all[:, b].index_select(2, idx))          # [L][H][n][D]
            for l in range(L):
                absdot = (absE @ np.abs(Ws[l].astype(np.float64))).reshape(len(rb), H, D)
                lo, hi = _round_bracket(exact_all[l, 0], absdot.transpose(1, 0, 2), dm, g.dtype)
                assert np.all(got[l] >= lo) and np.all(got[l] <= hi), (b, l)
                if g.dtype == "bf16":
                    worst = max(worst, max_abs(got[l], oracle.round_bf16(exact_all[l, 0])))
    assert worst <= TOL["bf16"]
    # Freivalds: K_l[b][h] . r == E_b . (W_l[:, h] r) for every slab, all rows
    rel, floor = _FREIVALDS[g.dtype]
    r = np.random.default_rng(78).choice([-1.0, 1.0], size=D)
    r_dev = torch.from_numpy(r).float().to(DEV)
    E64 = wt["E"].astype(np.float64)
    for got_all, Ws in ((cache.k, wt["WK"]), (cache.v, wt["WV"])):
        for l in range(L):
            slab = got_all[l].float()                                   # [B][H][T][D]
            y = to_np(slab @ r_dev)                                     # [B][H][T]
            mag = to_np(slab.abs().sum(-1))
            wr = Ws[l].astype(np.float64).reshape(dm, H, D) @ r         # [dm][H]
            want = (E64 @ wr).transpose(0, 2, 1)                        # [B][H][T]
            assert np.all(np.abs(y - want) <= rel * mag + floor), l


@pytest.mark.parametrize("name", ["large", "large_fp8"])
def test_full_size_decode_every_head(name):
    """Every (stream, head) output of the full-size decode, at the first and
    the last layer, with the cache holding seeded slabs of the projected
    spread (stored exactly in the cache type), against the oracle on the same
    slabs. A cache this large (K and V of 32 layers, far above the 256 MB
    MALL) is read with streaming loads, and of its 320 heads 256 run whole
    and 64 are split (in 8 over the bf16 cache, 4 over fp8) and merged in the
    same launch: this is those paths' full-size parity case."""
    g = synth.get(name)
    cache = pc.XattnCache(g.n_layers, g.n_streams, g.mem_len, g.d_model, g.n_heads, g.head_dim,
                          max_q=g.n_q, dtype=CACHE_DT[g.dtype])
    zeros_e = torch.zeros(g.n_streams, g.mem_len, g.d_model, dtype=torch.bfloat16, device=DEV)
    zeros_w = [torch.zeros(g.d_model, g.hd, dtype=torch.bfloat16, device=DEV)] * g.n_layers
    cache.populate(zeros_e, zeros_w, zeros_w)            # sets the ready flag
    del zeros_e
    shape = (g.n_streams, g.n_heads, g.mem_len, g.head_dim)
    for l in (0, g.n_layers - 1):
        kv = []
        for which, dst in ((0, cache.k[l]), (1, cache.v[l])):
            x = torch.from_numpy(synth.normal([g.seed, 90, l, which], shape, synth.q_std(g)))
            x = x.to(CACHE_DT[g.dtype])                  # the slab as stored (rounded)
            dst.copy_(x.to(DEV))
            kv.append(x.double().numpy())
        for step in (0, 5):
            q = synth.decode_call_inputs(g, step, l)["q_cross"]
            out = torch.full(q.shape, float("nan"), device=DEV)
            pc.cke_xattn_decode(t32(q), cache, l, g.scale, out)
            torch.cuda.synchronize()
            got = to_np(out)
            assert np.isfinite(got).all()
            want = oracle.cross_decode(q, kv[0], kv[1], g.scale)
            assert max_abs(got, want) <= TOL["f32"], (l, step)
    # the full-size heads are split and merged in launch
    assert pc.cke_xattn_num_splits(cache.geom) == (8 if g.dtype == "bf16" else 4)
    assert pc.cke_xattn_whole_pairs(cache.geom) == 256
    assert pc.cke_xattn_merges_in_launch(cache, g.n_q)


def test_large_self_attention_every_position():
    """Large workload's self-attention: 16 sequences x 20 heads, bf16 cache of
    capacity 448, all 128 decode positions; every output compared, stored rows
    bit-exact."""
    g = synth.get("large")
    kv = pc.KVLayer(g.n_seqs, g.n_heads, g.head_dim, g.max_pos, dtype=torch.bfloat16)
    Ks = np.zeros((g.n_seqs, g.n_heads, g.max_pos, g.head_dim))
    Vs = np.zeros_like(Ks)
    worst = 0.0
    for pos in range(g.steps):
        d = synth.decode_call_inputs(g, pos, 0)
        out = kv.append_attend(t32(d["q_self"]), t32(d["k_new"]), t32(d["v_new"]), pos, g.scale)
        want = oracle.self_append_attend(d["q_self"], d["k_new"], d["v_new"], Ks, Vs, pos,
                                         g.scale, round_bf16=True)
        worst = max(worst, max_abs(to_np(out), want))
    assert worst <= 1e-4
    np.testing.assert_array_equal(to_np(kv.k), Ks)
    np.testing.assert_array_equal(to_np(kv.v), Vs)


def test_qformer_memory_lift_full_size():
    """The Q-Former workload's lift at full size (1500 x 4096 -> 2048, 15
    position rows): every element against the oracle, per-tile split, split
    planes in the workspace, and (the path bench.py times) the weight split
    once into planes, with the product split over k in four slices."""
    g = synth.get("qformer")
    wt = synth.workload_tensors(g, ("X_lift", "W_lift", "pos"))
    rows = g.n_streams * g.mem_len
    want = oracle.lift_gelu(wt["X_lift"], wt["W_lift"], wt["pos"])
    need = pc.cke_memory_lift_workspace_bytes(rows, g.lift_in, g.d_model)
    assert need > 0
    for ws in (None, torch.full((need // 4,), float("nan"), device=DEV)):
        out = torch.full((rows, g.d_model), float("nan"), device=DEV)
        pc.cke_memory_lift_gelu(t32(wt["X_lift"]), t32(wt["W_lift"]), out, t32(wt["pos"]), ws=ws)
        torch.cuda.synchronize()
        assert max_abs(to_np(out), want) <= TOL["f32"], ws is None
    assert pc.cke_memory_lift_planes_workspace_bytes(rows, g.lift_in, g.d_model) > \
        pc.cke_row_planes_bytes(rows, g.lift_in)                     # split over k
    planes = pc.weight_planes([t32(wt["W_lift"])])
    rws = torch.full((pc.cke_memory_lift_planes_workspace_bytes(rows, g.lift_in, g.d_model) // 4,),
                     float("nan"), device=DEV)
    out = torch.full((rows, g.d_model), float("nan"), device=DEV)
    pc.cke_memory_lift_gelu_planes(t32(wt["X_lift"]), planes, g.d_model, out, rws, pos=t32(wt["pos"]))
    torch.cuda.synchronize()
    assert max_abs(to_np(out), want) <= TOL["f32"]


def test_qformer_populate_and_decode_full_size():
    """The Q-Former workload's projections and block-local decode at full
    size: populate from the lifted memory (the oracle's lift, rounded to fp32)
    compared on every element of both layers; decode of every block, query and
    head over the oracle's cache written into the library's cache."""
    g = synth.get("qformer")
    lt = synth.workload_tensors(g, ("X_lift", "W_lift", "pos"))
    E = oracle.lift_gelu(lt["X_lift"], lt["W_lift"], lt["pos"]).astype(np.float32)
    E = E.reshape(g.n_streams, g.mem_len, g.d_model)
    wt = synth.workload_tensors(g)
    cache = pc.XattnCache(g.n_layers, g.n_streams, g.mem_len, g.d_model, g.n_heads, g.head_dim,
                          max_q=g.n_q)
    Kc, Vc = oracle.populate(E, wt["WK"], wt["WV"], g.n_heads, g.head_dim)
    ws = cache.populate_workspace()
    assert ws is not None
    WK, WV = [t32(x) for x in wt["WK"]], [t32(x) for x in wt["WV"]]
    for mode in ("tile", "ws", "planes"):   # per-tile split, planes in the workspace, prepared planes
        _nan_fill(cache.k)
        _nan_fill(cache.v)
        if mode == "planes":
            rws = cache.row_planes_workspace()
            rws.fill_(float("nan"))
            cache.populate_planes(t32(E), cache.weight_planes(WK, WV), rws)
        else:
            if mode == "ws":
                ws.fill_(float("nan"))
            cache.populate(t32(E), WK, WV, ws=ws if mode == "ws" else None)
        torch.cuda.synchronize()
        assert max_abs(to_np(cache.k), Kc) <= TOL["f32"], mode
        assert max_abs(to_np(cache.v), Vc) <= TOL["f32"], mode
    K32, V32 = Kc.astype(np.float32), Vc.astype(np.float32)
    cache.k.copy_(t32(K32))
    cache.v.copy_(t32(V32))
    for l in range(g.n_layers):
        q = synth.decode_call_inputs(g, 0, l)["q_cross"]
        out = torch.full(q.shape, float("nan"), device=DEV)
        pc.cke_xattn_decode(t32(q), cache, l, g.scale, out)
        torch.cuda.synchronize()
        want = oracle.cross_decode(q, K32[l], V32[l], g.scale)
        assert max_abs(to_np(out), want) <= TOL["f32"], l


# ------------------------------------------- split count and resume from state
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_split_count_does_not_change_the_result(dtype):
    """The same head's keys and values, decoded in geometries whose key splits
    differ (32, 8 and 1 workgroups per head, the last with no merge), give the
    same output to within fp32 summation-order effects, and each matches the
    oracle."""
    T, H, D = 1500, 8, 64
    dm = H * D
    std = 0.02 * math.sqrt(dm)
    r = np.random.default_rng(404)
    kx = torch.from_numpy(r.standard_normal((H, T, D)) * std).float().to(CACHE_DT[dtype])
    vx = torch.from_numpy(r.standard_normal((H, T, D)) * std).float().to(CACHE_DT[dtype])
    q = (r.standard_normal((1, 2, H, D)) * std).astype(np.float32)
    want = oracle.cross_decode(q, kx.double().numpy()[None], vx.double().numpy()[None], 0.125)
    in_dt = torch.float32 if dtype == "f32" else torch.bfloat16
    outs, splits = [], []
    for B in (1, 4, 32):
        cache = pc.XattnCache(1, B, T, dm, H, D, max_q=2, dtype=CACHE_DT[dtype])
        cache.populate(torch.zeros(B, T, dm, dtype=in_dt, device=DEV),
                       [torch.zeros(dm, dm, dtype=in_dt, device=DEV)],
                       [torch.zeros(dm, dm, dtype=in_dt, device=DEV)])
        cache.k[0].copy_(kx.to(DEV).expand(B, H, T, D))
        cache.v[0].copy_(vx.to(DEV).expand(B, H, T, D))
        out = cache.decode(t32(q).expand(B, 2, H, D).contiguous(), 0, 0.125)
        torch.cuda.synchronize()
        o = to_np(out)
        for b in range(1, B):   # identical streams are computed identically
            np.testing.assert_array_equal(o[b], o[0])
        outs.append(o[0])
        splits.append(cache.n_splits)
        assert max_abs(o[0:1], want) <= TOL["f32"], B
    assert splits[0] > splits[1] > splits[2] == 1, splits
    for o in outs[1:]:
        assert max_abs(o, outs[0]) <= 2e-6


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_resumes_bit_identically_from_host_copies_of_its_state(dtype):
    """The caches are ordinary inputs and outputs ('Recurrence as feeds',
    'What it opened'): stop a decode window at step k, copy the projection
    cache, every layer's self cache and pos to host memory, drop every device
    buffer and handle, restore into fresh ones and continue. Every output of
    the resumed run equals the uninterrupted run's bit for bit."""
    if dtype == "f32":
        g = dataclasses.replace(synth.get("base"), steps=16)
    else:
        g = geometry(None, n_layers=2, n_streams=2, n_q=1, n_seqs=2, mem_len=700, d_model=512,
                     n_heads=8, head_dim=64, dtype="bf16", scale=0.125, steps=16, max_pos=32)
    k_stop = 7
    wt = synth.workload_tensors(g)
    sdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    calls = [[synth.decode_call_inputs(g, t, l) for l in range(g.n_layers)]
             for t in range(g.steps)]

    def fresh():
        cache, _, _ = make_cache(g, wt)
        kvs = [pc.KVLayer(g.n_seqs, g.n_heads, g.head_dim, g.max_pos, dtype=sdt)
               for _ in range(g.n_layers)]
        return cache, kvs

    def run(cache, kvs, t0, t1):
        outs = []
        for t in range(t0, t1):
            for l in range(g.n_layers):
                d = calls[t][l]
                so = kvs[l].append_attend(t32(d["q_self"]), t32(d["k_new"]), t32(d["v_new"]), t,
                                          g.scale)
                co = cache.decode(t32(d["q_cross"]), l, g.scale)
                outs += [so, co]
        torch.cuda.synchronize()
        return [o.cpu() for o in outs]

    cache, kvs = fresh()
    want = run(cache, kvs, 0, g.steps)
    del cache, kvs

    cache, kvs = fresh()
    got = run(cache, kvs, 0, k_stop)
    saved = {"pos": k_stop, "k": cache.k.cpu(), "v": cache.v.cpu(),
             "self": [(kv.k.cpu(), kv.v.cpu()) for kv in kvs]}
    cache.close()
    del cache, kvs
    torch.cuda.synchronize()

    cache, kvs = fresh()                 # new tensors and handles, populated afresh
    assert torch.equal(cache.k.cpu().view(torch.uint8), saved["k"].view(torch.uint8))
    cache.k.copy_(saved["k"].to(DEV))
    cache.v.copy_(saved["v"].to(DEV))
    for kv, (k, v) in zip(kvs, saved["self"]):
        kv.k.copy_(k.to(DEV))
        kv.v.copy_(v.to(DEV))
    got += run(cache, kvs, saved["pos"], g.steps)
    assert len(got) == len(want)
    for i, (a, b) in enumerate(zip(got, want)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), i


# ------------------------------------------------------------ graph replay
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_graph_replays_match_the_eager_window(dtype):
    """The call sequence bench.py times, captured once into a HIP graph:
    populate, then for four positions and both layers one self-attention append
    and one cross decode. Replayed three times, with eager resets and
    synchronisations in between, every replay must reproduce the eager run's
    outputs and self caches bit for bit (all kernels are deterministic)."""
    g = geometry(None, n_layers=2, n_streams=2, n_q=1, mem_len=300, d_model=256, n_heads=4,
                 head_dim=64, dtype=dtype, scale=0.125, max_pos=8)
    cache, wt, (E, WK, WV) = make_cache(g)
    S, H, D, P, L, steps = g.n_streams, g.n_heads, g.head_dim, g.max_pos, g.n_layers, 4
    kdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kvs = [pc.KVLayer(S, H, D, P, dtype=kdt) for _ in range(L)]
    r = np.random.default_rng(55)
    qs, kn, vn, qc = ([[t32(r.standard_normal((S, H, D)) * 0.45) for _ in range(L)] for _ in range(steps)]
                      for _ in range(4))
    qc = [[q.view(S, 1, H, D) for q in row] for row in qc]
    so = [[torch.empty(S, H, D, device=DEV) for _ in range(L)] for _ in range(steps)]
    co = [[torch.empty(S, 1, H, D, device=DEV) for _ in range(L)] for _ in range(steps)]

    def window():
        cache.populate(E, WK, WV)
        for t in range(steps):
            for l in range(L):
                kvs[l].append_attend(qs[t][l], kn[t][l], vn[t][l], t, g.scale, out=so[t][l])
                pc.cke_xattn_decode(qc[t][l], cache, l, g.scale, co[t][l])

    def reset():
        for kv in kvs:
            kv.k.zero_()
            kv.v.zero_()
        for row in so + co:
            for o in row:
                o.fill_(float("nan"))
        cache.k.fill_(float("nan"))
        cache.v.fill_(float("nan"))
        torch.cuda.synchronize()

    def snapshot():
        torch.cuda.synchronize()
        return ([o.clone() for row in so + co for o in row]
                + [x.clone() for kv in kvs for x in (kv.k, kv.v)] + [cache.k.clone(), cache.v.clone()])

    reset()
    window()
    want = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    reset()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        window()
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        graph.replay()
        got = snapshot()
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rep
        torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_graph_replays_of_decoder_layer_steps_match_eager(dtype):
    """Three positions of decoder-layer steps over both layers (seven launches
    each, workspace reused), captured once and replayed three times: the hidden
    state and the self caches match the eager run bit for bit."""
    g = geometry(None, n_layers=2, n_streams=2, n_q=2, n_seqs=4, mem_len=500, d_model=256,
                 n_heads=8, head_dim=32, dtype=dtype, scale=1 / math.sqrt(32), max_pos=8)
    st = _step_setup(g)
    x0 = t32(st["wt"]["x0"][:st["S"]])
    x = torch.empty_like(x0)

    def steps():
        for t in range(3):
            for l in range(g.n_layers):
                pc.cke_decoder_layer_step(x, st["descs"][l], st["kvs"][l], t, st["cache"], l,
                                          g.scale, st["ws"])

    def reset():
        x.copy_(x0)
        for kv in st["kvs"]:
            kv.k.zero_()
            kv.v.zero_()
        torch.cuda.synchronize()

    def snapshot():
        torch.cuda.synchronize()
        return [x.clone()] + [y.clone() for kv in st["kvs"] for y in (kv.k, kv.v)]

    reset()
    steps()
    want = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    reset()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        steps()
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        graph.replay()
        for a, b in zip(snapshot(), want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rep


def test_graph_replays_of_prepared_planes_lift_and_populate():
    """The fp32 path bench.py times for a projector memory, captured once into
    a HIP graph: the lift from prepared weight planes (split over k into four
    slices here), the populate from prepared planes, one cross decode per
    layer. Three replays, with eager resets and synchronisations in between,
    reproduce the eager run bit for bit; the eager memory is checked against
    the oracle's lift."""
    B, T, dm, H, D, L, k_in = 8, 25, 256, 4, 64, 2, 1024
    rows = B * T
    assert pc.cke_memory_lift_planes_workspace_bytes(rows, k_in, dm) > pc.cke_row_planes_bytes(rows, k_in)
    r = np.random.default_rng(77)
    xn = (r.standard_normal((rows, k_in)) * 0.5).astype(np.float32)
    wn = (r.standard_normal((k_in, dm)) * 0.03).astype(np.float32)
    pn = (r.standard_normal((T, dm)) * 0.02).astype(np.float32)
    x, Wl, pos = t32(xn), t32(wn), t32(pn)
    WK = [t32(r.standard_normal((dm, dm)) * 0.06) for _ in range(L)]
    WV = [t32(r.standard_normal((dm, dm)) * 0.06) for _ in range(L)]
    cache = pc.XattnCache(L, B, T, dm, H, D, max_q=2, dtype=torch.float32)
    E = torch.empty(B, T, dm, device=DEV)
    lp = pc.weight_planes([Wl])
    wp = cache.weight_planes(WK, WV)
    lws = torch.empty(pc.cke_memory_lift_planes_workspace_bytes(rows, k_in, dm) // 4, device=DEV)
    ews = cache.row_planes_workspace()
    q = [t32(r.standard_normal((B, 2, H, D)) * 0.5) for _ in range(L)]
    outs = [torch.empty(B, 2, H, D, device=DEV) for _ in range(L)]

    def window():
        pc.cke_memory_lift_gelu_planes(x, lp, dm, E.view(rows, dm), lws, pos=pos)
        cache.populate_planes(E, wp, ews)
        for l in range(L):
            pc.cke_xattn_decode(q[l], cache, l, 0.125, outs[l])

    def reset():
        for t in [E, cache.k, cache.v, lws, ews] + outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in [E, cache.k, cache.v] + outs]

    reset()
    window()
    want = snapshot()
    assert max_abs(to_np(E).reshape(rows, dm), oracle.lift_gelu(xn, wn, pn)) <= TOL["f32"]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    reset()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        window()
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        graph.replay()
        got = snapshot()
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rep
        torch.cuda.synchronize()
