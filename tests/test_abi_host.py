"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point the header declares, and validates arguments, geometry and
the ready flag before it would launch anything."""
import ctypes
import json
import os
import re

import pytest

import projection_cache_amd as pc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cke_xattn.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

FAKE = 0x100000  # an aligned non-NULL address; never dereferenced by these calls


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(cke_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 15
    lib = ctypes.CDLL(pc.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(pc.EXPORTED) == names


def test_version_string():
    assert "gfx950" in pc.cke_version()


def base_geom(**kw):
    d = dict(n_layers=6, n_streams=1, mem_len=1500, d_model=512, n_heads=8, head_dim=64,
             max_q=1, cache_dtype=pc.CKE_F32)
    d.update(kw)
    return pc.make_geom(**d)


def test_region_and_layer_offset_match_page():
    """C-Kernel-Engine 'View 2': layer 5's slab of Whisper Base (fp32) starts
    15,360,000 bytes into the cache region."""
    g = json.load(open(os.path.join(GOLDEN, "cke_whisper_base_geometry.json")))
    geom = base_geom()
    assert pc.cke_xattn_layer_offset_bytes(geom, 5) == g["layer5_k_offset_bytes"]
    assert pc.cke_xattn_region_bytes(geom) == 6 * 1500 * 512 * 4
    bf = base_geom(cache_dtype=pc.CKE_BF16)
    assert pc.cke_xattn_region_bytes(bf) == 6 * 1500 * 512 * 2
    with pytest.raises(pc.CkeError):
        pc.cke_xattn_layer_offset_bytes(geom, 6)


@pytest.mark.parametrize("bad", [
    dict(mem_len=0), dict(mem_len=-3), dict(d_model=500), dict(n_heads=7),
    dict(head_dim=48, d_model=384), dict(max_q=0), dict(max_q=9), dict(n_layers=0),
    dict(cache_dtype=7), dict(n_streams=0),
])
def test_geometry_fails_closed(bad):
    """C-Kernel-Engine 'View 3': non-positive memory length and
    num_heads * head_dim != embed_dim are hard errors, not defaults."""
    g = base_geom(**bad)
    assert pc.cke_xattn_region_bytes(g) == 0
    assert pc.cke_xattn_workspace_bytes(g) == 0
    with pytest.raises(pc.CkeError) as e:
        pc.cke_xattn_cache_create(g, FAKE, FAKE, FAKE)
    assert e.value.code == pc.CKE_EINVAL
    assert pc.cke_last_error()


def test_workspace_and_split_plan():
    for g in (base_geom(), base_geom(max_q=5),
              base_geom(n_layers=32, n_streams=16, d_model=1280, n_heads=20,
                        cache_dtype=pc.CKE_BF16),
              base_geom(n_layers=2, n_streams=100, mem_len=15, d_model=2048, n_heads=32,
                        max_q=3),
              base_geom(n_layers=1, mem_len=64, d_model=64, n_heads=2, head_dim=32)):
        s = pc.cke_xattn_num_splits(g)
        assert 1 <= s <= 64
        ws = pc.cke_xattn_workspace_bytes(g)
        al = lambda x: (x + 255) // 256 * 256
        need = g.n_streams * g.max_q * g.n_heads * s * (g.head_dim + 2) * 4
        stats = g.n_streams * g.max_q * g.n_heads * 2 * 4
        # partials, statistics, then one 128-byte arrival counter per head when split
        tickets = g.n_streams * g.n_heads * 128 if s > 1 else 0
        assert ws == max(256, al(al(need) + stats) + tickets)
    # Whisper Base splits its 1500 rows across workgroups, Q-Former does not
    assert pc.cke_xattn_num_splits(base_geom()) > 1
    assert pc.cke_xattn_num_splits(base_geom(n_layers=2, n_streams=100, mem_len=15, d_model=2048,
                                             n_heads=32, max_q=3)) == 1


def test_split_plan_evens_out_workgroups_per_compute_unit():
    """With at least 256 (stream, head) pairs the unsplit grid covers the 256
    compute units; the plan then splits a head into s pieces (2..8, >= 256
    rows each, at most 6 workgroups per unit for single-query bf16 caches and
    4 otherwise) only where that evens out the workgroups per unit, s
    minimising ceil(B*H*s/256)*256/(B*H*s); where B*H = 256k + R with R a
    multiple of 8 dividing 256, it runs the first 256k pairs whole and splits
    the last R pairs 256/R ways instead."""
    def splits(n_streams, n_heads, mem_len=1500, dt=pc.CKE_BF16, max_q=1):
        return pc.cke_xattn_num_splits(base_geom(n_layers=1, n_streams=n_streams, n_heads=n_heads,
                                                 d_model=64 * n_heads, mem_len=mem_len,
                                                 cache_dtype=dt, max_q=max_q))
    assert splits(16, 20) == 8                # Large: 320 = 256 + 64 pairs, 2 pieces per unit
    assert splits(16, 20, dt=pc.CKE_FP8) == 4  # one piece per unit
    assert splits(16, 20, mem_len=1000) == 4  # pieces of 8 would be < 128 rows: 4, one per unit
    assert splits(16, 20, mem_len=520) == 4   # 130 rows per piece of 4: one per unit
    assert splits(16, 20, mem_len=500) == 1   # < 128 rows per piece, and < 256 per uniform split
    assert splits(16, 20, dt=pc.CKE_F32) == 4
    assert splits(16, 20, max_q=2) == 4
    assert splits(32, 16) == 1                # 512 pairs: two per unit already
    assert splits(16, 16) == 1                # 256: one per unit
    assert splits(15, 20) == 5                # 300 pairs: 1.17 -> 1500 workgroups (5.86 per unit)
    assert splits(15, 20, dt=pc.CKE_FP8) == 3  # 900 workgroups (3.52 per unit)
    assert splits(64, 20) == 1                # 1280 pairs: five per unit; no room to split
    assert splits(15, 20, mem_len=600) == 2   # uniform: at least 256 rows per split
    assert splits(16, 20, mem_len=300) == 1
    # whole pairs: B*H = 256k + R, R a multiple of 8, split u*256/R ways (u = 2 for one-query bf16)
    def whole(n_streams, n_heads, mem_len=1500, dt=pc.CKE_BF16):
        return pc.cke_xattn_whole_pairs(base_geom(n_layers=1, n_streams=n_streams, n_heads=n_heads,
                                                  d_model=64 * n_heads, mem_len=mem_len,
                                                  cache_dtype=dt))
    assert whole(16, 20) == 256 and whole(16, 20, dt=pc.CKE_FP8) == 256
    assert whole(40, 8, mem_len=1024, dt=pc.CKE_F32) == 256
    assert splits(40, 8, mem_len=1024, dt=pc.CKE_F32) == 4
    assert whole(16, 20, mem_len=400) == 0    # pieces of 4 would be < 128 rows
    assert whole(15, 20) == 0                 # 300 = 256 + 44: 44 divides neither 256 nor 512
    assert whole(36, 8) == 256 and splits(36, 8) == 8    # 288 = 256 + 32: 16 pieces too many, 8
    assert whole(36, 8, mem_len=1000) == 0    # 8 pieces of 125 rows
    assert whole(32, 16) == 0 and whole(1, 8) == 0
    assert pc.lib().cke_xattn_whole_pairs(None) == 0
    # fewer pairs than units: about one workgroup per unit, as before (chunks
    # rounded up to whole passes of the waves: 64 bf16 rows, 16 fp32 rows)
    assert splits(1, 8, dt=pc.CKE_F32) == 32     # Whisper Base
    assert splits(1, 8) == 24
    assert splits(2, 8, dt=pc.CKE_F32) == 16


def test_merge_mode_switch_and_query():
    """cke_xattn_set_merge_mode takes 0 or 1 and returns the previous mode;
    cke_xattn_merges_in_launch is 0 for NULL, unsplit geometries, query
    counts outside [1, max_q] and in mode 0."""
    prev = pc.cke_xattn_set_merge_mode(0)
    try:
        assert prev in (0, 1)
        assert pc.cke_xattn_set_merge_mode(1) == 0
        assert pc.lib().cke_xattn_set_merge_mode(2) == pc.CKE_EINVAL
        assert "merge mode" in pc.cke_last_error()
        assert pc.lib().cke_xattn_set_merge_mode(-1) == pc.CKE_EINVAL
        assert pc.cke_xattn_set_merge_mode(1) == 1
        assert pc.lib().cke_xattn_merges_in_launch(None, 1) == 0
        unsplit = base_geom(n_layers=2, n_streams=100, mem_len=15, d_model=2048, n_heads=32, max_q=3)
        h = pc.cke_xattn_cache_create(unsplit, FAKE, FAKE, FAKE)
        try:
            assert pc.lib().cke_xattn_merges_in_launch(h, 1) == 0
        finally:
            pc.cke_xattn_cache_destroy(h)
        h = pc.cke_xattn_cache_create(base_geom(max_q=2), FAKE, FAKE, FAKE)
        try:
            for n_q in (0, 3, -1):
                assert pc.lib().cke_xattn_merges_in_launch(h, n_q) == 0
            pc.cke_xattn_set_merge_mode(0)
            assert pc.lib().cke_xattn_merges_in_launch(h, 1) == 0
        finally:
            pc.cke_xattn_cache_destroy(h)
    finally:
        pc.cke_xattn_set_merge_mode(prev)


def test_ready_flag_state_machine_without_gpu():
    """C-Kernel-Engine 'View 3': a cache is not ready until populated; after
    invalidation decode refuses with -2 before launching anything."""
    h = pc.cke_xattn_cache_create(base_geom(), FAKE, FAKE, FAKE)
    try:
        assert not pc.cke_xattn_is_ready(h)
        rc = pc.lib().cke_xattn_decode(FAKE, 1, h, 0, 0.125, FAKE, None)
        assert rc == pc.CKE_ENOTREADY == -2
        assert "not populated" in pc.cke_last_error()
        pc.cke_xattn_invalidate(h)
        assert pc.lib().cke_xattn_decode(FAKE, 1, h, 0, 0.125, FAKE, None) == -2
        # range checks come first
        assert pc.lib().cke_xattn_decode(FAKE, 1, h, 6, 0.125, FAKE, None) == pc.CKE_ERANGE
        assert pc.lib().cke_xattn_decode(FAKE, 2, h, 0, 0.125, FAKE, None) == pc.CKE_ERANGE
        assert pc.lib().cke_xattn_decode(FAKE, -1, h, 0, 0.125, FAKE, None) == pc.CKE_ERANGE
    finally:
        pc.cke_xattn_cache_destroy(h)


def test_populate_rejects_bad_arguments_before_launch():
    h = pc.cke_xattn_cache_create(base_geom(n_layers=2), FAKE, FAKE, FAKE)
    try:
        arr = ctypes.c_void_p * 2
        ok = arr(FAKE, FAKE)
        nul = arr(FAKE, None)
        L = pc.lib()
        assert L.cke_xattn_populate(h, None, 0, ok, ok, 0, None) == pc.CKE_EINVAL
        assert L.cke_xattn_populate(h, FAKE, 0, nul, ok, 0, None) == pc.CKE_EINVAL
        # fp32 cache with bf16 inputs: unsupported mix
        assert L.cke_xattn_populate(h, FAKE, 1, ok, ok, 1, None) == pc.CKE_EINVAL
        assert L.cke_xattn_populate(h, FAKE + 4, 0, ok, ok, 0, None) == pc.CKE_EINVAL
        assert not pc.cke_xattn_is_ready(h)
    finally:
        pc.cke_xattn_cache_destroy(h)


def test_fp8_cache_geometry_and_populate_checks():
    """fp8 E4M3 projection caches: one byte per element, populated only from
    bf16 E and weights, and only at widths n_heads*head_dim that are a
    multiple of 256; self-attention caches do not take fp8."""
    g = base_geom(cache_dtype=pc.CKE_FP8)
    assert pc.cke_xattn_region_bytes(g) == 6 * 1500 * 512
    assert pc.cke_xattn_layer_offset_bytes(g, 5) == 5 * 1500 * 512
    L = pc.lib()
    arr = ctypes.c_void_p * 6
    ok = arr(*([FAKE] * 6))
    h = pc.cke_xattn_cache_create(g, FAKE, FAKE, FAKE)
    try:
        assert L.cke_xattn_populate(h, FAKE, pc.CKE_F32, ok, ok, pc.CKE_F32, None) == pc.CKE_EINVAL
        assert L.cke_xattn_populate(h, FAKE, pc.CKE_FP8, ok, ok, pc.CKE_FP8, None) == pc.CKE_EINVAL
        assert not pc.cke_xattn_is_ready(h)
    finally:
        pc.cke_xattn_cache_destroy(h)
    narrow = base_geom(n_layers=1, d_model=96, n_heads=3, head_dim=32, cache_dtype=pc.CKE_FP8)
    h = pc.cke_xattn_cache_create(narrow, FAKE, FAKE, FAKE)
    try:
        rc = L.cke_xattn_populate(h, FAKE, pc.CKE_BF16, ok, ok, pc.CKE_BF16, None)
        assert rc == pc.CKE_EINVAL and "256" in pc.cke_last_error()
    finally:
        pc.cke_xattn_cache_destroy(h)
    kv = pc.cke_kv_layer(FAKE, FAKE, 1, 2, 64, 8, pc.CKE_FP8)
    rc = L.cke_selfattn_decode_append(FAKE, FAKE, FAKE, ctypes.byref(kv), 0, 0.125, FAKE, None)
    assert rc == pc.CKE_EINVAL


def test_decoder_step_workspace_and_argument_checks():
    """cke_decoder_layer_step validates before launching: NULL handle and
    descriptors, the layer range, then the ready flag (the checks behind the
    flag run in the GPU tests, which can populate)."""
    g = base_geom(n_layers=2, max_q=5)
    ws = pc.cke_decoder_step_workspace_bytes(g, 5)
    assert ws == 7 * ((5 * 512 * 4 + 255) // 256 * 256)
    assert pc.cke_decoder_step_workspace_bytes(g, 0) == 0
    L = pc.lib()
    w = pc.cke_decoder_layer(*([FAKE] * 6), pc.CKE_F32)
    kv = pc.cke_kv_layer(FAKE, FAKE, 5, 8, 64, 16, pc.CKE_F32)
    h = pc.cke_xattn_cache_create(g, FAKE, FAKE, FAKE)
    try:
        def step(w=w, kv=kv, pos=3, layer=1, x=FAKE, wsp=FAKE):
            return L.cke_decoder_layer_step(x, ctypes.byref(w), ctypes.byref(kv), pos, h, layer,
                                            0.125, wsp, None)
        assert step() == pc.CKE_ENOTREADY
        assert step(layer=2) == pc.CKE_ERANGE
        assert L.cke_decoder_layer_step(FAKE, None, ctypes.byref(kv), 0, None, 0, 0.1, FAKE,
                                        None) == pc.CKE_EINVAL
    finally:
        pc.cke_xattn_cache_destroy(h)


def test_memory_lift_rejects_bad_arguments_before_launch():
    L = pc.lib()
    ok = dict(x=FAKE, rows=30, k_in=64, w=FAKE, n=128, pos=FAKE, pos_rows=15, out=FAKE)
    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.cke_memory_lift_gelu(a["x"], a["rows"], a["k_in"], a["w"], a["n"], a["pos"],
                                      a["pos_rows"], a["out"], None)
    for bad in (dict(x=None), dict(out=None), dict(w=FAKE + 4), dict(rows=0), dict(k_in=48),
                dict(n=96), dict(pos_rows=0), dict(pos=FAKE + 8)):
        assert call(**bad) == pc.CKE_EINVAL, bad


def test_create_rejects_null_and_misaligned():
    g = base_geom()
    for k, v, w in ((None, FAKE, FAKE), (FAKE, None, FAKE), (FAKE, FAKE, None),
                    (FAKE + 8, FAKE, FAKE), (FAKE, FAKE, FAKE + 16)):
        with pytest.raises(pc.CkeError):
            pc.cke_xattn_cache_create(g, k, v, w)


def test_selfattn_rejects_bad_arguments_before_launch():
    L = pc.lib()

    def call(pos=0, **kw):
        d = dict(k=FAKE, v=FAKE, n_seqs=1, n_heads=8, head_dim=64, max_pos=448, dtype=0)
        d.update(kw)
        desc = pc.cke_kv_layer(**d)
        return L.cke_selfattn_decode_append(FAKE, FAKE, FAKE, ctypes.byref(desc), pos, 0.125,
                                            FAKE, None)

    assert call(pos=448) == pc.CKE_ERANGE
    assert call(pos=-1) == pc.CKE_ERANGE
    assert call(head_dim=48) == pc.CKE_EINVAL
    assert call(dtype=5) == pc.CKE_EINVAL
    assert call(k=None) == pc.CKE_EINVAL
    assert call(n_seqs=0) == pc.CKE_EINVAL
    assert L.cke_selfattn_decode_append(FAKE, FAKE, FAKE, None, 0, 0.125, FAKE, None) == pc.CKE_EINVAL


def test_prefill_rejects_bad_arguments_before_launch():
    L = pc.lib()

    def call(pos=0, n_new=3, n_q_heads=8, **kw):
        d = dict(k=FAKE, v=FAKE, n_seqs=1, n_heads=8, head_dim=64, max_pos=448, dtype=0)
        d.update(kw)
        desc = pc.cke_kv_layer(**d)
        return L.cke_selfattn_prefill_append(FAKE, FAKE, FAKE, ctypes.byref(desc), pos, n_new,
                                             n_q_heads, 0.125, FAKE, None)

    assert call(pos=446) == pc.CKE_ERANGE            # rows 446..448 run past max_pos
    assert call(pos=-1) == pc.CKE_ERANGE
    assert call(n_new=0) == pc.CKE_ERANGE
    assert call(n_q_heads=12) == pc.CKE_EINVAL       # not a multiple of the 8 kv heads
    assert call(n_q_heads=0) == pc.CKE_EINVAL
    assert call(head_dim=48) == pc.CKE_EINVAL
    assert call(k=None) == pc.CKE_EINVAL
    assert "n_q_heads" in (call(n_q_heads=4) and pc.cke_last_error())
    assert L.cke_selfattn_prefill_append(FAKE, FAKE, FAKE, None, 0, 1, 8, 0.125, FAKE, None) == pc.CKE_EINVAL


def test_decode_weights_rejects_bad_head_lists_before_launch():
    h = pc.cke_xattn_cache_create(base_geom(), FAKE, FAKE, FAKE)
    try:
        L = pc.lib()

        def call(heads, n=None):
            arr = (ctypes.c_int32 * max(1, len(heads)))(*heads)
            return L.cke_xattn_decode_weights(FAKE, 1, h, 0, 0.125, arr, len(heads) if n is None else n,
                                              FAKE, FAKE, None)

        assert call([0, 8]) == pc.CKE_ERANGE          # head 8 of 8
        assert call([-1]) == pc.CKE_ERANGE
        assert call([], 0) == pc.CKE_EINVAL
        assert call(list(range(8)) * 5) == pc.CKE_EINVAL   # more than 32 heads
        assert L.cke_xattn_decode_weights(FAKE, 1, h, 0, 0.125, None, 1, FAKE, FAKE, None) == pc.CKE_EINVAL
        # a valid list on an unpopulated cache: refused with -2 before any launch
        assert call([1, 3]) == pc.CKE_ENOTREADY
    finally:
        pc.cke_xattn_cache_destroy(h)


# ----------------------------------------------- Python binding argument checks
def _host_cache(geom):
    """An XattnCache over fake device addresses: enough for the binding's
    checks, which all run before anything reaches a device."""
    c = pc.XattnCache.__new__(pc.XattnCache)
    c.geom = geom
    c.handle = pc.cke_xattn_cache_create(geom, FAKE, FAKE, FAKE)
    return c


def test_binding_populate_checks_weight_count_and_shapes():
    import torch
    g = base_geom(n_layers=2, mem_len=10, d_model=64, n_heads=2, head_dim=32)
    c = _host_cache(g)
    try:
        E = torch.zeros(1, 10, 64)
        W = [torch.zeros(64, 64) for _ in range(2)]
        with pytest.raises(ValueError, match="one weight per layer"):
            pc.cke_xattn_populate(c, E, W[:1], W)              # short WK list
        with pytest.raises(ValueError, match="one weight per layer"):
            pc.cke_xattn_populate(c, E, W, W + W)              # uneven lists
        with pytest.raises(ValueError, match="E must have shape"):
            pc.cke_xattn_populate(c, torch.zeros(1, 11, 64), W, W)
        with pytest.raises(ValueError, match=r"WV\[1\] must have shape"):
            pc.cke_xattn_populate(c, E, W, [W[0], torch.zeros(64, 32)])
        with pytest.raises(ValueError, match="dtype"):
            pc.cke_xattn_populate(c, E, W, [W[0], W[1].bfloat16()])
        with pytest.raises(ValueError, match="device tensor"):
            pc.cke_xattn_populate(c, E, W, W)                 # host tensors
        with pytest.raises(TypeError):
            pc.cke_xattn_populate(c.handle, E, W, W)          # raw handle: no geometry
        assert not pc.cke_xattn_is_ready(c.handle)
    finally:
        c.close()


def test_binding_decode_and_self_calls_check_shapes_before_launch():
    import torch
    g = base_geom(n_layers=1, n_streams=2, mem_len=10, d_model=64, n_heads=2, head_dim=32,
                  max_q=3)
    c = _host_cache(g)
    try:
        q = torch.zeros(2, 3, 2, 32)
        with pytest.raises(ValueError, match="q must have shape"):
            pc.cke_xattn_decode(torch.zeros(1, 3, 2, 32), c, 0, 0.125, q)
        with pytest.raises(ValueError, match="out must have shape"):
            pc.cke_xattn_decode(q, c, 0, 0.125, torch.zeros(2, 2, 2, 32))
        with pytest.raises(ValueError, match="exceeds"):
            pc.cke_xattn_decode(q, c, 0, 0.125, q.clone(), n_q=4)
        with pytest.raises(ValueError, match="dtype"):
            pc.cke_xattn_decode(q.double(), c, 0, 0.125, q)
        with pytest.raises(ValueError, match="device tensor"):
            pc.cke_xattn_decode(q, c, 0, 0.125, q.clone())
        with pytest.raises(ValueError, match="weights must have shape"):
            pc.cke_xattn_decode_weights(q, c, 0, 0.125, [0], q.clone(), torch.zeros(2, 3, 9))
    finally:
        c.close()


def test_binding_kv_layer_takes_shape_and_dtype_from_its_tensors():
    import torch
    k = torch.zeros(2, 4, 16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="disagrees"):
        pc.KVLayer(2, 4, 64, 16, dtype=torch.float32, k=k, v=k.clone())   # bf16 described as fp32
    with pytest.raises(ValueError, match="disagrees"):
        pc.KVLayer(2, 4, 64, 32, k=k, v=k.clone())                        # wrong capacity
    with pytest.raises(ValueError, match="one shape"):
        pc.KVLayer(k=k, v=torch.zeros(2, 4, 16, 64))
    with pytest.raises(ValueError, match="both k and v"):
        pc.KVLayer(k=k)
    with pytest.raises(ValueError, match="device tensor"):
        pc.KVLayer(k=k, v=k.clone())
    with pytest.raises(TypeError, match="KVLayer"):
        pc.cke_selfattn_decode_append(None, None, None, pc.cke_kv_layer(), 0, 0.125, None)


def test_binding_lift_checks_shapes():
    import torch
    x, w = torch.zeros(30, 64), torch.zeros(64, 128)
    with pytest.raises(ValueError, match="w must have shape"):
        pc.cke_memory_lift_gelu(x, torch.zeros(32, 128), torch.zeros(30, 128))
    with pytest.raises(ValueError, match="out must hold"):
        pc.cke_memory_lift_gelu(x, w, torch.zeros(29, 128))
    with pytest.raises(ValueError, match="pos must have shape"):
        pc.cke_memory_lift_gelu(x, w, torch.zeros(30, 128), torch.zeros(15, 64))
    with pytest.raises(ValueError, match="device tensor"):
        pc.cke_memory_lift_gelu(x, w, torch.zeros(30, 128))


def test_populate_and_lift_workspace_sizes():
    """The split-planes workspace: E's hi and lo planes, then (256-byte
    aligned) a hi and a lo plane of every weight; none for bf16 inputs or
    widths the planes kernel does not take."""
    g = base_geom()
    e_planes = 2 * 1500 * 512 * 2
    w_planes = 12 * 2 * 512 * 512 * 2
    assert pc.cke_xattn_populate_workspace_bytes(g) == (e_planes + 255) // 256 * 256 + w_planes
    assert pc.cke_xattn_populate_workspace_bytes(g, pc.CKE_BF16, pc.CKE_BF16) == 0
    assert pc.cke_xattn_populate_workspace_bytes(base_geom(cache_dtype=pc.CKE_BF16)) == 0
    assert pc.cke_xattn_populate_workspace_bytes(base_geom(d_model=96, n_heads=3, head_dim=32)) == 0
    assert pc.cke_xattn_populate_workspace_bytes(base_geom(mem_len=0)) == 0
    # the Q-Former lift makes 64 tiles of 192 x 256: split over k in 4 slices of partial sums
    assert pc.cke_memory_lift_workspace_bytes(1500, 4096, 2048) == \
        2 * 1500 * 4096 * 2 + 2 * 4096 * 2048 * 2 + 4 * 1500 * 2048 * 4
    assert pc.cke_memory_lift_workspace_bytes(64, 4096, 64) == 0      # n not a multiple of 128
    assert pc.cke_memory_lift_workspace_bytes(0, 4096, 2048) == 0


def test_populate_ws_rejects_a_missing_or_short_workspace_before_launch():
    g = base_geom(n_layers=2)
    h = pc.cke_xattn_cache_create(g, FAKE, FAKE, FAKE)
    try:
        arr = ctypes.c_void_p * 2
        ok = arr(FAKE, FAKE)
        need = pc.cke_xattn_populate_workspace_bytes(g)
        L = pc.lib()
        assert L.cke_xattn_populate_ws(h, FAKE, 0, ok, ok, 0, None, need, None) == pc.CKE_EINVAL
        assert L.cke_xattn_populate_ws(h, FAKE, 0, ok, ok, 0, FAKE, need - 1, None) == pc.CKE_EINVAL
        assert "needs" in pc.cke_last_error()
        assert L.cke_xattn_populate_ws(h, FAKE, 0, ok, ok, 0, FAKE + 16, need, None) == pc.CKE_EINVAL
        assert not pc.cke_xattn_is_ready(h)
    finally:
        pc.cke_xattn_cache_destroy(h)
    Lb = pc.lib()
    assert Lb.cke_memory_lift_gelu_ws(FAKE, 30, 64, FAKE, 128, None, 0, FAKE, None, 0, None) == \
        pc.CKE_EINVAL


def test_prepared_weight_plane_sizes():
    """Prepared weight planes: [n_mat][hi, lo][n][k] bf16; per-call row
    planes [hi, lo][rows][k] bf16, rounded up to 256 bytes; 0 where the
    planes kernel does not take the shape."""
    assert pc.cke_weight_planes_bytes(12, 512, 512) == 12 * 2 * 512 * 512 * 2
    assert pc.cke_weight_planes_bytes(1, 4096, 2048) == 2 * 4096 * 2048 * 2
    assert pc.cke_weight_planes_bytes(2 * 128, 64, 128) == 256 * 2 * 64 * 128 * 2
    for bad in ((0, 512, 512), (257, 64, 128), (1, 32, 128), (1, 512, 64), (1, 0, 128),
                (1, 512, 0)):
        assert pc.cke_weight_planes_bytes(*bad) == 0, bad
    assert pc.cke_row_planes_bytes(1500, 512) == 2 * 1500 * 512 * 2
    assert pc.cke_row_planes_bytes(15, 64) == (2 * 15 * 64 * 2 + 255) // 256 * 256
    assert pc.cke_row_planes_bytes(0, 512) == 0
    assert pc.cke_row_planes_bytes(15, 96) == 0
    # the populate workspace is exactly the row planes followed by the weight planes
    g = base_geom()
    assert pc.cke_xattn_populate_workspace_bytes(g) == (
        pc.cke_row_planes_bytes(1500, 512) + pc.cke_weight_planes_bytes(12, 512, 512))
    slices = 4 * 1500 * 2048 * 4
    assert pc.cke_memory_lift_workspace_bytes(1500, 4096, 2048) == (
        pc.cke_row_planes_bytes(1500, 4096) + pc.cke_weight_planes_bytes(1, 4096, 2048) + slices)
    assert pc.cke_memory_lift_planes_workspace_bytes(1500, 4096, 2048) == (
        pc.cke_row_planes_bytes(1500, 4096) + slices)
    # split in two: 80 tiles of 192 x 256 in 4 slices would need 320 > 256 workgroups
    assert pc.cke_memory_lift_planes_workspace_bytes(1500, 1024, 2560) == (
        pc.cke_row_planes_bytes(1500, 1024) + 2 * 1500 * 2560 * 4)
    # no split: enough tiles (256), a short k, or widths that take 128 x 128 tiles
    assert pc.cke_memory_lift_planes_workspace_bytes(3000, 1024, 4096) == pc.cke_row_planes_bytes(3000, 1024)
    assert pc.cke_memory_lift_planes_workspace_bytes(200, 256, 256) == pc.cke_row_planes_bytes(200, 256)
    assert pc.cke_memory_lift_planes_workspace_bytes(130, 1024, 384) == pc.cke_row_planes_bytes(130, 1024)
    assert pc.cke_memory_lift_planes_workspace_bytes(130, 1024, 64) == 0
    assert pc.cke_memory_lift_planes_workspace_bytes(0, 1024, 256) == 0


def test_prepared_planes_calls_reject_bad_arguments_before_launch():
    L = pc.lib()
    arr = ctypes.c_void_p * 2
    need = pc.cke_weight_planes_bytes(2, 512, 512)
    ok = arr(FAKE, FAKE)
    for args in ((ok, 2, 512, 96, FAKE, need), (ok, 0, 512, 512, FAKE, need),
                 (None, 2, 512, 512, FAKE, need), (ok, 2, 512, 512, None, need),
                 (ok, 2, 512, 512, FAKE + 16, need), (ok, 2, 512, 512, FAKE, need - 1),
                 (arr(FAKE, None), 2, 512, 512, FAKE, need), (arr(FAKE, FAKE + 4), 2, 512, 512, FAKE, need)):
        assert L.cke_weight_planes(*args, None) == pc.CKE_EINVAL, args
    g = base_geom(n_layers=2)
    h = pc.cke_xattn_cache_create(g, FAKE, FAKE, FAKE)
    try:
        w_need = pc.cke_weight_planes_bytes(4, 512, 512)
        e_need = pc.cke_row_planes_bytes(1500, 512)
        for args in ((None, FAKE, FAKE, w_need, FAKE, e_need), (h, None, FAKE, w_need, FAKE, e_need),
                     (h, FAKE, None, w_need, FAKE, e_need), (h, FAKE, FAKE, w_need, None, e_need),
                     (h, FAKE + 4, FAKE, w_need, FAKE, e_need), (h, FAKE, FAKE + 16, w_need, FAKE, e_need),
                     (h, FAKE, FAKE, w_need, FAKE + 16, e_need), (h, FAKE, FAKE, w_need - 1, FAKE, e_need),
                     (h, FAKE, FAKE, w_need, FAKE, e_need - 1)):
            assert L.cke_xattn_populate_planes(*args, None) == pc.CKE_EINVAL, args
        assert pc.cke_xattn_is_ready(h) == 0
    finally:
        pc.cke_xattn_cache_destroy(h)
    for geom in (base_geom(cache_dtype=pc.CKE_BF16), base_geom(d_model=96, n_heads=3, head_dim=32)):
        h = pc.cke_xattn_cache_create(geom, FAKE, FAKE, FAKE)
        try:
            assert L.cke_xattn_populate_planes(h, FAKE, FAKE, 1 << 30, FAKE, 1 << 30,
                                               None) == pc.CKE_EINVAL
        finally:
            pc.cke_xattn_cache_destroy(h)
    w_need = pc.cke_weight_planes_bytes(1, 4096, 2048)
    e_need = pc.cke_memory_lift_planes_workspace_bytes(1500, 4096, 2048)
    for args in ((FAKE, 1500, 4096, FAKE, w_need, 2048, None, 0, FAKE, FAKE, e_need - 1),
                 (FAKE, 1500, 4096, FAKE, w_need - 1, 2048, None, 0, FAKE, FAKE, e_need),
                 (FAKE, 1500, 4096, FAKE + 16, w_need, 2048, None, 0, FAKE, FAKE, e_need),
                 (FAKE, 1500, 4096, FAKE, w_need, 2048, None, 0, FAKE, None, e_need),
                 (FAKE, 1500, 4096, FAKE, w_need, 2048, FAKE, 0, FAKE, FAKE, e_need),
                 (FAKE, 1500, 4096, FAKE, w_need, 2000, None, 0, FAKE, FAKE, e_need),
                 (FAKE, 1500, 4000, FAKE, w_need, 2048, None, 0, FAKE, FAKE, e_need),
                 (None, 1500, 4096, FAKE, w_need, 2048, None, 0, FAKE, FAKE, e_need)):
        assert L.cke_memory_lift_gelu_planes(*args, None) == pc.CKE_EINVAL, args


def test_binding_prepared_planes_check_shapes_before_launch():
    import torch
    x = torch.zeros(4, 64)
    with pytest.raises(ValueError):
        pc.cke_weight_planes([x], torch.zeros(16))
    with pytest.raises(ValueError):
        pc.cke_memory_lift_gelu_planes(torch.zeros(4), torch.zeros(16), 128, torch.zeros(512),
                                       torch.zeros(16))
    with pytest.raises(ValueError):
        pc.cke_memory_lift_gelu_planes(x, torch.zeros(16), 128, torch.zeros(4 * 127),
                                       torch.zeros(16))
    with pytest.raises(ValueError):
        pc.cke_memory_lift_gelu_planes(x, torch.zeros(16), 128, torch.zeros(4 * 128),
                                       torch.zeros(16))
