"""The C-ABI library on the host: it loads, exports every declared entry point, and
rejects bad arguments with the documented status before touching the device."""
import math
import os
import re

import numpy as np
import pytest

import __graft_entry__

__graft_entry__.ensure_built()

import global_paged_gqa_amd as g  # noqa: E402
from global_paged_gqa_amd import _native as nat  # noqa: E402
import workloads  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gattn_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert names == sorted(["gattn_abi_version", "gattn_status_str", "gattn_layer_family", "gattn_kv_offset",
                            "gattn_decode_workspace_bytes", "gattn_decode", "gattn_decode_noalloc",
                            "gattn_decode_fp8kv", "gattn_prefill", "gattn_combine", "gattn_kv_append",
                            "gattn_kv_append_fp8", "gattn_decode_graphs_create", "gattn_decode_graphs_bucket",
                            "gattn_decode_graphs_launch", "gattn_decode_graphs_destroy"])
    for n in names:
        assert hasattr(nat._lib, n), n
    assert g.gattn_abi_version() == 1


def test_status_strings():
    for s in range(7):
        assert g.gattn_status_str(s) and g.gattn_status_str(s) != "unknown status"
    assert g.gattn_status_str(99) == "unknown status"


def test_layer_family_schedule():
    fam = [g.gattn_layer_family(l, 60) for l in range(60)]
    assert fam.count(g.GLOBAL) == 10 and fam.count(g.LOCAL) == 50 and fam[59] == g.GLOBAL
    assert fam[:6] == [0, 0, 0, 0, 0, 1]
    assert g.gattn_layer_family(0, 59) == -1 and g.gattn_layer_family(60, 60) == -1
    assert g.gattn_layer_family(-1, 60) == -1


def test_kv_offset_hand_computed():
    lay = g.make_layer("global", 32, 4, 512)
    pt = np.array([[5, 2, -1, 7], [0, 1, 3, 6]], dtype=np.int32)
    cases = [  # (row, token, kv_head, expected)
        (0, 0, 0, ((5 * 4 + 0) * 16 + 0) * 512),
        (0, 15, 3, ((5 * 4 + 3) * 16 + 15) * 512),
        (0, 16, 1, ((2 * 4 + 1) * 16 + 0) * 512),
        (0, 31, 2, ((2 * 4 + 2) * 16 + 15) * 512),
        (0, 48, 0, ((7 * 4 + 0) * 16 + 0) * 512),
        (1, 0, 0, 0),
        (1, 17, 2, ((1 * 4 + 2) * 16 + 1) * 512),
        (1, 63, 3, ((6 * 4 + 3) * 16 + 15) * 512),
        (0, 32, 0, -1),      # page -1
        (0, 64, 0, -1),      # beyond the table
        (2, 0, 0, -1),       # row out of range
        (1, 0, 4, -1),       # kv head out of range
        (1, 40, 0, -1),      # page 3 >= num_pages 3
    ]
    for row, tok, kvh, want in cases:
        assert g.gattn_kv_offset(lay, pt, 2, 4, row, tok, kvh, 8 if want != -1 or row != 1 else 3) == want, \
            (row, tok, kvh)
    loc = g.make_layer("local", 32, 16, 256, window=1024)
    assert g.gattn_kv_offset(loc, pt, 2, 4, 1, 35, 9, 8) == ((3 * 16 + 9) * 16 + 3) * 256


def test_kv_offset_agrees_with_the_scatter():
    """The checked helper and the independent scatter in workloads agree on every stored token."""
    b = workloads.cfg1_tiny_decode()
    lay = g.make_layer("local", 4, 2, 256, 1024, scale=1 / 16)
    flat = b.k_pool.reshape(-1)
    for tok in (0, 1, 15, 16, 511, 1000, 1024):
        for kvh in (0, 1):
            off = g.gattn_kv_offset(lay, b.page_table, 1, b.pt_stride, 0, tok, kvh, b.num_pages)
            assert np.array_equal(flat[off:off + 256], b.k[tok, kvh])


def test_workspace_bytes():
    glob = g.make_layer("global", 32, 4, 512)
    assert g.gattn_decode_workspace_bytes(glob, 32, 8192, 512) == 32 * 32 * 16 * 513 * 4
    assert g.gattn_decode_workspace_bytes(glob, 32, 8192, 0) == 0          # one split per row
    assert g.gattn_decode_workspace_bytes(glob, 32, 512, 512) == 0
    assert g.gattn_decode_workspace_bytes(glob, 1, 65536, 1024) == 32 * 64 * 513 * 4
    loc = g.make_layer("local", 32, 16, 256, window=1024)
    # a 1024-key window touches at most 3 splits of 512 and 2 of 1024, whatever the context
    assert g.gattn_decode_workspace_bytes(loc, 64, 32768, 512) == 64 * 32 * 3 * 257 * 4
    assert g.gattn_decode_workspace_bytes(loc, 64, 32768, 1024) == 64 * 32 * 2 * 257 * 4
    assert g.gattn_decode_workspace_bytes(loc, 64, 32768, 16) == 64 * 32 * 65 * 257 * 4
    assert g.gattn_decode_workspace_bytes(glob, 32, 8192, 500) == 0        # bad split
    assert g.gattn_decode_workspace_bytes(glob, 32, 0, 512) == 0


def _decode_status(**over):
    lay = over.pop("layer", g.make_layer("global", 32, 4, 512))
    args = dict(q=1 << 20, k_pool=2 << 20, v_pool=3 << 20, num_pages=100, page_table=4 << 20, pt_stride=512,
                ctx_lens=5 << 20, batch=32, max_ctx=8192, split_tokens=512, workspace=6 << 20,
                workspace_bytes=1 << 30, out=7 << 20, lse=8 << 20)
    args.update(over)
    try:
        g.gattn_decode(lay, **args, stream=0)
    except g.GattnError as e:
        return e.status
    return 0


@pytest.mark.parametrize("over,status", [
    (dict(q=None), nat.ERR_NULL_PTR),
    (dict(k_pool=None), nat.ERR_NULL_PTR),
    (dict(v_pool=None), nat.ERR_NULL_PTR),
    (dict(page_table=None), nat.ERR_NULL_PTR),
    (dict(ctx_lens=None), nat.ERR_NULL_PTR),
    (dict(out=None), nat.ERR_NULL_PTR),
    (dict(lse=None), nat.ERR_NULL_PTR),
    (dict(workspace=None), nat.ERR_NULL_PTR),
    (dict(batch=-1), nat.ERR_BAD_SHAPE),
    (dict(max_ctx=0), nat.ERR_BAD_SHAPE),
    (dict(pt_stride=0), nat.ERR_BAD_SHAPE),
    (dict(pt_stride=511), nat.ERR_BAD_SHAPE),       # table cannot hold max_ctx tokens
    (dict(num_pages=0), nat.ERR_BAD_SHAPE),
    (dict(split_tokens=500), nat.ERR_BAD_SPLIT),
    (dict(split_tokens=-16), nat.ERR_BAD_SPLIT),
    (dict(workspace_bytes=100), nat.ERR_WORKSPACE_TOO_SMALL),
    (dict(layer=g.make_layer("global", 32, 4, 128)), nat.ERR_UNSUPPORTED),
    (dict(layer=g.make_layer("global", 32, 4, 512, page_size=32)), nat.ERR_UNSUPPORTED),
    (dict(layer=g.make_layer("global", 32, 5, 512)), nat.ERR_BAD_SHAPE),
    (dict(layer=g.make_layer("global", 64, 2, 512)), nat.ERR_UNSUPPORTED),   # group 32 > 16
    (dict(layer=g.make_layer("local", 32, 16, 256, window=0)), nat.ERR_BAD_SHAPE),
    (dict(layer=g.make_layer("global", 32, 4, 512, scale=math.inf)), nat.ERR_BAD_SHAPE),
    (dict(layer=g.make_layer(7, 32, 4, 512)), nat.ERR_UNSUPPORTED),
    (dict(layer=g.make_layer("global", 32, 4, 512, kv_shared=True)), nat.ERR_BAD_SHAPE),  # v_pool != k_pool
    (dict(batch=0), 0),
])
def test_decode_rejects_bad_arguments_without_a_device(over, status):
    assert _decode_status(**over) == status
    assert _decode_status(batch=0) == 0  # no sticky state after a rejected call


def _noalloc_status(**over):
    lay = over.pop("layer", g.make_layer("global", 32, 4, 512))
    args = dict(q=1 << 20, k_pool=2 << 20, v_pool=3 << 20, num_pages=100, page_table=4 << 20, pt_stride=512,
                ctx_lens=5 << 20, batch=32, max_ctx=8192, split_tokens=512, out=7 << 20, lse=8 << 20)
    args.update(over)
    try:
        g.gattn_decode_noalloc(lay, **args, stream=0)
    except g.GattnError as e:
        return e.status
    return 0


@pytest.mark.parametrize("over,status", [
    (dict(q=None), nat.ERR_NULL_PTR),
    (dict(v_pool=None), nat.ERR_NULL_PTR),
    (dict(lse=None), nat.ERR_NULL_PTR),
    (dict(batch=-1), nat.ERR_BAD_SHAPE),
    (dict(pt_stride=511), nat.ERR_BAD_SHAPE),
    (dict(split_tokens=500), nat.ERR_BAD_SPLIT),
    (dict(layer=g.make_layer("global", 32, 4, 128)), nat.ERR_UNSUPPORTED),
    # partials of 1000 rows x 32 heads x 16 splits x 513 words = 1.05 GB > the 64 MiB scratch
    (dict(batch=1000), nat.ERR_WORKSPACE_TOO_SMALL),
    (dict(batch=0), 0),
    (dict(batch=0, split_tokens=0), 0),
])
def test_decode_noalloc_rejects_bad_arguments_without_a_device(over, status):
    """The no-allocation decode checks its arguments exactly as gattn_decode does, and rejects a call
    whose partials would not fit its fixed scratch, all before any HIP call."""
    assert _noalloc_status(**over) == status


def _graphs_status(**over):
    lay = over.pop("layer", g.make_layer("global", 32, 4, 512))
    args = dict(q=1 << 20, k_pool=2 << 20, v_pool=3 << 20, num_pages=100, page_table=4 << 20, pt_stride=512,
                ctx_lens=5 << 20, max_ctx=8192, split_tokens=512, workspace=6 << 20, workspace_bytes=1 << 30,
                out=7 << 20, lse=8 << 20, buckets=[1, 8, 32])
    args.update(over)
    try:
        handle = g.gattn_decode_graphs_create(lay, **args)
    except g.GattnError as e:
        return e.status
    g.gattn_decode_graphs_destroy(handle)
    return 0


@pytest.mark.parametrize("over,status", [
    (dict(buckets=[]), nat.ERR_BAD_SHAPE),
    (dict(buckets=list(range(1, 18))), nat.ERR_BAD_SHAPE),      # more than 16 buckets
    (dict(buckets=[0, 8]), nat.ERR_BAD_SHAPE),
    (dict(buckets=[8, 4]), nat.ERR_BAD_SHAPE),                   # not increasing
    (dict(buckets=[4, 4]), nat.ERR_BAD_SHAPE),
    (dict(q=None), nat.ERR_NULL_PTR),
    (dict(v_pool=None), nat.ERR_NULL_PTR),
    (dict(workspace=None), nat.ERR_NULL_PTR),
    (dict(pt_stride=511), nat.ERR_BAD_SHAPE),
    (dict(split_tokens=500), nat.ERR_BAD_SPLIT),
    # the largest bucket sets the workspace: 32 rows need 32 x 32 x 16 x 513 x 4 B
    (dict(workspace_bytes=g.gattn_decode_workspace_bytes(g.make_layer("global", 32, 4, 512), 8, 8192, 512)),
     nat.ERR_WORKSPACE_TOO_SMALL),
    (dict(layer=g.make_layer("global", 32, 4, 128)), nat.ERR_UNSUPPORTED),
])
def test_decode_graphs_reject_bad_arguments_without_a_device(over, status):
    """The graph set checks its buckets and, for every bucket, the decode call it would capture,
    all before any HIP call."""
    assert _graphs_status(**over) == status


def test_decode_graphs_null_handles():
    assert g.gattn_decode_graphs_bucket(None, 4) == -1
    with pytest.raises(g.GattnError) as e:
        g.gattn_decode_graphs_launch(None, 4, stream=0)
    assert e.value.status == nat.ERR_NULL_PTR
    g.gattn_decode_graphs_destroy(None)
    rc = nat._lib.gattn_decode_graphs_create(None, None, None, None, 0, None, 0, None, 0, 0, None, 0, None, None,
                                             None, 0, None)
    assert rc == nat.ERR_NULL_PTR


def test_noalloc_scratch_limit():
    lay = g.make_layer("global", 32, 4, 512)
    assert nat.NOALLOC_SCRATCH_BYTES == 64 << 20
    # the largest batch of the 8192-context global workload at split 512 that fits: 63 rows
    per_row = g.gattn_decode_workspace_bytes(lay, 1, 8192, 512)
    fit = nat.NOALLOC_SCRATCH_BYTES // per_row
    assert fit == 63
    assert _noalloc_status(batch=fit + 1) == nat.ERR_WORKSPACE_TOO_SMALL


def test_prefill_and_combine_reject_bad_arguments():
    lay = g.make_layer("local", 32, 16, 256, window=1024)
    ok = dict(q=1, k_pool=2, v_pool=3, num_pages=10, page_table=4, pt_stride=8, cu_q=5, ctx_lens=6, batch=0,
              max_q=16, out=7, lse=8)

    def st(fn, *a, **kw):
        try:
            fn(*a, **kw, stream=0)
        except g.GattnError as e:
            return e.status
        return 0
    assert st(g.gattn_prefill, lay, **ok) == 0
    assert st(g.gattn_prefill, lay, **dict(ok, cu_q=None)) == nat.ERR_NULL_PTR
    assert st(g.gattn_prefill, lay, **dict(ok, max_q=-1)) == nat.ERR_BAD_SHAPE
    assert st(g.gattn_prefill, g.make_layer("local", 32, 16, 256, window=-5), **ok) == nat.ERR_BAD_SHAPE
    # a query tile's span of q must stay within 32-bit offsets: at most 16384 query heads
    assert st(g.gattn_prefill, g.make_layer("global", 32768, 2048, 512), **ok) == nat.ERR_UNSUPPORTED
    assert st(g.gattn_combine, 4, 32, 512, 0, 1, 2, 3, 4) == nat.ERR_BAD_SHAPE
    assert st(g.gattn_combine, 4, 32, 510, 3, 1, 2, 3, 4) == nat.ERR_UNSUPPORTED
    assert st(g.gattn_combine, 4, 32, 512, 3, None, 2, 3, 4) == nat.ERR_NULL_PTR
    assert st(g.gattn_combine, 0, 32, 512, 3, 1, 2, 3, 4) == 0


def test_kv_append_rejects_bad_arguments():
    lay = g.make_layer("global", 32, 4, 512)
    ok = dict(k_new=1, v_new=2, k_pool=3, v_pool=4, num_pages=10, page_table=5, pt_stride=8, cu_new=6, ctx_lens=7,
              batch=0, max_new=16, status=None)

    def st(layer, **kw):
        try:
            g.gattn_kv_append(layer, **kw, stream=0)
        except g.GattnError as e:
            return e.status
        return 0
    assert st(lay, **ok) == 0
    for key in ("k_new", "v_new", "k_pool", "v_pool", "page_table", "cu_new", "ctx_lens"):
        assert st(lay, **dict(ok, **{key: None})) == nat.ERR_NULL_PTR, key
    assert st(lay, **dict(ok, batch=-1)) == nat.ERR_BAD_SHAPE
    assert st(lay, **dict(ok, max_new=-1)) == nat.ERR_BAD_SHAPE
    assert st(lay, **dict(ok, pt_stride=0)) == nat.ERR_BAD_SHAPE
    assert st(lay, **dict(ok, num_pages=0)) == nat.ERR_BAD_SHAPE
    assert st(g.make_layer("global", 32, 4, 128), **ok) == nat.ERR_UNSUPPORTED
    shared = g.make_layer("global", 32, 4, 512, kv_shared=True)
    assert st(shared, **dict(ok, v_new=None, v_pool=None)) == 0
    assert st(shared, **dict(ok, v_new=None, v_pool=3)) == 0          # v_pool == k_pool
    assert st(shared, **dict(ok, v_new=2, v_pool=None)) == nat.ERR_BAD_SHAPE
    assert st(shared, **dict(ok, v_new=None, v_pool=4)) == nat.ERR_BAD_SHAPE


def test_decode_fp8kv_rejects_bad_arguments():
    """The FP8-pool decode validates like gattn_decode, serves head_dim 256 with separate K and V
    pools only, and needs positive finite scales; batch 0 with valid arguments is a no-op."""
    lay = g.make_layer("local", 32, 16, 256, window=1024)
    ok = dict(q=1, k_pool=2, v_pool=3, k_scale=0.5, v_scale=0.25, num_pages=10, page_table=4, pt_stride=8,
              ctx_lens=5, batch=0, max_ctx=128, split_tokens=64, workspace=None, workspace_bytes=0, out=6, lse=7)

    def st(layer, **kw):
        try:
            g.gattn_decode_fp8kv(layer, **kw, stream=0)
        except g.GattnError as e:
            return e.status
        return 0
    assert st(lay, **ok) == 0
    for key in ("q", "k_pool", "v_pool", "page_table", "ctx_lens", "out", "lse"):
        assert st(lay, **dict(ok, **{key: None})) == nat.ERR_NULL_PTR, key
    for bad in (0.0, -1.0, math.inf, math.nan):
        assert st(lay, **dict(ok, k_scale=bad)) == nat.ERR_BAD_SHAPE, bad
        assert st(lay, **dict(ok, v_scale=bad)) == nat.ERR_BAD_SHAPE, bad
    assert st(g.make_layer("global", 32, 4, 512), **ok) == 0
    shared = g.make_layer("global", 32, 4, 512, kv_shared=True)
    assert st(shared, **dict(ok, v_pool=None)) == 0
    assert st(shared, **dict(ok, v_pool=2)) == 0                        # v_pool == k_pool
    assert st(shared, **dict(ok, v_pool=3)) == nat.ERR_BAD_SHAPE
    assert st(shared, **dict(ok, v_pool=None, v_scale=math.nan)) == 0   # V uses k_scale
    assert st(g.make_layer("global", 32, 4, 128), **ok) == nat.ERR_UNSUPPORTED
    assert st(g.make_layer("local", 32, 16, 256, window=1024, kv_shared=True), **ok) == nat.ERR_UNSUPPORTED
    assert st(lay, **dict(ok, split_tokens=24)) == nat.ERR_BAD_SPLIT
    assert st(lay, **dict(ok, batch=2)) == nat.ERR_WORKSPACE_TOO_SMALL  # several splits need the workspace
    assert st(lay, **dict(ok, max_ctx=0)) == nat.ERR_BAD_SHAPE
    assert st(g.make_layer("global", 8, 2, 256), **ok) == 0  # any family at head_dim 256


def test_kv_append_fp8_rejects_bad_arguments():
    lay = g.make_layer("local", 32, 16, 256, window=1024)
    ok = dict(k_new=1, v_new=2, k_pool=3, v_pool=4, k_scale=0.5, v_scale=0.25, num_pages=10, page_table=5,
              pt_stride=8, cu_new=6, ctx_lens=7, batch=0, max_new=16, status=None)

    def st(layer, **kw):
        try:
            g.gattn_kv_append_fp8(layer, **kw, stream=0)
        except g.GattnError as e:
            return e.status
        return 0
    assert st(lay, **ok) == 0
    for key in ("k_new", "v_new", "k_pool", "v_pool", "page_table", "cu_new", "ctx_lens"):
        assert st(lay, **dict(ok, **{key: None})) == nat.ERR_NULL_PTR, key
    for bad in (0.0, -2.0, math.inf, math.nan):
        assert st(lay, **dict(ok, k_scale=bad)) == nat.ERR_BAD_SHAPE, bad
        assert st(lay, **dict(ok, v_scale=bad)) == nat.ERR_BAD_SHAPE, bad
    assert st(g.make_layer("global", 32, 4, 512), **ok) == 0
    shared = g.make_layer("global", 32, 4, 512, kv_shared=True)
    assert st(shared, **dict(ok, v_new=None, v_pool=None, v_scale=0.0)) == 0
    assert st(shared, **dict(ok, v_new=2, v_pool=None)) == nat.ERR_BAD_SHAPE
    assert st(g.make_layer("global", 32, 4, 128), **ok) == nat.ERR_UNSUPPORTED
    assert st(g.make_layer("local", 32, 16, 256, window=1024, kv_shared=True), **ok) == nat.ERR_UNSUPPORTED
    assert st(lay, **dict(ok, batch=-1)) == nat.ERR_BAD_SHAPE
    assert st(lay, **dict(ok, num_pages=0)) == nat.ERR_BAD_SHAPE


def test_one_hip_runtime_in_process():
    """The library must bind the HIP runtime torch uses: two runtimes in one process make
    torch's stream handles invalid for the library's launches."""
    import re
    maps = open("/proc/self/maps").read()
    libs = {os.path.basename(p).split(".so")[0] + "|" + os.path.dirname(p)
            for p in re.findall(r"\S*libamdhip64\.so\S*", maps)}
    assert len(libs) <= 1, libs
