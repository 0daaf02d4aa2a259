"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, and every argument error is reported on the host with its
status code before any HIP call (so nothing here ever launches a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest

from selective_recompute_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cacheblend.h")

# Fake, 16-byte aligned device addresses: every call below must fail validation
# before using them.
P = 0x10000
P2 = 0x20000
MISALIGNED = 0x10008


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from selective_recompute_amd import build
        build.build()
    return B.lib()


def test_exports_every_declared_symbol(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(cb_[a-z_]+)\s*\(", text))
    assert {"cb_rerotate", "cb_deviation_topk", "cb_fuse_scatter", "cb_partial_attn",
            "cb_blend_layer"} <= declared
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert lib.cb_abi_version() == 7


def test_struct_layouts_match_the_header(tmp_path):
    """The binding's ctypes structs have the sizes and field offsets a C
    compiler gives the header's structs (gcc, host only)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no host C compiler")
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "cacheblend.h"\n'
        'int main(void) {\n'
        '  printf("%zu %zu %zu %zu %zu %zu %zu\\n", sizeof(cb_layer_args),\n'
        '         offsetof(cb_layer_args, workspace_bytes), offsetof(cb_layer_args, order),\n'
        '         offsetof(cb_layer_args, flags), sizeof(cb_attn_plan), sizeof(cb_ragged),\n'
        '         sizeof(cb_geom));\n'
        '  return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    want = [ctypes.sizeof(B.LayerArgs), B.LayerArgs.workspace_bytes.offset,
            B.LayerArgs.order.offset, B.LayerArgs.flags.offset, ctypes.sizeof(B.AttnPlan),
            ctypes.sizeof(B.Ragged), ctypes.sizeof(B.Geom)]
    assert got == want


def test_check_indices_validates_on_the_host(lib):
    rg, keep = _ragged([0, 10, 25], [0, 6, 13], [0, 2, 5])
    assert lib.cb_check_indices(ctypes.byref(rg), P, P, P, None, None) == 1
    assert b"flags" in lib.cb_last_error()
    assert lib.cb_check_indices(None, P, P, P, P, None) == 1
    bad, keep2 = _ragged([0, 10, 5], [0, 6, 13], [0, 2, 5])   # offsets that go down
    assert lib.cb_check_indices(ctypes.byref(bad), P, P, P, P, None) == 1


def test_status_strings(lib):
    assert lib.cb_status_str(0) == b"CB_OK"
    assert lib.cb_status_str(1) == b"CB_ERR_INVALID_ARG"
    assert lib.cb_status_str(2) == b"CB_ERR_UNSUPPORTED"
    assert lib.cb_status_str(3) == b"CB_ERR_HIP"


def _geom(hq=32, hkv=8, d=128, dt=B.CB_DTYPE_BF16):
    return B.Geom(hq, hkv, d, dt)


def _rr(lib, g, k_out=P, k_in=P, delta=P, n_tok=16, n_layers=1, theta=1e4, style=0):
    gp = ctypes.byref(g) if g is not None else None
    return lib.cb_rerotate(gp, k_out, k_in, delta, n_tok, n_layers, theta, style, None)


@pytest.mark.parametrize("case,status,needle", [
    (dict(g=None), 1, "geom"),
    (dict(g=B.Geom(32, 8, 128, 7)), 2, "dtype"),
    (dict(g=B.Geom(30, 8, 128, 1)), 1, "multiple"),
    (dict(g=B.Geom(32, 8, 96, 1)), 2, "head_dim"),
    (dict(g=B.Geom(32, 0, 128, 1)), 1, "head counts"),
    (dict(k_in=MISALIGNED), 1, "aligned"),
    (dict(k_out=None), 1, "NULL"),
    (dict(delta=None), 1, "NULL"),
    (dict(n_layers=0), 1, "n_layers"),
    (dict(n_tok=-1), 1, "n_tok"),
    (dict(theta=0.0), 1, "rope_theta"),
    (dict(theta=float("nan")), 1, "rope_theta"),
    (dict(style=5), 1, "rope_style"),
    (dict(k_out=P + 64), 1, "overlap"),
])
def test_rerotate_argument_errors(lib, case, status, needle):
    args = dict(g=_geom())
    args.update(case)
    st = _rr(lib, **args)
    assert st == status
    assert needle in lib.cb_last_error().decode()


def _ragged(tok, cand, sel, n_req=None):
    arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in (tok, cand, sel)]
    ip = ctypes.POINTER(ctypes.c_int32)
    rg = B.Ragged(len(arrs[0]) - 1 if n_req is None else n_req, P, P, P,
                  *(a.ctypes.data_as(ip) for a in arrs))
    return rg, arrs


@pytest.mark.parametrize("tok,cand,sel,n_req,needle", [
    ([0, 10], [0, 10], [0, 11], None, "selects"),          # k > M
    ([0, 10], [0, 12], [0, 3], None, "candidates for"),    # M > N
    ([1, 10], [0, 10], [0, 3], None, "[0]"),               # offsets start at 0
    ([0, 10, 5], [0, 5, 5], [0, 1, 1], None, "decreases"),
    ([0, 10], [0, 10], [0, 3], 0, "n_req"),
])
def test_deviation_topk_ragged_errors(lib, tok, cand, sel, n_req, needle):
    rg, keep = _ragged(tok, cand, sel, n_req)
    g = _geom()
    st = lib.cb_deviation_topk(ctypes.byref(g), ctypes.byref(rg), P, P, P, P, P, P, None)
    assert st == B.CB_ERR_INVALID_ARG
    assert needle in lib.cb_last_error().decode()


def test_deviation_topk_pointer_errors(lib):
    rg, keep = _ragged([0, 10], [0, 10], [0, 3])
    g = _geom()
    st = lib.cb_deviation_topk(ctypes.byref(g), ctypes.byref(rg), P, None, P, P, P, P, None)
    assert st == 1 and "v_old" in lib.cb_last_error().decode()
    st = lib.cb_deviation_topk(ctypes.byref(g), ctypes.byref(rg), P, P, P, P, P + 2, P, None)
    assert st == 1 and "sel_local" in lib.cb_last_error().decode()
    st = lib.cb_deviation_topk(ctypes.byref(g), None, P, P, P, P, P, P, None)
    assert st == 1
    st = lib.cb_topk(ctypes.byref(rg), None, P, P, P, None)
    assert st == 1 and "dev" in lib.cb_last_error().decode()


def test_kv_deviation_source_errors(lib):
    """The source decides which tensors are needed; an unknown source is an
    argument error; V alone (source 0) needs no K pointer and K alone none of V."""
    rg, keep = _ragged([0, 10], [0, 10], [0, 3])
    g = _geom()

    def call(source, k_new=P, k_cached=P, v_new=P, v_old=P, dev=P):
        return lib.cb_kv_deviation_topk(ctypes.byref(g), ctypes.byref(rg), source, k_new,
                                        k_cached, v_new, v_old, P, dev, P, P, None)
    assert call(3) == 1 and "source" in lib.cb_last_error().decode()
    assert call(-1) == 1
    assert call(B.CB_DEV_K, k_cached=None) == 1 and "k_cached" in lib.cb_last_error().decode()
    assert call(B.CB_DEV_KV, k_new=MISALIGNED) == 1 and "aligned" in lib.cb_last_error().decode()
    assert call(B.CB_DEV_KV, v_old=None) == 1 and "v_old" in lib.cb_last_error().decode()
    assert call(B.CB_DEV_K, dev=None) == 1 and "dev" in lib.cb_last_error().decode()
    # no candidates: nothing to read, nothing launched
    rg0, keep0 = _ragged([0, 10], [0, 0], [0, 0])
    assert lib.cb_kv_deviation_topk(ctypes.byref(g), ctypes.byref(rg0), B.CB_DEV_KV, None, None,
                                    None, None, None, None, None, None, None) == 0


def test_fuse_and_attention_errors(lib):
    g = _geom()
    assert lib.cb_fuse_scatter(ctypes.byref(g), P, P, P, P, P, P, -1, None) == 1
    assert lib.cb_fuse_scatter(ctypes.byref(g), P, None, P, P, P, P, 4, None) == 1
    assert lib.cb_fuse_scatter(ctypes.byref(_geom(d=80)), P, P, P, P, P, P, 4, None) == 2
    rg, keep = _ragged([0, 10], [0, 10], [0, 3])
    assert lib.cb_partial_attn(ctypes.byref(g), ctypes.byref(rg), P, P, P, P, P, P, 0.0, None, 0, None) == 1
    assert "softmax_scale" in lib.cb_last_error().decode()
    assert lib.cb_partial_attn(ctypes.byref(g), ctypes.byref(rg), P, None, P, P, P, P, 0.1, None, 0, None) == 1
    # a workspace size with no pointer is an error
    assert lib.cb_partial_attn(ctypes.byref(g), ctypes.byref(rg), P, P, P, P, P, P, 0.1, None, 64, None) == 1
    assert "workspace" in lib.cb_last_error().decode()
    rg2, keep2 = _ragged([0, 10], [0, 10], [0, 11])
    assert lib.cb_partial_attn(ctypes.byref(g), ctypes.byref(rg2), P, P, P, P, P, P, 0.1, None, 0, None) == 1


def test_blend_layer_validates_every_stage_first(lib):
    assert lib.cb_blend_layer(None, None) == 1
    rg, keep = _ragged([0, 10], [0, 10], [0, 3])
    good = dict(geom=_geom(), rg=rg, k=P, v=P2, k_new_c=P, v_new_c=P, q_c=P, delta=P,
                cand_idx=P, rope_theta=1e4, rope_style=0, softmax_scale=0.1, dev=P,
                sel_local=P, sel_global=P, out=P, workspace=None, workspace_bytes=0)
    # a bad field of the LAST stage still fails before anything is enqueued
    for field, value, status in [("out", None, 1), ("softmax_scale", -1.0, 1),
                                 ("rope_style", 3, 1), ("cand_idx", None, 1),
                                 ("workspace_bytes", 1024, 1), ("dev_source", 7, 1),
                                 ("order", 3, 1), ("order", -1, 1), ("flags", 2, 1),
                                 ("flags", 0x80000000, 1),
                                 ("geom", B.Geom(32, 8, 128, 9), 2)]:
        args = dict(good)
        args[field] = value
        st = lib.cb_blend_layer(ctypes.byref(B.LayerArgs(**args)), None)
        assert st == status, field
    assert lib.cb_last_error() != b""
    # the select-first order scores V only: the keys are re-rotated after it
    for src in (B.CB_DEV_K, B.CB_DEV_KV):
        args = dict(good, order=B.CB_ORDER_SELECT_FIRST, dev_source=src)
        assert lib.cb_blend_layer(ctypes.byref(B.LayerArgs(**args)), None) == 1
        assert b"CB_ORDER_SELECT_FIRST" in lib.cb_last_error()


def test_blend_layer_noalloc_validates_and_refuses_a_workspace(lib):
    """cb_blend_layer_noalloc checks every stage as cb_blend_layer does and
    refuses a workspace (it brings its own static scratch), all before any
    HIP call, so nothing here touches a device."""
    assert lib.cb_blend_layer_noalloc(None, None) == 1
    rg, keep = _ragged([0, 10], [0, 10], [0, 3])
    good = dict(geom=_geom(), rg=rg, k=P, v=P2, k_new_c=P, v_new_c=P, q_c=P, delta=P,
                cand_idx=P, rope_theta=1e4, rope_style=0, softmax_scale=0.1, dev=P,
                sel_local=P, sel_global=P, out=P, workspace=None, workspace_bytes=0)
    for field, value, status, text in [("workspace", P, 1, b"static scratch"),
                                       ("workspace_bytes", 1024, 1, b"static scratch"),
                                       ("out", None, 1, b"out"),
                                       ("order", 3, 1, b"order"),
                                       ("flags", 4, 1, b"flags"),
                                       ("geom", B.Geom(32, 8, 128, 9), 2, b"dtype")]:
        args = dict(good)
        args[field] = value
        assert lib.cb_blend_layer_noalloc(ctypes.byref(B.LayerArgs(**args)), None) == status, field
        assert text in lib.cb_last_error(), field


def test_blend_layer_order_choice(lib):
    """CB_ORDER_AUTO selects first for a V deviation while the layer's K cache
    is at most CB_SELECT_FIRST_MAX_BYTES (16 MiB), or when the shared
    re-rotation + deviation launch does not cover the geometry."""
    def order(n_tok, g=None, **kw):
        rg, keep = _ragged([0, n_tok], [0, n_tok], [0, 1])
        args = dict(geom=g or _geom(), rg=rg, k=P, v=P2, k_new_c=P, v_new_c=P, q_c=P, delta=P,
                    cand_idx=P, rope_theta=1e4, rope_style=0, softmax_scale=0.1, dev=P,
                    sel_local=P, sel_global=P, out=P, workspace=None, workspace_bytes=0)
        args.update(kw)
        o = ctypes.c_int32(-1)
        st = lib.cb_blend_layer_order(ctypes.byref(B.LayerArgs(**args)), ctypes.byref(o))
        return st, o.value
    first, rot = (0, B.CB_ORDER_SELECT_FIRST), (0, B.CB_ORDER_ROTATE_FIRST)
    # 2 KiB rows (8 KV heads x 128, bf16): 8192 rows = 16 MiB
    assert order(2048) == first and order(6144) == first and order(8192) == first
    assert order(8193) == rot and order(32768) == rot
    assert order(32768, order=B.CB_ORDER_SELECT_FIRST) == first
    assert order(2048, order=B.CB_ORDER_ROTATE_FIRST) == rot
    assert order(2048, dev_source=B.CB_DEV_K) == rot and order(2048, dev_source=B.CB_DEV_KV) == rot
    assert order(2048, delta=None) == rot                       # nothing to re-rotate
    assert order(100000, g=_geom(64, 64, 128)) == first         # rows too wide for the shared launch
    assert order(2048, order=5)[0] == 1
    assert order(2048, order=B.CB_ORDER_SELECT_FIRST, dev_source=B.CB_DEV_K)[0] == 1
    assert lib.cb_blend_layer_order(None, None) == 1


def _rf(lib, g, k=P, v=P2, kn=P, vn=P2, delta=P, sl=P, sg=P, k_total=4, n_tok=16, theta=1e4,
        style=0):
    return lib.cb_rerotate_fuse(ctypes.byref(g), k, v, kn, vn, delta, sl, sg, k_total, n_tok,
                                theta, style, None)


def test_rerotate_fuse_errors(lib):
    """cb_rerotate_fuse checks what cb_rerotate and cb_fuse_scatter check, and
    that S fits the tokens (fake pointers: nothing may launch)."""
    g = _geom()
    for case, status, needle in [
        (dict(k_total=17), 1, "exceeds n_tok"),
        (dict(k_total=-1), 1, "k_total"),
        (dict(n_tok=-1), 1, "n_tok"),
        (dict(v=None), 1, "NULL"),
        (dict(kn=MISALIGNED), 1, "aligned"),
        (dict(delta=None), 1, "delta"),
        (dict(sg=None), 1, "sel_global"),
        (dict(sl=P + 2), 1, "4-byte"),
        (dict(theta=-1.0), 1, "rope_theta"),
        (dict(style=2), 1, "rope_style"),
    ]:
        assert _rf(lib, g, **case) == status, case
        assert needle in lib.cb_last_error().decode(), (case, lib.cb_last_error())
    assert _rf(lib, _geom(d=80)) == 2
    assert _rf(lib, B.Geom(32, 8, 128, 5)) == 2
    # nothing to do: no pointer is touched
    assert _rf(lib, g, k=None, v=None, kn=None, vn=None, delta=None, sl=None, sg=None,
               k_total=0, n_tok=0) == 0
    assert lib.cb_last_error() == b""


def test_zero_sized_calls_are_noops(lib):
    # nothing to do -> CB_OK without touching any pointer or the device
    g = _geom()
    assert _rr(lib, g, k_out=None, k_in=None, delta=None, n_tok=0) == 0
    assert lib.cb_fuse_scatter(ctypes.byref(g), None, None, None, None, None, None, 0, None) == 0
    assert lib.cb_last_error() == b""


SIZE_MAX = ctypes.c_size_t(-1).value


def _unit(ks, d=128):
    """Workspace bytes of one split unit: fp16 O of 256 / ks query vectors plus
    three fp32 values per vector."""
    q = 256 // ks
    return q * d * 2 + 3 * q * 4


def _split_ws(ks, workgroups, tiles, hkv, d=128):
    """A split's workspace: every workgroup's partial, then (256-byte aligned)
    one 4-byte arrival counter per (tile, KV head)."""
    return -(-workgroups * _unit(ks, d) // 256) * 256 + 4 * tiles * hkv


def _stream_ws(spans, tiles, hkv, d=128):
    """The balanced decomposition's workspace: two partial slots per
    workgroup, then (256-byte aligned) one arrival counter per (tile, KV head)."""
    return _split_ws(1, 2 * spans * hkv, tiles, hkv, d)


def _plan(lib, g, tok, sel, ws=SIZE_MAX):
    rg, keep = _ragged(tok, tok, sel)
    p = B.AttnPlan()
    assert lib.cb_partial_attn_plan(ctypes.byref(g), ctypes.byref(rg), ws, ctypes.byref(p)) == 0
    n = ctypes.c_size_t(123)
    assert lib.cb_partial_attn_workspace_size(ctypes.byref(g), ctypes.byref(rg), ctypes.byref(n)) == 0
    if ws == SIZE_MAX:
        assert n.value == p.workspace_bytes
    return p


def test_attention_plan_choices(lib):
    """The plan is a pure host computation.  Its cost model (fitted to MI355X
    timings of these shapes) splits the keys of each tile over two wave
    groups and / or long rows over key chunks when the query tiles leave the
    GPU idle, and does neither when the tiles fill it or the geometry runs on
    the plain kernel."""
    def fields(p):
        return (p.mfma, p.key_split, p.rows_per_tile, p.key_chunk, p.tiles, p.workgroups)
    # 308 of 2048 rows: key split 2 (32 rows per tile, 10 tiles), 4 chunks of
    # 512 keys, 216 working workgroups: measured 20.1 us against 22.2 for the
    # best key-split-1 plan (8 chunks of 256 keys) and 35.1 unsplit
    p = _plan(lib, _geom(), [0, 2048], [0, 308])
    assert fields(p) == (1, 2, 32, 512, 10, 320) and p.workspace_bytes == _split_ws(2, 320, 10, 8)
    # without workspace the same batch stays unsplit, still with key split 2
    p = _plan(lib, _geom(), [0, 2048], [0, 308], ws=0)
    assert fields(p) == (1, 2, 32, 0, 10, 80) and p.workspace_bytes == 0
    # 1844 of 6144 rows: two chunks of 3072 keys (the key-split-2 plans need
    # more than one round of the CUs, where they lose in the full step)
    p = _plan(lib, _geom(), [0, 6144], [0, 1844])
    assert fields(p) == (1, 1, 64, 3072, 29, 464) and p.workspace_bytes == _split_ws(1, 464, 29, 8)
    # 922 of 6144 rows: three chunks of 2048 keys (the 6k-token blend step:
    # 2.88 ms against 2.92 with key split 2 in two chunks of 3072 keys)
    p = _plan(lib, _geom(), [0, 6144], [0, 922])
    assert fields(p) == (1, 1, 64, 2048, 15, 360) and p.workspace_bytes == _split_ws(1, 360, 15, 8)
    # 3277 of 32768 rows: 52 tiles over four chunks of 8192 keys, launched
    # longest piece first (858 us against 912 unsplit and 867-889 for the
    # other chunkings, attention alone, one box)
    p = _plan(lib, _geom(), [0, 32768], [0, 3277])
    assert fields(p) == (1, 1, 64, 8192, 52, 1664)
    # 1024 workgroups or more: always key split 1 unsplit
    p = _plan(lib, _geom(), [0, 65536], [0, 16384])
    assert fields(p) == (1, 1, 64, 0, 256, 2048) and p.workspace_bytes == 0
    # the plain kernel: one workgroup per selected row and query head
    for g in (_geom(dt=B.CB_DTYPE_F32), _geom(d=16), _geom(24, 8, 128)):
        p = _plan(lib, g, [0, 2048], [0, 308])
        assert fields(p) == (0, 0, 0, 0, 0, 308 * g.n_q_heads) and p.workspace_bytes == 0
    rg, keep = _ragged([0, 2048], [0, 2048], [0, 308])
    assert lib.cb_partial_attn_workspace_size(ctypes.byref(_geom()), None, None) == 1
    assert lib.cb_partial_attn_plan(ctypes.byref(_geom()), ctypes.byref(rg), SIZE_MAX, None) == 1
    assert b"plan" in lib.cb_last_error()


def test_workspace_plan_properties(lib):
    """Random ragged batches: the plan's tiles, workgroups and workspace follow
    from its key split and key chunk (a multiple of the 64 * key_split keys
    of a tile, at least 256, at most 8 chunks for the longest request, one of
    the chunk counts 2..8); query tiles that alone give 1024 or more
    workgroups are never split; a workspace limit is respected."""
    rng = np.random.default_rng(11)
    seen = set()
    for i in range(300):
        hq, hkv = [(32, 8), (64, 8), (8, 2), (16, 1), (8, 8)][rng.integers(5)]
        lens = [int(x) for x in rng.integers(1, [40000, 4000][i % 2], size=rng.integers(1, 9))]
        ks = [min(n, int(n * rng.uniform(0, 0.3))) for n in lens]
        tok = np.concatenate([[0], np.cumsum(lens)])
        sel = np.concatenate([[0], np.cumsum(ks)])
        g = _geom(hq, hkv, 128)
        p = _plan(lib, g, tok, sel)
        assert p.mfma == 1 and p.key_split in (1, 2)
        rows = 256 // p.key_split // (hq // hkv)
        assert p.rows_per_tile == rows
        tiles = [-(-k // rows) for k in ks]
        assert p.tiles == sum(tiles)
        tiles1 = sum(-(-k // (256 // (hq // hkv))) for k in ks)
        if tiles1 * hkv >= 1024:
            assert (p.key_split, p.key_chunk, p.workspace_bytes) == (1, 0, 0)
        assert p.stream_spans == 0              # only a pinned plan is balanced
        seen.add((p.key_split, p.key_chunk > 0))
        if p.key_chunk == 0:
            assert p.workgroups == p.tiles * hkv and p.workspace_bytes == 0
            continue
        kt = 64 * p.key_split
        max_n = max(nn for nn, k in zip(lens, ks) if k)
        chunks = {max(256, -(-(-(-max_n // c)) // kt) * kt) for c in range(2, 9)}
        assert p.key_chunk in chunks and p.key_chunk < max_n
        units = sum(t * -(-nn // p.key_chunk) for t, nn in zip(tiles, lens))
        assert p.workgroups == units * hkv
        assert p.workspace_bytes == _split_ws(p.key_split, units * hkv, p.tiles, hkv)
        # a smaller workspace gives a plan that fits it
        q = _plan(lib, g, tok, sel, ws=p.workspace_bytes - 1)
        assert q.workspace_bytes <= p.workspace_bytes - 1
    assert seen == {(1, False), (1, True), (2, False), (2, True)}


def test_pinned_balanced_plans(lib):
    """The balanced decomposition, pinned: stream_spans workgroups per KV head,
    two partial slots each and a counter per (query tile, KV head); key split
    1 and no key chunk only; at most 1024 requests and 2048 query tiles."""
    tok, sel = [0, 3000, 3100, 9000], [0, 450, 470, 1000]
    rg, keep = _ragged(tok, tok, sel)
    g = _geom()

    def describe(ks, kc, spans, r=None):
        p = B.AttnPlan(1, ks, 0, kc, 0, 0, 0, spans)
        st = lib.cb_partial_attn_describe_plan(ctypes.byref(g), ctypes.byref(r or rg), ctypes.byref(p))
        return st, p

    tiles = -(-450 // 64) + -(-20 // 64) + -(-530 // 64)
    for spans in (1, 7, 32, 300):
        st, p = describe(1, 0, spans)
        assert st == 0 and p.stream_spans == spans and p.key_chunk == 0
        assert (p.tiles, p.workgroups) == (tiles, spans * 8)
        assert p.workspace_bytes == _stream_ws(spans, tiles, 8)
    for ks, kc, spans, status in [(2, 0, 8, 1), (1, 512, 8, 1), (1, 0, -1, 1), (1, 0, 65537, 1)]:
        st, p = describe(ks, kc, spans)
        assert st == status, (ks, kc, spans)
    assert b"stream_spans" in lib.cb_last_error()
    # more than 1024 requests, or more than 2048 query tiles
    n = 1100
    many, keep2 = _ragged(list(range(0, 10 * n + 1, 10)), list(range(0, 10 * n + 1, 10)),
                          list(range(0, n + 1)))
    assert describe(1, 0, 8, many)[0] == 2
    big, keep3 = _ragged([0, 200000], [0, 200000], [0, 2049 * 64])
    assert describe(1, 0, 8, big)[0] == 2
    assert b"2048" in lib.cb_last_error()
    # a workspace smaller than the plan's is refused before anything launches
    st, p = describe(1, 0, 32)
    P = ctypes.c_void_p(1 << 40)
    args = [ctypes.byref(g), ctypes.byref(rg), ctypes.byref(p), P, P, P, P, P, P, 0.1, P,
            p.workspace_bytes - 1, 0, None]
    assert lib.cb_partial_attn_with_plan(*args) == 1
    assert b"workspace" in lib.cb_last_error()


def test_pinned_plans(lib):
    """cb_partial_attn_describe_plan completes a pinned plan with the same
    counts as a chosen one, and it and cb_partial_attn_with_plan reject every
    invalid field on the host (fake device pointers: nothing may launch)."""
    tok, sel = [0, 3000, 3100], [0, 450, 470]
    rg, keep = _ragged(tok, tok, sel)

    def describe(g, mfma, ks, kc):
        p = B.AttnPlan(mfma, ks, 0, kc, 0, 0, 0)
        st = lib.cb_partial_attn_describe_plan(ctypes.byref(g), ctypes.byref(rg), ctypes.byref(p))
        return st, p

    for ks in (1, 2):
        rows = 64 // ks
        tiles = -(-450 // rows) + 1
        st, p = describe(_geom(), 1, ks, 0)
        assert st == 0 and (p.rows_per_tile, p.tiles, p.workgroups, p.workspace_bytes) == (rows, tiles, 8 * tiles, 0)
        for kc in (384, 768, 1024, 3072):
            if kc % (64 * ks):
                continue
            st, p = describe(_geom(), 1, ks, kc)
            units = -(-450 // rows) * -(-3000 // kc) + -(-100 // kc)
            split = -(-3000 // kc) > 1
            assert st == 0 and p.workgroups == 8 * units and p.key_chunk == (kc if split else 0)
            assert p.workspace_bytes == (_split_ws(ks, 8 * units, p.tiles, 8) if split else 0)
    st, p = describe(_geom(dt=B.CB_DTYPE_F32), 0, 0, 0)
    assert st == 0 and (p.mfma, p.workgroups) == (0, 470 * 32)
    bad = [
        (_geom(), 2, 1, 0, 1, "mfma"),
        (_geom(), 1, 3, 0, 1, "key_split"),
        (_geom(), 1, 1, 100, 1, "multiple of 64"),
        (_geom(), 1, 2, 192, 1, "multiple of 128"),
        (_geom(), 1, 1, -64, 1, "multiple"),
        (_geom(), 1, 1, 256, 1, "more than 8 chunks"),
        (_geom(dt=B.CB_DTYPE_F32), 1, 1, 0, 2, "MFMA"),
        (_geom(256, 1, 64), 1, 2, 0, 2, "key split 2"),
        (_geom(24, 8, 128), 1, 1, 0, 2, "MFMA"),
    ]
    for g, mfma, ks, kc, status, needle in bad:
        p = B.AttnPlan(mfma, ks, 7, kc, 7, 7, 7)
        assert lib.cb_partial_attn_describe_plan(ctypes.byref(g), ctypes.byref(rg), ctypes.byref(p)) == status
        assert needle.encode() in lib.cb_last_error(), lib.cb_last_error()
        assert (p.rows_per_tile, p.tiles, p.workgroups, p.workspace_bytes) == (7, 7, 7, 7)
        assert lib.cb_partial_attn_with_plan(ctypes.byref(g), ctypes.byref(rg), ctypes.byref(p), P, P, P, P,
                                             P, P, 0.1, None, 0, 0, None) == status
        assert needle.encode() in lib.cb_last_error()
    # a split needs its workspace
    p = B.AttnPlan(1, 1, 0, 1024, 0, 0, 0)
    assert lib.cb_partial_attn_with_plan(ctypes.byref(_geom()), ctypes.byref(rg), ctypes.byref(p), P, P, P, P,
                                         P, P, 0.1, P2, 4096, B.CB_ATTN_COUNTERS_ZERO, None) == 1
    assert b"smaller than the plan" in lib.cb_last_error()
    assert lib.cb_partial_attn_with_plan(ctypes.byref(_geom()), ctypes.byref(rg), None, P, P, P, P,
                                         P, P, 0.1, None, 0, 0, None) == 1
    # flags other than CB_ATTN_COUNTERS_ZERO
    for flags in (2, 0x80000000, 3):
        p = B.AttnPlan(1, 1, 0, 0, 0, 0, 0)
        assert lib.cb_partial_attn_with_plan(ctypes.byref(_geom()), ctypes.byref(rg), ctypes.byref(p), P, P, P, P,
                                             P, P, 0.1, None, 0, flags, None) == 1
        assert b"unknown flags" in lib.cb_last_error()
    assert lib.cb_partial_attn_describe_plan(ctypes.byref(_geom()), ctypes.byref(rg), None) == 1
