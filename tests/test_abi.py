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
    assert lib.cb_abi_version() == 3


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
                                 ("geom", B.Geom(32, 8, 128, 9), 2)]:
        args = dict(good)
        args[field] = value
        st = lib.cb_blend_layer(ctypes.byref(B.LayerArgs(**args)), None)
        assert st == status, field
    assert lib.cb_last_error() != b""


def test_zero_sized_calls_are_noops(lib):
    # nothing to do -> CB_OK without touching any pointer or the device
    g = _geom()
    assert _rr(lib, g, k_out=None, k_in=None, delta=None, n_tok=0) == 0
    assert lib.cb_fuse_scatter(ctypes.byref(g), None, None, None, None, None, None, 0, None) == 0
    assert lib.cb_last_error() == b""


def test_workspace_size_plan(lib):
    """The split plan is a pure host computation.  Its cost model splits when
    the query tiles leave the GPU idle or their rows are long, and not when
    the tiles already fill it or the geometry runs on the plain kernel."""
    def size(g, tok, sel):
        rg, keep = _ragged(tok, tok, sel)
        n = ctypes.c_size_t(123)
        assert lib.cb_partial_attn_workspace_size(ctypes.byref(g), ctypes.byref(rg), ctypes.byref(n)) == 0
        return n.value
    unit = 256 * 128 * 2 + 3 * 256 * 4
    # 256 query vectors per tile: 308 rows / 64 = 5 tiles x 8 heads, 2048 keys
    # in chunks of 256
    assert size(_geom(), [0, 2048], [0, 308]) == 5 * 8 * 8 * unit
    assert size(_geom(), [0, 65536], [0, 16384]) == 0           # enough tiles already
    # 922 of 6144 rows: 15 tiles; three chunks of 2048 keys fill two rounds of
    # the GPU better than eight of 768 (measured 79 against 99 us)
    assert size(_geom(), [0, 6144], [0, 922]) == 15 * 3 * 8 * unit
    # 3277 of 32768 rows: 52 tiles of up to 512 key tiles; a split only adds
    # partial traffic (measured 941 us unsplit against 1018 us in 5 chunks)
    assert size(_geom(), [0, 32768], [0, 3277]) == 0
    assert size(_geom(dt=B.CB_DTYPE_F32), [0, 2048], [0, 308]) == 0   # plain kernel
    assert size(_geom(d=16), [0, 2048], [0, 308]) == 0
    assert lib.cb_partial_attn_workspace_size(ctypes.byref(_geom()), None, None) == 1


def test_workspace_plan_properties(lib):
    """Random ragged batches: a split plan is a whole number of units, and its
    unit count is that of a chunk the planner may choose (a multiple of 64
    keys, at least 256, at most 8 chunks for the longest request); query
    tiles that alone give 1024 or more workgroups are never split."""
    rng = np.random.default_rng(11)
    unit = 256 * 128 * 2 + 3 * 256 * 4
    for _ in range(300):
        hq, hkv = [(32, 8), (64, 8), (8, 2), (16, 1), (8, 8)][rng.integers(5)]
        lens = [int(x) for x in rng.integers(1, 40000, size=rng.integers(1, 9))]
        ks = [min(n, int(n * rng.uniform(0, 0.3))) for n in lens]
        rg, keep = _ragged(np.concatenate([[0], np.cumsum(lens)]),
                           np.concatenate([[0], np.cumsum(lens)]),
                           np.concatenate([[0], np.cumsum(ks)]))
        g = _geom(hq, hkv, 128)
        n = ctypes.c_size_t(123)
        assert lib.cb_partial_attn_workspace_size(ctypes.byref(g), ctypes.byref(rg), ctypes.byref(n)) == 0
        rows = 256 // (hq // hkv)
        tiles = [-(-k // rows) for k in ks]
        if sum(tiles) * hkv >= 1024 or n.value == 0:
            assert sum(tiles) * hkv < 1024 or n.value == 0
            continue
        assert n.value % (hkv * unit) == 0
        units = n.value // (hkv * unit)
        max_n = max(nn for nn, k in zip(lens, ks) if k)
        chunks = set()
        for c in range(2, 9):
            kc = max(256, -(-(-(-max_n // c)) // 64) * 64)
            if kc < max_n:
                chunks.add(kc)
        assert any(units == sum(t * -(-nn // kc) for t, nn in zip(tiles, lens)) for kc in chunks)
