"""Host-side checks of the C ABI: the library loads, exports every function
include/fm.h declares, and rejects bad arguments before any GPU work (so these
run on machines without a GPU)."""

import ctypes
import os
import re

import pytest
import torch

from block_diffusion_drafter_all_amd import binding as B
from block_diffusion_drafter_all_amd.build import LIB_PATH, REPO_DIR

HEADER = os.path.join(REPO_DIR, "include", "fm.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fm_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        from block_diffusion_drafter_all_amd.build import build
        build()
    return B.load_library()


def test_every_declared_symbol_is_exported(lib):
    declared = _declared()
    assert set(declared) == set(B.SYMBOLS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_empty_error(lib):
    assert "gfx950" in B.fm_version()
    assert lib.fm_write_context_kv_workspace_size(10) > 0


def test_workspace_sizes(lib):
    small = lib.fm_cross_attention_workspace_size(1, 4, 64, 16, B.FM_BF16)
    big = lib.fm_cross_attention_workspace_size(64, 32, 128, 16, B.FM_BF16)
    assert 0 < small < big
    assert small % 256 == 0 and big % 256 == 0
    assert lib.fm_cross_attention_workspace_size(4, 0, 128, 16, B.FM_BF16) == 0
    assert lib.fm_cross_attention_workspace_size(4, 4, 96, 16, B.FM_BF16) == 0
    assert lib.fm_cross_attention_workspace_size(4, 4, 128, 65, B.FM_BF16) == 0
    # candidate blocks: 1, 2 or 4 query fragments per request
    one, two, four = (lib.fm_cross_attention_workspace_size(64, 32, 128, m, B.FM_BF16) for m in (16, 32, 64))
    assert big == one < two < four
    assert lib.fm_cross_attention_workspace_size(64, 32, 128, 17, B.FM_BF16) == two
    assert lib.fm_cross_attention_workspace_size(64, 32, 128, 48, B.FM_BF16) == four
    assert lib.fm_write_context_kv_workspace_size(1152) >= 256 + 4 * 4 * 1152
    # an e4m3 pool's plan cuts for twice the resident waves: more partial slots
    e4 = lib.fm_cross_attention_workspace_size(64, 32, 128, 16, B.FM_BF16_E4M3)
    assert e4 > one and lib.fm_cross_attention_workspace_size(64, 32, 128, 16, 7) == 0


FAKE = 1 << 20   # a non-null, 256-aligned host-side stand-in; never dereferenced


def _pool(num_pages=4):
    return B.fm_kv_pool(FAKE, FAKE, num_pages, 16 * 4 * 64, 4 * 64, 64)


def _cross(lib, **over):
    args = dict(q=FAKE, dt=B.FM_BF16, total_q=16, qn=FAKE, pool=_pool(), pt=FAKE, pt_stride=4, ps=16, ctx=FAKE,
                cu=FAKE, max_q=16, bs=1, H=4, Dh=64, scale=0.125, theta=1e6, eps=1e-6, out=FAKE, ws=FAKE,
                ws_bytes=1 << 30)
    args.update(over)
    pool = args["pool"]
    return lib.fm_paged_cross_attention(args["q"], args["dt"], args["total_q"], args["qn"],
                                        ctypes.byref(pool) if pool is not None else None,
                                        args["pt"], args["pt_stride"], args["ps"], args["ctx"], args["cu"],
                                        args["max_q"], args["bs"], args["H"], args["Dh"], args["scale"], args["theta"],
                                        args["eps"], args.get("fp8"), args["out"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("over,status,needle", [
    (dict(q=None), B.FM_E_INVALID, "null"),
    (dict(max_q=65), B.FM_E_UNSUPPORTED, "max_q"),
    (dict(max_q=-1), B.FM_E_INVALID, "max_q"),
    (dict(pool=None), B.FM_E_INVALID, "null"),
    (dict(Dh=96), B.FM_E_UNSUPPORTED, "head_dim"),
    (dict(dt=7), B.FM_E_UNSUPPORTED, "dtype"),
    (dict(dt=3), B.FM_E_UNSUPPORTED, "dtype"),
    # e4m3 elements are one byte: a stride of 72 elements is 144 bytes in bf16, 72 in e4m3
    (dict(dt=B.FM_BF16_E4M3, pool=B.fm_kv_pool(FAKE, FAKE, 4, 4096, 72, 64)), B.FM_E_INVALID, "16 bytes"),
    (dict(fp8=B._floats([0.0, 1.0, 1.0])), B.FM_E_INVALID, "e4m3 pool only"),
    (dict(dt=B.FM_BF16_E4M3, fp8=B._floats([-1.0, 1.0, 1.0])), B.FM_E_INVALID, "query scale"),
    (dict(dt=B.FM_BF16_E4M3, fp8=B._floats([0.0, 0.0, 1.0])), B.FM_E_INVALID, "descales"),
    (dict(dt=B.FM_BF16_E4M3, fp8=B._floats([0.0, 1.0, float("nan")])), B.FM_E_INVALID, "descales"),
    (dict(ps=12), B.FM_E_UNSUPPORTED, "page_size"),
    (dict(H=0), B.FM_E_INVALID, "H"),
    (dict(ws=None), B.FM_E_WORKSPACE, "workspace"),
    (dict(ws_bytes=1000), B.FM_E_WORKSPACE, "needed"),
    (dict(ws=FAKE + 64), B.FM_E_WORKSPACE, "aligned"),
    (dict(pool=B.fm_kv_pool(FAKE, FAKE, 0, 4096, 256, 64)), B.FM_E_INVALID, "num_pages"),
    (dict(pool=B.fm_kv_pool(FAKE, FAKE, 4, 4096, 250, 64)), B.FM_E_INVALID, "16 bytes"),
    (dict(eps=-1.0), B.FM_E_INVALID, "eps"),
    (dict(theta=0.0), B.FM_E_INVALID, "rope_theta"),
    (dict(scale=float("inf")), B.FM_E_INVALID, "softmax_scale"),
    (dict(pt_stride=0), B.FM_E_INVALID, "pt_stride"),
    (dict(pool=B.fm_kv_pool(FAKE, FAKE, 4, 1 << 32, 256, 64)), B.FM_E_UNSUPPORTED, "below 2^32"),
])
def test_cross_attention_rejects(lib, over, status, needle):
    assert _cross(lib, **over) == status
    assert needle in B.fm_last_error()


def test_timed_cross_attention_rejects(lib):
    """The timed call takes the untimed call's checks plus its record array."""
    pool = _pool()
    args = [FAKE, B.FM_BF16, 16, FAKE, ctypes.byref(pool), FAKE, 4, 16, FAKE, FAKE, 16, 1, 4, 64, 0.125, 1e6, 1e-6,
            None, FAKE, FAKE, 1 << 30]
    assert lib.fm_paged_cross_attention_timed(*args, None, 4096, None) == B.FM_E_INVALID
    assert "wave_clock is null" in B.fm_last_error()
    assert lib.fm_paged_cross_attention_timed(*args, FAKE, 3, None) == B.FM_E_INVALID
    assert "wave records" in B.fm_last_error()
    bad = list(args)
    bad[13] = 96  # head dim
    assert lib.fm_paged_cross_attention_timed(*bad, FAKE, 4096, None) == B.FM_E_UNSUPPORTED


def test_cross_attention_empty_is_noop(lib):
    assert _cross(lib, total_q=0, q=None) == B.FM_OK
    assert _cross(lib, bs=0) == B.FM_OK
    assert _cross(lib, total_q=-1) == B.FM_E_INVALID


def test_plan_rejects(lib):
    assert lib.fm_plan_cross_attention(FAKE, 4, 32, 128, 65, B.FM_BF16, FAKE, 1 << 30, None) == B.FM_E_UNSUPPORTED
    assert "max_q" in B.fm_last_error()
    assert lib.fm_plan_cross_attention(None, 4, 32, 128, 16, B.FM_BF16, FAKE, 1 << 30, None) == B.FM_E_INVALID
    assert lib.fm_plan_cross_attention(FAKE, -1, 32, 128, 16, B.FM_BF16, FAKE, 1 << 30, None) == B.FM_E_INVALID
    assert lib.fm_plan_cross_attention(FAKE, 4, 32, 128, 16, B.FM_BF16, FAKE, 10, None) == B.FM_E_WORKSPACE
    assert lib.fm_plan_cross_attention(FAKE, 4, 32, 96, 16, B.FM_BF16, FAKE, 1 << 30, None) == B.FM_E_UNSUPPORTED
    assert lib.fm_plan_cross_attention(FAKE, 4, 32, 128, 16, 9, FAKE, 1 << 30, None) == B.FM_E_UNSUPPORTED
    assert "dtype" in B.fm_last_error()


def test_weighted_plan_rejects(lib):
    """The XCD weights are checked on the host before anything is enqueued."""
    good = (ctypes.c_int32 * 8)(*([1000] * 8))
    assert lib.fm_plan_cross_attention_weighted(FAKE, 4, 32, 128, 16, B.FM_BF16, None, FAKE, 1 << 30,
                                                None) == B.FM_E_INVALID
    assert "xcd_weights is null" in B.fm_last_error()
    for bad in (499, 2001, 0, -1000):
        w = (ctypes.c_int32 * 8)(*([1000] * 7 + [bad]))
        assert lib.fm_plan_cross_attention_weighted(FAKE, 4, 32, 128, 16, B.FM_BF16, w, FAKE, 1 << 30,
                                                    None) == B.FM_E_INVALID
        assert "xcd_weights[7]" in B.fm_last_error()
    # the shape checks are the unweighted call's
    assert lib.fm_plan_cross_attention_weighted(FAKE, 4, 32, 96, 16, B.FM_BF16, good, FAKE, 1 << 30,
                                                None) == B.FM_E_UNSUPPORTED
    assert lib.fm_plan_cross_attention_weighted(FAKE, 4, 32, 128, 16, B.FM_BF16, good, FAKE, 10,
                                                None) == B.FM_E_WORKSPACE
    with pytest.raises(ValueError):
        B.fm_plan_cross_attention(torch.ones(1, dtype=torch.int32), 2, 64, torch.ones(1, dtype=torch.uint8),
                                  xcd_weights=[1000] * 7)


def _write(lib, **over):
    pools = (B.fm_kv_pool * 2)(_pool(), _pool())
    a = dict(x=FAKE, n_rows=8, d_in=512, dt=B.FM_BF16, w=FAKE, kn=FAKE, rr=FAKE, rp=FAKE, cl=None, win=0, pt=FAKE,
             pt_stride=4, ps=16, bs=1, pools=pools, L=2, H=4, Dh=64, eps=1e-6, theta=1e6, slots=None, ws=FAKE,
             ws_bytes=1 << 30)
    a.update(over)
    return lib.fm_write_context_kv(a["x"], a["n_rows"], a["d_in"], a["dt"], a["w"], a["kn"], a["rr"], a["rp"],
                                   a["cl"], a["win"], a["pt"], a["pt_stride"], a["ps"], a["bs"], a["pools"], a["L"],
                                   a["H"], a["Dh"], a["eps"], a["theta"], a.get("kvs"), a["slots"], a["ws"],
                                   a["ws_bytes"], None)


@pytest.mark.parametrize("over,status,needle", [
    (dict(x=None), B.FM_E_INVALID, "null"),
    (dict(d_in=100), B.FM_E_UNSUPPORTED, "d_in"),
    (dict(L=17), B.FM_E_UNSUPPORTED, "L ="),
    (dict(cl=FAKE, win=0), B.FM_E_INVALID, "window"),
    (dict(bs=0), B.FM_E_INVALID, "bs"),
    (dict(ws_bytes=100), B.FM_E_WORKSPACE, "needed"),
    (dict(ps=3), B.FM_E_UNSUPPORTED, "page_size"),
    (dict(n_rows=-1), B.FM_E_INVALID, "n_rows"),
    (dict(dt=B.FM_BF16_E4M3, pools=(B.fm_kv_pool * 2)(_pool(), B.fm_kv_pool(FAKE, FAKE, 4, 4096, 256, 8))),
     B.FM_E_INVALID, "16 bytes"),
    (dict(kvs=B._floats([1.0, 1.0, 1.0, 1.0])), B.FM_E_INVALID, "e4m3 pool only"),
    (dict(dt=B.FM_BF16_E4M3, kvs=B._floats([1.0, 1.0, 0.0, 1.0])), B.FM_E_INVALID, "kv_scales[2]"),
    (dict(dt=B.FM_BF16_E4M3, kvs=B._floats([1.0, float("inf"), 1.0, 1.0])), B.FM_E_INVALID, "kv_scales[1]"),
])
def test_write_rejects(lib, over, status, needle):
    assert _write(lib, **over) == status
    assert needle in B.fm_last_error()


def test_write_zero_rows_is_noop(lib):
    assert _write(lib, n_rows=0, x=None) == B.FM_OK


def _write_noalloc(lib, **over):
    pools = (B.fm_kv_pool * 2)(_pool(), _pool())
    a = dict(x=FAKE, n_rows=8, d_in=512, dt=B.FM_BF16, w=FAKE, kn=FAKE, rr=FAKE, rp=FAKE, cl=None, win=0, pt=FAKE,
             pt_stride=4, ps=16, bs=1, pools=pools, L=2, H=4, Dh=64, eps=1e-6, theta=1e6, slots=None)
    a.update(over)
    return lib.fm_write_context_kv_noalloc(a["x"], a["n_rows"], a["d_in"], a["dt"], a["w"], a["kn"], a["rr"],
                                           a["rp"], a["cl"], a["win"], a["pt"], a["pt_stride"], a["ps"], a["bs"],
                                           a["pools"], a["L"], a["H"], a["Dh"], a["eps"], a["theta"], None,
                                           a["slots"], None)


def test_noalloc_write_limits_and_validation(lib):
    """The no-allocation write refuses more rows than its static workspace
    serves, and validates like fm_write_context_kv, before any GPU call."""
    assert B.FM_WRITE_NOALLOC_MAX_ROWS == 65536
    assert _write_noalloc(lib, n_rows=65537) == B.FM_E_UNSUPPORTED
    assert "65536 rows its static workspace" in B.fm_last_error()
    assert _write_noalloc(lib, n_rows=0, x=None) == B.FM_OK
    assert _write_noalloc(lib, n_rows=-1) == B.FM_E_INVALID
    assert _write_noalloc(lib, Dh=96) == B.FM_E_UNSUPPORTED
    assert _write_noalloc(lib, x=None) == B.FM_E_INVALID
    assert _write_noalloc(lib, L=17) == B.FM_E_UNSUPPORTED
    # the static workspace covers the write layout of its largest call
    assert lib.fm_write_context_kv_workspace_size(65536) <= (1 << 20) + 1024


def test_self_attention_rejects(lib):
    f = lib.fm_block_self_attention
    assert f(FAKE, B.FM_BF16, 4, 65, FAKE, FAKE, FAKE, 4, 64, 0.1, 1e6, 1e-6, FAKE, None) == B.FM_E_UNSUPPORTED
    assert "block size 65" in B.fm_last_error()
    assert f(FAKE, B.FM_BF16, 4, 0, FAKE, FAKE, FAKE, 4, 64, 0.1, 1e6, 1e-6, FAKE, None) == B.FM_E_UNSUPPORTED
    assert f(None, B.FM_BF16, 4, 16, FAKE, FAKE, FAKE, 4, 64, 0.1, 1e6, 1e-6, FAKE, None) == B.FM_E_INVALID
    assert f(None, B.FM_BF16, 0, 16, FAKE, FAKE, FAKE, 4, 64, 0.1, 1e6, 1e-6, FAKE, None) == B.FM_OK
    # the block's own q, k, v are activations: an e4m3 pool type means nothing here
    assert f(FAKE, B.FM_BF16_E4M3, 4, 16, FAKE, FAKE, FAKE, 4, 64, 0.1, 1e6, 1e-6, FAKE, None) == B.FM_E_UNSUPPORTED
    assert "FM_BF16" in B.fm_last_error()


def test_launch_grid_limit(lib):
    """Sizes whose launch grid would reach 2^32 work-items are refused before
    anything is enqueued (the check runs ahead of every launch of the call)."""
    # 2^25 rows x 256 threads
    assert lib.fm_ada_layer_norm(FAKE, 1 << 25, 1024, FAKE, FAKE, 1e-6, FAKE, None) == B.FM_E_UNSUPPORTED
    assert "2^32" in B.fm_last_error()
    # 2^24 rows x 2^20 outputs: 2^16 x 2^12 tiles of 512 threads
    assert lib.fm_linear(FAKE, 1 << 24, 512, FAKE, 1 << 20, None, 0, None, FAKE, FAKE, 1 << 30, None) \
        == B.FM_E_UNSUPPORTED
    assert "2^32" in B.fm_last_error()
    # 2^25 blocks x 4 heads, one wave each
    assert lib.fm_block_self_attention(FAKE, B.FM_BF16, 1 << 25, 16, FAKE, FAKE, FAKE, 4, 64, 0.1, 1e6, 1e-6, FAKE,
                                       None) == B.FM_E_UNSUPPORTED
    assert "2^32" in B.fm_last_error()
    # blocks of 32 and 64 slots pass the size checks (one wave per 16-slot query
    # tile): 2^24 blocks x 4 heads x 2 or 4 tiles reach the grid limit instead
    for K in (32, 64):
        assert lib.fm_block_self_attention(FAKE, B.FM_BF16, 1 << 24, K, FAKE, FAKE, FAKE, 4, 64, 0.1, 1e6, 1e-6,
                                           FAKE, None) == B.FM_E_UNSUPPORTED
        assert "2^32" in B.fm_last_error()
    # the largest sizes the checks still pass are well inside the limit
    assert lib.fm_linear_workspace_size(1 << 24, 1 << 20, 512) == 0


def test_binding_dtype_pairs():
    bf, f32 = torch.zeros(1, dtype=torch.bfloat16), torch.zeros(1)
    assert B._dtype_code(bf) == B.FM_BF16 and B._dtype_code(f32) == B.FM_F32
    assert B._dtype_code(bf, torch.bfloat16) == B.FM_BF16
    assert B._dtype_code(bf, torch.float8_e4m3fn) == B.FM_BF16_E4M3
    with pytest.raises(TypeError):
        B._dtype_code(f32, torch.float8_e4m3fn)
    with pytest.raises(TypeError):
        B._dtype_code(bf, torch.float32)


def _rows(lib, **over):
    a = dict(hidden=FAKE, n_hidden=8, d_hidden=512, w_fc=FAKE, hn=FAKE, ids=FAKE, n_anchor=2, emb=FAKE, vocab=100,
             d_target=256, wap=FAKE, bap=FAKE, an=FAKE, dim=1024, cl=None, win=0, bs=0, eps=1e-6, rows=FAKE, ws=FAKE,
             ws_bytes=1 << 30)
    a.update(over)
    return lib.fm_context_rows(a["hidden"], a["n_hidden"], a["d_hidden"], a["w_fc"], a["hn"], a["ids"], a["n_anchor"],
                               a["emb"], a["vocab"], a["d_target"], a["wap"], a["bap"], a["an"], a["dim"], a["cl"],
                               a["win"], a["bs"], a["eps"], a["rows"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("over,status,needle", [
    (dict(hidden=None), B.FM_E_INVALID, "hidden-row pointer"),
    (dict(ids=None), B.FM_E_INVALID, "anchor-row pointer"),
    (dict(dim=1000), B.FM_E_UNSUPPORTED, "dim"),
    (dict(dim=9216), B.FM_E_UNSUPPORTED, "dim"),
    (dict(d_hidden=500), B.FM_E_UNSUPPORTED, "d_hidden"),
    (dict(d_hidden=96), B.FM_E_UNSUPPORTED, "multiple of 64"),
    (dict(d_target=100), B.FM_E_UNSUPPORTED, "d_target"),
    (dict(vocab=0), B.FM_E_INVALID, "vocab"),
    (dict(cl=FAKE, win=0, bs=1), B.FM_E_INVALID, "window"),
    (dict(cl=FAKE, win=5, bs=2), B.FM_E_INVALID, "bs * window"),
    (dict(rows=FAKE + 8), B.FM_E_INVALID, "aligned"),
    (dict(ws_bytes=100), B.FM_E_WORKSPACE, "needed"),
    (dict(eps=-1.0), B.FM_E_INVALID, "eps"),
    (dict(n_hidden=-1), B.FM_E_INVALID, "n_hidden"),
])
def test_context_rows_rejects(lib, over, status, needle):
    assert _rows(lib, **over) == status
    assert needle in B.fm_last_error()


def test_context_rows_empty_and_workspace(lib):
    assert _rows(lib, n_hidden=0, n_anchor=0, hidden=None, ids=None) == B.FM_OK
    # the partials of the contraction ranges dominate: more rows, more bytes
    small = lib.fm_context_rows_workspace_size(64, 64, 20480, 4096, 4096)
    big = lib.fm_context_rows_workspace_size(1088, 64, 20480, 4096, 4096)
    assert 0 < small < big and big >= 1088 * 4096 * 4
    assert lib.fm_context_rows_workspace_size(-1, 0, 64, 64, 1024) == 0
    # anchors alone need a workspace though they pass no hidden width (and hidden rows alone no target width)
    assert lib.fm_context_rows_workspace_size(0, 3, 0, 128, 1024) > 0
    assert lib.fm_context_rows_workspace_size(5, 0, 128, 0, 1024) > 0


def test_dit_entry_points_reject(lib):
    f = lib.fm_ada_layer_norm
    assert f(FAKE, 4, 1000, FAKE, FAKE, 1e-6, FAKE, None) == B.FM_E_UNSUPPORTED and "dim" in B.fm_last_error()
    assert f(None, 4, 1024, FAKE, FAKE, 1e-6, FAKE, None) == B.FM_E_INVALID
    assert f(FAKE, 4, 1024, FAKE, FAKE, -1.0, FAKE, None) == B.FM_E_INVALID and "eps" in B.fm_last_error()
    assert f(None, 0, 1024, None, None, 1e-6, None, None) == B.FM_OK
    g = lib.fm_linear
    assert g(FAKE, 8, 512, FAKE, 2000, None, 0, None, FAKE, FAKE, 1 << 30, None) == B.FM_E_UNSUPPORTED
    assert "N 2000" in B.fm_last_error()
    assert g(FAKE, 8, 500, FAKE, 2048, None, 0, None, FAKE, FAKE, 1 << 30, None) == B.FM_E_UNSUPPORTED
    # the tile streams the contraction in 64-wide stages
    assert g(FAKE, 8, 96, FAKE, 2048, None, 0, None, FAKE, FAKE, 1 << 30, None) == B.FM_E_UNSUPPORTED
    assert "multiple of 64" in B.fm_last_error()
    assert g(FAKE, 8, 512, FAKE, 2048, None, B.FM_LINEAR_RESIDUAL, None, FAKE, FAKE, 1 << 30, None) == B.FM_E_INVALID
    assert "gate" in B.fm_last_error()
    assert g(FAKE, 8, 512, FAKE, 2048, None, 7, None, FAKE, FAKE, 1 << 30, None) == B.FM_E_UNSUPPORTED
    assert g(None, 8, 512, FAKE, 2048, None, 0, None, FAKE, FAKE, 1 << 30, None) == B.FM_E_INVALID
    assert g(None, 0, 512, None, 2048, None, 0, None, None, None, 0, None) == B.FM_OK
    # a contraction split into ranges needs its partials' workspace
    need = lib.fm_linear_workspace_size(256, 1024, 4096)
    assert need >= 2 * 256 * 1024 * 4
    assert g(FAKE, 256, 4096, FAKE, 1024, None, 0, None, FAKE, FAKE, need - 1, None) == B.FM_E_WORKSPACE
    assert lib.fm_linear_workspace_size(1024, 16384, 4096) == 0   # 256 output tiles: no split


def test_binding_refuses_host_tensors(lib):
    # The C ABI takes bare device pointers: a host tensor reaching a kernel
    # would be a GPU memory fault, so the binding refuses it before any call.
    bf = dict(dtype=torch.bfloat16)
    i32 = dict(dtype=torch.int32)
    pool = B.KVPool(torch.zeros((4, 16, 2, 64), **bf), torch.zeros((4, 16, 2, 64), **bf))
    calls = {
        "fm_linear": lambda: B.fm_linear(torch.zeros((8, 64), **bf), torch.zeros((256, 64), **bf)),
        "fm_ada_layer_norm": lambda: B.fm_ada_layer_norm(torch.zeros((2, 256)), torch.ones(256), torch.zeros(256),
                                                         1e-6),
        "fm_plan_cross_attention": lambda: B.fm_plan_cross_attention(torch.ones(1, **i32), 2, 64,
                                                                     torch.zeros(4096, dtype=torch.uint8)),
        "fm_paged_cross_attention": lambda: B.fm_paged_cross_attention(
            torch.zeros((16, 2, 64), **bf), torch.ones(64), pool, torch.zeros((1, 4), **i32), torch.ones(1, **i32),
            torch.tensor([0, 16], **i32), 0.125, 1e6, 1e-6, torch.zeros(4096, dtype=torch.uint8)),
        "fm_block_self_attention": lambda: B.fm_block_self_attention(
            torch.zeros((1, 16, 3, 2, 64), **bf), torch.ones(64), torch.ones(64), torch.ones(1, **i32), 0.125, 1e6,
            1e-6),
        "fm_write_context_kv": lambda: B.fm_write_context_kv(
            torch.zeros((2, 64), **bf), torch.zeros((256, 64), **bf), torch.ones((1, 64)), torch.zeros(2, **i32),
            torch.zeros(2, **i32), torch.zeros((1, 4), **i32), [pool], 1e-6, 1e6),
        "fm_context_rows": lambda: B.fm_context_rows(
            torch.zeros((2, 64), **bf), torch.zeros((256, 64), **bf), torch.ones(256), None, None, None, None, None,
            1e-6),
    }
    for name, call in calls.items():
        with pytest.raises(ValueError, match="must be a GPU tensor"):
            call()
    with pytest.raises(ValueError, match="pool k must be a GPU tensor"):
        pool.descriptor()


def test_probe_library_exports_and_validation():
    """The benchmark's probe library exports what include/fm_probe.h declares
    and refuses bad arguments before launching anything."""
    from block_diffusion_drafter_all_amd.build import PROBE_LIB_PATH

    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(REPO_DIR, "include", "fm_probe.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(fm_probe_[a-z_0-9]+)\s*\(", text)))
    assert declared == ["fm_probe_stream_read", "fm_probe_tile_gather", "fm_probe_tile_gather_timed"]
    plib = ctypes.CDLL(PROBE_LIB_PATH)
    for name in declared:
        assert hasattr(plib, name), name
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    plib.fm_probe_stream_read.argtypes = [vp, sz, ctypes.c_int32, vp, ctypes.POINTER(sz), vp]
    plib.fm_probe_tile_gather.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp]
    n = ctypes.c_size_t(0)
    assert plib.fm_probe_stream_read(FAKE, 1 << 20, 6, FAKE, ctypes.byref(n), None) == -1      # waves not 4k
    assert plib.fm_probe_stream_read(FAKE, 4096, 4, FAKE, ctypes.byref(n), None) == -1         # under one block each
    assert plib.fm_probe_stream_read(None, 1 << 30, 4, FAKE, ctypes.byref(n), None) == -1
    assert plib.fm_probe_tile_gather(FAKE, FAKE, FAKE, 10, 3000, 8, FAKE, None) == -2          # tile not k KB
    assert plib.fm_probe_tile_gather(FAKE, FAKE, FAKE, 0, 4096, 8, FAKE, None) == -1           # no tiles
    assert plib.fm_probe_tile_gather(FAKE, FAKE + 8, FAKE, 10, 4096, 8, FAKE, None) == -1      # misaligned
    plib.fm_probe_tile_gather_timed.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp,
                                                vp]
    assert plib.fm_probe_tile_gather_timed(FAKE, FAKE, FAKE, 10, 4096, 8, FAKE, None, None) == -1  # no records
    assert plib.fm_probe_tile_gather_timed(FAKE, FAKE, FAKE, 10, 3000, 8, FAKE, FAKE, None) == -2
