"""ctypes binding of libfm (include/fm.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, passes their
device pointers, shapes and strides to the C ABI and enqueues the work on
torch's current HIP stream.  Nothing here computes any part of the draft step;
if libfm.so is missing, loading it raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from .build import LIB_PATH

FM_OK = 0
FM_E_INVALID = -1
FM_E_UNSUPPORTED = -2
FM_E_WORKSPACE = -3
FM_E_HIP = -4
FM_F32 = 0
FM_BF16 = 1
FM_BF16_E4M3 = 2
FM_LINEAR_BF16 = 0
FM_LINEAR_GELU_BF16 = 1
FM_LINEAR_RESIDUAL = 2
FM_LINEAR_ASSIGN_F32 = 3

SYMBOLS = (
    "fm_last_error",
    "fm_version",
    "fm_write_context_kv_workspace_size",
    "fm_write_context_kv",
    "fm_write_context_kv_noalloc",
    "fm_context_rows_workspace_size",
    "fm_context_rows",
    "fm_ada_layer_norm",
    "fm_linear_workspace_size",
    "fm_linear",
    "fm_cross_attention_workspace_size",
    "fm_plan_cross_attention",
    "fm_plan_cross_attention_weighted",
    "fm_paged_cross_attention",
    "fm_paged_cross_attention_timed",
    "fm_block_self_attention",
)


class FmError(RuntimeError):
    """A negative fm_status, with fm_last_error()'s message."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[fm status {status}] {message}")
        self.status = status


class fm_kv_pool(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64),
        ("page_stride", ctypes.c_int64),
        ("slot_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64),
    ]


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libfm.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with block_diffusion_drafter_all_amd.build.build()")
    lib = ctypes.CDLL(p)
    c_i32, c_i64, c_sz, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    f32 = ctypes.c_float
    lib.fm_last_error.restype = ctypes.c_char_p
    lib.fm_version.restype = ctypes.c_char_p
    lib.fm_write_context_kv_workspace_size.restype = c_sz
    lib.fm_write_context_kv_workspace_size.argtypes = [c_i64]
    lib.fm_write_context_kv.restype = ctypes.c_int
    lib.fm_write_context_kv.argtypes = [
        vp, c_i64, c_i32, ctypes.c_int, vp, vp, vp, vp, vp, c_i32, vp, c_i64, c_i32, c_i32,
        ctypes.POINTER(fm_kv_pool), c_i32, c_i32, c_i32, f32, f32, ctypes.POINTER(f32), vp, vp, c_sz, vp,
    ]
    lib.fm_write_context_kv_noalloc.restype = ctypes.c_int
    lib.fm_write_context_kv_noalloc.argtypes = [
        vp, c_i64, c_i32, ctypes.c_int, vp, vp, vp, vp, vp, c_i32, vp, c_i64, c_i32, c_i32,
        ctypes.POINTER(fm_kv_pool), c_i32, c_i32, c_i32, f32, f32, ctypes.POINTER(f32), vp, vp,
    ]
    lib.fm_context_rows_workspace_size.restype = c_sz
    lib.fm_context_rows_workspace_size.argtypes = [c_i64, c_i64, c_i32, c_i32, c_i32]
    lib.fm_context_rows.restype = ctypes.c_int
    lib.fm_context_rows.argtypes = [
        vp, c_i64, c_i32, vp, vp, vp, c_i64, vp, c_i64, c_i32, vp, vp, vp, c_i32, vp, c_i32, c_i32, f32, vp, vp,
        c_sz, vp,
    ]
    lib.fm_ada_layer_norm.restype = ctypes.c_int
    lib.fm_ada_layer_norm.argtypes = [vp, c_i64, c_i32, vp, vp, f32, vp, vp]
    lib.fm_linear_workspace_size.restype = c_sz
    lib.fm_linear_workspace_size.argtypes = [c_i64, c_i32, c_i32]
    lib.fm_linear.restype = ctypes.c_int
    lib.fm_linear.argtypes = [vp, c_i64, c_i32, vp, c_i32, vp, ctypes.c_int, vp, vp, vp, c_sz, vp]
    lib.fm_cross_attention_workspace_size.restype = c_sz
    lib.fm_cross_attention_workspace_size.argtypes = [c_i32, c_i32, c_i32, c_i32, ctypes.c_int]
    lib.fm_plan_cross_attention.restype = ctypes.c_int
    lib.fm_plan_cross_attention.argtypes = [vp, c_i32, c_i32, c_i32, c_i32, ctypes.c_int, vp, c_sz, vp]
    lib.fm_plan_cross_attention_weighted.restype = ctypes.c_int
    lib.fm_plan_cross_attention_weighted.argtypes = [vp, c_i32, c_i32, c_i32, c_i32, ctypes.c_int,
                                                     ctypes.POINTER(c_i32), vp, c_sz, vp]
    lib.fm_paged_cross_attention.restype = ctypes.c_int
    lib.fm_paged_cross_attention.argtypes = [
        vp, ctypes.c_int, c_i64, vp, ctypes.POINTER(fm_kv_pool), vp, c_i64, c_i32, vp, vp, c_i32, c_i32, c_i32,
        c_i32, f32, f32, f32, ctypes.POINTER(f32), vp, vp, c_sz, vp,
    ]
    lib.fm_paged_cross_attention_timed.restype = ctypes.c_int
    lib.fm_paged_cross_attention_timed.argtypes = [
        vp, ctypes.c_int, c_i64, vp, ctypes.POINTER(fm_kv_pool), vp, c_i64, c_i32, vp, vp, c_i32, c_i32, c_i32,
        c_i32, f32, f32, f32, ctypes.POINTER(f32), vp, vp, c_sz, vp, c_i64, vp,
    ]
    lib.fm_block_self_attention.restype = ctypes.c_int
    lib.fm_block_self_attention.argtypes = [
        vp, ctypes.c_int, c_i32, c_i32, vp, vp, vp, c_i32, c_i32, f32, f32, f32, vp, vp,
    ]
    if path is None:
        _lib = lib
    return lib


def fm_last_error() -> str:
    return load_library().fm_last_error().decode()


def fm_version() -> str:
    return load_library().fm_version().decode()


def _check(status: int) -> None:
    if status != FM_OK:
        raise FmError(status, fm_last_error())


def _dtype_code(t: torch.Tensor, pool_dtype=None) -> int:
    """fm_dtype of activations ``t`` over a pool of ``pool_dtype`` (None: no pool)."""
    if pool_dtype == torch.float8_e4m3fn:
        if t.dtype != torch.bfloat16:
            raise TypeError(f"an e4m3 pool takes bfloat16 activations, got {t.dtype}")
        return FM_BF16_E4M3
    if pool_dtype is not None and pool_dtype != t.dtype:
        raise TypeError(f"pool dtype {pool_dtype} does not go with activations of {t.dtype}")
    if t.dtype == torch.bfloat16:
        return FM_BF16
    if t.dtype == torch.float32:
        return FM_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None, contiguous=True, shape=None) -> None:
    """The C ABI takes bare pointers, so every extent it will touch is checked here."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}; the kernels run on the current device "
                         f"(cuda:{torch.cuda.current_device()})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


@dataclass
class KVPool:
    """One layer's paged pool: ``k`` and ``v`` viewed as ``(pages, page_size,
    H, Dh)`` with any strides (head_dim contiguous), e.g. a head-major
    ``(pages, H, page_size, Dh)`` tensor permuted to that view."""

    k: torch.Tensor
    v: torch.Tensor

    def descriptor(self) -> fm_kv_pool:
        k, v = self.k, self.v
        _need(k, "pool k", contiguous=False)
        _need(v, "pool v", contiguous=False)
        if k.dim() != 4 or v.shape != k.shape or v.stride() != k.stride() or v.dtype != k.dtype:
            raise ValueError("k and v must be (pages, page_size, H, Dh) views of one shape, stride and dtype")
        if k.stride(3) != 1:
            raise ValueError("head_dim must be contiguous")
        return fm_kv_pool(k.data_ptr(), v.data_ptr(), k.shape[0], k.stride(0), k.stride(1), k.stride(2))

    @property
    def page_size(self) -> int:
        return self.k.shape[1]


def fm_write_context_kv_workspace_size(n_rows: int) -> int:
    return load_library().fm_write_context_kv_workspace_size(n_rows)


def _floats(values):
    """A host float array for the C ABI, or None."""
    if values is None:
        return None
    flat = [float(v) for row in values for v in (row if hasattr(row, "__len__") else [row])]
    return (ctypes.c_float * len(flat))(*flat)


FM_WRITE_NOALLOC_MAX_ROWS = 65536


def _write_args(x, w_kv, k_norm_w, row_req, row_pos, page_table, pools, eps, rope_theta, commit_lens, window,
                out_slots, kv_scales):
    """Checked C-ABI arguments of the write, up to out_slots."""
    _need(x, "x")
    _need(w_kv, "w_kv", x.dtype)
    _need(k_norm_w, "k_norm_w", torch.float32)
    for name, t in (("row_req", row_req), ("row_pos", row_pos), ("page_table", page_table)):
        _need(t, name, torch.int32)
    if commit_lens is not None:
        _need(commit_lens, "commit_lens", torch.int32)
    if out_slots is not None:
        _need(out_slots, "out_slots", torch.int32)
    L = len(pools)
    H, Dh = pools[0].k.shape[2], pools[0].k.shape[3]
    if row_req.shape[0] != x.shape[0] or row_pos.shape[0] != x.shape[0]:
        raise ValueError("row_req and row_pos need one entry per row of x")
    if commit_lens is not None and commit_lens.shape[0] != page_table.shape[0]:
        raise ValueError("commit_lens needs one entry per request (page-table row)")
    if k_norm_w.shape != (L, Dh) or w_kv.shape != (L * 2 * H * Dh, x.shape[1]):
        raise ValueError("k_norm_w must be (L, Dh) and w_kv (L*2*H*Dh, d_in)")
    if out_slots is not None and out_slots.shape[0] != x.shape[0]:
        raise ValueError("out_slots needs one entry per row of x")
    descs = (fm_kv_pool * L)(*[p.descriptor() for p in pools])
    if any(p.k.dtype != pools[0].k.dtype for p in pools):
        raise TypeError("every layer's pool must have one dtype")
    if kv_scales is not None and len(kv_scales) != L:
        raise ValueError("kv_scales needs one (k_scale, v_scale) pair per layer")
    code = _dtype_code(x, pools[0].k.dtype)
    n_rows, d_in = x.shape
    return (_ptr(x), n_rows, d_in, code, _ptr(w_kv), _ptr(k_norm_w), _ptr(row_req), _ptr(row_pos),
            _ptr(commit_lens), window, _ptr(page_table), page_table.stride(0), pools[0].page_size,
            page_table.shape[0], descs, L, H, Dh, eps, rope_theta, _floats(kv_scales), _ptr(out_slots))


def fm_write_context_kv(x, w_kv, k_norm_w, row_req, row_pos, page_table, pools, eps, rope_theta,
                        commit_lens=None, window=0, out_slots=None, ws=None, kv_scales=None):
    """Project, k-norm, rotate and scatter every layer's context K/V rows into
    ``pools`` (a list of KVPool, one per layer).  Returns ``out_slots`` if given.
    ``kv_scales``: e4m3 pools only, one (k_scale, v_scale) per layer (the pool
    receives k / k_scale and v / v_scale); None = 1."""
    lib = load_library()
    args = _write_args(x, w_kv, k_norm_w, row_req, row_pos, page_table, pools, eps, rope_theta, commit_lens,
                       window, out_slots, kv_scales)
    if ws is not None:
        _need(ws, "ws", torch.uint8)
    if ws is None:
        ws = torch.empty(lib.fm_write_context_kv_workspace_size(x.shape[0]), dtype=torch.uint8, device=x.device)
    _check(lib.fm_write_context_kv(*args, _ptr(ws), ws.numel(), _stream()))
    return out_slots


def fm_write_context_kv_noalloc(x, w_kv, k_norm_w, row_req, row_pos, page_table, pools, eps, rope_theta,
                                commit_lens=None, window=0, out_slots=None, kv_scales=None):
    """fm_write_context_kv with the library's static per-GPU workspace (at most
    FM_WRITE_NOALLOC_MAX_ROWS rows; calls on one GPU must not overlap)."""
    lib = load_library()
    args = _write_args(x, w_kv, k_norm_w, row_req, row_pos, page_table, pools, eps, rope_theta, commit_lens,
                       window, out_slots, kv_scales)
    _check(lib.fm_write_context_kv_noalloc(*args, _stream()))
    return out_slots


def _pool_code(pool_dtype) -> int:
    """fm_dtype of the calls over a pool of ``pool_dtype``."""
    codes = {torch.float32: FM_F32, torch.bfloat16: FM_BF16, torch.float8_e4m3fn: FM_BF16_E4M3}
    if pool_dtype not in codes:
        raise TypeError(f"unsupported pool dtype {pool_dtype}")
    return codes[pool_dtype]


def fm_context_rows_workspace_size(n_hidden: int, n_anchor: int, d_hidden: int, d_target: int, dim: int) -> int:
    return load_library().fm_context_rows_workspace_size(n_hidden, n_anchor, d_hidden, d_target, dim)


def fm_context_rows(hidden, w_fc, hidden_norm_w, anchor_ids, embedding, w_anchor_proj, b_anchor_proj, anchor_norm_w,
                    eps, commit_lens=None, window=0, bs=None, rows=None, ws=None):
    """The rows fm_write_context_kv projects: ``hidden_norm(fc(hidden))`` for
    the committed hidden rows, then ``anchor_norm(anchor_proj(embedding[id]))``
    for the anchors.  ``hidden`` or ``anchor_ids`` may be None.  Returns
    ``rows (n_hidden + n_anchor, dim)`` bf16."""
    lib = load_library()
    n_hidden = 0 if hidden is None else hidden.shape[0]
    n_anchor = 0 if anchor_ids is None else anchor_ids.shape[0]
    dim = (w_fc if hidden is not None else w_anchor_proj).shape[0]
    d_hidden = 0 if hidden is None else hidden.shape[1]
    d_target = 0 if anchor_ids is None else embedding.shape[1]
    if hidden is not None:
        _need(hidden, "hidden", torch.bfloat16)
        _need(w_fc, "w_fc", torch.bfloat16)
        _need(hidden_norm_w, "hidden_norm_w", torch.float32)
        if w_fc.shape != (dim, d_hidden) or hidden_norm_w.shape != (dim,):
            raise ValueError("w_fc must be (dim, d_hidden) and hidden_norm_w (dim,)")
    if anchor_ids is not None:
        _need(anchor_ids, "anchor_ids", torch.int32)
        for name, t in (("embedding", embedding), ("w_anchor_proj", w_anchor_proj), ("b_anchor_proj", b_anchor_proj)):
            _need(t, name, torch.bfloat16)
        _need(anchor_norm_w, "anchor_norm_w", torch.float32)
        if w_anchor_proj.shape != (dim, d_target) or b_anchor_proj.shape != (dim,) or anchor_norm_w.shape != (dim,):
            raise ValueError("w_anchor_proj must be (dim, d_target), b_anchor_proj and anchor_norm_w (dim,)")
    if commit_lens is not None:
        _need(commit_lens, "commit_lens", torch.int32)
        bs = commit_lens.shape[0] if bs is None else bs
        if commit_lens.shape[0] < bs:
            raise ValueError("commit_lens needs an entry for each of the bs requests")
    if ws is not None:
        _need(ws, "ws", torch.uint8)
    dev = (hidden if hidden is not None else anchor_ids).device
    if rows is None:
        rows = torch.empty((n_hidden + n_anchor, dim), dtype=torch.bfloat16, device=dev)
    _need(rows, "rows", torch.bfloat16)
    if rows.shape != (n_hidden + n_anchor, dim):
        raise ValueError("rows must be (n_hidden + n_anchor, dim)")
    if ws is None:
        ws = torch.empty(lib.fm_context_rows_workspace_size(n_hidden, n_anchor, d_hidden, d_target, dim),
                         dtype=torch.uint8, device=dev)
    _check(lib.fm_context_rows(
        _ptr(hidden), n_hidden, d_hidden, _ptr(w_fc), _ptr(hidden_norm_w), _ptr(anchor_ids), n_anchor,
        _ptr(embedding), 0 if embedding is None else embedding.shape[0], d_target, _ptr(w_anchor_proj),
        _ptr(b_anchor_proj), _ptr(anchor_norm_w), dim, _ptr(commit_lens), window, 0 if bs is None else bs, eps,
        _ptr(rows), _ptr(ws), ws.numel(), _stream()))
    return rows


def fm_ada_layer_norm(h, scale, shift, eps, out=None):
    """``LayerNorm(h) * scale + shift`` of the fp32 residual stream ``h (rows,
    dim)`` into bf16 ``out``."""
    _need(h, "h", torch.float32)
    rows, dim = h.shape
    _need(scale, "scale", torch.float32, shape=(dim,))
    _need(shift, "shift", torch.float32, shape=(dim,))
    if out is None:
        out = torch.empty((rows, dim), dtype=torch.bfloat16, device=h.device)
    _need(out, "out", torch.bfloat16, shape=(rows, dim))
    _check(load_library().fm_ada_layer_norm(_ptr(h), rows, dim, _ptr(scale), _ptr(shift), eps, _ptr(out), _stream()))
    return out


def fm_linear_workspace_size(M: int, N: int, K: int) -> int:
    return load_library().fm_linear_workspace_size(M, N, K)


def fm_linear(x, w, bias=None, epilogue=FM_LINEAR_BF16, gate=None, out=None, ws=None):
    """``y = x w^T + bias`` with an epilogue: bf16 out, GELU bf16 out, the
    gated residual ``out += gate * y`` into an fp32 ``out``, or fp32 ``out = y``."""
    lib = load_library()
    _need(x, "x", torch.bfloat16)
    _need(w, "w", torch.bfloat16)
    M, K = x.shape
    N = w.shape[0]
    if w.shape != (N, K):
        raise ValueError("w must be (N, K) for x (M, K)")
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, shape=(N,))
    if gate is not None:
        _need(gate, "gate", torch.float32, shape=(N,))
    f32_out = epilogue in (FM_LINEAR_RESIDUAL, FM_LINEAR_ASSIGN_F32)
    if out is None:
        if epilogue == FM_LINEAR_RESIDUAL:
            raise ValueError("the residual epilogue updates an existing out")
        out = torch.empty((M, N), dtype=torch.float32 if f32_out else torch.bfloat16, device=x.device)
    _need(out, "out", torch.float32 if f32_out else torch.bfloat16, shape=(M, N))
    if ws is not None:
        _need(ws, "ws", torch.uint8)
    need = lib.fm_linear_workspace_size(M, N, K)
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(lib.fm_linear(_ptr(x), M, K, _ptr(w), N, _ptr(bias), epilogue, _ptr(gate), _ptr(out), _ptr(ws),
                         0 if ws is None else ws.numel(), _stream()))
    return out


def fm_cross_attention_workspace_size(bs: int, H: int, Dh: int, max_q: int = 16,
                                      pool_dtype=torch.bfloat16) -> int:
    return load_library().fm_cross_attention_workspace_size(bs, H, Dh, max_q, _pool_code(pool_dtype))


XCDS = 8


def fm_plan_cross_attention(ctx_lens, H, Dh, ws, max_q=16, pool_dtype=torch.bfloat16, xcd_weights=None):
    """Build the per-step tile schedule into ``ws`` (every layer reuses it) for
    calls over pools of ``pool_dtype``; ``xcd_weights`` (8 ints in [500,
    2000]) weight the wave shares by XCD instead of the library's default."""
    if xcd_weights is not None:
        weights = [int(x) for x in xcd_weights]
        if len(weights) != XCDS:
            raise ValueError(f"xcd_weights needs {XCDS} values, got {len(weights)}")
    lib = load_library()
    _need(ctx_lens, "ctx_lens", torch.int32)
    _need(ws, "ws", torch.uint8)
    if xcd_weights is None:
        _check(lib.fm_plan_cross_attention(_ptr(ctx_lens), ctx_lens.shape[0], H, Dh, max_q, _pool_code(pool_dtype),
                                           _ptr(ws), ws.numel(), _stream()))
        return
    arr = (ctypes.c_int32 * XCDS)(*weights)
    _check(lib.fm_plan_cross_attention_weighted(_ptr(ctx_lens), ctx_lens.shape[0], H, Dh, max_q,
                                                _pool_code(pool_dtype), arr, _ptr(ws), ws.numel(), _stream()))


def fm_paged_cross_attention(q, q_norm_w, pool: KVPool, page_table, ctx_lens, cu_seqlens_q, softmax_scale,
                             rope_theta, eps, ws, out=None, max_q=16, fp8_scales=None, wave_clock=None):
    """Paged cross-attention of ``q (total_q, H, Dh)`` onto ``pool``; the plan
    in ``ws`` must come from fm_plan_cross_attention with the same lengths and
    ``max_q`` (query rows per request: 16 per draft block, up to 4 blocks).
    ``fp8_scales``: e4m3 pools only, (q_scale, k_scale, v_scale): a fixed
    query scale (0 = per request and head) and the key/value descales.
    ``wave_clock`` (int64 device tensor of shape (waves, 4)): also time every
    wave (fm_paged_cross_attention_timed)."""
    lib = load_library()
    _need(q, "q")
    _need(q_norm_w, "q_norm_w", torch.float32)
    _need(page_table, "page_table", torch.int32, contiguous=False)
    if page_table.stride(1) != 1:
        raise ValueError("page_table rows must be contiguous")
    _need(ctx_lens, "ctx_lens", torch.int32)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, shape=q.shape)
    _need(ws, "ws", torch.uint8)
    total_q, H, Dh = q.shape
    _need(q_norm_w, "q_norm_w", torch.float32, shape=(Dh,))
    if tuple(pool.k.shape[2:]) != (H, Dh):
        raise ValueError(f"the pool holds {tuple(pool.k.shape[2:])} (H, Dh) per slot, q {(H, Dh)}")
    if page_table.shape[0] < ctx_lens.shape[0] or cu_seqlens_q.shape[0] != ctx_lens.shape[0] + 1:
        raise ValueError("page_table needs a row per request and cu_seqlens_q bs + 1 entries")
    desc = pool.descriptor()
    args = (_ptr(q), _dtype_code(q, pool.k.dtype), total_q, _ptr(q_norm_w), ctypes.byref(desc), _ptr(page_table),
            page_table.stride(0), pool.page_size, _ptr(ctx_lens), _ptr(cu_seqlens_q), max_q, ctx_lens.shape[0], H, Dh,
            softmax_scale, rope_theta, eps, _floats(fp8_scales), _ptr(out), _ptr(ws), ws.numel())
    if wave_clock is None:
        _check(lib.fm_paged_cross_attention(*args, _stream()))
    else:
        _need(wave_clock, "wave_clock", torch.int64)
        if wave_clock.dim() != 2 or wave_clock.shape[1] != 4:
            raise ValueError("wave_clock needs shape (waves, 4)")
        _check(lib.fm_paged_cross_attention_timed(*args, _ptr(wave_clock), wave_clock.shape[0], _stream()))
    return out


def fm_block_self_attention(qkv, q_norm_w, k_norm_w, ctx_lens, softmax_scale, rope_theta, eps, out=None):
    """Bidirectional attention within each block of ``qkv (n_blocks, K, 3, H, Dh)``."""
    lib = load_library()
    _need(qkv, "qkv")
    _need(q_norm_w, "q_norm_w", torch.float32)
    _need(k_norm_w, "k_norm_w", torch.float32)
    _need(ctx_lens, "ctx_lens", torch.int32)
    n_blocks, K, three, H, Dh = qkv.shape
    if three != 3:
        raise ValueError("qkv must be (n_blocks, K, 3, H, Dh)")
    _need(q_norm_w, "q_norm_w", torch.float32, shape=(Dh,))
    _need(k_norm_w, "k_norm_w", torch.float32, shape=(Dh,))
    _need(ctx_lens, "ctx_lens", torch.int32, shape=(n_blocks,))
    if out is None:
        out = torch.empty((n_blocks, K, H, Dh), dtype=qkv.dtype, device=qkv.device)
    _need(out, "out", qkv.dtype, shape=(n_blocks, K, H, Dh))
    _check(lib.fm_block_self_attention(
        _ptr(qkv), _dtype_code(qkv), n_blocks, K, _ptr(q_norm_w), _ptr(k_norm_w), _ptr(ctx_lens), H, Dh,
        softmax_scale, rope_theta, eps, _ptr(out), _stream()))
    return out
