"""Plain, slow CPU oracle of the FlashMap draft-step attention path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import or call this module.  The HIP path
never routes through it, and it shares no code, table or helper with the HIP
path: every formula below is written out again from the pages that define the
method.

Sources (the flashmap 0.1.0 wheel pages and the TokenSpeed DFlash page):
  * modeling_flashmap.py: ``rope_tables`` / ``apply_rope`` (interleaved-pair
    RoPE in float32), ``FlashMapRMSNorm``, ``FlashMapAttention.project_kv`` /
    ``forward`` (scaled dot-product attention, default scale), ``FlashMapCache``
    (dense per-layer context; the anchor's entry at position ``length``),
    ``draft`` (context ``0..anchor``, slots at ``anchor+1..anchor+K``).
  * sglang/model.py: ``rope_freqs``, ``_paged_cross_attention`` (page table,
    ``cache_seqlens``), ``write_target_hidden_kv`` / ``_kv_write`` (one GEMM over
    all layers' context K/V weights, k-norm, RoPE, write that skips the
    uncommitted verify columns), ``load_weights`` (the all-layer weight is the
    concatenation ``[k_0; v_0; k_1; v_1; ...]``), ``forward`` (the anchor is
    written at its own position; ``cache_seqlens = seq_lens + 1``),
    ``_paged_cross_attention_fp8`` and ``kv_norm_rope_write_fp8`` (the fp8 KV
    pool).
  * vllm/model.py: ``paged_cross_attention`` (cu_seqlens_q, seqused_k,
    block_table, softmax_scale = head_dim ** -0.5, non-causal), ``_prologue``
    (``seqused_k`` is 0 for empty rows), ``cache_layout`` (page, head, slot
    strides), ``_dit`` (slot positions = positions + 1).

Precision: every value is carried in float64, with two exceptions the pages
fix.  (1) The rotary angle is a float32 product of a float32 position and a
float32 inverse frequency (``rope_tables``: ``positions.float() * inv_freq``).
The inverse frequency itself is read as the float32 value nearest to
``theta ** (-2i / head_dim)``.  (2) A value stored into the KV pool takes the
pool's storage type (bf16, fp32 or e4m3 at scale 1), because the pool is the
interface between the write and the attention.  (3) Over an e4m3 pool the
query is itself cast to e4m3 under a per-(request, head) scale
(``_paged_cross_attention_fp8``).  Everything else, the GEMM, the norms, the
rotation, the softmax and the weighted sums, is exact up to float64 rounding.

Readings of points the pages leave open are listed in the design notes of the
repository; the ones that change arithmetic are repeated at the function that
takes them.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "rope_inv_freq",
    "rope_angles",
    "apply_rope",
    "rms_norm",
    "round_to_bfloat16",
    "round_to_e4m3",
    "round_to_storage",
    "quantize_query_e4m3",
    "attention",
    "context_slot",
    "live_rows",
    "project_context_rows",
    "context_input_rows",
    "anchor_input_rows",
    "write_context_kv",
    "scatter_into_pool",
    "paged_cross_attention",
    "block_self_attention",
    "layer_norm",
    "gelu",
    "ada_layer_norm",
    "dit_layer",
]


# --------------------------------------------------------------------- RoPE


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Inverse frequencies ``theta ** (-2i / head_dim)`` for ``i < head_dim / 2``.

    ``rope_tables`` computes ``1 / theta ** (arange(0, head_dim, 2) / head_dim)``
    in float32.  The reading taken here: the float32 value nearest to the exact
    power (computed in float64, rounded once), so any implementation can
    reproduce the same bits."""
    if head_dim % 2:
        raise ValueError("RoPE needs an even head_dim")
    # Python's float power is the C library's double pow, evaluated per element.
    exact = [float(theta) ** (-(2.0 * i) / head_dim) for i in range(head_dim // 2)]
    return np.array(exact, dtype=np.float64).astype(np.float32)


def rope_angles(positions, inv_freq: np.ndarray) -> np.ndarray:
    """float32 angles ``float32(position) * inv_freq`` (one float32 multiply),
    shape ``positions.shape + (head_dim / 2,)``, as ``rope_tables`` forms them."""
    pos = np.asarray(positions).astype(np.float32)
    return pos[..., None] * inv_freq.astype(np.float32)


def apply_rope(x: np.ndarray, positions, theta: float) -> np.ndarray:
    """Rotate the interleaved channel pairs ``(x[2i], x[2i+1])`` of ``x (..., D)``
    by the angles of ``positions`` (shape ``x.shape[:-1]``), ``apply_rope``:
    ``(x1 cos - x2 sin, x2 cos + x1 sin)``.  cos/sin are taken in float64 of the
    float32 angle."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = rope_angles(positions, rope_inv_freq(d, theta)).astype(np.float64)
    c, s = np.cos(ang), np.sin(ang)
    x1 = x[..., 0::2]
    x2 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * c - x2 * s
    out[..., 1::2] = x2 * c + x1 * s
    return out


# ------------------------------------------------------------------ RMSNorm


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """``x * weight / sqrt(mean(x^2) + eps)`` over the last axis
    (``FlashMapRMSNorm``; the scale is kept exact rather than rounded to the
    input's dtype, the plain definition of the norm)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * np.asarray(weight, dtype=np.float64) / np.sqrt(ms + float(eps))


# ------------------------------------------------------------ storage types


def round_to_bfloat16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits, nearest, ties to
    even), returned as float64.  Zeros stay zero; inputs are finite."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def round_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the OCP float8 e4m3 ("e4m3fn") grid, returned as
    float64: 3 mantissa bits, exponent bias 7, subnormals down to 2**-9, largest
    finite 448.  Nearest, ties to even; magnitudes past 448 saturate to 448 (the
    format has no infinity, and a pool entry must stay finite)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                       # a in [2**(e-1), 2**e)
    # spacing of the grid at a: 2**(e-1-3) for normals (e-1 >= -6), 2**-9 below
    step = np.where(e - 1 >= -6, np.ldexp(1.0, e - 4), 2.0 ** -9)
    r = np.minimum(np.rint(a / step) * step, 448.0)
    return np.copysign(r, x)


def quantize_query_e4m3(q_hat: np.ndarray, static_scale=None):
    """The fp8 pool's query: one scale per (request, head), the largest
    magnitude over the request's rows and the head's channels divided by 448
    (at least 1e-12 / 448), and the e4m3 query ``q_hat / scale`` (the sglang
    model's ``_paged_cross_attention_fp8``: ``q_scale = amax / 448``,
    ``query8 = query / q_scale``).  ``q_hat (rows, D)`` of one (request, head);
    returns ``(q8, scale)`` with ``q8 * scale`` the query the attention uses.
    ``static_scale``: a fixed per-tensor scale instead (the vLLM model's
    ``q_scale``: ``query / q_scale`` cast to e4m3, saturating here)."""
    q_hat = np.asarray(q_hat, dtype=np.float64)
    if static_scale is not None:
        scale = float(static_scale)
        return round_to_e4m3(q_hat / scale), scale
    scale = max(float(np.max(np.abs(q_hat), initial=0.0)), 1e-12) / 448.0
    return round_to_e4m3(q_hat / scale), scale


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """The value a pool of storage type ``dtype`` ("bf16", "f32" or "e4m3")
    holds (an e4m3 pool is written with scale 1)."""
    if dtype == "bf16":
        return round_to_bfloat16(x)
    if dtype == "e4m3":
        return round_to_e4m3(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown storage type {dtype!r}")


# ---------------------------------------------------------------- attention


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Non-causal softmax attention ``softmax(scale * q k^T) v`` for
    ``q (n, D)``, ``k, v (T, D)`` (``FlashMapAttention.forward``).  An empty
    context (``T == 0``) gives zeros (``_prologue``: no keys to read)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    s = float(scale) * (q @ k.T)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v) / p.sum(axis=1, keepdims=True)


# ------------------------------------------------------------------- paging


def context_slot(page_table_row: np.ndarray, pos: int, page_size: int) -> int:
    """Pool slot of logical position ``pos``: entry ``pos // page_size`` of the
    request's page table names the page, ``pos % page_size`` the slot in it
    (vLLM ``block_table`` semantics; a page of size 1 is sglang's
    ``req_to_token``)."""
    page = int(page_table_row[pos // page_size])
    return page * page_size + pos % page_size


def live_rows(n_rows: int, row_pos, commit_lens=None, window: int = 0) -> np.ndarray:
    """Which rows the write stores.  A row with a negative position is skipped.
    With ``commit_lens``, the first ``len(commit_lens) * window`` rows are verify
    windows, request-major: column ``j`` of request ``b``'s window is written
    only if ``j < commit_lens[b]`` (``write_target_hidden_kv``: only the
    committed columns are written).  Later rows (the anchors) are written."""
    row_pos = np.asarray(row_pos)
    live = row_pos >= 0
    if commit_lens is not None:
        commit_lens = np.asarray(commit_lens)
        for r in range(min(n_rows, len(commit_lens) * window)):
            b, j = divmod(r, window)
            if j >= commit_lens[b]:
                live[r] = False
    return live


def project_context_rows(x: np.ndarray, w_kv: np.ndarray, L: int, H: int, D: int) -> np.ndarray:
    """One GEMM over every layer's context K/V weight: ``x (n, d_in) @ w_kv^T``
    with ``w_kv`` rows ordered (layer, {k, v}, head, dim), viewed as
    ``(n, L, 2, H, D)`` (``load_weights`` concatenation; vLLM ``_write`` view)."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w_kv, dtype=np.float64).T
    return y.reshape(y.shape[0], L, 2, H, D)


def context_input_rows(target_hidden, w_fc, hidden_norm_w, eps):
    """The rows the context K/V GEMM takes for committed target positions:
    the concatenated hidden states of the target's chosen layers projected by
    ``fc`` (no bias) and RMS-normed with ``hidden_norm`` (the sglang model's
    ``_write_context``: ``rms_norm(fc(target_hidden), hidden_norm)``; vLLM
    ``combine_hidden_states`` then ``hidden_norm``).  ``target_hidden (n,
    n_aux * d_target)``, ``w_fc (dim, n_aux * d_target)``; returns ``(n, dim)``."""
    y = np.asarray(target_hidden, dtype=np.float64) @ np.asarray(w_fc, dtype=np.float64).T
    return rms_norm(y, hidden_norm_w, eps)


def anchor_input_rows(anchor_ids, embedding, w_anchor_proj, b_anchor_proj, anchor_norm_w, eps):
    """The rows the context K/V GEMM takes for anchors: the anchor token's
    embedding through ``anchor_proj`` (with bias) and ``anchor_norm`` (the
    sglang model's ``_anchor_kv_impl``; vLLM ``_prologue``).  ``embedding
    (vocab, d_target)``, ``w_anchor_proj (dim, d_target)``, ``b_anchor_proj
    (dim)``; returns ``(n, dim)``."""
    e = np.asarray(embedding, dtype=np.float64)[np.asarray(anchor_ids, dtype=np.int64)]
    y = e @ np.asarray(w_anchor_proj, dtype=np.float64).T + np.asarray(b_anchor_proj, dtype=np.float64)
    return rms_norm(y, anchor_norm_w, eps)


def write_context_kv(x, w_kv, k_norm_w, row_req, row_pos, page_table, page_size,
                     L, H, D, eps, theta, commit_lens=None, window=0):
    """The context/anchor K/V write of every layer.

    For each live row: ``y = W_kv x``; per layer ``l`` and head ``h``, the key
    is RMS-normed with ``k_norm_w[l]`` and rotated at the row's position, the
    value is left as projected (``project_kv``: no norm and no RoPE on v).

    Returns ``(slots, keys, values)``: ``slots (n_rows)`` int64, -1 for a
    skipped row; ``keys, values (n_rows, L, H, D)`` float64 (rows that are
    skipped hold zeros)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    row_req = np.asarray(row_req)
    row_pos = np.asarray(row_pos)
    live = live_rows(n, row_pos, commit_lens, window)
    slots = np.full(n, -1, dtype=np.int64)
    keys = np.zeros((n, L, H, D))
    values = np.zeros((n, L, H, D))
    idx = np.nonzero(live)[0]
    if idx.size == 0:
        return slots, keys, values
    y = project_context_rows(x[idx], w_kv, L, H, D)
    k_norm_w = np.asarray(k_norm_w, dtype=np.float64).reshape(L, D)
    for n_i, r in enumerate(idx):
        pos = int(row_pos[r])
        slots[r] = context_slot(page_table[int(row_req[r])], pos, page_size)
        for l in range(L):
            k = rms_norm(y[n_i, l, 0], k_norm_w[l], eps)          # (H, D)
            keys[r, l] = apply_rope(k, np.full(H, pos), theta)
            values[r, l] = y[n_i, l, 1]
    return slots, keys, values


def scatter_into_pool(pools_k, pools_v, slots, keys, values, page_size, dtype, kv_scales=None):
    """Store each written row into every layer's pool at its slot, rounded to
    the pool's storage type.  ``pools_k[l], pools_v[l]`` are logical float64
    arrays ``(pages, page_size, H, D)`` updated in place.  Live rows must name
    distinct slots (a precondition: the pages never write one slot twice in a
    call).  ``kv_scales (L, 2)``: an e4m3 pool's per-layer key and value
    scales; the pool holds ``k / k_scale`` and ``v / v_scale`` (vllm/model.py
    ``write_context_kv`` with ``kv_scales``; 1 when not given, as in sglang)."""
    live = np.nonzero(np.asarray(slots) >= 0)[0]
    taken = set()
    for r in live:
        s = int(slots[r])
        if s in taken:
            raise ValueError(f"slot {s} written twice")
        taken.add(s)
        page, off = divmod(s, page_size)
        for l in range(len(pools_k)):
            ks, vs = (1.0, 1.0) if kv_scales is None else (float(kv_scales[l][0]), float(kv_scales[l][1]))
            pools_k[l][page, off] = round_to_storage(keys[r, l] / ks, dtype)
            pools_v[l][page, off] = round_to_storage(values[r, l] / vs, dtype)


def paged_cross_attention(q, q_norm_w, pool_k, pool_v, page_table, ctx_lens,
                          cu_seqlens_q, page_size, scale, theta, eps,
                          requests=None, heads=None, block_size=16, kv_e4m3=False, q_scale=None,
                          k_scale=1.0, v_scale=1.0):
    """Cross-attention of each request's draft rows onto its paged context.

    Row ``r`` of request ``b`` (``cu_seqlens_q[b] <= r < cu_seqlens_q[b+1]``)
    is query slot ``k = (r - cu_seqlens_q[b]) mod block_size`` of candidate
    block ``(r - cu_seqlens_q[b]) // block_size``, at position
    ``ctx_lens[b] + k`` (slots sit at ``anchor + 1 + k`` and
    ``ctx_len = anchor + 1``; tree drafting puts a request's candidate blocks
    side by side, candidate-major, so that its context is read once: the
    sglang model's ``forward`` in the flashmap 0.1.0 wheel).  Its query is
    RMS-normed with ``q_norm_w`` and rotated there (``rms_norm_rope``), then
    attends, non-causally, to the keys/values at logical positions
    ``0 .. ctx_lens[b] - 1`` read through the page table.

    ``kv_e4m3``: the pool holds e4m3 codes and the query is quantized to
    e4m3 first (``quantize_query_e4m3``): per (request, head) with amax / 448
    (sglang), or with the fixed ``q_scale`` when given (vLLM).  The keys and
    values the attention sees are ``k_scale`` and ``v_scale`` times the codes
    (the descales; 1 in sglang), the query the descaled one.

    ``pool_k, pool_v``: logical ``(pages, page_size, H, D)`` arrays.  Returns
    float64 ``(total_q, H, D)``; rows of requests not in ``requests`` and heads
    not in ``heads`` (when given) are left as NaN."""
    q = np.asarray(q, dtype=np.float64)
    total_q, H, D = q.shape
    bs = len(ctx_lens)
    out = np.full((total_q, H, D), np.nan)
    reqs = range(bs) if requests is None else requests
    hs = list(range(H)) if heads is None else list(heads)
    for b in reqs:
        r0, r1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        if r1 == r0:
            continue
        ctx = int(ctx_lens[b])
        positions = ctx + np.arange(r1 - r0) % block_size
        # Dense context of request b, in logical order.
        n_pages = -(-ctx // page_size)
        pages = np.asarray(page_table[b][:n_pages], dtype=np.int64)
        k_b = pool_k[pages].reshape(-1, H, D)[:ctx]
        v_b = pool_v[pages].reshape(-1, H, D)[:ctx]
        for h in hs:
            qh = rms_norm(q[r0:r1, h], q_norm_w, eps)
            qh = apply_rope(qh, positions, theta)
            kh, vh = k_b[:, h], v_b[:, h]
            if kv_e4m3:
                q8, qs = quantize_query_e4m3(qh, q_scale)
                qh = q8 * qs
                kh, vh = kh * float(k_scale), vh * float(v_scale)
            out[r0:r1, h] = attention(qh, kh, vh, scale)
    return out


def block_self_attention(qkv, q_norm_w, k_norm_w, ctx_lens, scale, theta, eps):
    """Bidirectional attention within each draft block.

    ``qkv (n_blocks, K, 3, H, D)``: slot ``i`` of block ``b`` sits at position
    ``ctx_lens[b] + i``; its query and key are RMS-normed (``q_norm_w``,
    ``k_norm_w``) and rotated there, its value is used as given; every slot
    attends to all ``K`` slots of its own block (no mask).  Returns float64
    ``(n_blocks, K, H, D)``."""
    qkv = np.asarray(qkv, dtype=np.float64)
    n_blocks, K, _, H, D = qkv.shape
    out = np.zeros((n_blocks, K, H, D))
    for b in range(n_blocks):
        positions = int(ctx_lens[b]) + np.arange(K)
        for h in range(H):
            qh = apply_rope(rms_norm(qkv[b, :, 0, h], q_norm_w, eps), positions, theta)
            kh = apply_rope(rms_norm(qkv[b, :, 1, h], k_norm_w, eps), positions, theta)
            out[b, :, h] = attention(qh, kh, qkv[b, :, 2, h], scale)
    return out


# ---------------------------------------------------------- the DiT layer --


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm over the last axis without affine parameters
    (``F.layer_norm(x, (dim,), eps=eps)``)."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + float(eps))


def gelu(x: np.ndarray) -> np.ndarray:
    """GELU with the exact normal CDF (``F.gelu``'s default): x * Phi(x)."""
    from scipy.special import erf

    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def ada_layer_norm(h, scale, shift, eps):
    """A time-modulated LayerNorm: ``layer_norm(h) * scale + shift`` with the
    step's per-channel ``scale`` (already ``1 + scale``) and ``shift`` (the
    sglang model's ``_denoise``; modeling_flashmap.py ``FlashMapAdaLayerNorm``)."""
    return layer_norm(h, eps) * np.asarray(scale, dtype=np.float64) + np.asarray(shift, dtype=np.float64)


def dit_layer(h, mod, w, self_attention, cross_attention, eps):
    """One DiT block of the draft step (the sglang model's ``_denoise`` loop
    body; modeling_flashmap.py ``FlashMapLayer.forward``), on rows ``h (M,
    dim)``:

      h += s_gate * o_self(self_attention(qkv(ada_ln(h; s_scale, s_shift))))
      h += c_gate * o_cross(cross_attention(q(ada_ln(h; c_scale, c_shift))))
      h += m_gate * fc2(gelu(fc1(ada_ln(h; m_scale, m_shift)) + b1)) + b2)

    ``mod``: the step's per-layer vectors ``s_scale, s_shift, s_gate, c_scale,
    c_shift, c_gate, m_scale, m_shift, m_gate`` (dim,), scales already ``1 +
    scale``.  ``w``: ``qkv (3 dim, dim)`` (q, k, v heads), ``o_self``,
    ``q``, ``o_cross`` (dim, dim), ``fc1 (I, dim)``, ``b1 (I)``, ``fc2 (dim,
    I)``, ``b2 (dim)``; no bias elsewhere.  ``self_attention(qkv)`` maps the
    (M, 3 dim) projections to (M, dim) (norms and RoPE inside);
    ``cross_attention(q)`` maps the raw (M, dim) queries to (M, dim)."""
    f = lambda k: np.asarray(mod[k], dtype=np.float64)  # noqa: E731
    W = lambda k: np.asarray(w[k], dtype=np.float64)    # noqa: E731
    h = np.asarray(h, dtype=np.float64).copy()
    x = ada_layer_norm(h, f("s_scale"), f("s_shift"), eps)
    h = h + f("s_gate") * (self_attention(x @ W("qkv").T) @ W("o_self").T)
    x = ada_layer_norm(h, f("c_scale"), f("c_shift"), eps)
    h = h + f("c_gate") * (cross_attention(x @ W("q").T) @ W("o_cross").T)
    x = ada_layer_norm(h, f("m_scale"), f("m_shift"), eps)
    y = gelu(x @ W("fc1").T + W("b1")) @ W("fc2").T + W("b2")
    return h + f("m_gate") * y
