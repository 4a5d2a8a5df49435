"""One draft step's attention-path calls, in the order the method makes them.

For every DiT layer the draft step runs self-attention within the block, then
cross-attention onto the paged context (sglang/model.py ``_denoise``;
vllm/model.py ``_dit``).  Before the layers, the step writes the newly
committed context rows and the anchors into every layer's pool with one GEMM
(``write_target_hidden_kv`` / ``_prologue``) and builds the cross-attention
plan that every layer shares (``_cross_attention_schedule``).

This module only sequences calls into libfm; all arithmetic runs in its
kernels.  Buffers are allocated once, before the first step.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as B
from .workloads import Workload


@dataclass
class StepBuffers:
    cross_ws: torch.Tensor
    write_ws: torch.Tensor | None
    cross_out: list
    self_out: list
    out_slots: torch.Tensor | None
    rows_ws: torch.Tensor | None = None
    dit: dict | None = None               # the DiT blocks' activations and workspace
    xcd_weights: list | None = None       # the plan's per-XCD share weights (None: the library's default)


def allocate(w: Workload) -> StepBuffers:
    dev = w.ctx_lens.device
    cross_ws = torch.empty(B.fm_cross_attention_workspace_size(w.bs, w.H, w.Dh, w.max_q, w.pool_dtype),
                           dtype=torch.uint8, device=dev)
    write_ws = out_slots = None
    if w.write is not None:
        n_rows = w.write.x.shape[0]
        write_ws = torch.empty(B.fm_write_context_kv_workspace_size(n_rows), dtype=torch.uint8, device=dev)
        out_slots = torch.empty(n_rows, dtype=torch.int32, device=dev)
    cross_out = [torch.empty_like(q) for q in w.q]
    self_out = [torch.empty((w.bs * w.n_cand, w.K, w.H, w.Dh), dtype=w.dtype, device=dev) for _ in range(w.L)]
    rows_ws = None
    if w.upstream is not None:
        up = w.upstream
        rows_ws = torch.empty(B.fm_context_rows_workspace_size(up.hidden.shape[0], up.anchor_ids.shape[0],
                                                               up.hidden.shape[1], up.embedding.shape[1],
                                                               up.w_fc.shape[0]), dtype=torch.uint8, device=dev)
    dit = None
    if w.dit is not None:
        rows, dim = w.dit.embedded.shape[0], w.H * w.Dh
        inter = w.dit.layers[0]["fc1"].shape[0]
        f32, bf = dict(dtype=torch.float32, device=dev), dict(dtype=torch.bfloat16, device=dev)
        shapes = [(rows, 3 * dim, dim), (rows, dim, dim), (rows, inter, dim), (rows, dim, inter),
                  (rows, dim, w.dit.w_xe.shape[1])]
        dit = dict(h=torch.empty((rows, dim), **f32), xn=torch.empty((rows, dim), **bf),
                   qkv=torch.empty((rows, 3 * dim), **bf), q=torch.empty((rows, dim), **bf),
                   mlp=torch.empty((rows, inter), **bf), out=torch.empty((rows, dim), **bf),
                   ws=torch.empty(max(B.fm_linear_workspace_size(*s) for s in shapes) + 256, dtype=torch.uint8,
                                  device=dev))
    return StepBuffers(cross_ws, write_ws, cross_out, self_out, out_slots, rows_ws, dit)


def context_rows(w: Workload, buf: StepBuffers) -> None:
    """The write's rows from the target hidden states and the anchor tokens
    (sglang/model.py ``_write_context``, ``_anchor_kv_impl``)."""
    up, wr = w.upstream, w.write
    B.fm_context_rows(up.hidden, up.w_fc, up.hidden_norm_w, up.anchor_ids, up.embedding, up.w_anchor_proj,
                      up.b_anchor_proj, up.anchor_norm_w, w.eps, commit_lens=wr.commit_lens, window=wr.window,
                      bs=w.bs, rows=wr.x, ws=buf.rows_ws)


def write_context(w: Workload, buf: StepBuffers) -> None:
    """The context/anchor write, with its rows made first when the workload
    starts from the target hidden states."""
    if w.upstream is not None:
        context_rows(w, buf)
    write_kv(w, buf)


def write_kv(w: Workload, buf: StepBuffers) -> None:
    wr = w.write
    B.fm_write_context_kv(wr.x, wr.w_kv, wr.k_norm_w, wr.row_req, wr.row_pos, w.page_table, w.pools, w.eps,
                          w.theta, commit_lens=wr.commit_lens, window=wr.window, out_slots=buf.out_slots,
                          ws=buf.write_ws, kv_scales=w.kv_scales)


def plan(w: Workload, buf: StepBuffers) -> None:
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, buf.cross_ws, max_q=w.max_q, pool_dtype=w.pool_dtype,
                              xcd_weights=buf.xcd_weights)


def layer(w: Workload, buf: StepBuffers, l: int) -> None:
    B.fm_block_self_attention(w.qkv[l], w.self_q_norm_w[l], w.self_k_norm_w[l], w.block_ctx_lens, w.softmax_scale,
                              w.theta, w.eps, out=buf.self_out[l])
    B.fm_paged_cross_attention(w.q[l], w.q_norm_w[l], w.pools[l], w.page_table, w.ctx_lens, w.cu_seqlens_q,
                               w.softmax_scale, w.theta, w.eps, buf.cross_ws, out=buf.cross_out[l], max_q=w.max_q,
                               fp8_scales=w.fp8_scales(l))


def run_step(w: Workload, buf: StepBuffers) -> None:
    """Write (if the workload has one), plan, then every layer: the two
    attentions alone, or the whole DiT block around them."""
    if w.write is not None:
        write_context(w, buf)
    plan(w, buf)
    if w.dit is not None:
        dit_embed(w, buf)
        for l in range(w.L):
            dit_layer(w, buf, l)
        dit_final(w, buf)
        return
    for l in range(w.L):
        layer(w, buf, l)


def dit_embed(w: Workload, buf: StepBuffers) -> None:
    """The block's residual stream: x_embed of the jump's input rows."""
    d = w.dit
    B.fm_linear(d.embedded, d.w_xe, d.b_xe, B.FM_LINEAR_ASSIGN_F32, out=buf.dit["h"], ws=buf.dit["ws"])


def _untimed(kind, call):
    call()


def dit_layer(w: Workload, buf: StepBuffers, l: int, timed=_untimed) -> None:
    """One DiT block (sglang/model.py ``_denoise``): self-attention, then
    cross-attention, then the MLP, each behind a modulated LayerNorm and a
    gated residual into the fp32 stream ``h``.  ``timed(kind, call)`` runs
    each library call (kind: "norm", "linear", "self", "cross"), so a caller
    can bracket it with events."""
    a, lw, m = buf.dit, w.dit.layers[l], w.dit.mods[l]
    h, xn, ws = a["h"], a["xn"], a["ws"]
    rows = h.shape[0]
    sa, ca = buf.self_out[l], buf.cross_out[l]
    timed("norm", lambda: B.fm_ada_layer_norm(h, m["s_scale"], m["s_shift"], w.eps, out=xn))
    timed("linear", lambda: B.fm_linear(xn, lw["qkv"], out=a["qkv"], ws=ws))
    timed("self", lambda: B.fm_block_self_attention(
        a["qkv"].view(w.bs * w.n_cand, w.K, 3, w.H, w.Dh), w.self_q_norm_w[l], w.self_k_norm_w[l], w.block_ctx_lens,
        w.softmax_scale, w.theta, w.eps, out=sa))
    timed("linear", lambda: B.fm_linear(sa.view(rows, -1), lw["o_self"], epilogue=B.FM_LINEAR_RESIDUAL,
                                        gate=m["s_gate"], out=h, ws=ws))
    timed("norm", lambda: B.fm_ada_layer_norm(h, m["c_scale"], m["c_shift"], w.eps, out=xn))
    timed("linear", lambda: B.fm_linear(xn, lw["q"], out=a["q"], ws=ws))
    timed("cross", lambda: B.fm_paged_cross_attention(
        a["q"].view(rows, w.H, w.Dh), w.q_norm_w[l], w.pools[l], w.page_table, w.ctx_lens, w.cu_seqlens_q,
        w.softmax_scale, w.theta, w.eps, buf.cross_ws, out=ca, max_q=w.max_q, fp8_scales=w.fp8_scales(l)))
    timed("linear", lambda: B.fm_linear(ca.view(rows, -1), lw["o_cross"], epilogue=B.FM_LINEAR_RESIDUAL,
                                        gate=m["c_gate"], out=h, ws=ws))
    timed("norm", lambda: B.fm_ada_layer_norm(h, m["m_scale"], m["m_shift"], w.eps, out=xn))
    timed("linear", lambda: B.fm_linear(xn, lw["fc1"], lw["b1"], B.FM_LINEAR_GELU_BF16, out=a["mlp"], ws=ws))
    timed("linear", lambda: B.fm_linear(a["mlp"], lw["fc2"], lw["b2"], B.FM_LINEAR_RESIDUAL, gate=m["m_gate"],
                                        out=h, ws=ws))


def dit_final(w: Workload, buf: StepBuffers) -> None:
    """The final modulated LayerNorm of the block's rows."""
    B.fm_ada_layer_norm(buf.dit["h"], w.dit.final_scale, w.dit.final_shift, w.eps, out=buf.dit["out"])


PREFILL_CHUNK = 2048  # rows per write call in a prefill (sglang/model.py ``_WRITE_CHUNK``)


def write_prefill(hidden, positions, row_req, page_table, pools, w_fc, hidden_norm_w, w_kv, k_norm_w, eps, theta,
                  chunk=PREFILL_CHUNK, out_slots=None):
    """A prefill's context write (sglang/model.py ``write_target_hidden_kv``
    without verify windows): every row's hidden states through fc and
    hidden_norm, then the all-layer K/V write, ``chunk`` rows at a time so
    that the rows buffer and workspaces stay bounded.  Returns ``out_slots``."""
    n = hidden.shape[0]
    dim = w_fc.shape[0]
    dev = hidden.device
    rows = torch.empty((min(chunk, n), dim), dtype=torch.bfloat16, device=dev)
    rows_ws = torch.empty(B.fm_context_rows_workspace_size(min(chunk, n), 0, hidden.shape[1], 1, dim),
                          dtype=torch.uint8, device=dev)
    write_ws = torch.empty(B.fm_write_context_kv_workspace_size(min(chunk, n)), dtype=torch.uint8, device=dev)
    for s in range(0, n, chunk):
        e = min(s + chunk, n)
        r = rows[: e - s]
        B.fm_context_rows(hidden[s:e], w_fc, hidden_norm_w, None, None, None, None, None, eps, rows=r, ws=rows_ws)
        B.fm_write_context_kv(r, w_kv, k_norm_w, row_req[s:e], positions[s:e], page_table, pools, eps, theta,
                              out_slots=None if out_slots is None else out_slots[s:e], ws=write_ws)
    return out_slots
