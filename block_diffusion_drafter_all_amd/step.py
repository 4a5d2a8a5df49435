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
    return StepBuffers(cross_ws, write_ws, cross_out, self_out, out_slots, rows_ws)


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
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, buf.cross_ws, max_q=w.max_q, pool_dtype=w.pool_dtype)


def layer(w: Workload, buf: StepBuffers, l: int) -> None:
    B.fm_block_self_attention(w.qkv[l], w.self_q_norm_w[l], w.self_k_norm_w[l], w.block_ctx_lens, w.softmax_scale,
                              w.theta, w.eps, out=buf.self_out[l])
    B.fm_paged_cross_attention(w.q[l], w.q_norm_w[l], w.pools[l], w.page_table, w.ctx_lens, w.cu_seqlens_q,
                               w.softmax_scale, w.theta, w.eps, buf.cross_ws, out=buf.cross_out[l], max_q=w.max_q,
                               fp8_scales=w.fp8_scales(l))


def run_step(w: Workload, buf: StepBuffers) -> None:
    """Write (if the workload has one), plan, then every layer."""
    if w.write is not None:
        write_context(w, buf)
    plan(w, buf)
    for l in range(w.L):
        layer(w, buf, l)


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
