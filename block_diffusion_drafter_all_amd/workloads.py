"""Seeded synthetic inputs for the draft-step attention path.

This module only draws inputs: request lengths, page tables, pool contents,
queries, projections and weights, with the shapes and distributions of the
FlashMap drafting workloads.  It holds none of the method's arithmetic, and
it serves both the HIP path and the oracle (through host copies of the same
tensors).

Fixed draw order per workload, from one torch generator seeded
``1000 + workload id``: lengths -> commits (workload 5) -> page permutation ->
pool K -> pool V (per layer) -> q -> qkv -> X -> W -> norm weights.  Integer
uniforms are inclusive.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

from .binding import KVPool

BLOCK = 16          # draft slots per block
EPS = 1e-6          # q/k RMSNorm epsilon
THETA = 1e6         # RoPE base


@dataclass
class WriteInputs:
    x: torch.Tensor            # (n_rows, d_in)
    w_kv: torch.Tensor         # (L*2*H*Dh, d_in)
    k_norm_w: torch.Tensor     # (L, Dh) fp32
    row_req: torch.Tensor      # (n_rows,) int32
    row_pos: torch.Tensor      # (n_rows,) int32
    commit_lens: torch.Tensor | None  # (bs,) int32
    window: int


@dataclass
class UpstreamInputs:
    """What the write's rows are made from (fm_context_rows): the window rows'
    concatenated target hidden states through fc and hidden_norm, the anchors'
    token embeddings through anchor_proj and anchor_norm."""
    hidden: torch.Tensor          # (bs * window, n_aux * d_target) bf16
    w_fc: torch.Tensor            # (dim, n_aux * d_target) bf16
    hidden_norm_w: torch.Tensor   # (dim,) fp32
    anchor_ids: torch.Tensor      # (bs,) int32
    embedding: torch.Tensor       # (vocab, d_target) bf16
    w_anchor_proj: torch.Tensor   # (dim, d_target) bf16
    b_anchor_proj: torch.Tensor   # (dim,) bf16
    anchor_norm_w: torch.Tensor   # (dim,) fp32


@dataclass
class DitInputs:
    """The rest of the DiT blocks (fm_ada_layer_norm, fm_linear): the jump's
    input rows through x_embed, per layer the projections, the MLP and the
    step's modulation vectors, and the final modulation."""
    embedded: torch.Tensor        # (rows, d_target) bf16: the block's embedded state
    w_xe: torch.Tensor            # (dim, d_target) bf16
    b_xe: torch.Tensor            # (dim,) bf16
    layers: list                  # per layer: qkv, o_self, q, o_cross, fc1, b1, fc2, b2 (bf16)
    mods: list                    # per layer: s/c/m _scale (1 + scale), _shift, _gate (dim,) fp32
    final_scale: torch.Tensor     # (dim,) fp32, 1 + scale
    final_shift: torch.Tensor     # (dim,) fp32


@dataclass
class Workload:
    name: str
    workload_id: int
    bs: int
    K: int
    L: int
    H: int
    Dh: int
    page_size: int
    dtype: torch.dtype
    ctx_lens: torch.Tensor             # (bs,) int32: p + 1
    cu_seqlens_q: torch.Tensor         # (bs+1,) int32
    page_table: torch.Tensor           # (bs, width) int32
    pools: list                        # L x KVPool
    q: list                            # L x (total_q, H, Dh)
    qkv: list                          # L x (bs, K, 3, H, Dh)
    q_norm_w: list                     # L x (Dh,) fp32, cross-attention query norm
    self_q_norm_w: list                # L x (Dh,) fp32
    self_k_norm_w: list                # L x (Dh,) fp32
    write: WriteInputs | None = None
    n_cand: int = 1                    # candidate blocks per request (tree drafting)
    upstream: UpstreamInputs | None = None  # the write's rows made by fm_context_rows (write.x receives them)
    dit: DitInputs | None = None       # the rest of the DiT blocks around the two attentions
    kv_scales: list | None = None      # e4m3 pool: (k_scale, v_scale) per layer (None = 1)
    q_scales: list | None = None       # e4m3 pool: fixed query scale per layer (None = per request and head)
    eps: float = EPS
    theta: float = THETA
    meta: dict = field(default_factory=dict)

    @property
    def max_q(self) -> int:
        """Query rows per request: K per candidate block."""
        return self.K * self.n_cand

    @property
    def block_ctx_lens(self) -> torch.Tensor:
        """Context length of each self-attention block (every candidate of a
        request sits at the same positions)."""
        return self.ctx_lens if self.n_cand == 1 else self.ctx_lens.repeat_interleave(self.n_cand)

    @property
    def pool_dtype(self) -> torch.dtype:
        """Element type of the KV pool: the activation type, or e4m3."""
        return self.pools[0].k.dtype

    def fp8_scales(self, layer: int):
        """(q_scale, k_scale, v_scale) of a layer's cross-attention, or None."""
        if self.kv_scales is None and self.q_scales is None:
            return None
        q = 0.0 if self.q_scales is None else self.q_scales[layer]
        k, v = (1.0, 1.0) if self.kv_scales is None else self.kv_scales[layer]
        return (q, k, v)

    @property
    def softmax_scale(self) -> float:
        return self.Dh ** -0.5

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1].item())


def _randn(shape, gen, dtype, device, std=1.0, chunk=1 << 26):
    """N(0, std^2) drawn in float32 and rounded to ``dtype``, in chunks."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - s)
        flat[s:s + n] = (torch.randn(n, generator=gen, device=device, dtype=torch.float32) * std).to(dtype)
    return out


def _pool_tensors(n_pages, ps, H, Dh, dtype, device, gen, layout):
    """One layer's K and V pages filled N(0,1), as (pages, ps, H, Dh) views."""
    if layout == "head_major":          # (pages, H, ps, Dh): one (page, head) tile contiguous
        k = _randn((n_pages, H, ps, Dh), gen, dtype, device).permute(0, 2, 1, 3)
        v = _randn((n_pages, H, ps, Dh), gen, dtype, device).permute(0, 2, 1, 3)
    elif layout == "token_major":       # (pages, ps, H, Dh)
        k = _randn((n_pages, ps, H, Dh), gen, dtype, device)
        v = _randn((n_pages, ps, H, Dh), gen, dtype, device)
    else:
        raise ValueError(layout)
    return KVPool(k, v)


def _page_table(pages_needed, width, n_pages, gen, device):
    """Pages handed out from one permutation of the pool, in request order."""
    perm = torch.randperm(n_pages, generator=gen, device=device).to(torch.int32)
    pt = torch.zeros((len(pages_needed), width), dtype=torch.int32, device=device)
    at = 0
    for b, n in enumerate(pages_needed):
        pt[b, :n] = perm[at:at + n]
        at += n
    return pt


def _norm_weights(L, Dh, gen, device, kind):
    if kind == "ones":
        return [torch.ones(Dh, device=device) for _ in range(L)]
    return [1.0 + 0.1 * torch.randn(Dh, generator=gen, device=device) for _ in range(L)]


def _attention_inputs(bs, L, H, Dh, dtype, device, gen, cu_q, K):
    total_q = int(cu_q[-1].item())
    q = [_randn((total_q, H, Dh), gen, dtype, device) for _ in range(L)]
    qkv = [_randn((bs, K, 3, H, Dh), gen, dtype, device) for _ in range(L)]
    return q, qkv


def make_workload(workload_id: int, device="cuda", weights="ones", layout="head_major", scale_down=None,
                  q_scale=1.0, seed=None, n_cand=1, kv_fp8=False, upstream=False, dit=False) -> Workload:
    """The seeded inputs of one workload.

    1  tiny fp32 full step: 1 request, ctx 64, 1 layer, 4 x 64, page 16,
       pool = randperm of 4 pages, write of 64 rows with W = I (x = [k, v]).
    2  one bf16 layer: 8 requests, ctx U[512, 2048], 32 x 128, pool 4096 pages.
    3  five bf16 layers: 64 requests, ctx U[1024, 8192], one shared page table.
    4  long skewed batch: 256 requests ctx = clip(round(4096 e^Z), 64, 32768),
       Z ~ N(0,1), plus one of 131072 tokens (last); 1 layer.
    5  full draft step: 64 requests, ctx = p + 1 ~ U[1024, 8192], each commits
       c ~ U{1..17} verify columns at p-c .. p-1 plus its anchor at p; one GEMM
       from 4096 to 5 x 2 x 32 x 128 (W ~ N(0, 0.02^2)), then 5 layers.

    ``scale_down`` (dict) overrides bs / length bounds for small parity runs
    (and, for workloads 2 and 3, the activation and pool type: ``dtype``);
    ``q_scale`` multiplies the cross-attention query norm weight (a "peaky"
    softmax variant: the norm would cancel a scale on the raw queries, so the
    weight carries it and the scores' spread grows by that factor).
    ``n_cand`` candidate blocks per request (tree drafting): each request's
    cross-attention query holds ``n_cand * K`` rows, candidate-major, and the
    self-attention runs over ``bs * n_cand`` blocks.
    ``kv_fp8``: the pools hold e4m3 (the same N(0, 1) draws cast to e4m3;
    bf16 workloads only); the write stores e4m3 at scale 1 and cross-attention
    quantizes its queries (sglang/model.py ``_kv_fp8`` path).
    ``upstream`` (workload 5): the write's rows are made on the device from
    the window rows' concatenated target hidden states (``n_aux`` = 5 layers
    of ``d_target`` = 4096, N(0, 1)) through ``fc`` (N(0, 0.02^2)) and
    ``hidden_norm``, and from the anchors' token embeddings (vocab 151936,
    N(0, 1)) through ``anchor_proj`` (N(0, 0.02^2), bias N(0, 0.1^2)) and
    ``anchor_norm``; ``write.x`` is the buffer that receives them.
    ``dit``: the rest of every DiT block around the attentions (the sglang
    model's ``_denoise``): the block's rows start as ``x_embed`` of N(0, 1)
    embedded states (``d_target`` wide), each layer's projections are
    N(0, 0.02^2) (MLP width 4 dim, biases N(0, 0.1^2)), its modulations
    1 + 0.1 N(0, 1) (scales), 0.1 N(0, 1) (shifts) and 0.3 N(0, 1) (gates);
    the attentions take the projections' outputs instead of ``q``/``qkv``.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 + workload_id if seed is None else seed)
    sd = dict(scale_down or {})
    K = BLOCK
    write = None
    if workload_id == 1:
        bs, L, H, Dh, ps, dtype = 1, 1, 4, 64, 16, torch.float32
        ctx = torch.tensor([64], dtype=torch.int32, device=device)
        pages_needed = [4]
        n_pages = 4
        width = 4
    elif workload_id in (2, 3):
        bs = sd.get("bs", 8 if workload_id == 2 else 64)
        lo, hi = sd.get("ctx", (512, 2048) if workload_id == 2 else (1024, 8192))
        L = sd.get("L", 1 if workload_id == 2 else 5)
        H, Dh, ps, dtype = sd.get("H", 32), sd.get("Dh", 128), sd.get("ps", 16), sd.get("dtype", torch.bfloat16)
        ctx = torch.randint(lo, hi + 1, (bs,), generator=gen, device=device, dtype=torch.int32)
        if "ctx_list" in sd:                 # explicit lengths (edge cases)
            ctx = torch.tensor(sd["ctx_list"], dtype=torch.int32, device=device)
            bs = len(sd["ctx_list"])
        pages_needed = [math.ceil(int(c) / ps) for c in ctx.tolist()]
        width = max(max(pages_needed), 1)
        n_pages = sd.get("pool_pages", 4096 if workload_id == 2 else sum(pages_needed))
        n_pages = max(n_pages, sum(pages_needed), 1)
    elif workload_id == 4:
        bs_small = sd.get("bs", 256)
        lo, hi = sd.get("clip", (64, 32768))
        median = sd.get("median", 4096)
        long_len = sd.get("long", 131072)
        L, H, Dh, ps, dtype = 1, sd.get("H", 32), 128, 16, torch.bfloat16
        z = torch.randn(bs_small, generator=gen, device=device)
        small = torch.clamp(torch.round(median * torch.exp(z)), lo, hi).to(torch.int32)
        ctx = torch.cat([small, torch.tensor([long_len], dtype=torch.int32, device=device)])
        if sd.get("long_first"):
            ctx = torch.roll(ctx, 1)
        bs = bs_small + 1
        pages_needed = [math.ceil(int(c) / ps) for c in ctx.tolist()]
        width = max(pages_needed)
        n_pages = sum(pages_needed)
    elif workload_id == 5:
        bs = sd.get("bs", 64)
        lo, hi = sd.get("ctx", (1024, 8192))
        L, H, Dh, ps, dtype = sd.get("L", 5), sd.get("H", 32), 128, 16, torch.bfloat16
        d_in = sd.get("d_in", 4096)
        window = K + 1
        ctx = torch.randint(lo, hi + 1, (bs,), generator=gen, device=device, dtype=torch.int32)
        anchor = ctx - 1                                   # p
        # pages cover the whole verify window, so a write of an uncommitted
        # column would land inside the request's pages (and be caught)
        pages_needed = None
    else:
        raise ValueError(f"unknown workload {workload_id}")

    if workload_id == 5:
        commit = torch.randint(1, window + 1, (bs,), generator=gen, device=device, dtype=torch.int32)
        last_pos = anchor - commit + (window - 1)
        pages_needed = [math.ceil((int(lp) + 1) / ps) for lp in torch.maximum(last_pos, anchor).tolist()]
        width = max(pages_needed)
        n_pages = sum(pages_needed)
        pt = _page_table(pages_needed, width, n_pages, gen, device)
    else:
        pt = _page_table(pages_needed, width, n_pages, gen, device)

    if kv_fp8 and dtype != torch.bfloat16:
        raise ValueError("an e4m3 pool goes with bf16 activations")
    pool_dtype = torch.float8_e4m3fn if kv_fp8 else dtype
    pools = [_pool_tensors(n_pages, ps, H, Dh, pool_dtype, device, gen, layout) for _ in range(L)]
    cu_q = torch.arange(0, (bs + 1) * K * n_cand, K * n_cand, dtype=torch.int32, device=device)
    q, qkv = _attention_inputs(bs * n_cand, L, H, Dh, dtype, device, gen, cu_q, K)

    if workload_id == 1:
        # the write fills the whole context 0..63: x = [k | v] with W = I
        x = _randn((64, 2 * H * Dh), gen, dtype, device)
        w_kv = torch.eye(2 * H * Dh, dtype=dtype, device=device)
        write = WriteInputs(x=x, w_kv=w_kv, k_norm_w=None, row_req=torch.zeros(64, dtype=torch.int32, device=device),
                            row_pos=torch.arange(64, dtype=torch.int32, device=device), commit_lens=None, window=0)
    elif workload_id == 5:
        n_rows = bs * window + bs
        x = _randn((n_rows, d_in), gen, dtype, device)
        w_kv = _randn((L * 2 * H * Dh, d_in), gen, dtype, device, std=0.02)
        cols = torch.arange(window, dtype=torch.int32, device=device)
        win_pos = (anchor - commit)[:, None] + cols[None, :]
        row_pos = torch.cat([win_pos.reshape(-1), anchor]).to(torch.int32)
        row_req = torch.cat([torch.arange(bs, device=device).repeat_interleave(window),
                             torch.arange(bs, device=device)]).to(torch.int32)
        write = WriteInputs(x=x, w_kv=w_kv, k_norm_w=None, row_req=row_req, row_pos=row_pos,
                            commit_lens=commit, window=window)
        if upstream:
            n_aux, d_target, vocab = sd.get("n_aux", 5), sd.get("d_target", 4096), sd.get("vocab", 151936)
            hidden = _randn((bs * window, n_aux * d_target), gen, dtype, device)
            w_fc = _randn((d_in, n_aux * d_target), gen, dtype, device, std=0.02)
            anchor_ids = torch.randint(0, vocab, (bs,), generator=gen, device=device, dtype=torch.int32)
            embedding = _randn((vocab, d_target), gen, dtype, device)
            w_ap = _randn((d_in, d_target), gen, dtype, device, std=0.02)
            b_ap = _randn((d_in,), gen, dtype, device, std=0.1)
            up_norms = _norm_weights(2, d_in, gen, device, weights)
            upstream_inputs = UpstreamInputs(hidden=hidden, w_fc=w_fc, hidden_norm_w=up_norms[0],
                                             anchor_ids=anchor_ids, embedding=embedding, w_anchor_proj=w_ap,
                                             b_anchor_proj=b_ap, anchor_norm_w=up_norms[1])
            x.fill_(float("nan"))  # filled by fm_context_rows; skipped rows keep the NaN

    if not upstream or workload_id != 5:
        upstream_inputs = None
    dit_inputs = None
    if dit:
        dim, inter, d_target = H * Dh, 4 * H * Dh, sd.get("d_target", 4096)
        rows = bs * n_cand * K
        lw = []
        for _ in range(L):
            lw.append(dict(qkv=_randn((3 * dim, dim), gen, dtype, device, std=0.02),
                           o_self=_randn((dim, dim), gen, dtype, device, std=0.02),
                           q=_randn((dim, dim), gen, dtype, device, std=0.02),
                           o_cross=_randn((dim, dim), gen, dtype, device, std=0.02),
                           fc1=_randn((inter, dim), gen, dtype, device, std=0.02),
                           b1=_randn((inter,), gen, dtype, device, std=0.1),
                           fc2=_randn((dim, inter), gen, dtype, device, std=0.02),
                           b2=_randn((dim,), gen, dtype, device, std=0.1)))
        def mvec(kind):
            z = torch.randn(dim, generator=gen, device=device)
            return (1.0 + 0.1 * z) if kind == "scale" else (0.1 * z if kind == "shift" else 0.3 * z)
        mods = [{f"{b}_{k}": mvec(k) for b in ("s", "c", "m") for k in ("scale", "shift", "gate")} for _ in range(L)]
        dit_inputs = DitInputs(embedded=_randn((rows, d_target), gen, dtype, device),
                               w_xe=_randn((dim, d_target), gen, dtype, device, std=0.02),
                               b_xe=_randn((dim,), gen, dtype, device, std=0.1), layers=lw, mods=mods,
                               final_scale=mvec("scale"), final_shift=mvec("shift"))
    q_norm_w = [w * q_scale for w in _norm_weights(L, Dh, gen, device, weights)]
    self_q = _norm_weights(L, Dh, gen, device, weights)
    self_k = _norm_weights(L, Dh, gen, device, weights)
    if write is not None:
        write.k_norm_w = torch.stack(_norm_weights(L, Dh, gen, device, weights)).contiguous()
    names = {1: "tiny fp32 step", 2: "one-layer bf16 step", 3: "all-layers step", 4: "long skewed batch",
             5: "full draft step with context write"}
    return Workload(name=names[workload_id], workload_id=workload_id, bs=bs, K=K, L=L, H=H, Dh=Dh, page_size=ps,
                    dtype=dtype, ctx_lens=ctx.contiguous(), cu_seqlens_q=cu_q, page_table=pt, pools=pools, q=q,
                    qkv=qkv, q_norm_w=q_norm_w, self_q_norm_w=self_q, self_k_norm_w=self_k, write=write,
                    n_cand=n_cand, upstream=upstream_inputs, dit=dit_inputs,
                    meta=dict(layout=layout, weights=weights, n_pages=n_pages, scale_down=sd, q_scale=q_scale,
                              kv_fp8=kv_fp8))
