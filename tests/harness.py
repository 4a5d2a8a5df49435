"""Test-side plumbing between the GPU path and the oracle: host copies of the
seeded device inputs, page gathers for sampled requests, and the comparison
bar (max-abs <= 2e-2, mean-abs <= 2e-3 for floating outputs; exact for slots)."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle as O

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def storage_name(dtype: torch.dtype) -> str:
    return "bf16" if dtype == torch.bfloat16 else "f32"


def compare(gpu, ref, what: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    gpu = to_np(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(ref)), f"{what}: oracle produced non-finite values"
    assert np.all(np.isfinite(gpu)), f"{what}: GPU produced non-finite values"
    err = np.abs(gpu - ref)
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    log(f"  {what}: max-abs {mx:.3e}  mean-abs {mean:.3e}  ({err.size} values)")
    assert mx <= max_abs, f"{what}: max-abs {mx} > {max_abs}"
    assert mean <= mean_abs, f"{what}: mean-abs {mean} > {mean_abs}"
    return mx, mean


def pages_of(w, b: int, upto: int | None = None) -> torch.Tensor:
    n = math.ceil((int(w.ctx_lens[b]) if upto is None else upto) / w.page_size)
    return w.page_table[b, :n].long()


def gather_pages(pool_view: torch.Tensor, page_ids: torch.Tensor) -> np.ndarray:
    """Logical (n, ps, H, Dh) float64 copy of the listed pages."""
    if page_ids.numel() == 0:
        return np.zeros((0,) + tuple(pool_view.shape[1:]))
    return to_np(pool_view[page_ids])


def compact_context(w, layer: int, reqs, pools=None):
    """Pages of ``reqs`` copied to the host with a compact page table: returns
    (pk, pv, pt_rows) where pt_rows[i] indexes pk/pv for request reqs[i]."""
    pools = pools if pools is not None else w.pools
    ids, rows, at = [], [], 0
    for b in reqs:
        p = pages_of(w, b)
        ids.append(p)
        rows.append(np.arange(at, at + p.numel()))
        at += p.numel()
    idx = torch.cat(ids) if ids else torch.zeros(0, dtype=torch.long, device=w.page_table.device)
    pk = gather_pages(pools[layer].k, idx)
    pv = gather_pages(pools[layer].v, idx)
    return pk, pv, rows


def oracle_cross(w, layer: int, reqs, pk, pv, pt_rows, q=None):
    """Oracle cross-attention outputs for the rows of ``reqs`` (dict b -> (nq, H, Dh))."""
    q = to_np(w.q[layer] if q is None else q)
    cu = w.cu_seqlens_q.cpu().numpy()
    ctx = w.ctx_lens.cpu().numpy()
    out = {}
    width = max([len(r) for r in pt_rows] + [1])
    for i, b in enumerate(reqs):
        pt = np.zeros((1, width), dtype=np.int64)
        pt[0, :len(pt_rows[i])] = pt_rows[i]
        r0, r1 = cu[b], cu[b + 1]
        o = O.paged_cross_attention(q[r0:r1], to_np(w.q_norm_w[layer]), pk, pv, pt, [ctx[b]], [0, r1 - r0],
                                    w.page_size, w.softmax_scale, w.theta, w.eps)
        out[b] = o
    return out


def rows_of(w, reqs, t: torch.Tensor) -> np.ndarray:
    cu = w.cu_seqlens_q.cpu().numpy()
    return np.concatenate([to_np(t[cu[b]:cu[b + 1]]) for b in reqs])


def ws_error_word(ws: torch.Tensor) -> int:
    return int(ws[4:8].view(torch.int32).item())
