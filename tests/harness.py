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
    if dtype == torch.float8_e4m3fn:
        return "e4m3"
    return "bf16" if dtype == torch.bfloat16 else "f32"


def bits_view(t: torch.Tensor) -> torch.Tensor:
    """The tensor's raw elements as integers of the same width."""
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def check_e4m3_rounding(got, exact, what: str, max_other=1e-3):
    """Codes written from fp32 against the oracle's unrounded values: each is
    the nearest-even e4m3 of the exact value, except that a value within fp32
    noise of a midpoint may take the other neighbour (at most ``max_other`` of
    them)."""
    got = to_np(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    assert got.shape == exact.shape, (what, got.shape, exact.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite codes"
    want = O.round_to_e4m3(exact)
    a = np.minimum(np.abs(exact), 448.0)
    _, e = np.frexp(a)
    half = np.where(e - 1 >= -6, np.ldexp(1.0, e - 4), 2.0 ** -9) / 2
    other = got != want
    err = np.abs(got - np.clip(exact, -448.0, 448.0))
    bad = other & (err > half + np.maximum(1e-3 * half, 1e-6))
    frac = float(other.mean()) if other.size else 0.0
    log(f"  {what}: {int(other.sum())} of {other.size} codes at the other neighbour of a midpoint")
    assert not bad.any(), f"{what}: {int(bad.sum())} codes are not a nearest e4m3 of the exact value"
    assert frac <= max_other, f"{what}: {frac:.2e} of the codes off the nearest-even one"


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
    fp8 = w.fp8_scales(layer)
    scales = {} if fp8 is None else dict(q_scale=fp8[0] or None, k_scale=fp8[1], v_scale=fp8[2])
    for i, b in enumerate(reqs):
        pt = np.zeros((1, width), dtype=np.int64)
        pt[0, :len(pt_rows[i])] = pt_rows[i]
        r0, r1 = cu[b], cu[b + 1]
        o = O.paged_cross_attention(q[r0:r1], to_np(w.q_norm_w[layer]), pk, pv, pt, [ctx[b]], [0, r1 - r0],
                                    w.page_size, w.softmax_scale, w.theta, w.eps,
                                    kv_e4m3=w.pools[layer].k.dtype == torch.float8_e4m3fn, **scales)
        out[b] = o
    return out


def rows_of(w, reqs, t: torch.Tensor) -> np.ndarray:
    cu = w.cu_seqlens_q.cpu().numpy()
    return np.concatenate([to_np(t[cu[b]:cu[b + 1]]) for b in reqs])


def ws_error_word(ws: torch.Tensor) -> int:
    return int(ws[4:8].view(torch.int32).item())
