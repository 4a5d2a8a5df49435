"""The no-allocation context K/V write (fm_write_context_kv_noalloc, through
the C ABI) against fm_write_context_kv with its own workspace: two calls in a
row on one GPU, the second with fewer rows, each bit for bit (slots and every
pool byte), and an oversized call refused before anything is enqueued."""

from __future__ import annotations

import pytest
import torch

from harness import bits_view, log

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU machines
    pytest.skip("needs a GPU", allow_module_level=True)

from block_diffusion_drafter_all_amd import binding as B  # noqa: E402
from block_diffusion_drafter_all_amd.workloads import make_workload  # noqa: E402


def _write_both_ways(w):
    """The same write into two copies of the pools: with a workspace, then
    with the static one.  Returns both slot arrays and both pool copies."""
    wr = w.write
    pools_ws = w.pools
    pools_st = [type(p)(p.k.clone(), p.v.clone()) for p in w.pools]
    n = wr.x.shape[0]
    slots_ws = torch.full((n,), -7, dtype=torch.int32, device=wr.x.device)
    slots_st = torch.full((n,), -7, dtype=torch.int32, device=wr.x.device)
    B.fm_write_context_kv(wr.x, wr.w_kv, wr.k_norm_w, wr.row_req, wr.row_pos, w.page_table, pools_ws, w.eps,
                          w.theta, commit_lens=wr.commit_lens, window=wr.window, out_slots=slots_ws)
    B.fm_write_context_kv_noalloc(wr.x, wr.w_kv, wr.k_norm_w, wr.row_req, wr.row_pos, w.page_table, pools_st,
                                  w.eps, w.theta, commit_lens=wr.commit_lens, window=wr.window, out_slots=slots_st)
    torch.cuda.synchronize()
    return slots_ws, slots_st, pools_ws, pools_st


def _same_bits(a, b, what):
    assert torch.equal(bits_view(a.contiguous()), bits_view(b.contiguous())), f"{what}: bits differ"


def test_noalloc_write_equals_workspace_write():
    # First call: the full draft step's write (1152 rows, 5 layers x 32 heads,
    # the tiled bf16 GEMM); second: a smaller one on the same GPU, which
    # finds the first call's contents in the static array.
    cases = [
        ("full step: 64 requests, 1152 rows, 5 layers", dict(seed=None, scale_down=None, kv_fp8=False)),
        ("small step: 6 requests, 2 layers, 4 heads, d_in 256",
         dict(seed=2024, scale_down=dict(bs=6, ctx=(20, 300), L=2, H=4, d_in=256), kv_fp8=False)),
        ("small step over an e4m3 pool", dict(seed=2025, scale_down=dict(bs=3, ctx=(20, 90), L=1, H=2, d_in=128),
                                              kv_fp8=True)),
    ]
    prev_rows = None
    for what, kw in cases:
        log(f"no-alloc write: {what}")
        w = make_workload(5, weights="random", **kw)
        n = w.write.x.shape[0]
        assert prev_rows is None or n < prev_rows
        prev_rows = n
        slots_ws, slots_st, pools_ws, pools_st = _write_both_ways(w)
        live = int((slots_ws >= 0).sum())
        log(f"  {live} of {n} rows written")
        assert live > 0
        _same_bits(slots_ws, slots_st, "out_slots")
        for l, (a, b) in enumerate(zip(pools_ws, pools_st)):
            _same_bits(a.k, b.k, f"layer {l} K pool")
            _same_bits(a.v, b.v, f"layer {l} V pool")
        del w, pools_st
        torch.cuda.empty_cache()


def test_noalloc_write_refuses_more_rows_than_its_workspace():
    w = make_workload(5, weights="random", seed=11, scale_down=dict(bs=2, ctx=(20, 60), L=1, H=2, d_in=64))
    wr = w.write
    n = B.FM_WRITE_NOALLOC_MAX_ROWS + 1
    x = torch.zeros((n, wr.x.shape[1]), dtype=wr.x.dtype, device=wr.x.device)
    req = torch.zeros(n, dtype=torch.int32, device=x.device)
    pos = torch.full((n,), -1, dtype=torch.int32, device=x.device)
    before = [(p.k.clone(), p.v.clone()) for p in w.pools]
    with pytest.raises(B.FmError) as e:
        B.fm_write_context_kv_noalloc(x, wr.w_kv, wr.k_norm_w, req, pos, w.page_table, w.pools, w.eps, w.theta)
    assert e.value.status == B.FM_E_UNSUPPORTED and "static workspace" in str(e.value)
    torch.cuda.synchronize()
    for (k0, v0), p in zip(before, w.pools):
        _same_bits(k0, p.k, "K pool after a refused call")
        _same_bits(v0, p.v, "V pool after a refused call")
