"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Floating outputs: max-abs <= 2e-2 and mean-abs <= 2e-3;
slots and placement: exact."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle as O
from harness import (bits_view, check_e4m3_rounding, compact_context, compare, log, oracle_cross, rows_of,
                     storage_name, to_np, ws_error_word)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU machines
    pytest.skip("needs a GPU", allow_module_level=True)

from block_diffusion_drafter_all_amd import binding as B  # noqa: E402
from block_diffusion_drafter_all_amd import step as S  # noqa: E402
from block_diffusion_drafter_all_amd.workloads import make_workload  # noqa: E402


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _oracle_self(w, layer, blocks=None):
    blocks = range(w.bs) if blocks is None else blocks
    qkv = to_np(w.qkv[layer][list(blocks)])
    return O.block_self_attention(qkv, to_np(w.self_q_norm_w[layer]), to_np(w.self_k_norm_w[layer]),
                                  w.block_ctx_lens.cpu().numpy()[list(blocks)], w.softmax_scale, w.theta, w.eps)


def _check_attention(w, buf, reqs, layers=None, self_blocks=None, pools=None):
    layers = range(w.L) if layers is None else layers
    for l in layers:
        pk, pv, rows = compact_context(w, l, reqs, pools)
        ref = oracle_cross(w, l, reqs, pk, pv, rows)
        compare(rows_of(w, reqs, buf.cross_out[l]), np.concatenate([ref[b] for b in reqs]), f"cross L{l}")
        sb = list(range(w.bs)) if self_blocks is None else list(self_blocks)
        compare(buf.self_out[l][sb], _oracle_self(w, l, sb), f"self L{l}")
    assert ws_error_word(buf.cross_ws) == 0


def _write_oracle(w):
    wr = w.write
    return O.write_context_kv(to_np(wr.x), to_np(wr.w_kv), to_np(wr.k_norm_w), wr.row_req.cpu().numpy(),
                              wr.row_pos.cpu().numpy(), w.page_table.cpu().numpy(), w.page_size, w.L, w.H, w.Dh,
                              w.eps, w.theta,
                              commit_lens=None if wr.commit_lens is None else wr.commit_lens.cpu().numpy(),
                              window=wr.window)


def _snapshot(w):
    return [(p.k.clone(), p.v.clone()) for p in w.pools]


def _check_write(w, buf, before, slots, keys, values):
    """Slots exact; the set of changed slots exact; written values in tolerance."""
    np.testing.assert_array_equal(buf.out_slots.cpu().numpy(), slots)
    assert int(buf.write_ws[4:8].view(torch.int32).item()) == 0
    live = np.nonzero(slots >= 0)[0]
    ps = w.page_size
    expect = set(int(s) for s in slots[live])
    for l in range(w.L):
        for t_before, t_after, name in ((before[l][0], w.pools[l].k, "k"), (before[l][1], w.pools[l].v, "v")):
            diff = (bits_view(t_before) != bits_view(t_after)).any(dim=3).any(dim=2)   # (pages, ps)
            changed = torch.nonzero(diff.reshape(-1)).flatten().cpu().numpy()
            assert set(changed.tolist()) == expect, f"layer {l} {name}: changed slots differ"
        sl = torch.as_tensor(slots[live], device=w.page_table.device, dtype=torch.long)
        got_k = w.pools[l].k[sl // ps, sl % ps]
        got_v = w.pools[l].v[sl // ps, sl % ps]
        if w.pool_dtype == torch.float8_e4m3fn:
            ks, vs = (1.0, 1.0) if w.kv_scales is None else w.kv_scales[l]
            check_e4m3_rounding(got_k, keys[live, l] / ks, f"written K L{l} (e4m3)")
            check_e4m3_rounding(got_v, values[live, l] / vs, f"written V L{l} (e4m3)")
        else:
            compare(got_k, keys[live, l], f"written K L{l}")
            compare(got_v, values[live, l], f"written V L{l}")


def test_config1_full_step():
    log("config 1: tiny fp32 full step")
    w = make_workload(1)
    buf = S.allocate(w)
    before = _snapshot(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    slots, keys, values = _write_oracle(w)
    _check_write(w, buf, before, slots, keys, values)
    # oracle pool = pre-write pages + the oracle's own write
    pk = [to_np(before[0][0])]
    pv = [to_np(before[0][1])]
    O.scatter_into_pool(pk, pv, slots, keys, values, w.page_size, storage_name(w.pool_dtype), kv_scales=w.kv_scales)
    ref = O.paged_cross_attention(to_np(w.q[0]), to_np(w.q_norm_w[0]), pk[0], pv[0], w.page_table.cpu().numpy(),
                                  w.ctx_lens.cpu().numpy(), w.cu_seqlens_q.cpu().numpy(), w.page_size,
                                  w.softmax_scale, w.theta, w.eps)
    mx, _ = compare(buf.cross_out[0], ref, "cross (fp32)")
    assert mx < 1e-4  # fp32 storage and MFMA: far inside the bf16 bar
    mx, _ = compare(buf.self_out[0], _oracle_self(w, 0), "self (fp32)")
    assert mx < 1e-4


@pytest.mark.parametrize("variant", ["default", "token_major", "peaky_f32", "peaky_bf16"])
def test_config2_all_rows(variant):
    # 8 requests x 32 heads over ~2048 waves: most pairs are cut between waves,
    # so the merge path is exercised as well as whole pairs.  The peaky
    # variants widen the scores (query norm weight x8: std 8, so the running
    # max moves past the lazy-rescale slack tile after tile) in fp32, where
    # the operands carry no rounding; over bf16 operands x2 (std 2): past
    # that, the bf16 query operand alone moves outputs beyond the bar.
    log(f"config 2: {variant}")
    kw = {}
    if variant == "token_major":
        kw = dict(weights="random", layout="token_major")
    elif variant == "peaky_f32":
        kw = dict(weights="random", q_scale=8.0, scale_down=dict(dtype=torch.float32))
    elif variant == "peaky_bf16":
        kw = dict(weights="random", q_scale=2.0)
    w = make_workload(2, **kw)
    buf = S.allocate(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    _check_attention(w, buf, list(range(w.bs)))


@pytest.mark.parametrize("n_cand", [2, 4])
def test_candidate_blocks_share_one_context_read(n_cand):
    # Tree drafting: each request's n_cand candidate blocks (16 rows each) sit
    # side by side on the query axis and attend to one read of its context;
    # config 2's shape, random norm weights, all rows against the oracle.
    log(f"config 2 with {n_cand} candidate blocks per request")
    w = make_workload(2, weights="random", n_cand=n_cand)
    buf = S.allocate(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    _check_attention(w, buf, list(range(w.bs)), self_blocks=range(w.bs * n_cand))


def test_candidate_blocks_ragged_rows_and_empty_context():
    # max_q 64 (four fragments) with 0, 1, 16, 17, 40 and 64 rows per request,
    # including an empty context and a context shorter than one tile.
    log("candidate blocks: ragged rows, empty context")
    ctx = [300, 0, 5, 1000, 77, 2100]
    nq = [40, 17, 64, 1, 0, 16]
    w = make_workload(3, weights="random", scale_down=dict(ctx_list=ctx, L=1, H=3), n_cand=4)
    dev = w.ctx_lens.device
    cu = torch.tensor(np.concatenate([[0], np.cumsum(nq)]), dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    q = torch.randn((int(cu[-1]), w.H, w.Dh), generator=gen, device=dev).to(torch.bfloat16)
    w.q[0], w.cu_seqlens_q = q, cu
    ws = torch.empty(B.fm_cross_attention_workspace_size(w.bs, w.H, w.Dh, 64, w.pool_dtype), dtype=torch.uint8,
                     device=dev)
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws, max_q=64, pool_dtype=w.pool_dtype)
    out = torch.full_like(q, float("nan"))
    B.fm_paged_cross_attention(q, w.q_norm_w[0], w.pools[0], w.page_table, w.ctx_lens, cu, w.softmax_scale,
                               w.theta, w.eps, ws, out=out, max_q=64)
    torch.cuda.synchronize()
    reqs = list(range(w.bs))
    pk, pv, rows = compact_context(w, 0, reqs)
    ref = oracle_cross(w, 0, reqs, pk, pv, rows, q=q)
    compare(rows_of(w, reqs, out), np.concatenate([ref[b] for b in reqs]), "cross 4 fragments ragged")
    assert torch.all(out[cu[1]:cu[2]] == 0), "an empty context must give exactly zero"
    assert ws_error_word(ws) == 0


@pytest.mark.parametrize("ps", [1, 8, 32, 64])
def test_page_sizes_and_ragged_lengths(ps):
    log(f"page size {ps}")
    ctx = [0, 1, 15, 16, 17, 100, 257, 1000]
    w = make_workload(3, weights="random", scale_down=dict(ctx_list=ctx, L=2, H=4, ps=ps))
    buf = S.allocate(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    _check_attention(w, buf, list(range(w.bs)))
    for l in range(w.L):   # empty context -> exactly zero
        assert torch.count_nonzero(buf.cross_out[l][:16]) == 0


def test_head_dim_64_bf16_and_ragged_query_rows():
    log("Dh 64 bf16, ragged cu_seqlens_q")
    w = make_workload(3, weights="random", scale_down=dict(ctx_list=[40, 300, 7, 129], L=1, H=3, Dh=64))
    dev = w.ctx_lens.device
    nq = [16, 3, 0, 9]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(nq)]), dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    q = torch.randn((int(cu[-1]), w.H, w.Dh), generator=gen, device=dev).to(torch.bfloat16)
    w.q[0], w.cu_seqlens_q = q, cu
    ws = torch.empty(B.fm_cross_attention_workspace_size(w.bs, w.H, w.Dh, 16, w.pool_dtype), dtype=torch.uint8,
                     device=dev)
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws, pool_dtype=w.pool_dtype)
    out = B.fm_paged_cross_attention(q, w.q_norm_w[0], w.pools[0], w.page_table, w.ctx_lens, cu,
                                     w.softmax_scale, w.theta, w.eps, ws)
    torch.cuda.synchronize()
    reqs = list(range(w.bs))
    pk, pv, rows = compact_context(w, 0, reqs)
    ref = oracle_cross(w, 0, reqs, pk, pv, rows, q=q)
    compare(rows_of(w, reqs, out), np.concatenate([ref[b] for b in reqs]), "cross Dh64 ragged q")


def test_self_attention_small_blocks_fp32_dh128():
    log("self-attention K < 16, fp32, Dh 128")
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    for K, dtype in ((1, torch.float32), (5, torch.bfloat16), (16, torch.float32)):
        qkv = torch.randn((7, K, 3, 2, 128), generator=gen, device=dev).to(dtype)
        wq = 1 + 0.1 * torch.randn(128, generator=gen, device=dev)
        wk = 1 + 0.1 * torch.randn(128, generator=gen, device=dev)
        ctx = torch.randint(0, 5000, (7,), generator=gen, device=dev, dtype=torch.int32)
        out = B.fm_block_self_attention(qkv, wq, wk, ctx, 128 ** -0.5, 1e6, 1e-6)
        torch.cuda.synchronize()
        ref = O.block_self_attention(to_np(qkv), to_np(wq), to_np(wk), ctx.cpu().numpy(), 128 ** -0.5, 1e6, 1e-6)
        compare(out, ref, f"self K={K} {dtype}")


@pytest.mark.parametrize("K", [17, 24, 32, 33, 48, 64])
def test_self_attention_large_blocks(K):
    # Blocks of more than 16 slots: one wave per 16-slot query tile, each
    # scoring all K keys (up to four key tiles) with one exact softmax.
    log(f"self-attention K = {K}: bf16 and fp32, Dh 128 and 64")
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(40 + K)
    for Dh, dtype in ((128, torch.bfloat16), (64, torch.float32), (64, torch.bfloat16)):
        qkv = torch.randn((5, K, 3, 3, Dh), generator=gen, device=dev).to(dtype)
        wq = 1 + 0.1 * torch.randn(Dh, generator=gen, device=dev)
        wk = 1 + 0.1 * torch.randn(Dh, generator=gen, device=dev)
        ctx = torch.randint(0, 9000, (5,), generator=gen, device=dev, dtype=torch.int32)
        out = B.fm_block_self_attention(qkv, wq, wk, ctx, Dh ** -0.5, 1e6, 1e-6)
        torch.cuda.synchronize()
        ref = O.block_self_attention(to_np(qkv), to_np(wq), to_np(wk), ctx.cpu().numpy(), Dh ** -0.5, 1e6, 1e-6)
        compare(out, ref, f"self K={K} Dh {Dh} {dtype}")
    # peaky scores (std 8) in fp32: the softmax max must span every key tile
    # (over bf16 operands the rounding of the normed q and k alone would move
    # such outputs past the bar)
    qkv = torch.randn((3, K, 3, 2, 128), generator=gen, device=dev)
    wq = torch.ones(128, device=dev)
    out = B.fm_block_self_attention(qkv, wq, wq, torch.zeros(3, dtype=torch.int32, device=dev),
                                    128 ** -0.5 * 8, 1e6, 1e-6)
    torch.cuda.synchronize()
    ref = O.block_self_attention(to_np(qkv), to_np(wq), to_np(wq), np.zeros(3), 128 ** -0.5 * 8, 1e6, 1e-6)
    compare(out, ref, f"self K={K} peaky")


@pytest.mark.parametrize("n_cand", [1, 4])
def test_cross_attention_deterministic(n_cand):
    w = make_workload(2, weights="random", n_cand=n_cand)
    buf = S.allocate(w)
    S.run_step(w, buf)
    first = buf.cross_out[0].clone()
    S.run_step(w, buf)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), buf.cross_out[0].view(torch.int16))


def test_write_commit_rule_and_placement_small():
    log("write: commit rule and placement on a small full step")
    w = make_workload(5, weights="random", scale_down=dict(bs=6, ctx=(20, 90), L=2, H=4, d_in=256))
    buf = S.allocate(w)
    before = _snapshot(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    slots, keys, values = _write_oracle(w)
    _check_write(w, buf, before, slots, keys, values)
    _check_full_step_attention(w, buf, before, slots, keys, values, list(range(w.bs)))


def _check_full_step_attention(w, buf, before, slots, keys, values, reqs):
    """Cross-attention against the oracle's own pool: the pre-write pages plus
    the oracle's write."""
    ps = w.page_size
    for l in range(w.L):
        pk, pv, rows = compact_context(w, l, reqs, pools=[type(p)(b[0], b[1]) for p, b in zip(w.pools, before)])
        # move the oracle's written rows of these requests into the compact pages
        remap = {}
        for i, b in enumerate(reqs):
            for j, page in enumerate(w.page_table[b, :len(rows[i])].cpu().numpy()):
                remap[int(page)] = int(rows[i][j])
        sel = [r for r in np.nonzero(slots >= 0)[0] if int(slots[r]) // ps in remap]
        cslots = np.full_like(slots, -1)
        for r in sel:
            cslots[r] = remap[int(slots[r]) // ps] * ps + int(slots[r]) % ps
        pkl, pvl = [pk], [pv]
        O.scatter_into_pool(pkl, pvl, cslots, keys[:, l:l + 1], values[:, l:l + 1], ps, storage_name(w.pool_dtype),
                            kv_scales=None if w.kv_scales is None else w.kv_scales[l:l + 1])
        ref = oracle_cross(w, l, reqs, pk, pv, rows)
        compare(rows_of(w, reqs, buf.cross_out[l]), np.concatenate([ref[b] for b in reqs]), f"cross L{l}")
        compare(buf.self_out[l], _oracle_self(w, l), f"self L{l}")
    assert ws_error_word(buf.cross_ws) == 0


# ------------------------------------------------------------ full sizes


def _sample(w, n_extra, seed):
    ctx = w.ctx_lens.cpu().numpy()
    rng = np.random.default_rng(seed)
    picks = {int(np.argmax(ctx)), int(np.argmin(ctx))}
    picks.update(int(b) for b in rng.choice(w.bs, size=min(n_extra, w.bs), replace=False))
    return sorted(picks)


def test_config3_full_size_sampled():
    log("config 3: 64 requests, ctx U[1024, 8192], 5 layers (sampled requests)")
    w = make_workload(3)
    buf = S.allocate(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    reqs = _sample(w, 4, 3)
    log(f"  sampled requests {reqs}")
    _check_attention(w, buf, reqs, self_blocks=range(w.bs))


def test_config4_full_size_sampled():
    log("config 4: 256 lognormal requests + one of 131072 tokens (sampled requests)")
    w = make_workload(4)
    buf = S.allocate(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    reqs = _sample(w, 3, 4)
    log(f"  sampled requests {reqs} ctx {[int(w.ctx_lens[b]) for b in reqs]}")
    _check_attention(w, buf, reqs, self_blocks=range(w.bs))


def test_config4_long_request_first_sampled():
    # The 131072-token request first: its 32 heads' pairs open the tile stream,
    # so wave 0 starts inside it and the plan cuts it into many shares.
    log("config 4 with the 131072-token request first (sampled requests)")
    w = make_workload(4, scale_down=dict(long_first=True))
    assert int(w.ctx_lens[0]) == 131072
    buf = S.allocate(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    reqs = sorted({0, 1, 2} | set(_sample(w, 2, 44)))
    log(f"  sampled requests {reqs} ctx {[int(w.ctx_lens[b]) for b in reqs]}")
    _check_attention(w, buf, reqs, self_blocks=range(w.bs))


def test_config5_full_step_full_size():
    log("config 5: full draft step, write of 64 x 17 windows + anchors, 5 layers")
    w = make_workload(5)
    buf = S.allocate(w)
    before = _snapshot(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    log("  oracle write (one fp64 GEMM over the live rows)")
    slots, keys, values = _write_oracle(w)
    live = int((slots >= 0).sum())
    log(f"  live rows {live} of {len(slots)}")
    _check_write(w, buf, before, slots, keys, values)
    reqs = _sample(w, 3, 5)
    log(f"  sampled requests {reqs}")
    _check_full_step_attention(w, buf, before, slots, keys, values, reqs)


# ------------------------------------------------------------ e4m3 KV pool
# sglang/model.py ``_kv_fp8``: the write stores e4m3 at scale 1, cross-attention
# quantizes each (request, head)'s query with scale amax / 448.


@pytest.mark.parametrize("variant", ["default", "peaky", "token_major"])
def test_fp8_pool_config2_all_rows(variant):
    log(f"e4m3 pool, config 2 shape: {variant}")
    kw = dict(weights="random")
    if variant == "peaky":
        kw["q_scale"] = 2.0
    elif variant == "token_major":
        kw["layout"] = "token_major"
    w = make_workload(2, kv_fp8=True, **kw)
    buf = S.allocate(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    _check_attention(w, buf, list(range(w.bs)))


@pytest.mark.parametrize("n_cand", [2, 4])
def test_fp8_pool_candidate_blocks(n_cand):
    log(f"e4m3 pool, {n_cand} candidate blocks per request")
    w = make_workload(2, weights="random", n_cand=n_cand, kv_fp8=True)
    buf = S.allocate(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    _check_attention(w, buf, list(range(w.bs)), self_blocks=range(w.bs * n_cand))


@pytest.mark.parametrize("ps,Dh", [(1, 128), (32, 128), (16, 64), (4, 64)])
def test_fp8_pool_page_sizes_ragged(ps, Dh):
    # empty and sub-tile contexts, one query row, a request with no rows
    log(f"e4m3 pool, page size {ps}, Dh {Dh}, ragged rows")
    ctx = [0, 1, 15, 17, 300, 1000]
    nq = [16, 1, 16, 0, 9, 16]
    w = make_workload(3, weights="random", scale_down=dict(ctx_list=ctx, L=1, H=3, Dh=Dh, ps=ps), kv_fp8=True)
    dev = w.ctx_lens.device
    cu = torch.tensor(np.concatenate([[0], np.cumsum(nq)]), dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(13)
    q = torch.randn((int(cu[-1]), w.H, w.Dh), generator=gen, device=dev).to(torch.bfloat16)
    w.q[0], w.cu_seqlens_q = q, cu
    ws = torch.empty(B.fm_cross_attention_workspace_size(w.bs, w.H, w.Dh, 16, w.pool_dtype), dtype=torch.uint8,
                     device=dev)
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws, pool_dtype=w.pool_dtype)
    out = torch.full_like(q, float("nan"))
    B.fm_paged_cross_attention(q, w.q_norm_w[0], w.pools[0], w.page_table, w.ctx_lens, cu, w.softmax_scale,
                               w.theta, w.eps, ws, out=out)
    torch.cuda.synchronize()
    reqs = list(range(w.bs))
    pk, pv, rows = compact_context(w, 0, reqs)
    ref = oracle_cross(w, 0, reqs, pk, pv, rows, q=q)
    compare(rows_of(w, reqs, out), np.concatenate([ref[b] for b in reqs]), f"cross e4m3 ps{ps} Dh{Dh}")
    assert torch.all(out[:16] == 0), "an empty context must give exactly zero"
    assert ws_error_word(ws) == 0


def test_fp8_pool_write_and_step_small():
    log("e4m3 pool: write (commit rule, placement, rounding) and the step on it")
    w = make_workload(5, weights="random", scale_down=dict(bs=6, ctx=(20, 90), L=2, H=4, d_in=256), kv_fp8=True)
    buf = S.allocate(w)
    before = _snapshot(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    slots, keys, values = _write_oracle(w)
    _check_write(w, buf, before, slots, keys, values)
    _check_full_step_attention(w, buf, before, slots, keys, values, list(range(w.bs)))


def test_fp8_pool_deterministic():
    w = make_workload(2, weights="random", kv_fp8=True)
    buf = S.allocate(w)
    S.run_step(w, buf)
    first = buf.cross_out[0].clone()
    S.run_step(w, buf)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), buf.cross_out[0].view(torch.int16))


def test_fp8_pool_full_step_full_size():
    log("e4m3 pool: full draft step at full size (sampled requests)")
    w = make_workload(5, kv_fp8=True)
    buf = S.allocate(w)
    before = _snapshot(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    slots, keys, values = _write_oracle(w)
    _check_write(w, buf, before, slots, keys, values)
    reqs = _sample(w, 2, 6)
    log(f"  sampled requests {reqs}")
    _check_full_step_attention(w, buf, before, slots, keys, values, reqs)


@pytest.mark.parametrize("q_static", [True, False])
def test_fp8_pool_per_tensor_scales_small_step(q_static):
    # vLLM's calibrated fp8 cache: per-layer k/v scales in the write and as
    # descales in the attention, a fixed per-layer query scale (or, with
    # q_static False, sglang's per-(request, head) one with the k/v scales).
    log(f"e4m3 pool with per-tensor scales, static q scale: {q_static}")
    w = make_workload(5, weights="random", scale_down=dict(bs=6, ctx=(20, 90), L=2, H=4, d_in=256), kv_fp8=True)
    w.kv_scales = [(0.25, 0.5), (2.0, 0.125)]
    if q_static:
        w.q_scales = [1.0 / 64, 1.0 / 128]
    buf = S.allocate(w)
    before = _snapshot(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    slots, keys, values = _write_oracle(w)
    _check_write(w, buf, before, slots, keys, values)
    _check_full_step_attention(w, buf, before, slots, keys, values, list(range(w.bs)))


def test_fp8_pool_static_q_scale_saturates():
    # a fixed query scale small enough that q^ / scale passes 448: codes saturate
    log("e4m3 pool: static query scale with saturation")
    w = make_workload(3, weights="random", scale_down=dict(ctx_list=[40, 300, 1000], L=1, H=2), kv_fp8=True)
    w.q_scales = [1.0 / 512]
    buf = S.allocate(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    _check_attention(w, buf, list(range(w.bs)))


# ------------------------------------------------- rows of the K/V write
# sglang/model.py ``_write_context`` (fc, hidden_norm) and ``_anchor_kv_impl``
# (embedding, anchor_proj, anchor_norm).  The rows buffer is bf16: the write
# reads it as its x, so each stage is checked against the oracle from its own
# inputs.


def _oracle_rows(w, rows_idx=None, anchors=None):
    """Oracle rows for the given committed window rows and anchors."""
    up = w.upstream
    out = {}
    if rows_idx:
        out["hidden"] = O.context_input_rows(to_np(up.hidden[torch.as_tensor(rows_idx, device=up.hidden.device)]),
                                             to_np(up.w_fc), to_np(up.hidden_norm_w), w.eps)
    if anchors:
        ids = up.anchor_ids.cpu().numpy()[anchors]
        uniq, inv = np.unique(ids, return_inverse=True)
        emb = to_np(up.embedding[torch.as_tensor(uniq, device=up.embedding.device, dtype=torch.long)])
        out["anchor"] = O.anchor_input_rows(inv, emb, to_np(up.w_anchor_proj), to_np(up.b_anchor_proj),
                                            to_np(up.anchor_norm_w), w.eps)
    return out


def _committed_rows(w):
    wr = w.write
    cl = wr.commit_lens.cpu().numpy()
    return [b * wr.window + j for b in range(w.bs) for j in range(int(cl[b]))]


def test_context_rows_small_step():
    log("rows of the write: fc + hidden_norm, anchor_proj + anchor_norm, then the step")
    w = make_workload(5, weights="random", upstream=True,
                      scale_down=dict(bs=6, ctx=(20, 90), L=2, H=4, d_in=1024, n_aux=2, d_target=256, vocab=1000))
    buf = S.allocate(w)
    before = _snapshot(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    wr = w.write
    live = _committed_rows(w)
    n_win = w.bs * wr.window
    ref = _oracle_rows(w, live, list(range(w.bs)))
    compare(wr.x[torch.as_tensor(live, device=wr.x.device)], ref["hidden"], "rows: fc + hidden_norm")
    compare(wr.x[n_win:], ref["anchor"], "rows: anchor_proj + anchor_norm")
    skipped = sorted(set(range(n_win)) - set(live))
    assert skipped and torch.isnan(wr.x[torch.as_tensor(skipped, device=wr.x.device)].float()).all(), \
        "rows the commit rule skips must be left untouched"
    assert int(buf.rows_ws[4:8].view(torch.int32).item()) == 0
    slots, keys, values = _write_oracle(w)
    _check_write(w, buf, before, slots, keys, values)
    _check_full_step_attention(w, buf, before, slots, keys, values, list(range(w.bs)))


def test_context_rows_full_size_sampled():
    log("rows of the write at full size: 5 x 4096 -> 4096 (fc), vocab 151936 (sampled rows)")
    w = make_workload(5, upstream=True)
    buf = S.allocate(w)
    before = _snapshot(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    wr = w.write
    live = _committed_rows(w)
    rng = np.random.default_rng(21)
    pick = sorted(rng.choice(live, size=48, replace=False).tolist())
    ref = _oracle_rows(w, pick, list(range(w.bs)))
    compare(wr.x[torch.as_tensor(pick, device=wr.x.device)], ref["hidden"], "rows: fc + hidden_norm (48 rows)")
    compare(wr.x[w.bs * wr.window:], ref["anchor"], "rows: anchors (all 64)")
    slots, keys, values = _write_oracle(w)
    np.testing.assert_array_equal(buf.out_slots.cpu().numpy(), slots)
    reqs = _sample(w, 2, 7)
    _check_full_step_attention(w, buf, before, slots, keys, values, reqs)


def test_context_rows_edge_cases():
    # Nothing committed (the hidden rows are left as they were, the anchors
    # still computed), anchors only, and anchor ids outside [0, vocab) (read as
    # the clamped row, error bit 0 set).
    log("rows of the write: nothing committed; anchors only; out-of-vocabulary anchor ids")
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(41)
    bs, window, d_hidden, d_target, dim, vocab = 3, 16, 256, 128, 1024, 97
    hidden = torch.randn((bs * window, d_hidden), generator=gen, device=dev).to(torch.bfloat16)
    w_fc = (0.05 * torch.randn((dim, d_hidden), generator=gen, device=dev)).to(torch.bfloat16)
    g_h = 1 + 0.1 * torch.randn(dim, generator=gen, device=dev)
    emb = torch.randn((vocab, d_target), generator=gen, device=dev).to(torch.bfloat16)
    w_ap = (0.05 * torch.randn((dim, d_target), generator=gen, device=dev)).to(torch.bfloat16)
    b_ap = (0.1 * torch.randn(dim, generator=gen, device=dev)).to(torch.bfloat16)
    g_a = 1 + 0.1 * torch.randn(dim, generator=gen, device=dev)
    ids = torch.tensor([5, vocab - 1, 0], dtype=torch.int32, device=dev)
    ref = O.anchor_input_rows(ids.cpu().numpy(), to_np(emb), to_np(w_ap), to_np(b_ap), to_np(g_a), 1e-6)

    commit = torch.zeros(bs, dtype=torch.int32, device=dev)
    rows = torch.full((bs * window + bs, dim), float("nan"), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(B.fm_context_rows_workspace_size(bs * window, bs, d_hidden, d_target, dim), dtype=torch.uint8,
                     device=dev)
    B.fm_context_rows(hidden, w_fc, g_h, ids, emb, w_ap, b_ap, g_a, 1e-6, commit_lens=commit, window=window,
                      rows=rows, ws=ws)
    torch.cuda.synchronize()
    assert torch.isnan(rows[: bs * window].float()).all(), "no committed column: no hidden row is written"
    compare(rows[bs * window:], ref, "anchors, nothing committed")
    assert int(ws[4:8].view(torch.int32).item()) == 0

    only = B.fm_context_rows(None, None, None, ids, emb, w_ap, b_ap, g_a, 1e-6)
    torch.cuda.synchronize()
    compare(only, ref, "anchors only")

    bad = torch.tensor([5, vocab + 3, -2], dtype=torch.int32, device=dev)
    ws3 = torch.zeros(B.fm_context_rows_workspace_size(0, 3, 0, d_target, dim), dtype=torch.uint8, device=dev)
    out = B.fm_context_rows(None, None, None, bad, emb, w_ap, b_ap, g_a, 1e-6, ws=ws3)
    torch.cuda.synchronize()
    assert int(ws3[4:8].view(torch.int32).item()) & 1, "an id outside the vocabulary sets error bit 0"
    clamped = np.clip(bad.cpu().numpy(), 0, vocab - 1)
    compare(out, O.anchor_input_rows(clamped, to_np(emb), to_np(w_ap), to_np(b_ap), to_np(g_a), 1e-6),
            "out-of-range ids read the clamped rows")


def test_prefill_in_chunks():
    # a prefill of 4100 rows (two full chunks of 2048 and a ragged one) of one
    # request: the pool against the oracle's write of the oracle's rows (rounded
    # to bf16, the rows buffer's type)
    log("prefill: 4100 rows in chunks of 2048")
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(31)
    n, d_hidden, dim, L, H, Dh, ps = 4100, 512, 1024, 2, 4, 128, 16
    n_pages = math.ceil(n / ps) + 5
    hidden = torch.randn((n, d_hidden), generator=gen, device=dev).to(torch.bfloat16)
    w_fc = (0.05 * torch.randn((dim, d_hidden), generator=gen, device=dev)).to(torch.bfloat16)
    g_h = 1 + 0.1 * torch.randn(dim, generator=gen, device=dev)
    w_kv = (0.03 * torch.randn((L * 2 * H * Dh, dim), generator=gen, device=dev)).to(torch.bfloat16)
    k_norm_w = 1 + 0.1 * torch.randn((L, Dh), generator=gen, device=dev)
    perm = torch.randperm(n_pages, generator=gen, device=dev).to(torch.int32)
    page_table = perm[: math.ceil(n / ps)][None, :].contiguous()
    pools = [B.KVPool(torch.zeros((n_pages, H, ps, Dh), dtype=torch.bfloat16, device=dev).permute(0, 2, 1, 3),
                      torch.zeros((n_pages, H, ps, Dh), dtype=torch.bfloat16, device=dev).permute(0, 2, 1, 3))
             for _ in range(L)]
    positions = torch.arange(n, dtype=torch.int32, device=dev)
    row_req = torch.zeros(n, dtype=torch.int32, device=dev)
    out_slots = torch.empty(n, dtype=torch.int32, device=dev)
    S.write_prefill(hidden, positions, row_req, page_table, pools, w_fc, g_h, w_kv, k_norm_w, 1e-6, 1e6,
                    out_slots=out_slots)
    torch.cuda.synchronize()
    rows = O.round_to_bfloat16(O.context_input_rows(to_np(hidden), to_np(w_fc), to_np(g_h), 1e-6))
    slots, keys, values = O.write_context_kv(rows, to_np(w_kv), to_np(k_norm_w), np.zeros(n, dtype=np.int64),
                                             np.arange(n), page_table.cpu().numpy(), ps, L, H, Dh, 1e-6, 1e6)
    np.testing.assert_array_equal(out_slots.cpu().numpy(), slots)
    for l in range(L):
        sl = torch.as_tensor(slots, device=dev, dtype=torch.long)
        compare(pools[l].k[sl // ps, sl % ps], keys[:, l], f"prefill K L{l}")
        compare(pools[l].v[sl // ps, sl % ps], values[:, l], f"prefill V L{l}")



# ------------------------------------------------------- the DiT blocks
# sglang/model.py ``_denoise``: modulated LayerNorms, the projections with
# gated residuals, the GELU MLP, around the two attentions.


@pytest.mark.parametrize("M,K,N", [(300, 512, 2048), (1024, 1024, 16384), (37, 4096, 1024), (1, 64, 1024),
                                   (257, 512, 1024)])
def test_linear_epilogues(M, K, N):
    _check_linear(M, K, N)


@pytest.mark.parametrize("case", range(8))
def test_linear_seeded_shapes(case):
    # Seeded shapes: any row count (partial last tiles, waves of padding rows),
    # contractions that split into ranges or not, and widths 1024..4096 (the
    # entry point takes N in multiples of 1024).
    rng = np.random.default_rng(300 + case)
    _check_linear(int(rng.integers(1, 700)), 64 * int(rng.integers(1, 33)), 1024 * int(rng.integers(1, 5)))


def _check_linear(M, K, N):
    log(f"fm_linear M={M} K={K} N={N} (ranges: {B.fm_linear_workspace_size(M, N, K) > 0})")
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(M + K + N)
    x = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=gen, device=dev) / math.sqrt(K)).to(torch.bfloat16)
    b = (0.1 * torch.randn(N, generator=gen, device=dev)).to(torch.bfloat16)
    gate = 0.3 * torch.randn(N, generator=gen, device=dev)
    h0 = torch.randn((M, N), generator=gen, device=dev)
    y = B.fm_linear(x, w)
    yg = B.fm_linear(x, w, b, B.FM_LINEAR_GELU_BF16)
    ya = B.fm_linear(x, w, b, B.FM_LINEAR_ASSIGN_F32)
    h = h0.clone()
    B.fm_linear(x, w, b, B.FM_LINEAR_RESIDUAL, gate=gate, out=h)
    torch.cuda.synchronize()
    ref = to_np(x) @ to_np(w).T
    compare(y, ref, "linear bf16")
    compare(yg, O.gelu(ref + to_np(b)), "linear + bias + gelu")
    compare(ya, ref + to_np(b), "linear + bias (fp32)", max_abs=1e-3, mean_abs=1e-4)
    compare(h, to_np(h0) + to_np(gate) * (ref + to_np(b)), "gated residual (fp32)", max_abs=1e-3, mean_abs=1e-4)


def test_ada_layer_norm():
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    for dim in (1024, 4096):
        h = 2 * torch.randn((77, dim), generator=gen, device=dev) + 5.0   # a large mean: the two-pass variance
        sc = 1 + 0.1 * torch.randn(dim, generator=gen, device=dev)
        sh = 0.1 * torch.randn(dim, generator=gen, device=dev)
        out = B.fm_ada_layer_norm(h, sc, sh, 1e-6)
        torch.cuda.synchronize()
        compare(out, O.ada_layer_norm(to_np(h), to_np(sc), to_np(sh), 1e-6), f"ada layer norm dim {dim}")


def _oracle_dit_layer(w, buf, l, h_in, reqs):
    """Oracle DiT block on the rows of requests ``reqs`` from the GPU's own
    residual stream, with the attentions reading the GPU-written pools."""
    K, H, Dh, nc = w.K, w.H, w.Dh, w.n_cand
    rows = np.concatenate([np.arange(b * nc * K, (b + 1) * nc * K) for b in reqs])
    blocks = [b * nc + i for b in reqs for i in range(nc)]
    pk, pv, pt_rows = compact_context(w, l, reqs)
    ctx = w.ctx_lens.cpu().numpy()
    bctx = w.block_ctx_lens.cpu().numpy()[blocks]
    width = max([len(r) for r in pt_rows] + [1])
    pt = np.zeros((len(reqs), width), dtype=np.int64)
    for i, r in enumerate(pt_rows):
        pt[i, :len(r)] = r
    cu = np.arange(len(reqs) + 1) * nc * K
    fp8 = w.fp8_scales(l)
    sc = {} if fp8 is None else dict(q_scale=fp8[0] or None, k_scale=fp8[1], v_scale=fp8[2])

    def self_attention(qkv):
        o = O.block_self_attention(qkv.reshape(len(blocks), K, 3, H, Dh), to_np(w.self_q_norm_w[l]),
                                   to_np(w.self_k_norm_w[l]), bctx, w.softmax_scale, w.theta, w.eps)
        return o.reshape(len(rows), H * Dh)

    def cross_attention(q):
        o = O.paged_cross_attention(q.reshape(len(rows), H, Dh), to_np(w.q_norm_w[l]), pk, pv, pt, ctx[reqs], cu,
                                    w.page_size, w.softmax_scale, w.theta, w.eps,
                                    kv_e4m3=w.pool_dtype == torch.float8_e4m3fn, **sc)
        return o.reshape(len(rows), H * Dh)

    lw = {k: to_np(v) for k, v in w.dit.layers[l].items()}
    mod = {k: to_np(v) for k, v in w.dit.mods[l].items()}
    return rows, O.dit_layer(h_in[rows], mod, lw, self_attention, cross_attention, w.eps)


def _compare_stream(gpu, ref, what):
    """The fp32 residual stream against the oracle.  Every operand a
    projection takes is rounded once to bf16 (relative error up to 2^-9), and
    fc2 contracts 16384 such GELU outputs, so the stream's error scales with
    the magnitude of the values carried: the bar is the bf16 bar times the
    stream's RMS (at least 1)."""
    s = max(1.0, float(np.sqrt(np.mean(np.asarray(ref, dtype=np.float64) ** 2))))
    log(f"  {what}: stream RMS {s:.2f}")
    compare(gpu, ref, what, max_abs=2e-2 * s, mean_abs=2e-3 * s)


def _run_dit_stagewise(w, buf):
    """The step with the residual stream captured around every block."""
    if w.write is not None:
        S.write_context(w, buf)
    S.plan(w, buf)
    S.dit_embed(w, buf)
    hs = [buf.dit["h"].clone()]
    for l in range(w.L):
        S.dit_layer(w, buf, l)
        hs.append(buf.dit["h"].clone())
    S.dit_final(w, buf)
    torch.cuda.synchronize()
    return [to_np(h) for h in hs]


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_dit_step_small(kv_fp8):
    log(f"DiT blocks around the attentions, small step (e4m3 pool: {kv_fp8})")
    w = make_workload(5, weights="random", dit=True, kv_fp8=kv_fp8,
                      scale_down=dict(bs=4, ctx=(20, 300), L=2, H=8, d_in=1024, d_target=512))
    buf = S.allocate(w)
    hs = _run_dit_stagewise(w, buf)
    d = w.dit
    ref0 = to_np(d.embedded) @ to_np(d.w_xe).T + to_np(d.b_xe)
    compare(hs[0], ref0, "x_embed (fp32)", max_abs=1e-3, mean_abs=1e-4)
    reqs = list(range(w.bs))
    for l in range(w.L):
        rows, ref = _oracle_dit_layer(w, buf, l, hs[l], reqs)
        _compare_stream(hs[l + 1][rows], ref, f"DiT block {l}: residual stream")
    compare(buf.dit["out"], O.ada_layer_norm(hs[-1], to_np(d.final_scale), to_np(d.final_shift), w.eps),
            "final modulated LayerNorm")
    assert ws_error_word(buf.cross_ws) == 0


def test_dit_step_full_size_sampled():
    log("DiT blocks at full size (64 requests, 5 layers, dim 4096, MLP 16384): block 0 on sampled requests")
    w = make_workload(5, dit=True)
    buf = S.allocate(w)
    hs = _run_dit_stagewise(w, buf)
    reqs = _sample(w, 2, 8)
    log(f"  sampled requests {reqs}")
    rows, ref = _oracle_dit_layer(w, buf, 0, hs[0], reqs)
    _compare_stream(hs[1][rows], ref, "DiT block 0: residual stream (sampled)")
    d = w.dit
    compare(buf.dit["out"][torch.as_tensor(rows, device=buf.dit["out"].device)],
            O.ada_layer_norm(hs[-1][rows], to_np(d.final_scale), to_np(d.final_shift), w.eps), "final LayerNorm")


def test_binding_refuses_mismatched_extents():
    # The C ABI takes bare pointers; the binding checks every extent it passes
    # (nothing is launched for these calls).
    dev = torch.device("cuda")
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((1024, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="out must have shape"):
        B.fm_linear(x, w, out=torch.empty((4, 1024), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError, match="bias must have shape"):
        B.fm_linear(x, w, torch.zeros(512, dtype=torch.bfloat16, device=dev))
    h = torch.zeros((3, 1024), device=dev)
    with pytest.raises(ValueError, match="scale must have shape"):
        B.fm_ada_layer_norm(h, torch.ones(512, device=dev), torch.zeros(1024, device=dev), 1e-6)
    q = torch.zeros((16, 4, 64), dtype=torch.bfloat16, device=dev)
    pool = B.KVPool(torch.zeros((4, 16, 2, 64), dtype=torch.bfloat16, device=dev),
                    torch.zeros((4, 16, 2, 64), dtype=torch.bfloat16, device=dev))
    one = torch.ones(1, dtype=torch.int32, device=dev)
    ws = torch.zeros(B.fm_cross_attention_workspace_size(1, 4, 64), dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="pool holds"):
        B.fm_paged_cross_attention(q, torch.ones(64, device=dev), pool, torch.zeros((1, 4), dtype=torch.int32,
                                   device=dev), one, torch.tensor([0, 16], dtype=torch.int32, device=dev),
                                   0.125, 1e6, 1e-6, ws)
    qkv = torch.zeros((2, 16, 3, 4, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="ctx_lens must have shape"):
        B.fm_block_self_attention(qkv, torch.ones(64, device=dev), torch.ones(64, device=dev), one, 0.125, 1e6, 1e-6)


@pytest.mark.parametrize("ps", [16, 4])
def test_bad_page_ids_are_skipped_and_flagged(ps):
    # Page-table entries outside [0, num_pages) (too large or negative): the
    # tokens of that page are skipped and bit 0 of the workspace error word is
    # set (the C ABI's device-side index checks); every other token and
    # request is computed as usual.  Page size 16 reads page ids through the
    # scalar cache, 4 through the per-wave window.
    log(f"page-table entries outside the pool, page size {ps}: tokens skipped, error bit set")
    ctx = [40, 70, 33, 90]
    w = make_workload(3, weights="random", scale_down=dict(ctx_list=ctx, L=1, H=2, Dh=128, ps=ps))
    dev = w.ctx_lens.device
    n_pages = w.pools[0].k.shape[0]
    bad = {1: (2, n_pages + 7), 2: (0, -3)}  # request -> (logical page, out-of-range id)
    pt = w.page_table.clone()
    for b, (j, v) in bad.items():
        pt[b, j] = v
    ws = torch.zeros(B.fm_cross_attention_workspace_size(w.bs, w.H, w.Dh, 16), dtype=torch.uint8, device=dev)
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws)
    out = torch.full_like(w.q[0], float("nan"))
    B.fm_paged_cross_attention(w.q[0], w.q_norm_w[0], w.pools[0], pt, w.ctx_lens, w.cu_seqlens_q, w.softmax_scale,
                               w.theta, w.eps, ws, out=out)
    torch.cuda.synchronize()
    assert ws_error_word(ws) & 1, "an out-of-range page id sets error bit 0"
    # expected: each request's context without the bad page's tokens (oracle steps)
    q, qnw = to_np(w.q[0]), to_np(w.q_norm_w[0])
    pk, pv = to_np(w.pools[0].k), to_np(w.pools[0].v)
    good_pt = w.page_table.cpu().numpy()
    cu = w.cu_seqlens_q.cpu().numpy()
    ref = np.zeros(q.shape)
    for b, n in enumerate(ctx):
        pages = good_pt[b][: -(-n // ps)]
        kb = pk[pages].reshape(-1, w.H, w.Dh)[:n]
        vb = pv[pages].reshape(-1, w.H, w.Dh)[:n]
        keep = np.ones(n, dtype=bool)
        if b in bad:
            j = bad[b][0]
            keep[j * ps:(j + 1) * ps] = False
        r0, r1 = cu[b], cu[b + 1]
        positions = n + np.arange(r1 - r0) % 16
        for h in range(w.H):
            qh = O.apply_rope(O.rms_norm(q[r0:r1, h], qnw, w.eps), positions, w.theta)
            ref[r0:r1, h] = O.attention(qh, kb[keep, h], vb[keep, h], w.softmax_scale)
    compare(out, ref, f"cross-attention with bad page ids, ps {ps}")


def test_write_skips_rows_of_bad_pages():
    # A row whose page-table entry lies outside the pool is not written (its
    # slot reads -1) and sets error bit 0; the other rows land as usual.
    log("write: rows on an out-of-range page are skipped and flagged")
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(51)
    L, H, Dh, ps, d_in, n_pages = 1, 2, 128, 16, 256, 6
    n = 40  # positions 0..39 of one request: pages 0, 1, 2 of its row
    x = torch.randn((n, d_in), generator=gen, device=dev).to(torch.bfloat16)
    w_kv = (0.05 * torch.randn((L * 2 * H * Dh, d_in), generator=gen, device=dev)).to(torch.bfloat16)
    knw = 1 + 0.1 * torch.randn((L, Dh), generator=gen, device=dev)
    pt = torch.tensor([[3, n_pages + 2, 1]], dtype=torch.int32, device=dev)  # logical page 1 is outside the pool
    sentinel = -7.0
    pools = [B.KVPool(torch.full((n_pages, ps, H, Dh), sentinel, dtype=torch.bfloat16, device=dev),
                      torch.full((n_pages, ps, H, Dh), sentinel, dtype=torch.bfloat16, device=dev))]
    row_req = torch.zeros(n, dtype=torch.int32, device=dev)
    row_pos = torch.arange(n, dtype=torch.int32, device=dev)
    slots = torch.empty(n, dtype=torch.int32, device=dev)
    ws = torch.zeros(B.fm_write_context_kv_workspace_size(n), dtype=torch.uint8, device=dev)
    B.fm_write_context_kv(x, w_kv, knw, row_req, row_pos, pt, pools, 1e-6, 1e6, out_slots=slots, ws=ws)
    torch.cuda.synchronize()
    assert ws_error_word(ws) & 1, "a row on an out-of-range page sets error bit 0"
    got = slots.cpu().numpy()
    want = np.array([3 * ps + p if p < 16 else (-1 if p < 32 else 1 * ps + p - 32) for p in range(n)])
    np.testing.assert_array_equal(got, want)
    live = np.nonzero(want >= 0)[0]
    s_, keys, values = O.write_context_kv(to_np(x)[live], to_np(w_kv), to_np(knw), np.zeros(len(live), np.int64),
                                          live, np.array([[3, 0, 1]]), ps, L, H, Dh, 1e-6, 1e6)
    kk = pools[0].k.reshape(-1, H, Dh)
    vv = pools[0].v.reshape(-1, H, Dh)
    sl = torch.as_tensor(want[live], device=dev, dtype=torch.long)
    compare(kk[sl], keys[:, 0], "keys of the rows on valid pages")
    compare(vv[sl], values[:, 0], "values of the rows on valid pages")
    untouched = np.setdiff1d(np.arange(n_pages * ps), want[live])
    assert (kk[torch.as_tensor(untouched, device=dev)].float() == sentinel).all(), "no other slot is written"


def test_cross_attention_with_a_plan_for_other_sizes():
    # A plan made with another max_q (or other shapes) computes nothing but the
    # zero rows of empty contexts and sets bit 2 of the error word.
    log("cross-attention called with a plan made for another max_q")
    ctx = [40, 0, 70]
    w = make_workload(3, weights="random", scale_down=dict(ctx_list=ctx, L=1, H=2, Dh=128, ps=16))
    dev = w.ctx_lens.device
    ws = torch.zeros(B.fm_cross_attention_workspace_size(w.bs, w.H, w.Dh, 32), dtype=torch.uint8, device=dev)
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws, max_q=16)
    out = torch.full_like(w.q[0], float("nan"))
    B.fm_paged_cross_attention(w.q[0], w.q_norm_w[0], w.pools[0], w.page_table, w.ctx_lens, w.cu_seqlens_q,
                               w.softmax_scale, w.theta, w.eps, ws, out=out, max_q=32)
    torch.cuda.synchronize()
    assert ws_error_word(ws) & 4, "a plan for other sizes sets error bit 2"
    cu = w.cu_seqlens_q.cpu().numpy()
    for b, n in enumerate(ctx):
        rows = out[cu[b]:cu[b + 1]].float()
        if n == 0:
            assert (rows == 0).all(), "empty contexts still get their zero rows"
        else:
            assert torch.isnan(rows).all(), "nothing else is written"
    # planned again with the call's max_q, the same call computes and clears nothing else
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws, max_q=32)
    B.fm_paged_cross_attention(w.q[0], w.q_norm_w[0], w.pools[0], w.page_table, w.ctx_lens, w.cu_seqlens_q,
                               w.softmax_scale, w.theta, w.eps, ws, out=out, max_q=32)
    torch.cuda.synchronize()
    assert ws_error_word(ws) == 0
    reqs = list(range(w.bs))
    pk, pv, rows = compact_context(w, 0, reqs)
    ref = oracle_cross(w, 0, reqs, pk, pv, rows)
    compare(rows_of(w, reqs, out), np.concatenate([ref[b] for b in reqs]), "cross-attention after planning again")


def test_plan_records_head_dim_and_pool_type():
    # The plan header records Dh and the pool type.  A call with another Dh
    # (whose workspace layout differs past the header) or another pool type
    # computes nothing, sets bit 2 and leaves the plan's records intact, so a
    # later call that matches the plan still computes the right result.
    log("cross-attention with a plan made for another head dim or pool type")
    ctx = [40, 0, 300]
    w64 = make_workload(3, weights="random", scale_down=dict(ctx_list=ctx, L=1, H=2, Dh=64, ps=16))
    w128 = make_workload(3, weights="random", scale_down=dict(ctx_list=ctx, L=1, H=2, Dh=128, ps=16), seed=77)
    dev = w64.ctx_lens.device
    n = max(B.fm_cross_attention_workspace_size(3, 2, D, 16) for D in (64, 128))
    ws = torch.zeros(n, dtype=torch.uint8, device=dev)
    B.fm_plan_cross_attention(w64.ctx_lens, 2, 64, ws)
    out = torch.full_like(w128.q[0], float("nan"))
    B.fm_paged_cross_attention(w128.q[0], w128.q_norm_w[0], w128.pools[0], w128.page_table, w128.ctx_lens,
                               w128.cu_seqlens_q, w128.softmax_scale, w128.theta, w128.eps, ws, out=out)
    torch.cuda.synchronize()
    assert ws_error_word(ws) & 4, "a plan for another head dim sets error bit 2"
    cu = w128.cu_seqlens_q.cpu().numpy()
    for b, c in enumerate(ctx):
        rows = out[cu[b]:cu[b + 1]].float()
        assert (rows == 0).all() if c == 0 else torch.isnan(rows).all()
    # the Dh = 64 plan is still whole: its own call computes the right rows
    ws[4:8].zero_()
    out64 = B.fm_paged_cross_attention(w64.q[0], w64.q_norm_w[0], w64.pools[0], w64.page_table, w64.ctx_lens,
                                       w64.cu_seqlens_q, w64.softmax_scale, w64.theta, w64.eps, ws)
    torch.cuda.synchronize()
    assert ws_error_word(ws) == 0
    reqs = list(range(3))
    pk, pv, rows = compact_context(w64, 0, reqs)
    ref = oracle_cross(w64, 0, reqs, pk, pv, rows)
    compare(rows_of(w64, reqs, out64), np.concatenate([ref[b] for b in reqs]), "Dh 64 after a Dh 128 call")
    # a bf16 plan (same sizes) serving an fp32 call
    w1 = make_workload(1)
    ws1 = torch.zeros(B.fm_cross_attention_workspace_size(1, w1.H, w1.Dh, 16), dtype=torch.uint8, device=dev)
    B.fm_plan_cross_attention(w1.ctx_lens, w1.H, w1.Dh, ws1, pool_dtype=torch.bfloat16)
    out1 = torch.full_like(w1.q[0], float("nan"))
    B.fm_paged_cross_attention(w1.q[0], w1.q_norm_w[0], w1.pools[0], w1.page_table, w1.ctx_lens, w1.cu_seqlens_q,
                               w1.softmax_scale, w1.theta, w1.eps, ws1, out=out1)
    torch.cuda.synchronize()
    assert ws_error_word(ws1) & 4, "a plan for another pool type sets error bit 2"
    assert torch.isnan(out1).all(), "nothing is computed"


def test_plan_xcd_weights():
    # The plan's per-XCD weights move the cut points and nothing else: the
    # default weights given explicitly reproduce the default plan bit for bit;
    # skewed weights give the oracle's result, and the same bits on every call.
    log("cross-attention planned with explicit XCD weights")
    w = make_workload(2, weights="random")  # 8 requests: most pairs are cut between waves
    dev = w.ctx_lens.device
    ws = torch.zeros(B.fm_cross_attention_workspace_size(w.bs, w.H, w.Dh, 16), dtype=torch.uint8, device=dev)

    def call():
        return B.fm_paged_cross_attention(w.q[0], w.q_norm_w[0], w.pools[0], w.page_table, w.ctx_lens,
                                          w.cu_seqlens_q, w.softmax_scale, w.theta, w.eps, ws).clone()

    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws)
    base = call()
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws, xcd_weights=[1045, 955] * 4)
    assert torch.equal(call(), base), "the default weights, given explicitly, are the default plan"
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws, xcd_weights=[700, 1300, 900, 1100, 1000, 1000, 1500, 500])
    a, b = call(), call()
    torch.cuda.synchronize()
    assert ws_error_word(ws) == 0
    assert torch.equal(a, b), "one plan, one result"
    reqs = list(range(w.bs))
    pk, pv, rows = compact_context(w, 0, reqs)
    ref = oracle_cross(w, 0, reqs, pk, pv, rows)
    compare(rows_of(w, reqs, a), np.concatenate([ref[b] for b in reqs]), "cross-attention, skewed XCD weights")


def test_timed_cross_attention():
    # The timed call computes the untimed call's bits, and every wave with
    # tiles records its XCD, its tile count and a loop time that moves forward;
    # the counts add up to the plan's tile stream.
    log("cross-attention with its waves timed")
    w = make_workload(2, weights="random")
    dev = w.ctx_lens.device
    ws = torch.zeros(B.fm_cross_attention_workspace_size(w.bs, w.H, w.Dh, 16), dtype=torch.uint8, device=dev)
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws)
    args = (w.q[0], w.q_norm_w[0], w.pools[0], w.page_table, w.ctx_lens, w.cu_seqlens_q, w.softmax_scale, w.theta,
            w.eps, ws)
    base = B.fm_paged_cross_attention(*args).clone()
    waves = torch.cuda.get_device_properties(0).multi_processor_count * 4
    clock = torch.zeros((waves, 4), dtype=torch.int64, device=dev)
    timed = B.fm_paged_cross_attention(*args, wave_clock=clock)
    torch.cuda.synchronize()
    assert torch.equal(timed, base)
    r = clock.cpu().numpy()
    live = r[:, 3] > 0
    assert live.sum() > 0
    assert (r[live, 1] > r[live, 0]).all()
    assert ((r[live, 2] >= 0) & (r[live, 2] < 8)).all()
    total = sum((int(c) + 15) // 16 for c in w.ctx_lens.cpu().tolist()) * w.H
    assert int(r[:, 3].sum()) == total
    with pytest.raises(B.FmError):
        B.fm_paged_cross_attention(*args, wave_clock=clock[: waves // 2])


def test_cross_attention_after_lengths_shrank_flags_bit1():
    # Lengths shortened after the plan so that a wave's planned share runs past
    # the last tile: every request after the first emptied, so the waves that
    # cross out of request 0 find no tiles left.  The outputs are unspecified,
    # nothing outside the buffers is touched, and bit 1 of the error word is
    # set; planning again gives the right result.  (Many more tiles than
    # waves, so that shares cross from one request into the next.)
    log("cross-attention with lengths shortened after the plan")
    ctx = [1500, 1200, 1800, 1500, 900, 1650, 1400, 1100]
    w = make_workload(3, weights="random", scale_down=dict(ctx_list=ctx, L=1, H=32, Dh=128, ps=16))
    dev = w.ctx_lens.device
    ws = torch.zeros(B.fm_cross_attention_workspace_size(w.bs, w.H, w.Dh, 16), dtype=torch.uint8, device=dev)
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws)
    shorter = torch.zeros_like(w.ctx_lens)
    shorter[0] = w.ctx_lens[0]
    out = torch.empty_like(w.q[0])
    B.fm_paged_cross_attention(w.q[0], w.q_norm_w[0], w.pools[0], w.page_table, shorter, w.cu_seqlens_q,
                               w.softmax_scale, w.theta, w.eps, ws, out=out)
    torch.cuda.synchronize()
    assert ws_error_word(ws) & 2, "a share running past the last tile sets error bit 1"
    w.ctx_lens = shorter
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws)
    B.fm_paged_cross_attention(w.q[0], w.q_norm_w[0], w.pools[0], w.page_table, w.ctx_lens, w.cu_seqlens_q,
                               w.softmax_scale, w.theta, w.eps, ws, out=out)
    torch.cuda.synchronize()
    assert ws_error_word(ws) == 0
    reqs = list(range(w.bs))
    pk, pv, rows = compact_context(w, 0, reqs)
    ref = oracle_cross(w, 0, reqs, pk, pv, rows)
    compare(rows_of(w, reqs, out), np.concatenate([ref[b] for b in reqs]), "cross-attention after planning again")


@pytest.mark.parametrize("kind,ps", [("bf16", 16), ("bf16", 4), ("fp32", 16), ("e4m3", 16), ("e4m3", 1)])
def test_one_fragment_query_rows_and_other_plan(kind, ps):
    # The one-fragment kernels norm and rotate their query rows themselves and
    # write the zero rows of empty contexts: ragged row counts (a request with
    # no rows, one with one), empty and sub-tile contexts; then a plan made for
    # two fragments, which leaves only those zero rows and sets error bit 2.
    log(f"one-fragment query rows, {kind} pool, page size {ps}")
    ctx = [0, 1, 15, 0, 300, 1000, 0]
    nq = [16, 1, 16, 5, 0, 9, 16]
    sd = dict(ctx_list=ctx, L=1, H=3, Dh=128, ps=ps)
    if kind == "fp32":
        sd["dtype"] = torch.float32
    w = make_workload(3, weights="random", scale_down=sd, kv_fp8=kind == "e4m3", seed=31)
    dev = w.ctx_lens.device
    cu = torch.tensor(np.concatenate([[0], np.cumsum(nq)]), dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(17)
    q = torch.randn((int(cu[-1]), w.H, w.Dh), generator=gen, device=dev).to(w.q[0].dtype)
    w.q[0], w.cu_seqlens_q = q, cu
    ws = torch.zeros(B.fm_cross_attention_workspace_size(w.bs, w.H, w.Dh, 32, w.pool_dtype), dtype=torch.uint8,
                     device=dev)
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws, max_q=16, pool_dtype=w.pool_dtype)
    out = torch.full_like(q, float("nan"))
    B.fm_paged_cross_attention(q, w.q_norm_w[0], w.pools[0], w.page_table, w.ctx_lens, cu, w.softmax_scale,
                               w.theta, w.eps, ws, out=out, max_q=16)
    torch.cuda.synchronize()
    assert ws_error_word(ws) == 0
    reqs = list(range(w.bs))
    pk, pv, rows = compact_context(w, 0, reqs)
    ref = oracle_cross(w, 0, reqs, pk, pv, rows, q=q)
    compare(rows_of(w, reqs, out), np.concatenate([ref[b] for b in reqs]), f"one-fragment cross {kind} ps{ps}")
    cuh = cu.cpu().numpy()
    for b, n in enumerate(ctx):
        if n == 0:
            assert (out[cuh[b]:cuh[b + 1]] == 0).all(), "an empty context must give exactly zero"
    # a plan for two fragments: the one-fragment call computes nothing else
    B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws, max_q=32, pool_dtype=w.pool_dtype)
    out2 = torch.full_like(q, float("nan"))
    B.fm_paged_cross_attention(q, w.q_norm_w[0], w.pools[0], w.page_table, w.ctx_lens, cu, w.softmax_scale,
                               w.theta, w.eps, ws, out=out2, max_q=16)
    torch.cuda.synchronize()
    assert ws_error_word(ws) & 4, "a plan for other sizes sets error bit 2"
    for b, n in enumerate(ctx):
        r = out2[cuh[b]:cuh[b + 1]].float()
        if n == 0:
            assert (r == 0).all(), "empty contexts still get their zero rows"
        else:
            assert torch.isnan(r).all(), "nothing else is written"


@pytest.mark.parametrize("case", range(16))
def test_seeded_sweep_of_shapes(case):
    # Seeded draws over the combinations the parametrized tests above take one
    # at a time: page size, head dim, heads, layout, candidate blocks, pool
    # type, and a request mix of empty, sub-tile, tile-edge and long contexts.
    rng = np.random.default_rng(500 + case)
    ps = int(rng.choice([1, 4, 8, 16, 32, 64]))
    Dh = int(rng.choice([64, 128]))
    H = int(rng.choice([1, 2, 3, 5, 8]))
    n_cand = int(rng.choice([1, 2, 4]))
    fp8 = bool(rng.integers(2))
    layout = str(rng.choice(["head_major", "token_major"]))
    bs = int(rng.integers(1, 10))
    ctx = [int(rng.choice([0, 1, 15, 16, 17, 63, 64, 65])) if rng.random() < 0.4 else int(rng.integers(1, 3000))
           for _ in range(bs)]
    log(f"sweep {case}: ps {ps} Dh {Dh} H {H} candidates {n_cand} e4m3 {fp8} {layout} ctx {ctx}")
    w = make_workload(3, weights="random", layout=layout, n_cand=n_cand, kv_fp8=fp8,
                      scale_down=dict(ctx_list=ctx, L=1, H=H, Dh=Dh, ps=ps), seed=900 + case)
    buf = S.allocate(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    _check_attention(w, buf, list(range(w.bs)), self_blocks=range(w.bs * n_cand))
    rows = w.cu_seqlens_q.cpu().numpy()
    for b in range(w.bs):  # an empty context gives exactly zero
        if ctx[b] == 0:
            assert torch.count_nonzero(buf.cross_out[0][int(rows[b]):int(rows[b + 1])]) == 0


@pytest.mark.parametrize("bs", [2048, 2100])
def test_plan_many_requests(bs):
    # The plan keeps per-request tables in LDS up to 2048 requests and reads
    # them back from the workspace beyond: both sides of that line, with
    # short, empty and tile-edge contexts, on sampled requests.
    rng = np.random.default_rng(bs)
    ctx = [int(rng.choice([0, 1, 16, 17])) if rng.random() < 0.2 else int(rng.integers(1, 120)) for _ in range(bs)]
    log(f"plan over {bs} requests")
    w = make_workload(3, weights="random", scale_down=dict(ctx_list=ctx, L=1, H=2, Dh=64, ps=16), seed=bs)
    buf = S.allocate(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    assert ws_error_word(buf.cross_ws) == 0
    reqs = sorted(set([0, 1, bs // 2, bs - 2, bs - 1] + [int(x) for x in rng.choice(bs, 40, replace=False)]))
    _check_attention(w, buf, reqs, self_blocks=reqs)
    rows = w.cu_seqlens_q.cpu().numpy()
    empty = [b for b in range(bs) if ctx[b] == 0]
    assert max(empty) > 1024  # requests past the first wave stride
    for b in empty:  # every empty context gives exactly zero
        assert torch.count_nonzero(buf.cross_out[0][int(rows[b]):int(rows[b + 1])]) == 0


@pytest.mark.parametrize("case", range(8))
def test_seeded_sweep_of_writes(case):
    # Seeded draws of the write's shape: request count and commits (so the
    # live rows end anywhere inside a 256-row tile and its 64-row waves),
    # layers, heads, d_in and pool type; then the step's attention on the
    # written pool.
    rng = np.random.default_rng(700 + case)
    bs = int(rng.integers(1, 40))
    L = int(rng.integers(1, 4))
    H = int(rng.choice([1, 2, 3, 4]))
    d_in = int(rng.choice([64, 192, 256, 512]))
    fp8 = bool(rng.integers(2))
    log(f"write sweep {case}: bs {bs} L {L} H {H} d_in {d_in} e4m3 {fp8}")
    w = make_workload(5, weights="random", kv_fp8=fp8, seed=1700 + case,
                      scale_down=dict(bs=bs, ctx=(20, 400), L=L, H=H, d_in=d_in))
    buf = S.allocate(w)
    before = _snapshot(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    slots, keys, values = _write_oracle(w)
    log(f"  live rows {int((slots >= 0).sum())} of {slots.shape[0]}")
    _check_write(w, buf, before, slots, keys, values)
    _check_full_step_attention(w, buf, before, slots, keys, values, list(range(w.bs)))
