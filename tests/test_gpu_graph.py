"""HIP graph replay of the draft step: every entry point on the path takes
its buffers from the caller, launches on the caller's stream and neither
allocates nor synchronises, so one step can be captured in a graph and
replayed.  Each replay must reproduce the eager step bit for bit (the
kernels are deterministic); between replays the outputs are poisoned and
ordinary eager work runs."""

from __future__ import annotations

import pytest
import torch

from harness import log, ws_error_word

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU machines
    pytest.skip("needs a GPU", allow_module_level=True)

from block_diffusion_drafter_all_amd import step as S  # noqa: E402
from block_diffusion_drafter_all_amd.workloads import make_workload  # noqa: E402

SMALL = dict(bs=6, ctx=(20, 90), L=2, H=4, d_in=256)
CASES = {
    "attention": dict(scale_down=SMALL),
    "e4m3_pool": dict(scale_down=SMALL, kv_fp8=True),
    "upstream_rows": dict(upstream=True, scale_down=dict(bs=6, ctx=(20, 90), L=2, H=4, d_in=1024, n_aux=2,
                                                         d_target=256, vocab=1000)),
    "dit_blocks": dict(dit=True, scale_down=dict(bs=4, ctx=(20, 300), L=2, H=8, d_in=1024, d_target=512)),
    "full_draft_step": dict(),
}


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _outputs(w, buf):
    """(tensor, rows compared or None for all) of every output the step writes."""
    outs = [(t, None) for t in list(buf.cross_out) + list(buf.self_out)]
    if buf.out_slots is not None:
        outs.append((buf.out_slots, None))
    if w.upstream is not None:  # the write's rows: committed window rows and the anchors
        wr = w.write
        cl = wr.commit_lens.cpu().tolist()
        rows = [b * wr.window + j for b in range(w.bs) for j in range(int(cl[b]))]
        rows += list(range(w.bs * wr.window, wr.x.shape[0]))
        outs.append((wr.x, torch.as_tensor(rows, device=wr.x.device)))
    if buf.dit is not None:
        outs += [(buf.dit["out"], None), (buf.dit["h"], None)]
    return outs


def _poison(outs):
    for t, rows in outs:
        if rows is not None:
            t.index_fill_(0, rows, float("nan"))
        elif t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


def _take(t, rows):
    return t if rows is None else t.index_select(0, rows)


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32) if t.element_size() == 4 else t


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replay_matches_eager(case):
    log(f"graph replay of the step: {case}")
    w = make_workload(5, weights="random", **CASES[case])
    buf = S.allocate(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    outs = _outputs(w, buf)
    ref = [_take(t, rows).clone() for t, rows in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        S.run_step(w, buf)  # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        S.run_step(w, buf)
    torch.cuda.synchronize()

    scratch = torch.randn(1 << 20, device="cuda")
    for replay in range(3):
        _poison(outs)
        scratch.mul_(0.5).add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, ((t, rows), want) in enumerate(zip(outs, ref)):
            got = _take(t, rows)
            assert torch.equal(_bits(got), _bits(want)), f"replay {replay}: output {i} differs from the eager step"
        assert ws_error_word(buf.cross_ws) == 0
    del graph


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_graph_replay_reads_new_inputs(kv_fp8):
    # A serving loop captures once and updates the inputs in place: new query
    # rows and shorter context lengths (the plan is rebuilt on the device from
    # the lengths at every replay).  Each replay must equal an eager step on
    # the same inputs, bit for bit.
    log(f"graph replay over inputs updated in place (e4m3 pool: {kv_fp8})")
    w = make_workload(5, weights="random", scale_down=SMALL, kv_fp8=kv_fp8)
    buf = S.allocate(w)
    S.run_step(w, buf)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        S.run_step(w, buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        S.run_step(w, buf)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda")
    for replay in range(3):
        gen.manual_seed(40 + replay)
        for q in w.q:
            q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(q.dtype))
        shrink = torch.randint(0, 9, w.ctx_lens.shape, generator=gen, device="cuda", dtype=torch.int32)
        w.ctx_lens.copy_(torch.clamp(w.ctx_lens - shrink, min=0))
        torch.cuda.synchronize()
        S.run_step(w, buf)
        torch.cuda.synchronize()
        ref = [t.clone() for t in buf.cross_out]
        for t in buf.cross_out:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for l, (got, want) in enumerate(zip(buf.cross_out, ref)):
            assert torch.equal(_bits(got), _bits(want)), f"replay {replay}: layer {l} differs from the eager step"
        assert ws_error_word(buf.cross_ws) == 0
    del graph
