"""Benchmark of the FlashMap draft-step attention path on one MI355X.

A step is one pass of the whole path over one batch: the context/anchor K/V
write (one GEMM over every layer's weight, k-norm, RoPE, paged scatter that
skips uncommitted columns), the cross-attention plan, and for every layer the
block self-attention and the paged cross-attention.  The default workload is
the full draft step: 64 requests, context lengths U[1024, 8192], block 16,
5 layers, 32 heads x 128, page size 16, bf16 pool; each request commits
U{1..17} verify columns plus its anchor through the write.  ``--kv-fp8``
runs the same step over an e4m3 pool (bf16 activations).

Prints ONE JSON line (see the fields below).  Inputs are resident in HBM
before timing starts; timing brackets exactly --steps steps with device
synchronization on both sides.  The steps are timed twice: first as eager
launches, with events around every cross-attention call (the roofline's
figures), then as --steps replays of one step captured in a HIP graph, which
give ``value`` (``--no-graph``: the eager figure instead).  Both passes run
the same kernels on the same buffers.

Two helper modes feed the ``roofline.traffic`` field (HBM bytes per
cross-attention launch from rocprofv3's FETCH_SIZE / WRITE_SIZE counters):
  --copy-calibration      one plain 1 GiB device-to-device copy, the known-size
                          kernel the counters are scaled by;
  --write-traffic DIRS    (CPU only) turns four counter-collection outputs
                          into an entry of profiles/cross_attention_traffic.json
                          for the workload the other options name, keyed by a
                          hash of the kernel sources: the bench reports the
                          traffic only for that workload and only while the
                          sources still match.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft query rows/s over paged context + achieved KV-read HBM GB/s (% of peak)"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "cross_attention_traffic.json")
# Sources whose code the cross-attention launch runs; a change in any of them
# invalidates counters taken before it.
KERNEL_SOURCES = ("cross_attention.hip", "fm_device.h", "fm_internal.h", "abi.cpp")
CROSS_KERNELS = ("cross_attn_kernel", "q_prologue_kernel")
COPY_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5],
                    help="workload: 5 = full draft step (default); 3 = attention of 5 layers; 2, 4, 1")
    ap.add_argument("--layout", default="head_major", choices=["head_major", "token_major"])
    ap.add_argument("--candidates", type=int, default=1, choices=[1, 2, 4],
                    help="candidate blocks per request (tree drafting): 16 query rows each, one context read")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="e4m3 KV pool (written at scale 1; queries quantized per request and head)")
    ap.add_argument("--dit", action="store_true",
                    help="the whole one-jump draft step: x_embed, every DiT block (modulated LayerNorms, "
                         "projections, gated residuals, GELU MLP) around the two attentions, the final norm")
    ap.add_argument("--upstream", action="store_true",
                    help="config 5: make the write's rows on the device from the target hidden states (fc + "
                         "hidden_norm) and the anchor tokens (embedding + anchor_proj + anchor_norm) in the step")
    ap.add_argument("--flush-mall", action="store_true",
                    help="before each timed step, read a 1 GiB scratch buffer (untimed) so the step starts with "
                         "a cold MALL; ms_per_step is then the mean of the per-step events")
    ap.add_argument("--no-graph", action="store_true",
                    help="report the eager launches' time as value.  By default one step is also captured in a HIP "
                         "graph and --steps replays of it give value; the eager pass (first) still gives the "
                         "per-call events of the roofline and is reported under \"eager\"")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-xcd-calibration", action="store_true",
                    help="plan with the library's default XCD weights instead of weights measured on this box on "
                         "the attention kernel itself (its waves timed) before the timed steps")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the sweep that also times the cross-attention of workloads 1, 2 (warm and with the "
                         "MALL flushed), 3 and 4 in the same run (reported under \"configs\")")
    ap.add_argument("--config-steps", type=int, default=10,
                    help="timed steps of each workload of the sweep (after 3 untimed ones)")
    ap.add_argument("--cpu-configs", action="store_true",
                    help="also time the oracle on a sample of each workload of the sweep")
    ap.add_argument("--cpu-sample-requests", type=int, default=0,
                    help="requests in the oracle's timed sample (0 = 24, about 10-20 s of CPU work)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--write-traffic", nargs=4, metavar=("CROSS_FETCH", "CROSS_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc output directories: write the traffic record and exit (no GPU)")
    ap.add_argument("--traffic-command", default="", help="the commands that produced --write-traffic's inputs")
    return ap.parse_args()


def kernel_sources_hash() -> str:
    """SHA-256 of the attention kernel's sources and of the build script that
    sets their compiler flags."""
    h = hashlib.sha256()
    paths = [os.path.join(ROOT, "block_diffusion_drafter_all_amd", "csrc", n) for n in KERNEL_SOURCES]
    paths.append(os.path.join(ROOT, "block_diffusion_drafter_all_amd", "build.py"))
    for path in paths:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()


def _counter_rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _kib_per_dispatch(rows, match):
    """Mean counter value (KiB) per dispatch of kernels whose name contains ``match``, and the count."""
    per = {}
    for r in rows:
        if match in r["Kernel_Name"]:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return (sum(per.values()) / len(per), len(per)) if per else (0.0, 0)


def workload_key(args) -> str:
    """Names the workload a traffic record was measured on."""
    return (f"config={args.config},layout={args.layout},candidates={args.candidates},"
            f"kv={'e4m3' if args.kv_fp8 else 'activation-type'}" + (",upstream" if args.upstream else "")
            + (",dit" if args.dit else ""))


def _traffic_records() -> dict:
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return {}
    return data.get("records", {}) if isinstance(data, dict) else {}


def write_traffic(dirs, command: str, key: str) -> None:
    cross_fetch, cross_write, copy_fetch, copy_write = (_counter_rows(d) for d in dirs)
    # the calibration copy: the largest copy dispatch of the run
    def largest(rows):
        best = {}
        for r in rows:
            if "copy" in r["Kernel_Name"].lower():
                best[r["Dispatch_Id"]] = best.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        return max(best.values())
    fetch_scale = COPY_BYTES / (largest(copy_fetch) * 1024.0)
    write_scale = COPY_BYTES / (largest(copy_write) * 1024.0)
    rec = {"workload": key, "sources_sha256": kernel_sources_hash(), "kernels": {}, "fetch_scale": fetch_scale,
           "write_scale": write_scale, "calibration": f"plain {COPY_BYTES} B device copy (bench.py --copy-calibration)",
           "command": command}
    fetch = write = 0.0
    for k in CROSS_KERNELS:
        fk, n = _kib_per_dispatch(cross_fetch, k)
        wk, _ = _kib_per_dispatch(cross_write, k)
        rec["kernels"][k] = {"dispatches": n, "FETCH_SIZE_KiB": fk, "WRITE_SIZE_KiB": wk}
        fetch += fk * 1024.0 * fetch_scale
        write += wk * 1024.0 * write_scale
    rec["fetch_bytes_per_launch"] = fetch
    rec["write_bytes_per_launch"] = write
    rec["traffic_bytes_per_launch"] = fetch + write
    records = _traffic_records()
    records[key] = rec
    with open(TRAFFIC_FILE, "w") as f:
        json.dump({"records": records}, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec))


def measured_traffic(key: str):
    """HBM bytes per cross-attention launch from the committed counter record
    of workload ``key``, or None when there is none or the kernel sources
    changed since it was taken."""
    rec = _traffic_records().get(key)
    if rec is None or rec.get("sources_sha256") != kernel_sources_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cpu() -> dict:
    """The host's processor as lscpu describes it, and the cores this process
    may run on."""
    info = {"model_name": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count()}
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        keep = ("Model name", "Vendor ID", "CPU family", "Model", "Stepping", "Socket(s)", "Core(s) per socket",
                "Thread(s) per core", "CPU(s)", "CPU max MHz")
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() in keep:
                info["lscpu " + k.strip()] = v.strip()
    except (OSError, ValueError):
        pass
    return info


def oracle_threads() -> int:
    """Threads for the oracle's BLAS: every core this process may run on,
    within the CPU share the environment sets (OMP_NUM_THREADS)."""
    cores = len(os.sched_getaffinity(0))
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        share = 0
    return min(cores, share) if share > 0 else cores


def hbm_ceilings() -> dict:
    """Context for the HBM figures: torch's plain 1 GiB device-to-device copy,
    bytes read + written per second, best of 5 after one warm-up."""
    import torch

    src = torch.ones((COPY_BYTES // 2,), dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1))
    return {"torch_copy_GBps": 2 * COPY_BYTES / (min(t) * 1e-3) / 1e9, "copy_bytes": COPY_BYTES}


def _probe_lib():
    import ctypes

    from block_diffusion_drafter_all_amd.build import PROBE_LIB_PATH

    if not os.path.exists(PROBE_LIB_PATH):
        raise SystemExit(f"{PROBE_LIB_PATH} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.fm_probe_stream_read.restype = ctypes.c_int
    lib.fm_probe_stream_read.argtypes = [vp, sz, ctypes.c_int32, vp, ctypes.POINTER(sz), vp]
    lib.fm_probe_tile_gather.restype = ctypes.c_int
    lib.fm_probe_tile_gather.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp]
    lib.fm_probe_tile_gather_timed.restype = ctypes.c_int
    lib.fm_probe_tile_gather_timed.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp,
                                               vp]
    return lib


class MallFlush:
    """Evicts the step's data from the MALL (256 MB) before a timed step: one
    streaming read of a 1 GiB buffer (the probe library's read kernel).  The
    flush only reads, so it leaves clean lines behind: a flush that also wrote
    its buffer would leave up to 256 MB of dirty lines, whose write-back to
    HBM would then share the bandwidth with the timed step's reads."""

    def __init__(self):
        import ctypes

        import torch

        self._lib = _probe_lib()
        self._buf = torch.ones((COPY_BYTES // 4,), dtype=torch.int32, device="cuda")
        self._sink = torch.empty(2048 * 64, dtype=torch.int32, device="cuda")
        self._n = ctypes.c_size_t(0)

    def __call__(self):
        import ctypes

        import torch

        if self._lib.fm_probe_stream_read(self._buf.data_ptr(), self._buf.numel() * 4, 2048, self._sink.data_ptr(),
                                          ctypes.byref(self._n), torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("fm_probe_stream_read failed")


def _best_rate(launch, nbytes: float, reps: int = 5) -> float:
    """GB/s of the fastest of ``reps`` timed launches (one untimed first)."""
    import torch

    launch()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        launch()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    return nbytes / (best * 1e-3) / 1e9


def tile_offsets(w, layer: int):
    """Byte offsets (int64, on the device) of the K/V tiles one cross-attention
    call of ``w`` reads, in the plan's order: (request, head) pairs, then
    16-token tiles in position order.  None unless a tile is one contiguous run
    (pages of at least 16 tokens in the head-major layout)."""
    import torch

    k = w.pools[layer].k
    s = k.element_size()
    if w.page_size < 16 or k.stride(1) * s != w.Dh * s:
        return None
    page_b, slot_b, head_b = k.stride(0) * s, k.stride(1) * s, k.stride(2) * s
    pt = w.page_table.to(torch.int64)
    out = []
    for b, c in enumerate(w.ctx_lens.cpu().tolist()):
        n = (c + 15) // 16
        if n == 0:
            continue
        t = torch.arange(n, device=pt.device) * 16
        base = pt[b, t // w.page_size] * page_b + (t % w.page_size) * slot_b
        out.append((torch.arange(w.H, device=pt.device)[:, None] * head_b + base[None, :]).reshape(-1))
    return torch.cat(out)


def probe_ceilings(w, n_waves: int) -> dict:
    """What the memory system delivers on this machine: a streaming read of 4 GiB,
    and the tiles one cross-attention call of ``w`` reads, gathered in the
    plan's order over the plan's number of waves with no arithmetic (layer 0's
    pool).  Both best of 5."""
    import ctypes

    import torch

    lib = _probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    buf = torch.ones((1 << 32) // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(4096 * 64, dtype=torch.int32, device="cuda")
    nread = ctypes.c_size_t(0)

    def read():
        if lib.fm_probe_stream_read(buf.data_ptr(), buf.numel() * 4, 2048, sink.data_ptr(), ctypes.byref(nread),
                                    stream) != 0:
            raise RuntimeError("fm_probe_stream_read failed")

    read()
    out["stream_read_GBps"] = _best_rate(read, float(nread.value))
    out["stream_read_bytes"] = int(nread.value)
    del buf
    off = tile_offsets(w, 0)
    if off is not None:
        tb = 16 * w.Dh * w.pools[0].k.element_size()
        pk, pv = w.pools[0].k, w.pools[0].v

        def gather():
            if lib.fm_probe_tile_gather(pk.data_ptr(), pv.data_ptr(), off.data_ptr(), off.numel(), tb, n_waves,
                                        sink.data_ptr(), stream) != 0:
                raise RuntimeError("fm_probe_tile_gather failed")

        out["tile_gather_GBps"] = _best_rate(gather, float(off.numel()) * 2 * tb)
        out["tile_gather"] = (f"{off.numel()} K/V tile pairs of {tb} B (layer 0's call), {n_waves} waves, "
                              f"plan order, no arithmetic")
    return out


def xcd_calibration(w, reps: int = 3, rounds: int = 2) -> dict | None:
    """Weights of the plan's wave shares by XCD for this box, measured on the
    attention kernel itself: layer 0's cross-attention call is run timed
    (fm_paged_cross_attention_timed), every wave's loop time per tile is
    averaged by XCD, and an XCD's weight is proportional to its rate (tiles per
    unit time), normalised to a mean of 1000 and clamped to [800, 1200].  The
    first round plans with the library's default weights, the next with the
    weights measured so far; the per-tile times of all rounds are averaged."""
    import torch

    from block_diffusion_drafter_all_amd import binding as B

    nw = 4096  # records for the most waves a plan has; waves without tiles leave theirs at zero
    ws = torch.zeros(B.fm_cross_attention_workspace_size(w.bs, w.H, w.Dh, w.max_q, w.pool_dtype), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(w.q[0])
    clock = torch.zeros((nw, 4), dtype=torch.int64, device="cuda")
    per_tile = [[] for _ in range(8)]
    weights = None
    n_timed = 0
    for _ in range(rounds):
        B.fm_plan_cross_attention(w.ctx_lens, w.H, w.Dh, ws, max_q=w.max_q, pool_dtype=w.pool_dtype,
                                  xcd_weights=weights)
        for rep in range(reps + 1):
            clock.zero_()
            B.fm_paged_cross_attention(w.q[0], w.q_norm_w[0], w.pools[0], w.page_table, w.ctx_lens, w.cu_seqlens_q,
                                       w.softmax_scale, w.theta, w.eps, ws, out=out, max_q=w.max_q,
                                       fp8_scales=w.fp8_scales(0), wave_clock=clock)
            torch.cuda.synchronize()
            if rep == 0:
                continue  # untimed first run
            recs = [r for r in clock.cpu().tolist() if r[3] > 0]
            n_timed = len(recs)
            for t0, t1, xcd, tiles in recs:
                per_tile[int(xcd) % 8].append((t1 - t0) / tiles)
        if any(not v for v in per_tile):
            return None
        t = [sum(v) / len(v) for v in per_tile]
        rate = [1.0 / x for x in t]
        mean_rate = sum(rate) / 8
        weights = [int(round(min(1200.0, max(800.0, 1000.0 * r / mean_rate)))) for r in rate]
    return {"xcd_weights": weights, "xcd_us_per_tile": [round(x * 0.01, 4) for x in t],
            "xcd_calibration": (f"layer 0's cross-attention call timed per wave ({n_timed} waves with tiles), "
                                f"{rounds} rounds of {reps} timed calls")}


def copy_calibration() -> None:
    import torch

    src = torch.full((COPY_BYTES,), 7, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "ok": bool(dst[-1].item() == 7)}), flush=True)


def kv_bytes_per_row(L: int, H: int, Dh: int, elem_bytes: int) -> int:
    """Bytes one context row's keys and values take in every layer's pool."""
    return L * 2 * H * Dh * elem_bytes


def cross_bytes(w) -> int:
    """Algorithmic bytes of one cross-attention call: every context key and
    value read once, the queries read and the outputs written once, the page
    ids, lengths, cu_seqlens and the norm weight."""
    s = w.dtype.itemsize          # queries and outputs
    skv = w.pool_dtype.itemsize   # pool elements
    ctx = w.ctx_lens.cpu().tolist()
    kv = sum(ctx) * w.H * w.Dh * 2 * skv
    qo = 2 * w.total_q * w.H * w.Dh * s
    pages = 4 * sum(math.ceil(c / w.page_size) for c in ctx)
    return kv + qo + pages + 4 * (2 * w.bs + 1) + 4 * w.Dh


def cross_flops(w) -> int:
    ctx = w.ctx_lens.cpu().tolist()
    cu = w.cu_seqlens_q.cpu().tolist()
    return sum(4 * (cu[b + 1] - cu[b]) * ctx[b] * w.H * w.Dh for b in range(w.bs))


def write_flops_bytes(w):
    import torch

    wr = w.write
    if wr is None:
        return 0, 0
    n_rows, d_in = wr.x.shape
    pos = wr.row_pos.cpu()
    live = pos >= 0
    if wr.commit_lens is not None:
        cl = wr.commit_lens.cpu()
        r = torch.arange(n_rows)
        win = r < w.bs * wr.window
        col = r % wr.window
        b = torch.clamp(r // wr.window, max=w.bs - 1)
        live &= ~(win & (col >= cl[b]))
    m = int(live.sum())
    s = wr.x.element_size()
    n = w.L * 2 * w.H * w.Dh
    flops = 2 * m * d_in * n
    nbytes = (s * (n * d_in + m * d_in) + m * kv_bytes_per_row(w.L, w.H, w.Dh, w.pool_dtype.itemsize)
              + 4 * w.L * w.Dh + 12 * n_rows)
    return flops, nbytes


def context_rows_flops(w) -> int:
    """MFMA flops of fm_context_rows: fc over the committed window rows and
    anchor_proj over the anchors."""
    up = w.upstream
    if up is None:
        return 0
    live = int(w.write.commit_lens.sum().item())
    dim = up.w_fc.shape[0]
    return 2 * live * up.hidden.shape[1] * dim + 2 * up.anchor_ids.shape[0] * up.embedding.shape[1] * dim


def dit_linear_flops(w) -> int:
    """MFMA flops of one step's DiT projections (x_embed and, per layer,
    qkv, q, the two o_proj, fc1, fc2)."""
    d = w.dit
    if d is None:
        return 0
    rows, dim = d.embedded.shape[0], w.H * w.Dh
    inter = d.layers[0]["fc1"].shape[0]
    per_layer = 2 * rows * dim * (3 * dim + 3 * dim + 2 * inter)
    return w.L * per_layer + 2 * rows * d.embedded.shape[1] * dim


def describe(w) -> dict:
    ctx = w.ctx_lens.cpu().tolist()
    d = {
        "workload": {1: "tiny fp32 step (1 request, ctx 64, 4 x 64)",
                     2: "one-layer bf16 step (8 requests, ctx U[512,2048])",
                     3: "all-layers attention step (64 requests, ctx U[1024,8192], 5 layers)",
                     4: "long skewed batch (256 lognormal + one 131072-token request)",
                     5: "full draft step: context write + 5-layer attention (64 requests, ctx U[1024,8192])"}[
            w.workload_id],
        "requests": w.bs, "block_size": w.K, "candidate_blocks": w.n_cand, "layers": w.L, "heads": w.H,
        "head_dim": w.Dh,
        "page_size": w.page_size, "total_context_tokens": int(sum(ctx)), "pool_layout": w.meta["layout"],
        "kv_pool": {1: "e4m3", 2: "bf16", 4: "fp32"}[w.pool_dtype.itemsize],
    }
    if w.write is not None:
        d["write_rows"] = int(w.write.x.shape[0])
        d["write_d_in"] = int(w.write.x.shape[1])
    if w.dit is not None:
        d["dit"] = {"dim": w.H * w.Dh, "mlp": int(w.dit.layers[0]["fc1"].shape[0]),
                    "x_embed_in": int(w.dit.embedded.shape[1])}
    if w.upstream is not None:
        d["upstream"] = {"hidden_width": int(w.upstream.hidden.shape[1]), "vocab": int(w.upstream.embedding.shape[0]),
                         "dim": int(w.upstream.w_fc.shape[0])}
    return d


def cpu_baseline_inputs(w, n_req: int) -> dict:
    """Host copies (float32, exact for the bf16 / e4m3 / fp32 values) of what
    the oracle needs for a bounded sample of ``w``'s step: ``n_req`` requests'
    write rows, and per layer their self-attention blocks, query rows and
    context pages."""
    import numpy as np
    import torch

    import oracle as O

    def host(t):
        return t.detach().to(torch.float32).cpu().numpy()

    rng = np.random.default_rng(0)
    reqs = sorted(rng.choice(w.bs, size=min(n_req, w.bs), replace=False).tolist())
    ps = w.page_size
    pages = []
    for l in range(w.L):
        ids, rows, at = [], [], 0
        for b in reqs:
            n = math.ceil(int(w.ctx_lens[b]) / ps)
            ids.append(w.page_table[b, :n].long())
            rows.append(np.arange(at, at + n))
            at += n
        idx = torch.cat(ids)
        pages.append((host(w.pools[l].k[idx]), host(w.pools[l].v[idx]), rows))
    wr_in = None
    if w.write is not None:
        wr = w.write
        row_req = wr.row_req.cpu().numpy()
        sel = np.nonzero(np.isin(row_req, reqs))[0]
        cl = None if wr.commit_lens is None else wr.commit_lens.cpu().numpy()
        live = O.live_rows(len(wr.row_pos), wr.row_pos.cpu().numpy(), cl, wr.window)[sel]
        keep = sel[np.nonzero(live)[0]]
        wr_in = dict(x=host(wr.x[torch.as_tensor(keep, device=wr.x.device)]), w=host(wr.w_kv), kn=host(wr.k_norm_w),
                     pos=wr.row_pos.cpu().numpy()[keep], req=row_req[keep], pt=w.page_table.cpu().numpy())
    blocks = [b * w.n_cand + i for b in reqs for i in range(w.n_cand)]   # candidate blocks of the sample
    return dict(
        reqs=reqs, bs=w.bs, L=w.L, H=w.H, Dh=w.Dh, ps=ps, eps=w.eps, theta=w.theta, scale=w.softmax_scale,
        e4m3=w.pool_dtype.itemsize == 1, pages=pages, write=wr_in, cu=w.cu_seqlens_q.cpu().numpy(),
        ctx=w.ctx_lens.cpu().numpy(), q=[host(w.q[l]) for l in range(w.L)],
        q_norm=[host(w.q_norm_w[l]) for l in range(w.L)],
        qkv=[host(w.qkv[l][torch.as_tensor(blocks, device=w.qkv[l].device)]) for l in range(w.L)],
        self_q=[host(w.self_q_norm_w[l]) for l in range(w.L)], self_k=[host(w.self_k_norm_w[l]) for l in range(w.L)],
        block_ctx=w.block_ctx_lens.cpu().numpy()[blocks])


def cpu_baseline_run(smp: dict) -> dict:
    """Time the oracle (as it stands) on a sample from cpu_baseline_inputs:
    the sampled requests' write rows, then for every layer their
    self-attention blocks and their cross-attention rows."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle as O

    cores = oracle_threads()
    reqs, cu, ctx = smp["reqs"], smp["cu"], smp["ctx"]
    with threadpool_limits(limits=cores):
        blas = [i.get("num_threads") for i in threadpool_info()]
        t0 = time.perf_counter()
        wr = smp["write"]
        if wr is not None:
            O.write_context_kv(wr["x"], wr["w"], wr["kn"], wr["req"], wr["pos"], wr["pt"], smp["ps"], smp["L"],
                               smp["H"], smp["Dh"], smp["eps"], smp["theta"])
        for l in range(smp["L"]):
            O.block_self_attention(smp["qkv"][l], smp["self_q"][l], smp["self_k"][l], smp["block_ctx"], smp["scale"],
                                   smp["theta"], smp["eps"])
            pk, pv, rows = smp["pages"][l]
            for i, b in enumerate(reqs):
                O.paged_cross_attention(smp["q"][l][cu[b]:cu[b + 1]], smp["q_norm"][l], pk, pv, rows[i][None, :],
                                        [ctx[b]], [0, cu[b + 1] - cu[b]], smp["ps"], smp["scale"], smp["theta"],
                                        smp["eps"], kv_e4m3=smp["e4m3"])
        dt = time.perf_counter() - t0
    rows = sum(int(cu[b + 1] - cu[b]) for b in reqs) * smp["L"]
    return {"value": rows / dt, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": (f"{len(reqs)} of {smp['bs']} requests (ids {reqs}): their written rows and, for all "
                       f"{smp['L']} layers, their self-attention blocks and cross-attention rows; {dt:.1f} s wall; "
                       f"numpy fp64, BLAS threads {blas}"),
            "seconds": dt, "cpu_model": cpu_model(), "host": host_cpu()}


def plan_waves(pool_dtype) -> int:
    """Resident cross-attention waves the plan cuts for (CUs x 4 SIMDs x the
    pool type's waves per SIMD, at most 4096)."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return min(cus * 4 * (2 if pool_dtype == torch.float8_e4m3fn else 1), 4096)


def time_attention(w, steps: int, warmup: int, flush_mall: bool, warm_seconds: float = 0.3,
                   xcd_weights=None) -> dict:
    """The attention step of ``w`` (plan, then per layer self- and
    cross-attention), ``steps`` timed steps with events around every step and
    every cross-attention call; with ``flush_mall`` a 1 GiB buffer is read
    (untimed, between the events) before each step.  Untimed steps run first,
    at least ``warmup`` of them and at least ``warm_seconds`` of them, so the
    timed ones do not see clocks still ramping after an idle stretch."""
    import torch

    from block_diffusion_drafter_all_amd import binding as B
    from block_diffusion_drafter_all_amd import step as S

    buf = S.allocate(w)
    buf.xcd_weights = xcd_weights
    flush = MallFlush() if flush_mall else None
    E = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))  # noqa: E731

    def step(ev=None):
        S.plan(w, buf)
        for l in range(w.L):
            B.fm_block_self_attention(w.qkv[l], w.self_q_norm_w[l], w.self_k_norm_w[l], w.block_ctx_lens,
                                      w.softmax_scale, w.theta, w.eps, out=buf.self_out[l])
            if ev is not None:
                ev["cross"][l][0].record()
            B.fm_paged_cross_attention(w.q[l], w.q_norm_w[l], w.pools[l], w.page_table, w.ctx_lens,
                                       w.cu_seqlens_q, w.softmax_scale, w.theta, w.eps, buf.cross_ws,
                                       out=buf.cross_out[l], max_q=w.max_q, fp8_scales=w.fp8_scales(l))
            if ev is not None:
                ev["cross"][l][1].record()

    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < warm_seconds:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [dict(step=E(), cross=[E() for _ in range(w.L)]) for _ in range(steps)]
    for s in range(steps):
        if flush is not None:
            flush()
        evs[s]["step"][0].record()
        step(evs[s])
        evs[s]["step"][1].record()
    torch.cuda.synchronize()
    step_ms = sorted(e["step"][0].elapsed_time(e["step"][1]) for e in evs)
    cross_ms = [c[0].elapsed_time(c[1]) for e in evs for c in e["cross"]]
    first_ms = [e["cross"][0][0].elapsed_time(e["cross"][0][1]) for e in evs]
    avg_cross = sum(cross_ms) / len(cross_ms)
    nbytes = cross_bytes(w)
    rows = w.total_q * w.L
    mean_step = sum(step_ms) / len(step_ms)
    res = {"steps": steps, "step_ms_mean": mean_step, "step_ms_p50": step_ms[len(step_ms) // 2],
           "rows_per_s": rows / (mean_step * 1e-3), "cross_avg_ms": avg_cross,
           "cross_first_layer_avg_ms": sum(first_ms) / len(first_ms), "bytes_per_launch": nbytes,
           "mall": "flushed before each step" if flush_mall else "warm (data left by the previous step)"}
    per_call = avg_cross
    if not flush_mall:
        # Calls whose kernels take less than the host needs to launch them leave
        # launch gaps inside per-call events; calls enqueued back to back give
        # the device's own time per call (the last layer's call, its plan kept).
        n = 20
        e0, e1 = E()
        e0.record()
        for _ in range(n):
            B.fm_paged_cross_attention(w.q[-1], w.q_norm_w[-1], w.pools[-1], w.page_table, w.ctx_lens,
                                       w.cu_seqlens_q, w.softmax_scale, w.theta, w.eps, buf.cross_ws,
                                       out=buf.cross_out[-1], max_q=w.max_q, fp8_scales=w.fp8_scales(w.L - 1))
        e1.record()
        torch.cuda.synchronize()
        res["cross_back_to_back_ms"] = e0.elapsed_time(e1) / n
        per_call = min(per_call, res["cross_back_to_back_ms"])
    res["kv_read_GBps"] = nbytes / (per_call * 1e-3) / 1e9
    res["frac"] = res["kv_read_GBps"] / HBM_PEAK_GBPS
    res["frac_basis"] = ("per-call events (each call after a MALL flush)" if flush_mall else
                         "the shorter of per-call events and back-to-back calls")
    return res


def sweep_configs(args, xcd_weights=None) -> dict:
    """The cross-attention of workloads 1, 2 (warm and MALL-flushed), 3 and 4,
    timed in this run with the main workload's pool options (and its plan
    weights: the XCDs' rates are the box's, not the workload's)."""
    import torch

    from block_diffusion_drafter_all_amd.workloads import make_workload

    res, samples = {}, {}
    for name, cid, flush in (("1", 1, False), ("2_warm", 2, False), ("2_flushed", 2, True), ("3", 3, False),
                             ("4", 4, False)):
        if cid == 1 and (args.kv_fp8 or args.candidates != 1):
            continue  # the tiny workload is fp32, one block per request
        print(f"[bench] timing workload {name}", file=sys.stderr, flush=True)
        w = make_workload(cid, layout=args.layout, n_cand=args.candidates, kv_fp8=args.kv_fp8)
        torch.cuda.synchronize()
        r = {"workload": describe(w)}
        r.update(time_attention(w, args.config_steps, 3, flush, xcd_weights=xcd_weights))
        key = (f"config={cid},layout={args.layout},candidates={args.candidates},"
               f"kv={'e4m3' if args.kv_fp8 else 'activation-type'}")
        r["traffic"] = measured_traffic(key)
        if args.cpu_configs and not flush:
            samples[name] = cpu_baseline_inputs(w, min(w.bs, args.cpu_sample_requests or 24))
        res[name] = r
        del w
        torch.cuda.empty_cache()
    for name, smp in samples.items():  # the oracle after all of the sweep's GPU timing
        res[name]["cpu_baseline"] = cpu_baseline_run(smp)
    return res


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args.write_traffic, args.traffic_command, workload_key(args))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU; --gpus must be 1",
                          "requested_gpus": args.gpus}))
        sys.exit(2)
    import torch

    from block_diffusion_drafter_all_amd import step as S
    from block_diffusion_drafter_all_amd.workloads import make_workload

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.upstream and args.config != 5:
        raise SystemExit("--upstream applies to config 5 (the full draft step)")
    if args.dit and args.config != 5:
        raise SystemExit("--dit applies to config 5 (the full draft step)")
    w = make_workload(args.config, layout=args.layout, n_cand=args.candidates, kv_fp8=args.kv_fp8,
                      upstream=args.upstream, dit=args.dit)
    buf = S.allocate(w)
    calib = None if args.no_xcd_calibration else xcd_calibration(w)
    xcd_weights = None if calib is None else calib["xcd_weights"]
    buf.xcd_weights = xcd_weights
    torch.cuda.synchronize()

    def one_step(events=None):
        if w.upstream is not None:
            if events is not None:
                events["rows"][0].record()
            S.context_rows(w, buf)
            if events is not None:
                events["rows"][1].record()
        if w.write is not None:
            if events is not None:
                events["write"][0].record()
            S.write_kv(w, buf)
            if events is not None:
                events["write"][1].record()
        S.plan(w, buf)
        if w.dit is not None:
            def timed(kind, call):
                if events is None:
                    call()
                    return
                e0, e1 = E()
                e0.record()
                call()
                e1.record()
                events.setdefault(kind, []).append((e0, e1))
            timed("linear", lambda: S.dit_embed(w, buf))
            for l in range(w.L):
                S.dit_layer(w, buf, l, timed)
            timed("norm", lambda: S.dit_final(w, buf))
            return
        for l in range(w.L):
            if events is not None:
                events["self"][l][0].record()
            from block_diffusion_drafter_all_amd import binding as B
            B.fm_block_self_attention(w.qkv[l], w.self_q_norm_w[l], w.self_k_norm_w[l], w.block_ctx_lens,
                                      w.softmax_scale, w.theta, w.eps, out=buf.self_out[l])
            if events is not None:
                events["self"][l][1].record()
                events["cross"][l][0].record()
            B.fm_paged_cross_attention(w.q[l], w.q_norm_w[l], w.pools[l], w.page_table, w.ctx_lens,
                                       w.cu_seqlens_q, w.softmax_scale, w.theta, w.eps, buf.cross_ws,
                                       out=buf.cross_out[l], max_q=w.max_q, fp8_scales=w.fp8_scales(l))
            if events is not None:
                events["cross"][l][1].record()

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    # Timed region: exactly --steps steps.  Events bracket each cross-attention
    # call on the stream it is launched on (torch's current stream).
    E = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))  # noqa: E731
    n_pre = 0 if w.dit is not None else w.L   # the DiT step appends its own events per call
    per_step = [dict(step=E(), rows=E(), write=E(), self=[E() for _ in range(n_pre)],
                     cross=[E() for _ in range(n_pre)]) for _ in range(args.steps)]
    flush = MallFlush() if args.flush_mall else None
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        if flush is not None:
            flush()  # 1 GiB read: the MALL (256 MB) holds none of the step's data
        per_step[s]["step"][0].record()
        one_step(per_step[s])
        per_step[s]["step"][1].record()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_total = start.elapsed_time(end)
    step_ms = sorted(st["step"][0].elapsed_time(st["step"][1]) for st in per_step)
    ms_step = sum(step_ms) / len(step_ms) if flush is not None else ms_total / args.steps

    def pct(p):
        return step_ms[min(len(step_ms) - 1, int(round(p / 100 * (len(step_ms) - 1))))]

    cross_ms = [ev[0].elapsed_time(ev[1]) for st in per_step for ev in st["cross"]]
    self_ms = [ev[0].elapsed_time(ev[1]) for st in per_step for ev in st["self"]]
    write_ms = [st["write"][0].elapsed_time(st["write"][1]) for st in per_step] if w.write is not None else []
    rows_ms = [st["rows"][0].elapsed_time(st["rows"][1]) for st in per_step] if w.upstream is not None else []
    avg_cross = sum(cross_ms) / len(cross_ms)
    cb = cross_bytes(w)
    achieved = cb / (avg_cross * 1e-3) / 1e9
    rows = w.total_q * w.L
    out = {
        "metric": METRIC,
        "value": rows / (ms_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # activations; over an e4m3 pool QK^T runs on fp8 MFMA and PV on bf16
        "dtype": ("bf16" if w.dtype == torch.bfloat16 else "f32") + ("+e4m3-kv" if args.kv_fp8 else ""),
        "data": "synthetic (seeded; shapes and distributions of the drafting workload)",
        "config": describe(w),
        "roofline": {"bound": "hbm",
                     "kernel": ("fm_paged_cross_attention (cross_attn_kernel"
                                + (", after q_prologue_kernel)" if args.candidates > 1 else ")")),
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(workload_key(args)), "bytes_per_launch": cb,
                     "avg_launch_ms": avg_cross},
        "step_ms": {"p10": pct(10), "p50": pct(50), "p90": pct(90), "mall": "flushed" if flush is not None else "warm"},
        "kv_read_GBps": achieved,
        "kv_read_pct_peak": 100.0 * achieved / HBM_PEAK_GBPS,
        "attention_rows_per_s": rows / (sum(cross_ms + self_ms) / args.steps * 1e-3),
        "self_attention_avg_ms": sum(self_ms) / len(self_ms),
        "wall_s_timed": t_wall,
    }
    if write_ms:
        wf, wb = write_flops_bytes(w)
        avg_w = sum(write_ms) / len(write_ms)
        out["write"] = {"avg_ms": avg_w, "flops": wf, "tflops": wf / (avg_w * 1e-3) / 1e12,
                        "mfma_frac_of_bf16_peak": wf / (avg_w * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                        "algorithmic_bytes": wb}
    if w.dit is not None:
        lin_ms = sum(ev[0].elapsed_time(ev[1]) for st in per_step for ev in st.get("linear", [])) / args.steps
        norm_ms = sum(ev[0].elapsed_time(ev[1]) for st in per_step for ev in st.get("norm", [])) / args.steps
        lf = dit_linear_flops(w)
        out["dit"] = {"linear_ms_per_step": lin_ms, "norm_ms_per_step": norm_ms, "linear_flops_per_step": lf,
                      "linear_tflops": lf / (lin_ms * 1e-3) / 1e12,
                      "mfma_frac_of_bf16_peak": lf / (lin_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    if rows_ms:
        rf = context_rows_flops(w)
        avg_r = sum(rows_ms) / len(rows_ms)
        out["context_rows"] = {"avg_ms": avg_r, "flops": rf, "tflops": rf / (avg_r * 1e-3) / 1e12,
                               "mfma_frac_of_bf16_peak": rf / (avg_r * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    if not args.no_graph and flush is None:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            one_step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        graph.replay()
        torch.cuda.synchronize()
        g_ev = [E() for _ in range(args.steps)]
        start.record()
        for s in range(args.steps):
            g_ev[s][0].record()
            graph.replay()
            g_ev[s][1].record()
        end.record()
        torch.cuda.synchronize()
        g_ms = start.elapsed_time(end) / args.steps
        step_ms = sorted(ev[0].elapsed_time(ev[1]) for ev in g_ev)
        out["eager"] = {"ms_per_step": out["ms_per_step"], "rows_per_s": out["value"], "step_ms": out["step_ms"]}
        out["value"] = rows / (g_ms * 1e-3)
        out["ms_per_step"] = g_ms
        out["step_ms"] = {"p10": pct(10), "p50": pct(50), "p90": pct(90), "mall": "warm"}
        out["timing"] = ("HIP graph: one captured step replayed --steps times; the roofline comes from the eager "
                         "pass's per-call events")
        del graph
    else:
        out["timing"] = "eager launches"
    props = torch.cuda.get_device_properties(0)
    out["context"] = {"device": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
                      "rocm_hip": torch.version.hip, "torch": torch.__version__, **hbm_ceilings(),
                      **probe_ceilings(w, plan_waves(w.pool_dtype))}
    if calib is not None:
        out["context"].update(calib)
    else:
        out["context"]["xcd_weights"] = "library default"
    for k in ("stream_read_GBps", "tile_gather_GBps"):
        if k in out["context"]:
            out["roofline"]["frac_of_" + k[:-5]] = achieved / out["context"][k]
    # The oracle (CPU only) runs last: every GPU figure is taken with the GPU busy.
    cpu_sample = None
    if not args.no_cpu_baseline:
        n_req = args.cpu_sample_requests or max(1, min(w.bs, 24))
        cpu_sample = cpu_baseline_inputs(w, n_req)
    if not args.no_configs:
        del w, buf
        torch.cuda.empty_cache()
        out["configs"] = sweep_configs(args, xcd_weights)
    if cpu_sample is not None:
        out["cpu_baseline"] = cpu_baseline_run(cpu_sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
