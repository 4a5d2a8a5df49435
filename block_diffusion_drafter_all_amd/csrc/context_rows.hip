// The rows the all-layer context K/V GEMM takes (flashmap 0.1.0 wheel:
// sglang/model.py ``_write_context`` and ``_anchor_kv_impl``; vllm/model.py
// ``combine_hidden_states``, ``precompute_and_store_context_kv``, ``_prologue``):
//   committed target positions:  hidden_norm(fc(concatenated target hidden))
//   anchors:                     anchor_norm(anchor_proj(embedding[token]) + bias)
//
// Three launches, no host synchronization between them:
//   1. prep: the commit rule over the hidden rows (the same rule as the K/V
//      write: uncommitted verify columns are skipped), compacted in row order;
//      anchor ids checked against the vocabulary;
//   2. the two projections in one launch on the shared 256 x 256 MFMA tile
//      (gemm_core.h), the contraction split into a few ranges so the small row
//      counts still fill the chip; each range leaves an fp32 partial
//      (deterministic: no atomics).  The anchor tiles run on the CUs the
//      hidden-row tiles leave free;
//   3. per row: the partials summed in order (plus the bias), RMS-normed with
//      the row kind's weight from the fp32 sum, rounded once to bf16.

#include "gemm_core.h"

namespace fm {

namespace {

// The commit rule and the anchor-id check.  One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void ctx_prep_kernel(CtxRowsArgs a) {
  CtxRowsHeader* hdr = (CtxRowsHeader*)a.ws;
  int32_t* live_idx = (int32_t*)(a.ws + a.lay.live_idx);
  int base = 0;
  for (int64_t r0 = 0; r0 < a.n_hidden; r0 += 1024) {
    const int64_t r = r0 + threadIdx.x;
    bool live = r < a.n_hidden;
    if (live && a.commit_lens != nullptr && r < (int64_t)a.bs * a.window) {
      const int b = (int)(r / a.window), col = (int)(r - (int64_t)b * a.window);
      live = col < a.commit_lens[b];
    }
    int total;
    const int before = block_exclusive_scan(live ? 1 : 0, &total);
    if (live) live_idx[base + before] = (int32_t)r;
    base += total;
  }
  int bad = 0;
  for (int64_t i = threadIdx.x; i < a.n_anchor; i += 1024) {
    const int32_t id = a.anchor_ids[i];
    bad |= (id < 0 || (int64_t)id >= a.vocab) ? 1 : 0;
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) {
    hdr->live_count = base;
    hdr->error = bad;
    __hip_atomic_store(&hdr->magic, kCtxMagic, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Workgroups of one projection in the shared launch.
struct ProjGrid {
  int m_tiles, splits, wgs;
};

// One 256 x 256 tile of one contraction range of a projection: rows of the
// compacted committed hidden rows (the first hid.wgs workgroups: X = hidden,
// W = w_fc) or of the anchors (the rest: X = embedding rows of the anchor
// ids, W = w_anchor).  The partial of range sp goes to part[sp][row][column].
// Workgroups go round-robin over the 8 XCDs (hid.wgs is a multiple of 8);
// consecutive groups of 8 are ordered (W tile, range)-major, so the row tiles
// that share one W tile and range run on the same XCD and find W in its L2.
__global__ __launch_bounds__(64 * kGemmWaves, 1) void proj_gemm_kernel(CtxRowsArgs a, int n_tiles, ProjGrid hid,
                                                                        ProjGrid anc) {
  FM_GEMM_RING;
  const int lane = lane_id();
  const int wv = wave_in_block();
  const int wm = wv >> 1, wn = wv & 1;
  const bool ANCHOR = (int)blockIdx.x >= hid.wgs;
  const int wg = ANCHOR ? (int)blockIdx.x - hid.wgs : (int)blockIdx.x;
  const int m_tiles = ANCHOR ? anc.m_tiles : hid.m_tiles;
  const int splits = ANCHOR ? anc.splits : hid.splits;
  const int ns = ((wg >> 3) / m_tiles) * 8 + (wg & 7);
  const int mt = (wg >> 3) % m_tiles;
  const int n = ns / splits, sp = ns - (ns / splits) * splits;
  if (n >= n_tiles) return;
  const CtxRowsHeader* hdr = (const CtxRowsHeader*)a.ws;
  if (hdr->magic != kCtxMagic) return;
  const int64_t M = ANCHOR ? a.n_anchor : (int64_t)hdr->live_count;
  const int64_t m0 = (int64_t)mt * kGM;
  if (m0 >= M) return;
  const int64_t K = ANCHOR ? a.d_target : a.d_hidden;
  const int64_t Ks = K / splits, k_begin = (int64_t)sp * Ks;
  const uint16_t* W = (const uint16_t*)(ANCHOR ? a.w_anchor : a.w_fc);
  const int32_t* live_idx = (const int32_t*)(a.ws + a.lay.live_idx);

  const uint16_t* src[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const GemmLoad g = gemm_load_of(wv, lane, i);
    if (g.is_w) {
      src[i] = W + ((int64_t)n * kGN + g.row) * K + k_begin + g.chunk * 8;
    } else {
      const int64_t m = min(m0 + g.row, M - 1);  // rows past the last re-read it (never stored)
      int64_t xr;
      const uint16_t* X;
      if (ANCHOR) {
        xr = min(max((int64_t)a.anchor_ids[m], (int64_t)0), a.vocab - 1);
        X = (const uint16_t*)a.embedding;
      } else {
        xr = live_idx[m];
        X = (const uint16_t*)a.hidden;
      }
      src[i] = X + xr * K + k_begin + g.chunk * 8;
    }
  }
  f32x16_t acc[4][2];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg)
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[cg][rg][i] = 0.f;
  gemm256_mainloop_rows(acc, src, (int)(Ks / kGK), wv, wm, wn, buf0, buf1, M - (m0 + 64 * wm));

  // acc[cg][rg][i] (lane l) = Y[row m0 + 64 wm + 32 rg + l % 32]
  //                            [column 256 n + 128 wn + 32 cg + 8 (i / 4) + 4 (l / 32) + i % 4]
  const int frow = lane & 31, fchunk = lane >> 5;
  const int64_t rows_max = ANCHOR ? a.n_anchor : a.n_hidden;
  float* part = (float*)(a.ws + (ANCHOR ? a.lay.part_anchor : a.lay.part_fc)) + (int64_t)sp * rows_max * a.dim;
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int64_t m = m0 + 64 * wm + 32 * rg + frow;
    if (m >= M) continue;
    float* prow = part + m * a.dim + (int64_t)n * kGN + 128 * wn + 4 * fchunk;
#pragma unroll
    for (int cg = 0; cg < 4; ++cg)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4_t*)(prow + 32 * cg + 8 * q) = (f32x4_t){acc[cg][rg][4 * q], acc[cg][rg][4 * q + 1],
                                                        acc[cg][rg][4 * q + 2], acc[cg][rg][4 * q + 3]};
  }
}

// One output row per workgroup of 256 threads: the ranges' partials summed in
// range order (plus the anchor bias), then RMSNorm with the row kind's weight,
// rounded once to bf16.  Thread t holds columns 4 (t + 256 j) .. +3.
constexpr int kMaxDimGroups = 8;  // dim <= 8192
__global__ __launch_bounds__(256) void rows_norm_kernel(CtxRowsArgs a) {
  const CtxRowsHeader* hdr = (const CtxRowsHeader*)a.ws;
  if (hdr->magic != kCtxMagic) return;
  const int64_t i = blockIdx.x;
  const bool anchor = i >= a.n_hidden;
  int64_t row, out_row, rows_max;
  int splits;
  if (anchor) {
    row = i - a.n_hidden;
    out_row = i;
    rows_max = a.n_anchor;
    splits = a.lay.s_anchor;
  } else {
    if (i >= hdr->live_count) return;
    row = i;
    out_row = ((const int32_t*)(a.ws + a.lay.live_idx))[i];
    rows_max = a.n_hidden;
    splits = a.lay.s_fc;
  }
  const float* part = (const float*)(a.ws + (anchor ? a.lay.part_anchor : a.lay.part_fc)) + row * a.dim;
  const int groups = a.dim / 1024;
  const int t = threadIdx.x;
  f32x4_t y[kMaxDimGroups];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxDimGroups; ++j) {
    if (j >= groups) break;
    const int64_t c = 4 * (t + 256 * j);
    f32x4_t v = *(const f32x4_t*)(part + c);
    for (int s = 1; s < splits; ++s) v += *(const f32x4_t*)(part + (int64_t)s * rows_max * a.dim + c);
    if (anchor) {
      const uint32_t* bb = (const uint32_t*)((const uint16_t*)a.b_anchor + c);
      const uint32_t b01 = bb[0], b23 = bb[1];
      v += (f32x4_t){bf16_bits_to_f32(b01 & 0xFFFFu), bf16_bits_to_f32(b01 >> 16), bf16_bits_to_f32(b23 & 0xFFFFu),
                     bf16_bits_to_f32(b23 >> 16)};
    }
    y[j] = v;
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  // block sum of squares: within the wave, then across the four waves
  ss = wave_sum_groups(ss);
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) ss += __shfl_xor(ss, d);
  __shared__ float wave_ss[4];
  if ((t & 63) == 0) wave_ss[t >> 6] = ss;
  __syncthreads();
  ss = wave_ss[0] + wave_ss[1] + wave_ss[2] + wave_ss[3];
  const float rs = 1.0f / sqrtf(ss / (float)a.dim + a.eps);
  const float* w = anchor ? a.anchor_norm_w : a.hidden_norm_w;
  uint16_t* out = (uint16_t*)a.rows + out_row * a.dim;
#pragma unroll
  for (int j = 0; j < kMaxDimGroups; ++j) {
    if (j >= groups) break;
    const int64_t c = 4 * (t + 256 * j);
    const f32x4_t ww = *(const f32x4_t*)(w + c);
    store4<Bf16>(out + c, y[j] * ww, rs);
  }
}

}  // namespace

hipError_t launch_context_rows(const CtxRowsArgs& a, hipStream_t s) {
  const int n_tiles = a.dim / kGN;
  auto grid_of = [&](int64_t rows, int splits, int64_t* wgs) {
    ProjGrid g{};
    *wgs = 0;
    if (rows == 0) return g;
    g.m_tiles = (int)((rows + kGM - 1) / kGM);
    g.splits = splits;
    *wgs = (((int64_t)n_tiles * splits + 7) / 8) * 8 * g.m_tiles;
    g.wgs = (int)std::min<int64_t>(*wgs, INT32_MAX);
    return g;
  };
  int64_t hid_wgs, anc_wgs;
  const ProjGrid hid = grid_of(a.n_hidden, a.lay.s_fc, &hid_wgs), anc = grid_of(a.n_anchor, a.lay.s_anchor, &anc_wgs);
  const int64_t rows = a.n_hidden + a.n_anchor;
  if (!grid_fits(hid_wgs + anc_wgs, 64 * kGemmWaves) || !grid_fits(rows, 256)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(ctx_prep_kernel, dim3(1), dim3(1024), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(proj_gemm_kernel, dim3((unsigned)(hid_wgs + anc_wgs)), dim3(64 * kGemmWaves), 0, s, a, n_tiles,
                     hid, anc);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(rows_norm_kernel, dim3((unsigned)rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fm
