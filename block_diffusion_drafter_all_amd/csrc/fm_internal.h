// Internal host/device interface of libfm: kernel argument blocks, workspace
// layouts and the launchers the C ABI calls.  Not installed; include/fm.h is
// the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include "fm_device.h"

namespace fm {

constexpr int kMaxLayers = 16;
constexpr int kQRows = 16;          // query rows of one MFMA fragment (one draft block)
constexpr int kMaxQFrags = 4;       // fragments per request: up to 64 query rows (4 candidate blocks)

// Fragments the plan and the kernel use for at most max_q query rows per request
// (1, 2 or 4; 0 when max_q is out of range).
inline int q_frags(int max_q) {
  if (max_q < 0 || max_q > kQRows * kMaxQFrags) return 0;
  const int f = (max_q + kQRows - 1) / kQRows;
  return f <= 1 ? 1 : (f <= 2 ? 2 : 4);
}
constexpr int32_t kPlanMagic = 0x464d504c;   // "FMPL"
constexpr int32_t kWriteMagic = 0x464d5752;  // "FMWR"
constexpr int32_t kCtxMagic = 0x464d4358;    // "FMCX"
// Resident cross-attention waves per SIMD, by pool type: a bf16 or fp32 tile
// keeps one wave busy; e4m3 tiles (half the bytes for the same instructions)
// run two waves per SIMD so that one issues while the other waits.  The plan
// cuts the tile stream for exactly the waves the kernel keeps resident.
#ifndef FM_CROSS_OCC_BF16
#define FM_CROSS_OCC_BF16 1
#endif
#ifndef FM_CROSS_OCC_FP8
#define FM_CROSS_OCC_FP8 2
#endif
constexpr int cross_occupancy(int dtype) { return dtype == 2 ? FM_CROSS_OCC_FP8 : (dtype == 1 ? FM_CROSS_OCC_BF16 : 1); }
constexpr int kMaxPlanWaves = 4096;  // most attention waves one plan describes

// One dispatch holds fewer than 2^32 work-items per grid dimension.  The
// launchers check every grid of a call before its first launch and return
// hipErrorInvalidConfiguration (nothing enqueued) when one does not fit.
inline bool grid_fits(int64_t workgroups, int threads) {
  return workgroups >= 0 && workgroups <= (((int64_t)1 << 32) - 1) / threads;
}

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ------------------------------------------------------------ pool descriptor

struct PoolDesc {
  uint64_t k, v;            // device addresses
  int64_t num_pages;
  int64_t page_stride, slot_stride, head_stride;
};

// ------------------------------------------------------------------- plan --

// Cross-attention schedule.  The work of one call is the stream of 16-token
// K/V tiles of every (request, head) pair, pairs in (request, head) order and
// tiles in position order.  The plan cuts that stream into n_waves equal
// contiguous ranges, one per resident wavefront of the attention kernel, so
// every wave streams the same number of tiles across pair boundaries with no
// per-unit restart.  A pair cut by a range boundary leaves (m, l, O) partials
// (at most two per wave: its first and its last segment); the last of the
// pair's waves to finish combines them in wave order.

// Header at byte 0 of a cross-attention workspace.  error at byte 4 (see fm.h).
struct PlanHeader {
  int32_t magic;
  int32_t error;
  int32_t n_waves;
  int32_t bs;
  int32_t H;
  int32_t nqf;        // query fragments per request
  int64_t total_tiles;
  int32_t Dh;         // head dim: the workspace layout past the header depends on it
  int32_t dtype;      // pool type (0 fp32, 1 bf16, 2 e4m3) the plan was cut for
};

// One wave's range: it starts at tile ``k`` of pair (b, h), which is tile
// ``start`` of the stream, and covers ``count`` tiles; ``ctx`` is request b's
// context length.
struct WaveRec {
  int32_t b, h, k, count;
  int32_t ctx, pad;
  int64_t start;
};

// Where a pair's tiles lie among the wave ranges: the first and last wave
// holding them, how many waves hold a part (1: the pair is whole), and the
// partial slot of its first wave (1 when that wave's range starts in an
// earlier pair, whose partial takes slot 0; every later wave starts inside
// the pair and uses slot 0).
struct PairRec {
  int32_t w0, w1, parts, slot0;
};

struct PlanLayout {
  size_t q_hat;       // [bs][16 nqf][H][Dh] of the pool's type: normed, rotated queries (0 past a request's rows);
                      // over an e4m3 pool, the queries divided by their (request, head) scale
  size_t q_scale;     // float [bs][H]: e4m3 pool only, the query scale of each (request, head)
  size_t pair_off;    // int64 [bs + 1]: first tile of request b's pairs in the stream
  size_t wave_rec;    // WaveRec [n_waves]
  size_t pair_rec;    // PairRec [bs * H]
  size_t merge_cnt;   // int32 [n_waves]: partials counted in for the cut pair whose first wave is w
  size_t partial_ml;  // float2 [n_waves][2][nqf][64 lanes]: running max (log2) and denominator of the lane's row
  size_t partial_o;   // f32x4 [n_waves][2][nqf][Dh/16][64 lanes]: unnormalized outputs in MFMA fragment order
  size_t total;
  int n_waves;
  int nqf;
};

inline PlanLayout plan_layout(int bs, int H, int Dh, int n_waves, int nqf) {
  PlanLayout p;
  p.n_waves = n_waves;
  p.nqf = nqf;
  size_t off = 256;
  p.q_hat = off;      off = align256(off + (size_t)bs * kQRows * nqf * H * Dh * 4);
  p.q_scale = off;    off = align256(off + (size_t)bs * H * 4);
  p.pair_off = off;   off = align256(off + (size_t)(bs + 1) * 8);
  p.wave_rec = off;   off = align256(off + (size_t)n_waves * sizeof(WaveRec));
  p.pair_rec = off;   off = align256(off + (size_t)bs * H * sizeof(PairRec));
  p.merge_cnt = off;  off = align256(off + (size_t)n_waves * 4);
  p.partial_ml = off; off = align256(off + (size_t)n_waves * 2 * nqf * 64 * 8);
  p.partial_o = off;  off = align256(off + (size_t)n_waves * 2 * nqf * kQRows * Dh * 4);
  p.total = off;
  return p;
}

// The weights of the plan's wave shares by XCD: workgroups go round-robin
// over the 8 XCDs, so wave w (4 per workgroup) runs on XCD (w / 4) mod 8 and
// its share of the tile stream is proportional to xcd_w[(w / 4) mod 8].
constexpr int kXcds = 8;
constexpr int32_t kXcdWeightMin = 500, kXcdWeightMax = 2000;

struct PlanArgs {
  const int32_t* ctx_lens;
  int32_t bs, H;
  int32_t Dh, dtype;  // recorded in the header: a call checks them against its own
  int32_t xcd_w[kXcds];
  uint8_t* ws;
  PlanLayout lay;
};

struct CrossArgs {
  const void* q;
  void* out;
  const float* q_norm_w;
  PoolDesc pool;
  const int32_t* page_table;
  int64_t pt_stride;
  int32_t log2ps;
  // The pool's strides (elements, each below 2^32), its page count and the
  // page-table row length clamped to 2^31 - 1, as 32-bit scalars for the
  // loader's per-tile arithmetic.
  uint32_t page_stride32, slot_stride32, head_stride32;
  int32_t num_pages32, pt_stride32;
  const int32_t* ctx_lens;
  const int32_t* cu_q;
  int32_t bs, H;
  int32_t total_q;          // rows of q / out; rows at or past it are never touched
  float qscale_log2;        // softmax_scale * log2(e) (times the key descale over e4m3)
  float eps;
  float q_static;           // e4m3 pool: a fixed query scale, or 0 for amax / 448 per (request, head)
  float q_static_inv;       // 1 / q_static
  float v_descale;          // e4m3 pool: the value descale (1 otherwise)
  uint8_t* ws;
  PlanLayout lay;
  RopeFreqs rope;
  uint64_t* wave_clock;     // or null: per wave, [start, end of its tile loop, XCD, tiles] on the 100 MHz clock
};

struct SelfArgs {
  const void* qkv;
  void* out;
  const float* q_norm_w;
  const float* k_norm_w;
  const int32_t* ctx_lens;
  int32_t n_blocks, K, H;
  float qscale_log2;
  float eps;
  RopeFreqs rope;
};

// ------------------------------------------------------------------ write --

struct WriteHeader {
  int32_t magic;
  int32_t error;
  int32_t live_count;
  int32_t reserved[5];
};

struct WriteLayout {
  size_t live_row, live_pos, live_page, live_off, total;
};

constexpr WriteLayout write_layout(int64_t n_rows) {
  WriteLayout w{};
  size_t off = 256;
  size_t n = (size_t)(n_rows > 0 ? n_rows : 0);
  w.live_row = off;  off = align256(off + n * 4);
  w.live_pos = off;  off = align256(off + n * 4);
  w.live_page = off; off = align256(off + n * 4);
  w.live_off = off;  off = align256(off + n * 4);
  w.total = off;
  return w;
}

// Rows the no-allocation write (fm_write_context_kv_noalloc) serves: its
// workspace is a static device array of write_layout(kWriteScratchRows).total
// bytes (about 1 MB), one copy per GPU.
constexpr int64_t kWriteScratchRows = 65536;
constexpr size_t kWriteScratchBytes = write_layout(kWriteScratchRows).total;

// Device address of the current device's copy of that array (looked up once
// per device, then cached); ``bytes`` receives its size.
hipError_t write_scratch(uint8_t** ptr, size_t* bytes);

struct WritePrepArgs {
  const int32_t* row_req;
  const int32_t* row_pos;
  const int32_t* commit_lens;
  int32_t window;
  int32_t bs;
  int64_t n_rows;
  const int32_t* page_table;
  int64_t pt_stride;
  int32_t log2ps;
  int64_t min_pages;        // smallest num_pages over the layers' pools
  int32_t* out_slots;
  uint8_t* ws;
  WriteLayout lay;
};

struct WriteGemmArgs {
  const void* x;
  const void* w;
  const float* k_norm_w;
  int32_t d_in;
  int32_t L, H;
  float eps;
  uint8_t* ws;
  WriteLayout lay;
  PoolDesc pools[kMaxLayers];
  float inv_scale[kMaxLayers][2];  // e4m3 pool: 1 / (key, value) scale of each layer (1 otherwise)
  RopeFreqs rope;
};

// ------------------------------------------------------------ context rows --

struct CtxRowsHeader {
  int32_t magic;
  int32_t error;       // bit 0: an anchor id outside [0, vocab) (read as a clamped row)
  int32_t live_count;  // committed hidden rows
  int32_t reserved[5];
};

struct CtxRowsLayout {
  size_t live_idx, part_fc, part_anchor, total;
  int s_fc, s_anchor;  // contraction splits of the two projections
};

// Contraction splits of the two projections that share one launch of the
// context rows (m_tiles x n_tiles output tiles of 256 x 256, a k-wide
// contraction): enough (1..8, a power of two dividing k / 64, at least two
// 64-wide stages per range) to give the chip about 256 workgroups, so the two
// together fill it.
inline int proj_splits(int64_t m_tiles, int64_t n_tiles, int64_t k) {
  const int64_t tiles = m_tiles * n_tiles > 0 ? m_tiles * n_tiles : 1;
  int s = 1;
  while (s < 8 && tiles * s < 256 && (k / 64) % (2 * s) == 0 && k / 64 / (2 * s) >= 2) s *= 2;
  return s;
}

inline CtxRowsLayout ctx_rows_layout(int64_t n_hidden, int64_t n_anchor, int64_t d_hidden, int64_t d_target,
                                     int64_t dim) {
  CtxRowsLayout c;
  const int64_t nt = dim / 256;
  c.s_fc = proj_splits((n_hidden + 255) / 256, nt, d_hidden);
  c.s_anchor = proj_splits((n_anchor + 255) / 256, nt, d_target);
  size_t off = 256;
  c.live_idx = off;    off = align256(off + (size_t)n_hidden * 4);
  c.part_fc = off;     off = align256(off + (size_t)c.s_fc * n_hidden * dim * 4);
  c.part_anchor = off; off = align256(off + (size_t)c.s_anchor * n_anchor * dim * 4);
  c.total = off;
  return c;
}

struct CtxRowsArgs {
  const void* hidden;           // bf16 [n_hidden, d_hidden]
  int64_t n_hidden;
  int32_t d_hidden;
  const void* w_fc;             // bf16 [dim, d_hidden]
  const float* hidden_norm_w;   // [dim]
  const int32_t* anchor_ids;    // [n_anchor]
  int64_t n_anchor;
  const void* embedding;        // bf16 [vocab, d_target]
  int64_t vocab;
  int32_t d_target;
  const void* w_anchor;         // bf16 [dim, d_target]
  const void* b_anchor;         // bf16 [dim]
  const float* anchor_norm_w;   // [dim]
  int32_t dim;
  const int32_t* commit_lens;   // or null
  int32_t window, bs;
  float eps;
  void* rows;                   // bf16 [n_hidden + n_anchor, dim]
  uint8_t* ws;
  CtxRowsLayout lay;
};

// -------------------------------------------------------------- DiT layer --

struct AdaLnArgs {
  const float* h;      // fp32 [rows, dim]
  int64_t rows;
  int32_t dim;
  const float* scale;  // [dim], already 1 + scale
  const float* shift;  // [dim]
  float eps;
  void* out;           // bf16 [rows, dim]
};

// Epilogues of fm_linear (the values of fm_linear_epilogue in fm.h).
constexpr int kLinBf16 = 0, kLinGeluBf16 = 1, kLinResidual = 2, kLinAssignF32 = 3;

struct LinearArgs {
  const void* x;       // bf16 [M, K]
  const void* w;       // bf16 [N, K]
  const void* bias;    // bf16 [N] or null
  const float* gate;   // [N] (residual epilogue)
  void* out;           // bf16 [M, N], or the fp32 stream [M, N]
  float* part;         // fp32 [splits][M][N] when splits > 1
  int64_t M, K, N;
  int32_t splits, epilogue;
};

// Contraction ranges of a projection: enough to give the chip ~256 workgroups.
// Contraction splits of one projection launch (M x N outputs in 256 x 256
// tiles, a K-wide contraction): the s in {1, 2, 4, 8} (dividing K / 64, at
// least two 64-wide stages per range) with the least modelled time, the
// smallest on a tie.  One workgroup fills a CU, so the tiles run in rounds of
// kGemmCUs; a range takes about a microsecond per 32 of its K / s when the
// chip is full; with s > 1 the partials (s fp32 outputs) are written,
// then read back with the output by a row kernel at about 5 TB/s.  A split that
// only adds a round (192 tiles in two ranges: 384 workgroups, two rounds of half
// the work) gains nothing and pays the partials, so it is not taken.
constexpr int64_t kGemmCUs = 256;
inline int linear_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = std::max<int64_t>(((M + 255) / 256) * (N / 256), 1);
  const double out_bytes = (double)tiles * 256.0 * 256.0 * 4.0;
  int best = 1;
  double best_us = 0.0;
  for (int s = 1; s <= 8; s *= 2) {
    if ((K / 64) % s != 0 || (s > 1 && K / 64 / s < 2)) break;
    const int64_t rounds = (tiles * s + kGemmCUs - 1) / kGemmCUs;
    const double us = (double)rounds * (double)(K / 32 / s) + (s > 1 ? (s + 1) * out_bytes / 5.0e6 : 0.0);
    if (s == 1 || us < best_us) best = s, best_us = us;
  }
  return best;
}

// -------------------------------------------------------------- launchers --
// Each returns hipSuccess or the launch error.  dtype: 0 = fp32, 1 = bf16,
// 2 = bf16 activations over an e4m3 pool (write and cross-attention only).

hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_cross_attention(const CrossArgs& a, int dtype, int Dh, hipStream_t s);
hipError_t launch_self_attention(const SelfArgs& a, int dtype, int Dh, hipStream_t s);
hipError_t launch_write(const WritePrepArgs& p, const WriteGemmArgs& g, int dtype, int Dh,
                        int64_t n_rows, hipStream_t s);
hipError_t launch_context_rows(const CtxRowsArgs& a, hipStream_t s);
hipError_t launch_ada_layer_norm(const AdaLnArgs& a, hipStream_t s);
hipError_t launch_linear(const LinearArgs& a, hipStream_t s);

}  // namespace fm
