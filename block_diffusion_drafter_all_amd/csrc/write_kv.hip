// Context/anchor K/V write of every DiT layer for gfx950 (flashmap 0.1.0 wheel:
// sglang/model.py ``write_target_hidden_kv`` / ``_write_context`` /
// ``_kv_write``; vllm/model.py ``_prologue`` / ``_write``).
//
// Two kernels, no host synchronization between them:
//   1. prep: decides which rows are written (negative position, or a verify
//      column at or past the request's commit length, is skipped), compacts
//      the written rows in row order and resolves each one's page and slot;
//   2. GEMM + epilogue: Y = X W^T over the compacted rows only, one output
//      tile = 64 rows x one (layer, {k|v}, head) of head_dim columns, so the
//      tile holds whole heads: the epilogue RMS-norms and rotates keys in
//      registers (fp32 from the MFMA accumulator) and stores every row's
//      head straight to its page slot, rounded once to the pool's type (an
//      e4m3 pool is written with scale 1: sglang/model.py ``_kv_write`` with
//      ``kv_norm_rope_write_fp8``).

#include <mutex>

#include "gemm_core.h"

// Workspace of the no-allocation write: one static array per GPU, held until
// the process ends.  Host code must not pass this name to a kernel (on the
// host it is a stand-in, not a device address): fm::write_scratch looks up
// each device's address once and every launch takes that address.
static __device__ __align__(256) uint8_t scratch[fm::kWriteScratchBytes];

namespace fm {

namespace {

constexpr int kDhGemm = 128;  // head_dim of the MFMA-tiled bf16 GEMM

__global__ __launch_bounds__(1024) void write_prep_kernel(WritePrepArgs a) {
  uint8_t* ws = a.ws;
  WriteHeader* hdr = (WriteHeader*)ws;
  int32_t* live_row = (int32_t*)(ws + a.lay.live_row);
  int32_t* live_pos = (int32_t*)(ws + a.lay.live_pos);
  int32_t* live_page = (int32_t*)(ws + a.lay.live_page);
  int32_t* live_off = (int32_t*)(ws + a.lay.live_off);
  if (threadIdx.x == 0) hdr->error = 0;
  __syncthreads();
  const int ps_mask = (1 << a.log2ps) - 1;
  int carry = 0;
  bool bad = false;
  for (int64_t base = 0; base < a.n_rows; base += 1024) {
    const int64_t r = base + threadIdx.x;
    int live = 0, pos = -1, page = 0;
    if (r < a.n_rows) {
      pos = a.row_pos[r];
      bool want = pos >= 0;
      if (want && a.commit_lens != nullptr && r < (int64_t)a.bs * a.window) {
        const int64_t b = r / a.window;
        const int64_t j = r - b * a.window;
        if (j >= a.commit_lens[b]) want = false;
      }
      if (want) {
        const int b = a.row_req[r];
        const int64_t pidx = (int64_t)pos >> a.log2ps;
        bool ok = b >= 0 && b < a.bs && pidx < a.pt_stride;
        if (ok) {
          page = a.page_table[(int64_t)b * a.pt_stride + pidx];
          ok = page >= 0 && (int64_t)page < a.min_pages;
        }
        if (ok) live = 1;
        else bad = true;
      }
      if (a.out_slots != nullptr) a.out_slots[r] = live ? (page << a.log2ps) + (pos & ps_mask) : -1;
    }
    int block_total;
    const int idx = carry + block_exclusive_scan(live, &block_total);
    if (live) {
      live_row[idx] = (int32_t)r;
      live_pos[idx] = pos;
      live_page[idx] = page;
      live_off[idx] = pos & ps_mask;
    }
    carry += block_total;
  }
  if (bad) atomicOr(&hdr->error, 1);
  if (threadIdx.x == 0) {
    hdr->magic = kWriteMagic;
    hdr->live_count = carry;
  }
}

// T: x and W; PT: the pool (T itself, or e4m3 under bf16 operands).
template <class T, class PT, int D>
__global__ __launch_bounds__(256) void write_gemm_kernel(WriteGemmArgs a) {
  typedef typename T::storage st;
  typedef typename PT::storage pst;
  constexpr int EPC = T::EPC;
  constexpr int KC = 4 * EPC;   // contraction elements per 16-byte chunk per lane group
  constexpr int NDT = D / 16;   // 16-column tiles of one head
  const int lane = lane_id(), g = lane >> 4, c = lane & 15;
  const uint8_t* ws = a.ws;
  const WriteHeader* hdr = (const WriteHeader*)ws;
  if (hdr->magic != kWriteMagic) return;
  const int live = hdr->live_count;
  const int m0 = blockIdx.y * 64 + wave_in_block() * 16;
  if (m0 >= live) return;
  const int n = blockIdx.x;  // (layer, {k, v}, head)
  const int l = n / (2 * a.H);
  const int kv = (n / a.H) & 1;
  const int h = n - (n / a.H) * a.H;
  const int li = m0 + c;
  const bool has = li < live;
  const int32_t* live_row = (const int32_t*)(ws + a.lay.live_row);
  const int xr = live_row[has ? li : m0];

  // Row fragments: X row of this lane's data row, W rows of this lane's columns.
  const st* xrow = (const st*)a.x + (int64_t)xr * a.d_in + g * EPC;
  const st* wrow = (const st*)a.w + ((int64_t)n * D + c) * a.d_in + g * EPC;
  const int64_t wstep = (int64_t)16 * a.d_in;
  f32x4_t acc[NDT];
#pragma unroll
  for (int ct = 0; ct < NDT; ++ct) acc[ct] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < a.d_in; k0 += KC) {
    const u32x4_t xb = load16(xrow + k0);
    u32x4_t wa[NDT];
#pragma unroll
    for (int ct = 0; ct < NDT; ++ct) wa[ct] = load16(wrow + ct * wstep + k0);
#pragma unroll
    for (int ct = 0; ct < NDT; ++ct) mma_chunk<T>(acc[ct], wa[ct], xb);
  }
  // acc[ct][i] (lane (g, c)) = Y[data row c][column 16ct + 4g + i] of this head.

  const int pos = has ? ((const int32_t*)(ws + a.lay.live_pos))[li] : 0;
  if (kv == 0) {
    float ss = 0.f;
#pragma unroll
    for (int ct = 0; ct < NDT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) ss += acc[ct][i] * acc[ct][i];
    ss = wave_sum_groups(ss);
    const float rs = 1.0f / sqrtf(ss / (float)D + a.eps);
    const float* kw = a.k_norm_w + (int64_t)l * D;
    const float fpos = (float)pos;
#pragma unroll
    for (int ct = 0; ct < NDT; ++ct) {
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const int col = 16 * ct + 4 * g + i;
        // frequency index col / 2 = 8ct + 2g + i/2, selected by lane group
        const int f0 = 8 * ct + i / 2;
        const float inv = sel4(g, a.rope.inv[f0], a.rope.inv[f0 + 2], a.rope.inv[f0 + 4], a.rope.inv[f0 + 6]);
        float sn, cs;
        angle_sincos(fpos * inv, &sn, &cs);
        const float y0 = acc[ct][i] * rs * kw[col];
        const float y1 = acc[ct][i + 1] * rs * kw[col + 1];
        acc[ct][i] = y0 * cs - y1 * sn;
        acc[ct][i + 1] = y1 * cs + y0 * sn;
      }
    }
  }
  if (has) {
    const int page = ((const int32_t*)(ws + a.lay.live_page))[li];
    const int off = ((const int32_t*)(ws + a.lay.live_off))[li];
    const PoolDesc& P = a.pools[l];
    pst* dst = (pst*)(kv ? P.v : P.k) + (int64_t)page * P.page_stride + (int64_t)off * P.slot_stride +
               (int64_t)h * P.head_stride + 4 * g;
    const float sc = a.inv_scale[l][kv];
#pragma unroll
    for (int ct = 0; ct < NDT; ++ct) store4<PT>(dst + 16 * ct, acc[ct], sc);
  }
}

// The epilogue of the bf16 tile works on 32-column blocks of one head: lane l
// holds one compacted row (its own) and, in c[i], columns
// col0 + 8 (i / 4) + 4 (l / 32) + i % 4.  It only reads the accumulators.

// The key head of layer l in acc[0..3][rg] (block cg = columns 32 cg ..):
// k-normed, rotated and stored to head h of the key pool at (page, slot off)
// when ``has``.  The sum of squares over the head's 128 columns is 64 in this
// lane and 64 in lane l ^ 32.  kw: the layer's k-norm weight, inv: the inverse
// RoPE frequencies (both in LDS).
template <class PT>
__device__ __forceinline__ void store_key_head(const WriteGemmArgs& a, const f32x16_t (&acc)[4][2], int rg, int l,
                                               int h, const float* kw, const float* inv_tab, float fpos, int page,
                                               int off, bool has) {
  typedef typename PT::storage pst;
  const int fchunk = lane_id() >> 5;
  float ss = 0.f;
#pragma unroll
  for (int cg = 0; cg < 4; ++cg)
#pragma unroll
    for (int i = 0; i < 16; ++i) ss += acc[cg][rg][i] * acc[cg][rg][i];
  ss += __shfl_xor(ss, 32);
  const float rs = 1.0f / sqrtf(ss / (float)kDhGemm + a.eps);
  const PoolDesc& P = a.pools[l];
  pst* dst = (pst*)P.k + (int64_t)page * P.page_stride + (int64_t)off * P.slot_stride + (int64_t)h * P.head_stride +
             4 * fchunk;
  const float sc = a.inv_scale[l][0];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int p2 = 0; p2 < 4; p2 += 2) {
        // columns 32 cg + 8 q + 4 (l/32) + p2, + 1: one interleaved RoPE pair,
        // frequency index col / 2 = 16 cg + 4 q + 2 (l/32) + p2/2
        const int col = 32 * cg + 8 * q + 4 * fchunk + p2;
        float sn, cs;
        angle_sincos(fpos * inv_tab[16 * cg + 4 * q + p2 / 2 + 2 * fchunk], &sn, &cs);
        const float y0 = acc[cg][rg][4 * q + p2] * rs * kw[col];
        const float y1 = acc[cg][rg][4 * q + p2 + 1] * rs * kw[col + 1];
        v[p2] = y0 * cs - y1 * sn;
        v[p2 + 1] = y1 * cs + y0 * sn;
      }
      if (has) store4<PT>(dst + 32 * cg + 8 * q, (f32x4_t){v[0], v[1], v[2], v[3]}, sc);
    }
}

// Stores one block to head h of layer l's {k|v} pool at (page, slot off),
// rounded once to the pool's type.
template <class PT>
__device__ __forceinline__ void store_block(const WriteGemmArgs& a, const f32x16_t& c, int l, int kv, int h, int col0,
                                            int page, int off) {
  typedef typename PT::storage pst;
  const PoolDesc& P = a.pools[l];
  pst* dst = (pst*)(kv ? P.v : P.k) + (int64_t)page * P.page_stride + (int64_t)off * P.slot_stride +
             (int64_t)h * P.head_stride + col0 + 4 * (lane_id() >> 5);
  const float sc = a.inv_scale[l][kv];
#pragma unroll
  for (int q = 0; q < 4; ++q) store4<PT>(dst + 8 * q, (f32x4_t){c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]}, sc);
}

// bf16 activations with head_dim 128: the MFMA-tiled GEMM (gemm_core.h), one
// 256 x 256 tile of Y^T = W X^T per workgroup: two (layer, {k|v}, head) blocks
// of W against 256 compacted rows, each wave one whole head for 64 rows.  Tiles
// are ordered so the row tiles that share one W tile run back to back on the
// same XCD (workgroups go round-robin over the 8 XCDs), so W streams from HBM
// once and the other row tiles find it in that XCD's L2.  A wave holds all 128
// columns of its head, so the k-norm's sum of squares needs one cross-lane
// exchange.
template <class PT>
__global__ __launch_bounds__(64 * kGemmWaves, 1) void write_gemm_bf16_kernel(WriteGemmArgs a, int n_tiles,
                                                                              int m_tiles) {
  FM_GEMM_RING;
  // per head wn of the tile: the k-norm weight of its layer and the inverse
  // RoPE frequencies, for the epilogue
  __shared__ float epi_lds[2][kDhGemm + kDhGemm / 2];
  const int lane = lane_id();
  const int wv = wave_in_block();
  const int wm = wv >> 1, wn = wv & 1;  // rows 64 wm .. +63 of the tile, head wn
  const int wg = blockIdx.x;
  const int n = ((wg >> 3) / m_tiles) * 8 + (wg & 7);
  const int mt = (wg >> 3) % m_tiles;
  if (n >= n_tiles) return;
  const uint8_t* ws = a.ws;
  const WriteHeader* hdr = (const WriteHeader*)ws;
  if (hdr->magic != kWriteMagic) return;
  const int live = hdr->live_count;
  const int m0 = mt * kGM;
  if (m0 >= live) return;
  const int hn = 2 * n + wn;  // this wave's (layer, k|v, head) block of W
  const int l = hn / (2 * a.H);
  const int kv = (hn / a.H) & 1;
  const int h = hn - (hn / a.H) * a.H;
  const int32_t* live_row = (const int32_t*)(ws + a.lay.live_row);
  const int frow = lane & 31;

  const uint16_t* src[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const GemmLoad g = gemm_load_of(wv, lane, i);
    if (g.is_w) {
      src[i] = (const uint16_t*)a.w + ((int64_t)n * kGN + g.row) * a.d_in + g.chunk * 8;
    } else {
      const int xr = live_row[min(m0 + g.row, live - 1)];
      src[i] = (const uint16_t*)a.x + (int64_t)xr * a.d_in + g.chunk * 8;
    }
  }
  // The epilogue's inputs, fetched while the contraction runs: each row's
  // page, slot and position, and (key heads) the norm weight, which goes to
  // LDS with the frequencies once the contraction is done.
  int page[2], off[2];
  float fpos[2];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int li = m0 + 64 * wm + 32 * rg + frow;
    const int lic = li < live ? li : m0;
    page[rg] = ((const int32_t*)(ws + a.lay.live_page))[lic];
    off[rg] = ((const int32_t*)(ws + a.lay.live_off))[lic];
    fpos[rg] = (float)((const int32_t*)(ws + a.lay.live_pos))[lic];
  }
  float kw_reg[2] = {0.f, 0.f};
  if (kv == 0 && wm == 0) {
    kw_reg[0] = a.k_norm_w[(int64_t)l * kDhGemm + lane];
    kw_reg[1] = a.k_norm_w[(int64_t)l * kDhGemm + lane + 64];
  }
  f32x16_t acc[4][2];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg)
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[cg][rg][i] = 0.f;
  gemm256_mainloop_rows(acc, src, a.d_in / kGK, wv, wm, wn, buf0, buf1, live - (m0 + 64 * wm));
  // acc[cg][rg][i] (lane l) = Y[tile row 64 wm + 32 rg + l % 32]
  //                            [head column 32 cg + 8 (i / 4) + 4 (l / 32) + i % 4]
  float* kw = epi_lds[wn];
  float* inv_tab = kw + kDhGemm;
  if (kv == 0 && wm == 0) {
    kw[lane] = kw_reg[0];
    kw[lane + 64] = kw_reg[1];
    if (lane == 0) {  // (a per-lane index into the kernel argument would cost scratch)
#pragma unroll
      for (int i = 0; i < kDhGemm / 2; ++i) inv_tab[i] = a.rope.inv[i];
    }
  }
  __syncthreads();
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const bool has = m0 + 64 * wm + 32 * rg + frow < live;
    if (kv == 0) {
      store_key_head<PT>(a, acc, rg, l, h, kw, inv_tab, fpos[rg], page[rg], off[rg], has);
    } else if (has) {
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) store_block<PT>(a, acc[cg][rg], l, 1, h, 32 * cg, page[rg], off[rg]);
    }
  }
}

template <class T, class PT, int D>
hipError_t launch_write_typed(const WritePrepArgs& p, const WriteGemmArgs& g, int64_t n_rows, hipStream_t s) {
  const int n_tiles = g.L * 2 * g.H;
  constexpr bool tiled = sizeof(typename T::storage) == 2 && D == kDhGemm;
  const int64_t m_tiles = tiled ? (n_rows + kGM - 1) / kGM : (n_rows + 63) / 64;
  const int64_t groups = (n_tiles / 2 + 7) / 8;  // 256-row tiles of W: two heads each
  if (tiled ? !grid_fits(groups * 8 * m_tiles, 64 * kGemmWaves) : (!grid_fits(n_tiles, 256) || m_tiles > INT32_MAX))
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(write_prep_kernel, dim3(1), dim3(1024), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (tiled) {
    hipLaunchKernelGGL(write_gemm_bf16_kernel<PT>, dim3((unsigned)(groups * 8 * m_tiles)), dim3(64 * kGemmWaves), 0,
                       s, g, n_tiles / 2, (int)m_tiles);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((write_gemm_kernel<T, PT, D>), dim3((unsigned)n_tiles, (unsigned)m_tiles), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t write_scratch(uint8_t** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static uint8_t* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {  // with this device current: its own copy of the array
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<uint8_t*>(p);
  }
  *ptr = addr[dev];
  *bytes = kWriteScratchBytes;
  return hipSuccess;
}

hipError_t launch_write(const WritePrepArgs& p, const WriteGemmArgs& g, int dtype, int Dh, int64_t n_rows,
                        hipStream_t s) {
  if (dtype == 1) return Dh == 128 ? launch_write_typed<Bf16, Bf16, 128>(p, g, n_rows, s)
                                   : launch_write_typed<Bf16, Bf16, 64>(p, g, n_rows, s);
  if (dtype == 2) return Dh == 128 ? launch_write_typed<Bf16, E4m3, 128>(p, g, n_rows, s)
                                   : launch_write_typed<Bf16, E4m3, 64>(p, g, n_rows, s);
  return Dh == 128 ? launch_write_typed<F32, F32, 128>(p, g, n_rows, s)
                   : launch_write_typed<F32, F32, 64>(p, g, n_rows, s);
}

}  // namespace fm
