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
//      head straight to its page slot, rounded once to the pool's type.

#include "fm_internal.h"

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

template <class T, int D>
__global__ __launch_bounds__(256) void write_gemm_kernel(WriteGemmArgs a) {
  typedef typename T::storage st;
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
#pragma unroll 2
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
        sincosf(fpos * inv, &sn, &cs);
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
    st* dst = (st*)(kv ? P.v : P.k) + (int64_t)page * P.page_stride + (int64_t)off * P.slot_stride +
              (int64_t)h * P.head_stride + 4 * g;
#pragma unroll
    for (int ct = 0; ct < NDT; ++ct) store4<T>(dst + 16 * ct, acc[ct], 1.0f);
  }
}

// bf16 pools with head_dim 128: the MFMA-tiled GEMM.  One workgroup (4 waves
// in a 2 x 2 arrangement) computes a 128-row x 128-column tile of
// Y^T = W X^T, i.e. one (layer, {k|v}, head) for 128 compacted rows, with
// v_mfma_f32_32x32x16_bf16 (each wave a 64 x 64 quarter).  Both operands are
// staged through double-buffered LDS in 64-wide slices of d_in; rows are
// padded to 144 bytes so the fragment reads do not collide in LDS banks.
// Tiles are ordered so the row tiles that share one W tile run back to back
// on the same XCD (workgroups go round-robin over the 8 XCDs), so W streams
// from HBM once and the other row tiles find it in that XCD's L2.
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kGM = 128, kGN = 128, kGK = 64;
constexpr int kLdsRow = kGK * 2 + 16;  // bytes per staged row

__global__ __launch_bounds__(256, 2) void write_gemm_bf16_kernel(WriteGemmArgs a, int n_tiles, int m_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_w[2][kGN * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t lds_x[2][kGM * kLdsRow];
  __shared__ float ss_part[2][2][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = wave_in_block();
  const int wm = wv >> 1, wn = wv & 1;
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
  const int l = n / (2 * a.H);
  const int kv = (n / a.H) & 1;
  const int h = n - (n / a.H) * a.H;
  const int32_t* live_row = (const int32_t*)(ws + a.lay.live_row);

  // Global -> LDS staging: each operand slice is 128 rows x 8 chunks of 16 B.
  // thread t moves rows (t >> 3) + 32 i, 16-byte segment t & 7, of each slice
  const int srow = tid >> 3, seg = tid & 7;
  const uint16_t* W = (const uint16_t*)a.w + ((int64_t)n * kGN + srow) * a.d_in + seg * 8;
  const uint16_t* X = (const uint16_t*)a.x + seg * 8;
  int32_t xrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xrow[i] = live_row[min(m0 + srow + 32 * i, live - 1)];
  const int64_t w_step = (int64_t)32 * a.d_in;
  u32x4_t gw[4], gx[4];
  auto gload = [&](int kc) {
    const int k0 = kc * kGK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gw[i] = load16(W + i * w_step + k0);
      gx[i] = load16(X + (int64_t)xrow[i] * a.d_in + k0);
    }
  };
  auto lstore = [&](int b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(u32x4_t*)(lds_w[b] + (srow + 32 * i) * kLdsRow + seg * 16) = gw[i];
      *(u32x4_t*)(lds_x[b] + (srow + 32 * i) * kLdsRow + seg * 16) = gx[i];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int cg = 0; cg < 2; ++cg)
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[cg][rg][i] = 0.f;

  // Fragment rows: lane l reads row (l % 32) of a 32-row group and the 16-byte
  // chunk 2*kk + l/32 of the 64-wide slice (8 consecutive k per lane).
  const int frow = lane & 31, fchunk = lane >> 5;
  const int nk = a.d_in / kGK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    gload(min(kc + 1, nk - 1));
    const uint8_t* bw = lds_w[kc & 1];
    const uint8_t* bx = lds_x[kc & 1];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int co = (2 * kk + fchunk) * 16;
      const u32x4_t a0 = *(const u32x4_t*)(bw + (64 * wn + frow) * kLdsRow + co);
      const u32x4_t a1 = *(const u32x4_t*)(bw + (64 * wn + 32 + frow) * kLdsRow + co);
      const u32x4_t b0 = *(const u32x4_t*)(bx + (64 * wm + frow) * kLdsRow + co);
      const u32x4_t b1 = *(const u32x4_t*)(bx + (64 * wm + 32 + frow) * kLdsRow + co);
      const bf16x8_t A0 = __builtin_bit_cast(bf16x8_t, a0), A1 = __builtin_bit_cast(bf16x8_t, a1);
      const bf16x8_t B0 = __builtin_bit_cast(bf16x8_t, b0), B1 = __builtin_bit_cast(bf16x8_t, b1);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B1, acc[1][1], 0, 0, 0);
    }
    lstore((kc + 1) & 1);
    __syncthreads();
  }
  // acc[cg][rg][i] (lane l) = Y[tile row 64 wm + 32 rg + l % 32]
  //                            [head column 64 wn + 32 cg + 8 (i / 4) + 4 (l / 32) + i % 4]

  float rs[2] = {1.f, 1.f};
  if (kv == 0) {  // k-norm over the head's 128 columns: this wave's 64, then its partner's
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      float ss = 0.f;
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int i = 0; i < 16; ++i) ss += acc[cg][rg][i] * acc[cg][rg][i];
      ss += __shfl_xor(ss, 32);
      if (lane < 32) ss_part[wm][wn][32 * rg + lane] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const int r = 32 * rg + frow;
      rs[rg] = 1.0f / sqrtf((ss_part[wm][0][r] + ss_part[wm][1][r]) / (float)kDhGemm + a.eps);
    }
  }
  const PoolDesc& P = a.pools[l];
  const float* kw = a.k_norm_w + (int64_t)l * kDhGemm;
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int li = m0 + 64 * wm + 32 * rg + frow;
    const bool has = li < live;
    const int lic = has ? li : m0;
    const int page = ((const int32_t*)(ws + a.lay.live_page))[lic];
    const int off = ((const int32_t*)(ws + a.lay.live_off))[lic];
    const float fpos = (float)((const int32_t*)(ws + a.lay.live_pos))[lic];
    uint16_t* dst = (uint16_t*)(kv ? P.v : P.k) + (int64_t)page * P.page_stride + (int64_t)off * P.slot_stride +
                    (int64_t)h * P.head_stride + 64 * wn + 4 * fchunk;
#pragma unroll
    for (int cg = 0; cg < 2; ++cg)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // columns 64 wn + 32 cg + 8 q + 4 (l/32) + 0..3: two interleaved RoPE pairs
        float v[4] = {acc[cg][rg][4 * q], acc[cg][rg][4 * q + 1], acc[cg][rg][4 * q + 2], acc[cg][rg][4 * q + 3]};
        if (kv == 0) {
#pragma unroll
          for (int p2 = 0; p2 < 4; p2 += 2) {
            const int col = 64 * wn + 32 * cg + 8 * q + 4 * fchunk + p2;
            // frequency index col / 2 = 32 wn + 16 cg + 4 q + 2 (l/32) + p2/2
            const int f0 = 32 * wn + 16 * cg + 4 * q + p2 / 2;
            const float inv = fchunk ? a.rope.inv[f0 + 2] : a.rope.inv[f0];
            float sn, cs;
            sincosf(fpos * inv, &sn, &cs);
            const float y0 = v[p2] * rs[rg] * kw[col];
            const float y1 = v[p2 + 1] * rs[rg] * kw[col + 1];
            v[p2] = y0 * cs - y1 * sn;
            v[p2 + 1] = y1 * cs + y0 * sn;
          }
        }
        if (has) store4<Bf16>(dst + 32 * cg + 8 * q, (f32x4_t){v[0], v[1], v[2], v[3]}, 1.0f);
      }
  }
}

template <class T, int D>
hipError_t launch_write_typed(const WritePrepArgs& p, const WriteGemmArgs& g, int64_t n_rows, hipStream_t s) {
  hipLaunchKernelGGL(write_prep_kernel, dim3(1), dim3(1024), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_tiles = g.L * 2 * g.H;
  if (sizeof(typename T::storage) == 2 && D == kDhGemm) {
    const int m_tiles = (int)((n_rows + kGM - 1) / kGM);
    const int64_t groups = (n_tiles + 7) / 8;
    hipLaunchKernelGGL(write_gemm_bf16_kernel, dim3((unsigned)(groups * 8 * m_tiles)), dim3(256), 0, s, g, n_tiles,
                       m_tiles);
    return hipGetLastError();
  }
  const unsigned m_tiles = (unsigned)((n_rows + 63) / 64);
  hipLaunchKernelGGL((write_gemm_kernel<T, D>), dim3((unsigned)n_tiles, m_tiles), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_write(const WritePrepArgs& p, const WriteGemmArgs& g, int dtype, int Dh, int64_t n_rows,
                        hipStream_t s) {
  if (dtype == 1) return Dh == 128 ? launch_write_typed<Bf16, 128>(p, g, n_rows, s)
                                   : launch_write_typed<Bf16, 64>(p, g, n_rows, s);
  return Dh == 128 ? launch_write_typed<F32, 128>(p, g, n_rows, s) : launch_write_typed<F32, 64>(p, g, n_rows, s);
}

}  // namespace fm
