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

template <class T, int D>
hipError_t launch_write_typed(const WritePrepArgs& p, const WriteGemmArgs& g, int64_t n_rows, hipStream_t s) {
  hipLaunchKernelGGL(write_prep_kernel, dim3(1), dim3(1024), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned n_tiles = (unsigned)(g.L * 2 * g.H);
  const unsigned m_tiles = (unsigned)((n_rows + 63) / 64);
  hipLaunchKernelGGL((write_gemm_kernel<T, D>), dim3(n_tiles, m_tiles), dim3(256), 0, s, g);
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
