// The rest of a DiT block of the draft step (flashmap 0.1.0 wheel:
// sglang/model.py ``_denoise``; vllm/model.py ``_dit``; modeling_flashmap.py
// ``FlashMapLayer``, ``FlashMapAdaLayerNorm``, ``FlashMapMLP``):
//   - the time-modulated LayerNorm, LayerNorm(h) * (1 + scale) + shift, from
//     the fp32 residual stream to the bf16 operand of the next projection;
//   - the projections (qkv, q, the two o_proj, fc1, fc2, x_embed) on the
//     shared 256 x 256 MFMA tile, with the epilogue the layer needs: bf16 out,
//     bias + GELU, or the gated residual h += gate * (y + bias) into the fp32
//     stream.  A projection whose output tiles alone would leave the chip
//     idle splits its contraction into ranges that leave fp32 partials, summed
//     in range order by a row kernel that applies the same epilogue
//     (deterministic: no atomics).

#include "gemm_core.h"

namespace fm {

namespace {

constexpr int kMaxRowGroups = 8;  // row kernels: dim <= 8192, 4 columns x 256 threads per group

// Block reduction of one value over the 256 threads (four waves); every thread gets the sum.
__device__ __forceinline__ float block256_sum(float v, float* scratch4) {
  v = wave_sum_groups(v);
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) v += __shfl_xor(v, d);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch4[threadIdx.x >> 6] = v;
  __syncthreads();
  return scratch4[0] + scratch4[1] + scratch4[2] + scratch4[3];
}

// LayerNorm(h) * scale + shift of one row per workgroup of 256 threads; the
// mean first, then the variance from the centred values (two passes over
// registers), rounded once to bf16.
__global__ __launch_bounds__(256) void ada_ln_kernel(AdaLnArgs a) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x, groups = a.dim / 1024;
  const float* hr = a.h + row * a.dim;
  f32x4_t x[kMaxRowGroups];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxRowGroups; ++j) {
    if (j >= groups) break;
    x[j] = *(const f32x4_t*)(hr + 4 * (t + 256 * j));
    s += (x[j][0] + x[j][1]) + (x[j][2] + x[j][3]);
  }
  const float mu = block256_sum(s, red) / (float)a.dim;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxRowGroups; ++j) {
    if (j >= groups) break;
    x[j] -= mu;
    ss += (x[j][0] * x[j][0] + x[j][1] * x[j][1]) + (x[j][2] * x[j][2] + x[j][3] * x[j][3]);
  }
  const float rstd = 1.0f / sqrtf(block256_sum(ss, red) / (float)a.dim + a.eps);
  uint16_t* out = (uint16_t*)a.out + row * a.dim;
#pragma unroll
  for (int j = 0; j < kMaxRowGroups; ++j) {
    if (j >= groups) break;
    const int c = 4 * (t + 256 * j);
    const f32x4_t sc = *(const f32x4_t*)(a.scale + c), sh = *(const f32x4_t*)(a.shift + c);
    store4<Bf16>(out + c, x[j] * rstd * sc + sh, 1.0f);
  }
}

__device__ __forceinline__ float gelu_exact(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

__device__ __forceinline__ f32x4_t bias4(const uint16_t* b, int64_t c) {
  if (b == nullptr) return (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const u32x2_t v = *(const u32x2_t*)(b + c);
  return (f32x4_t){bf16_bits_to_f32(v[0] & 0xFFFFu), bf16_bits_to_f32(v[0] >> 16), bf16_bits_to_f32(v[1] & 0xFFFFu),
                   bf16_bits_to_f32(v[1] >> 16)};
}

// The epilogue of four consecutive outputs y (the contraction's full sum) of
// row m, columns c .. c+3.
__device__ __forceinline__ void linear_epilogue(const LinearArgs& a, int64_t m, int64_t c, f32x4_t y) {
  y += bias4((const uint16_t*)a.bias, c);
  switch (a.epilogue) {
    case kLinBf16:
      store4<Bf16>((uint16_t*)a.out + m * a.N + c, y, 1.0f);
      break;
    case kLinGeluBf16:
      store4<Bf16>((uint16_t*)a.out + m * a.N + c,
                   (f32x4_t){gelu_exact(y[0]), gelu_exact(y[1]), gelu_exact(y[2]), gelu_exact(y[3])}, 1.0f);
      break;
    case kLinResidual: {
      float* h = (float*)a.out + m * a.N + c;
      *(f32x4_t*)h = *(const f32x4_t*)h + *(const f32x4_t*)(a.gate + c) * y;
      break;
    }
    default:  // kLinAssignF32
      *(f32x4_t*)((float*)a.out + m * a.N + c) = y;
  }
}

// One 256 x 256 tile of one contraction range of Y = X W^T.  With one range
// the epilogue runs here; with more, the range's partial goes to
// part[sp][m][n].  Workgroups go round-robin over the 8 XCDs; consecutive
// groups of 8 are (W tile, range)-major, so the row tiles sharing a W tile
// and range run on one XCD and find W in its L2.
__global__ __launch_bounds__(64 * kGemmWaves, 1) void linear_gemm_kernel(LinearArgs a, int n_tiles, int m_tiles,
                                                                          int splits) {
  FM_GEMM_RING;
  const int lane = lane_id();
  const int wv = wave_in_block();
  const int wm = wv >> 1, wn = wv & 1;
  const int wg = blockIdx.x;
  const int ns = ((wg >> 3) / m_tiles) * 8 + (wg & 7);
  const int mt = (wg >> 3) % m_tiles;
  const int n = ns / splits, sp = ns - (ns / splits) * splits;
  if (n >= n_tiles) return;
  const int64_t M = a.M, K = a.K;
  const int64_t m0 = (int64_t)mt * kGM;
  const int64_t Ks = K / splits, k_begin = (int64_t)sp * Ks;
  const uint16_t* src[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const GemmLoad g = gemm_load_of(wv, lane, i);
    if (g.is_w)
      src[i] = (const uint16_t*)a.w + ((int64_t)n * kGN + g.row) * K + k_begin + g.chunk * 8;
    else  // rows past the last re-read it (never stored)
      src[i] = (const uint16_t*)a.x + min(m0 + g.row, M - 1) * K + k_begin + g.chunk * 8;
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
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int64_t m = m0 + 64 * wm + 32 * rg + frow;
    if (m >= M) continue;
    const int64_t c0 = (int64_t)n * kGN + 128 * wn + 4 * fchunk;
#pragma unroll
    for (int cg = 0; cg < 4; ++cg)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t y = {acc[cg][rg][4 * q], acc[cg][rg][4 * q + 1], acc[cg][rg][4 * q + 2], acc[cg][rg][4 * q + 3]};
        const int64_t c = c0 + 32 * cg + 8 * q;
        if (splits == 1)
          linear_epilogue(a, m, c, y);
        else
          *(f32x4_t*)(a.part + ((int64_t)sp * M + m) * a.N + c) = y;
      }
  }
}

// One output row per workgroup of 256 threads: the ranges' partials summed in
// range order, then the epilogue.  Thread t holds columns 4 (t + 256 j) .. +3.
__global__ __launch_bounds__(256) void linear_reduce_kernel(LinearArgs a, int splits) {
  const int64_t m = blockIdx.x;
  const int groups = (int)(a.N / 1024);
  for (int j = 0; j < groups; ++j) {
    const int64_t c = 4 * ((int64_t)threadIdx.x + 256 * j);
    f32x4_t y = *(const f32x4_t*)(a.part + m * a.N + c);
    for (int s = 1; s < splits; ++s) y += *(const f32x4_t*)(a.part + ((int64_t)s * a.M + m) * a.N + c);
    linear_epilogue(a, m, c, y);
  }
}

}  // namespace

hipError_t launch_ada_layer_norm(const AdaLnArgs& a, hipStream_t s) {
  if (!grid_fits(a.rows, 256)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(ada_ln_kernel, dim3((unsigned)a.rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_linear(const LinearArgs& a, hipStream_t s) {
  const int n_tiles = (int)(a.N / kGN), m_tiles = (int)((a.M + kGM - 1) / kGM);
  const int splits = a.splits;
  const int64_t groups = ((int64_t)n_tiles * splits + 7) / 8;
  if (!grid_fits(groups * 8 * m_tiles, 64 * kGemmWaves) || (splits > 1 && !grid_fits(a.M, 256)))
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(linear_gemm_kernel, dim3((unsigned)(groups * 8 * m_tiles)), dim3(64 * kGemmWaves), 0, s, a,
                     n_tiles, m_tiles, splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(linear_reduce_kernel, dim3((unsigned)a.M), dim3(256), 0, s, a, splits);
  return hipGetLastError();
}

}  // namespace fm
