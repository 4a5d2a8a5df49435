// The bf16 MFMA GEMM tile shared by the context K/V write, the context /
// anchor input projections and the DiT projections: one workgroup (8 waves in
// a 4 x 2 arrangement) computes a 256 x 256 tile of Y^T = W X^T, 256 rows of W
// against 256 rows of X, each wave 128 W rows x 64 X rows with
// v_mfma_f32_32x32x16_bf16 (4 x 2 accumulator blocks of 32 x 32); two waves
// share each SIMD.
//
// Operands stream through two LDS stages of 64 KB, each a 64-wide slice of
// the contraction (256 rows x 128 bytes per operand), filled by direct
// global->LDS loads that hold no registers while in flight.  Each 1 KB load
// moves 8 whole rows of 128 contiguous bytes: a full L2 line per row, which
// the memory system streams ~1.6x faster than the half-line rows of a
// 32-wide slice.  The 16-byte chunks of a row are stored XOR-swizzled by
// (row >> 1) & 7, so the 16 lanes of each phase of a fragment read (16 rows,
// one chunk) hit 64 distinct banks.
//
// The MFMA operands are pipelined through registers: each 16-wide k step's
// fragments are read while the previous step's MFMAs run, interleaved one
// read per MFMA.  One barrier per stage, three quarters of the way through
// it: by then every wave has issued its last read of the stage's buffer and
// the next stage has landed, so the stage after next is issued into the
// buffer just finished and the next stage's first fragments are read in the
// shadow of the current stage's last MFMAs.
#pragma once

#include "fm_internal.h"

namespace fm {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kGM = 256, kGN = 256, kGK = 64;  // tile rows of X and W; contraction per stage
constexpr int kGemmWaves = 8;
constexpr int kStageBytes = 65536;              // W 32 KB + X 32 KB
constexpr int kLoadsPerWave = 64 / kGemmWaves;  // 1 KB loads each wave issues per stage

// s_waitcnt with vmcnt(n) only (expcnt and lgkmcnt left at their maxima).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0) only

// Load i of wave wv (f = kLoadsPerWave wv + i: W for f < 32, X for f >= 32)
// fills rows 8 (f & 31) .. +7 of its operand: lane l takes row 8 (f & 31) +
// l / 8 and, at slot position l % 8 of the row, the 16-byte chunk
// (l % 8) ^ ((row >> 1) & 7) of the row's 128-byte slice.
struct GemmLoad {
  bool is_w;
  int row;    // tile row, 0..255
  int chunk;  // 16-byte chunk (8 bf16) of the 64-wide slice
};
__device__ __forceinline__ GemmLoad gemm_load_of(int wv, int lane, int i) {
  const int f = kLoadsPerWave * wv + i;
  GemmLoad g;
  g.is_w = f < 32;
  g.row = 8 * (f & 31) + (lane >> 3);
  g.chunk = (lane & 7) ^ ((g.row >> 1) & 7);
  return g;
}

// acc += the tile's product over ns stages.  src[i]: the start of this lane's
// load i at stage 0 (row start + 8 chunk elements); stage s reads src[i] +
// 64 s.  Afterwards acc[cg][rg][i] (lane l) = Y[X row 64 wm + 32 rg + l % 32]
// [W row 128 wn + 32 cg + 8 (i / 4) + 4 (l / 32) + i % 4], for the wave's
// first RG blocks of 32 X rows (rg < RG; the others are left untouched).
// With RG = 0 the wave only issues its share of the loads and meets every
// barrier (the same sequence in every case) and reads no fragments.
template <int RG = 2>
__device__ __forceinline__ void gemm256_mainloop(f32x16_t (&acc)[4][2], const uint16_t* const (&src)[kLoadsPerWave],
                                                 int ns, int wv, int wm, int wn, uint8_t* buf0, uint8_t* buf1) {
  constexpr bool MMA = RG > 0;
  const int lane = lane_id();
  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto issue = [&](int s, uint8_t* b) {  // stage s into a buffer
    const int k0 = s * kGK;
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + k0), (lds_ptr)(b + (kLoadsPerWave * wv + i) * 1024), 16,
                                       0, 0);
  };
  // k step t (16 k: chunks 2t, 2t + 1): lane l reads row 32 q + l % 32 (4 KB per 32 rows), chunk 2t + l / 32
  const int frow = lane & 31, fhalf = lane >> 5;
  int off[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) off[t] = frow * 128 + (((2 * t + fhalf) ^ ((frow >> 1) & 7)) * 16);
  struct Frags {
    bf16x8_t A[4], B[2];  // W, X
  };
  auto read = [&](const uint8_t* b, int t, Frags& f) {
    if constexpr (!MMA) return;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      f.A[q] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(b + off[t] + (4 * wn + q) * 4096));
#pragma unroll
    for (int q = 0; q < RG; ++q)
      f.B[q] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(b + 32768 + off[t] + (2 * wm + q) * 4096));
  };
  auto mma = [&](const Frags& f) {
    if constexpr (!MMA) return;
#pragma unroll
    for (int cg = 0; cg < 4; ++cg)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
        acc[cg][rg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.A[cg], f.B[rg], acc[cg][rg], 0, 0, 0);
  };
  // the order of issue in a k step: each fragment read (then each load) behind one MFMA
  // (4 RG MFMAs and 4 + RG reads a step: with one block the fifth read follows the fourth)
  auto interleave = [&](bool loads) {
    if constexpr (!MMA) return;
    constexpr int kPairs = RG == 2 ? 6 : 4;
#pragma unroll
    for (int j = 0; j < kPairs; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    if constexpr (RG == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the fifth read
    if constexpr (RG == 2) {
      if (loads) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, kLoadsPerWave / 2, 0);  // global->LDS loads
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    } else if (loads) {
      __builtin_amdgcn_sched_group_barrier(0x020, kLoadsPerWave, 0);  // global->LDS loads
    }
  };
  Frags fa, fb;
  // Stage s from buffer cur; the other buffer nxt holds stage s + 1.
  auto stage = [&](int s, uint8_t* cur, uint8_t* nxt) {
    read(cur, 1, fb);
    mma(fa);
    interleave(false);
    read(cur, 2, fa);
    mma(fb);
    interleave(false);
    read(cur, 3, fb);
    mma(fa);
    interleave(false);
    // this wave's reads of cur are done and stage s + 1 (its only loads in flight) has landed;
    // after the barrier, every wave's are
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0) & kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    issue(min(s + 2, ns - 1), cur);  // past the end: a re-read of the last stage, never used
    read(nxt, 0, fa);                // past the end: a stale stage, never multiplied
    mma(fb);
    interleave(true);
  };
  issue(0, buf0);
  issue(min(1, ns - 1), buf1);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoadsPerWave));  // stage 0 landed
  __builtin_amdgcn_s_barrier();
  read(buf0, 0, fa);
  int s = 0;
  for (; s + 2 <= ns; s += 2) {  // the buffers named statically in each step
    stage(s, buf0, buf1);
    stage(s + 1, buf1, buf0);
  }
  if (s < ns) stage(s, buf0, buf1);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0) & kWaitLgkm0);  // drain the trailing loads and reads
}

// The mainloop for a wave with ``rows`` live X rows (wave-uniform, clamped to
// 0..64): the 32-row MFMA blocks past them (the padding of a partial tile)
// are not multiplied, and a wave with none still moves its share of each
// stage through LDS but reads no fragments, leaving the matrix core of its
// SIMD to the other wave there.
__device__ __forceinline__ void gemm256_mainloop_rows(f32x16_t (&acc)[4][2],
                                                      const uint16_t* const (&src)[kLoadsPerWave], int ns, int wv,
                                                      int wm, int wn, uint8_t* buf0, uint8_t* buf1, int64_t rows) {
  if (rows > 32)
    gemm256_mainloop<2>(acc, src, ns, wv, wm, wn, buf0, buf1);
  else if (rows > 0)
    gemm256_mainloop<1>(acc, src, ns, wv, wm, wn, buf0, buf1);
  else
    gemm256_mainloop<0>(acc, src, ns, wv, wm, wn, buf0, buf1);
}

// Declares the two LDS stages of a GEMM kernel.
#define FM_GEMM_RING                                                     \
  __shared__ __attribute__((aligned(1024))) uint8_t buf0[kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[kStageBytes]

}  // namespace fm
