// The bf16 MFMA GEMM tile shared by the context K/V write and the context /
// anchor input projections: one workgroup (8 waves in a 4 x 2 arrangement)
// computes a 256 x 256 tile of Y^T = W X^T, 256 rows of W against 256 rows of
// X, each wave 128 W rows x 64 X rows with v_mfma_f32_32x32x16_bf16 (4 x 2
// accumulator blocks of 32 x 32, held in AGPRs); two waves share each SIMD.
//
// Operands stream through a ring of five LDS buffers (5 x 32 KB: gfx950's 160
// KB per workgroup), each a 32-wide slice of the contraction, filled by direct
// global->LDS loads that hold no registers while in flight.  A staged operand
// slice is 256 rows x 4 chunks of 16 bytes; each 1 KB load moves 16 whole rows
// (64 contiguous bytes each: one L2 request per row), and the chunk order
// within a row is swizzled by XOR with (row >> 2) & 3 so that the 16 lanes of
// each phase of an MFMA fragment read (16 rows, one chunk) hit 64 distinct
// banks.  Per slice: wait until the slice three steps back has landed, one
// barrier (after it every wave is also done with the buffer consumed last
// step), refill that buffer, then 16 MFMAs per wave.  The buffers are named
// statically in each unrolled step, so the compiler can tell the buffer being
// read from the ones being filled and never waits for every load in flight.
#pragma once

#include "fm_internal.h"

namespace fm {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kGM = 256, kGN = 256, kGK = 32;
constexpr int kGemmWaves = 8;
constexpr int kStages = 5;                      // LDS ring buffers of 32 KB
constexpr int kFrag = 1024;                     // bytes of one 32-row x 16-k fragment
constexpr int kStageBytes = 2 * 16 * kFrag;     // 16 W fragments + 16 X fragments
constexpr int kLoadsPerWave = 32 / kGemmWaves;  // fragments each wave loads per slice

// s_waitcnt with vmcnt(n) only (expcnt and lgkmcnt left at their maxima).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0) only

// Load i of wave wv fills LDS slots 64 (f & 15) .. +63 of its operand (f =
// 4 wv + i: W for f < 16, X for f >= 16): lane l takes tile row
// 16 (f & 15) + l/4 and, at slot position l % 4, the 16-byte chunk
// (l % 4) ^ ((row >> 2) & 3) of the row's 64-byte slice.
struct GemmLoad {
  bool is_w;
  int row;    // tile row, 0..255
  int chunk;  // 16-byte chunk (8 bf16) of the 32-wide slice
};
__device__ __forceinline__ GemmLoad gemm_load_of(int wv, int lane, int i) {
  const int f = kLoadsPerWave * wv + i, fl = f & 15;
  GemmLoad g;
  g.is_w = f < 16;
  g.row = 16 * fl + (lane >> 2);
  g.chunk = (lane & 3) ^ ((g.row >> 2) & 3);
  return g;
}

// acc += the tile's product over nk slices.  src[i]: the start of this lane's
// load i at slice 0 (row start + 8 chunk elements); slice kc reads src[i] +
// 32 kc.  Afterwards acc[cg][rg][i] (lane l) = Y[X row 64 wm + 32 rg + l % 32]
// [W row 128 wn + 32 cg + 8 (i / 4) + 4 (l / 32) + i % 4].
__device__ __forceinline__ void gemm256_mainloop(f32x16_t (&acc)[4][2], const uint16_t* const (&src)[kLoadsPerWave],
                                                 int nk, int wv, int wm, int wn, uint8_t* ring0, uint8_t* ring1,
                                                 uint8_t* ring2, uint8_t* ring3, uint8_t* ring4) {
  const int lane = lane_id();
  const int frow = lane & 31, fchunk = lane >> 5;
  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto issue = [&](int kc, uint8_t* base) {  // slice kc into a ring buffer
    const int k0 = kc * kGK;
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + k0), (lds_ptr)(base + (kLoadsPerWave * wv + i) * kFrag),
                                       16, 0, 0);
  };
  // Byte offset of this lane's fragment element in a staged operand, for k
  // chunk pair kk: row l % 32 (plus 32 q rows = 2048 q bytes), chunk 2 kk + l/32
  // at its swizzled position.
  int frag_off[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) frag_off[kk] = frow * 64 + (((2 * kk + fchunk) ^ ((frow >> 2) & 3)) * 16);

  // One step of the ring: slice kc is read from ``cur``; slice kc + 4 goes
  // into ``refill``, the buffer every wave finished reading last step.
  auto step = [&](int kc, const uint8_t* cur, uint8_t* refill) {
    // slice kc landed (the three slices issued after it may still be in flight)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoadsPerWave * (kStages - 2)));
    __builtin_amdgcn_s_barrier();
    // past the end: a re-read of the last slice into a buffer nobody reads again
    issue(min(kc + kStages - 1, nk - 1), refill);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // lane l reads row 32 q + l % 32 (rows of one fragment are 2 KB apart per 32) and chunk 2 kk + l/32
      const uint8_t* buf = cur + frag_off[kk];
      bf16x8_t A[4], B[2];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        A[q] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(buf + (4 * wn + q) * 2048));
#pragma unroll
      for (int q = 0; q < 2; ++q)
        B[q] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(buf + 16 * kFrag + (2 * wm + q) * 2048));
#pragma unroll
      for (int cg = 0; cg < 4; ++cg)
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
          acc[cg][rg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[cg], B[rg], acc[cg][rg], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this wave's reads of the buffer are done
  };
  issue(0, ring0);
  issue(min(1, nk - 1), ring1);
  issue(min(2, nk - 1), ring2);
  issue(min(3, nk - 1), ring3);
  int kc = 0;
  for (; kc + 5 <= nk; kc += 5) {
    step(kc, ring0, ring4);
    step(kc + 1, ring1, ring0);
    step(kc + 2, ring2, ring1);
    step(kc + 3, ring3, ring2);
    step(kc + 4, ring4, ring3);
  }
  // the last nk % 5 slices, in ring order (each step's buffers named statically)
  const int rem = nk - kc;
  if (rem > 0) step(kc, ring0, ring4);
  if (rem > 1) step(kc + 1, ring1, ring0);
  if (rem > 2) step(kc + 2, ring2, ring1);
  if (rem > 3) step(kc + 3, ring3, ring2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // drain the ring's trailing loads
}

// Declares the five ring buffers of a GEMM kernel.
#define FM_GEMM_RING                                                       \
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t ring4[kStageBytes]

}  // namespace fm
