// Device-side building blocks shared by the gfx950 kernels of the draft-step
// attention path: register fragments in MFMA operand layout, the MFMA
// contractions, RMSNorm + interleaved RoPE on a fragment, and conversions.
//
// Fragment layout.  A "row fragment" holds 16 rows of a [rows, D] matrix in one
// wave: lane l owns row (l % 16) and, for each 16-byte chunk ch, the EPC
// consecutive elements starting at column ch*4*EPC + (l / 16)*EPC, where EPC
// is the number of elements per 16 bytes (8 for bf16, 4 for fp32).  This is at
// once the A-operand layout (rows = M) and the B-operand layout (rows = N) of
// the 16x16 MFMA family, with the contraction index permuted consistently, so
// a product of two row fragments over their columns needs no data movement:
//   acc[i] (lane l) = sum_d A[4*(l/16) + i][d] * B[l % 16][d].
// The result lane l therefore holds column (l % 16) of B against rows
// 4*(l/16) .. 4*(l/16)+3 of A (the "C layout").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct Bf16 {
  typedef uint16_t storage;
  static constexpr int EPC = 8;  // elements per 16-byte chunk
};
struct F32 {
  typedef float storage;
  static constexpr int EPC = 4;
};
// OCP float8 e4m3 ("e4m3fn": bias 7, largest finite 448, no infinity): the
// fp8 KV pool, written with scale 1.  Its row fragments hold 16 elements per
// chunk, so a 16-byte load covers the same 16 rows x 64 bytes as for bf16.
struct E4m3 {
  typedef uint8_t storage;
  static constexpr int EPC = 16;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float round_bf16(float f) {
  return bf16_bits_to_f32(f32_to_bf16_bits(f));
}

// Four fp32 values -> four OCP e4m3 codes (the first in the low byte):
// nearest, ties to even, magnitudes past 448 saturating to 448 (the pool must
// stay finite).  Clamped first, then converted by gfx950's packed fp8
// conversion; over every multiple of 2^-13 below 520 (both signs), every
// midpoint of the e4m3 grid and 2M random values of 2^-14..2^9 it gives the
// same codes as rounding the significand to 3 bits (2^-9 steps below 2^-6).
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  auto sat = [](float x) { return fminf(fmaxf(x, -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
  return (uint32_t)w;
}

template <class T>
__device__ __forceinline__ float chunk_elem(const u32x4_t& v, int j);

template <>
__device__ __forceinline__ float chunk_elem<Bf16>(const u32x4_t& v, int j) {
  uint32_t w = v[j >> 1];
  return (j & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
}

template <>
__device__ __forceinline__ float chunk_elem<F32>(const u32x4_t& v, int j) {
  return __uint_as_float(v[j]);
}

// Pack EPC floats into one 16-byte chunk of storage type T.
template <class T>
__device__ __forceinline__ u32x4_t pack_chunk(const float* x);

template <>
__device__ __forceinline__ u32x4_t pack_chunk<Bf16>(const float* x) {
  u32x4_t r;
#pragma unroll
  for (int w = 0; w < 4; ++w) r[w] = f32_to_bf16_bits(x[2 * w]) | (f32_to_bf16_bits(x[2 * w + 1]) << 16);
  return r;
}

template <>
__device__ __forceinline__ u32x4_t pack_chunk<F32>(const float* x) {
  u32x4_t r;
#pragma unroll
  for (int w = 0; w < 4; ++w) r[w] = __float_as_uint(x[w]);
  return r;
}

// 16-byte load from global memory (device allocations only): an explicit
// global-address-space access, so the compiler emits global_load_dwordx4
// (counted by vmcnt alone) rather than a flat load.
typedef const __attribute__((address_space(1))) u32x4_t* gptr_u32x4;
__device__ __forceinline__ u32x4_t load16(const void* p) { return *(gptr_u32x4)(p); }

// Streaming 16-byte load (K/V tiles are read once): nontemporal hint.
__device__ __forceinline__ u32x4_t load16_stream(const void* p) {
#ifdef FM_KV_NT
  return __builtin_nontemporal_load((gptr_u32x4)(p));
#else
  return *(gptr_u32x4)(p);
#endif
}

typedef const __attribute__((address_space(1))) int32_t* gptr_i32;
__device__ __forceinline__ int32_t load_i32(const int32_t* p) { return *(gptr_i32)(p); }

// s_waitcnt vmcnt(0) through the builtin, so that the compiler's wait
// bookkeeping knows every vector load has completed here.
__device__ __forceinline__ void wait_all_vector_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wave-uniform load through the scalar unit (constant address space): for
// small read-only tables such as lengths, so that waiting for the value never
// waits for vector loads in flight.  Reads only; the data must not change
// while the kernel runs.
typedef const __attribute__((address_space(4))) int32_t* cptr_i32;
__device__ __forceinline__ int32_t sload_i32(const int32_t* p) { return *(cptr_i32)(p); }
typedef const __attribute__((address_space(4))) float* cptr_f32;
__device__ __forceinline__ float sload_f32(const float* p) { return *(cptr_f32)(p); }

typedef const __attribute__((address_space(1))) float* gptr_f32;
__device__ __forceinline__ float load_f32(const float* p) { return *(gptr_f32)(p); }

// acc += A_chunk x B_chunk^T over one 16-byte chunk of each row fragment.
template <class T>
__device__ __forceinline__ void mma_chunk(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b);

template <>
__device__ __forceinline__ void mma_chunk<Bf16>(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma_chunk<F32>(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[j]), __uint_as_float(b[j]), acc, 0, 0, 0);
}

__device__ __forceinline__ long u64_of(uint32_t lo, uint32_t hi) {
  return (long)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// e4m3 chunks: two 16x16x32 fp8 MFMAs, one per 8-byte half.  Every product of
// two e4m3 values is exact in fp32.
template <>
__device__ __forceinline__ void mma_chunk<E4m3>(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(u64_of(a[0], a[1]), u64_of(b[0], b[1]), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(u64_of(a[2], a[3]), u64_of(b[2], b[3]), acc, 0, 0, 0);
}

// Two e4m3 chunks of each lane (32 codes) in one gfx950 16x16x128 fp8 MFMA
// (unit block scales: exponent 127).  The contraction pairs the operands'
// codes position by position, so any assignment of the 128 contraction
// indices to (lane group, byte) that A and B share gives the same products;
// here that of the chunks the lanes already hold.
__device__ __forceinline__ void mma_two_chunks_e4m3(f32x4_t& acc, const u32x4_t& a0, const u32x4_t& a1,
                                                    const u32x4_t& b0, const u32x4_t& b1) {
  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  const i32x8_t a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8_t b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
}

// Selection operands that move a row fragment into the C layout ("column
// fragment"): for column tile dt (16 columns), transpose_tile returns, in lane
// l, M[4*(l/16) + i][16*dt + l%16] for i < 4 -- four consecutive rows of one
// column.  It is the MFMA product of the fragment with a 0/1 selection matrix,
// exact for finite inputs.
template <class T>
struct Selector;

template <>
struct Selector<Bf16> {
  u32x4_t sel[2];  // sel[h]: element j of lane (g, c) is 1 iff 8g + j == 16h + c
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = (8 * g + j == 16 * h + c) ? 1.0f : 0.0f;
      sel[h] = pack_chunk<Bf16>(e);
    }
  }
  template <int NCH>
  __device__ __forceinline__ f32x4_t transpose_tile(const u32x4_t (&frag)[NCH], int dt) const {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    mma_chunk<Bf16>(acc, frag[dt >> 1], sel[dt & 1]);
    return acc;
  }
};

template <>
struct Selector<F32> {
  float sel[4];  // sel[j] of lane (g, c) is 1 iff 4g + j == c
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j) sel[j] = (4 * g + j == c) ? 1.0f : 0.0f;
  }
  template <int NCH>
  __device__ __forceinline__ f32x4_t transpose_tile(const u32x4_t (&frag)[NCH], int dt) const {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(frag[dt][j]), sel[j], acc, 0, 0, 0);
    return acc;
  }
};

// e4m3 fragments: each 8-byte half of a chunk is one fp8 MFMA operand, whose
// element j in lane group g is "virtual column" 8g + j of that half; the
// selection matrix (e4m3 1.0 = 0x38) is the bf16 one on 8-byte operands, and
// the products are exact.  Tile dt = 4 ch + 2 half + hsel of chunk ch yields,
// in lane (g, c), V[key 4g+i][virtual column 16 hsel + c] as fp32; the real
// column of an output lane is given by out_col<E4m3>.
template <>
struct Selector<E4m3> {
  long sel[2];  // sel[h]: byte j of lane (g, c) is 1.0 iff 8g + j == 16h + c
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint64_t v = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (8 * g + j == 16 * h + c) v |= (uint64_t)0x38u << (8 * j);
      sel[h] = (long)v;
    }
  }
  template <int NCH>
  __device__ __forceinline__ f32x4_t transpose_tile(const u32x4_t (&frag)[NCH], int dt) const {
    const u32x4_t& ch = frag[dt >> 2];
    const long a = ((dt >> 1) & 1) ? u64_of(ch[2], ch[3]) : u64_of(ch[0], ch[1]);
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, sel[dt & 1], (f32x4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
};

// First of the four consecutive output columns lane group g holds after the
// PV product of column tile dt (the tile order transpose_tile defines).
template <class T>
__device__ __forceinline__ int out_col(int dt, int g) {
  return 16 * dt + 4 * g;
}
template <>
__device__ __forceinline__ int out_col<E4m3>(int dt, int g) {
  // virtual column 16 hsel + 4g + i of half ``half`` of chunk ch is real column
  // 64 ch + 16 (2 hsel + g/2) + 8 half + 4 (g%2) + i
  return 64 * (dt >> 2) + 32 * (dt & 1) + 16 * (g >> 1) + 8 * ((dt >> 1) & 1) + 4 * (g & 1);
}

// acc (C layout, lane (g, c) = out[4g+i][c]) += Vt x P, the weighted sum of
// four keys: vt[i] (lane (g, c)) is column c of key 4g+i, p[i] the weight of
// key 4g+i for query row c.  Afterwards lane (g, c) holds, for query row c,
// output columns 4g .. 4g+3 of the tile.
template <class T>
__device__ __forceinline__ void mma_pv(f32x4_t& acc, const f32x4_t& vt, const f32x4_t& p);

// bf16 bits of two fp32 values that bf16 holds exactly (their high halves),
// packed lo | hi << 16 by one byte permute.
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Two fp32 values rounded to bf16 (nearest even) in one v_cvt_pk_bf16_f32:
// lo in the low half, hi in the high half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Four e4m3 codes (byte i = element i) as bf16, exact (bf16 holds every
// e4m3 value): two packed conversions with a unit scale.
__device__ __forceinline__ i16x4_t e4m3x4_to_bf16x4(uint32_t codes) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t r = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true))};
  return __builtin_bit_cast(i16x4_t, r);
}

// The PV product with the weights already packed as bf16 pairs (pb: keys
// 4g, 4g+1 | 4g+2, 4g+3 of lane (g, c)); vt as for mma_pv<Bf16>.
__device__ __forceinline__ void mma_pv_packed(f32x4_t& acc, const f32x4_t& vt, const u32x2_t& pb) {
  const u32x2_t a = {pack_hi16(vt[0], vt[1]), pack_hi16(vt[2], vt[3])};
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, pb),
                                                  acc, 0, 0, 0);
}

// bf16 operands: vt comes from transpose_tile of bf16 or e4m3 data and p from
// operand_value<Bf16>, so every value is bf16-representable and packing its
// high half is exact.
template <>
__device__ __forceinline__ void mma_pv<Bf16>(f32x4_t& acc, const f32x4_t& vt, const f32x4_t& p) {
  const u32x2_t a = {pack_hi16(vt[0], vt[1]), pack_hi16(vt[2], vt[3])};
  const u32x2_t b = {pack_hi16(p[0], p[1]), pack_hi16(p[2], p[3])};
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, b),
                                                  acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma_pv<F32>(f32x4_t& acc, const f32x4_t& vt, const f32x4_t& p) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(vt[i], p[i], acc, 0, 0, 0);
}

// The probability a weight takes into the PV contraction: bf16 operands round it.
template <class T>
__device__ __forceinline__ float operand_value(float p);
template <>
__device__ __forceinline__ float operand_value<Bf16>(float p) { return round_bf16(p); }
template <>
__device__ __forceinline__ float operand_value<F32>(float p) { return p; }

__device__ __forceinline__ float sel4(int g, float a0, float a1, float a2, float a3) {
  return g == 0 ? a0 : (g == 1 ? a1 : (g == 2 ? a2 : a3));
}

// Reductions over the four lane groups (lanes c, c+16, c+32, c+48) with the
// gfx950 row swaps: v_permlane16_swap of x with itself leaves x's and its
// xor-16 partner's values in the two results (in some order), and
// v_permlane32_swap does the same for xor 32; no LDS round trip.
__device__ __forceinline__ u32x2_t swap16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (u32x2_t){r[0], r[1]};
}
__device__ __forceinline__ u32x2_t swap32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (u32x2_t){r[0], r[1]};
}

__device__ __forceinline__ float wave_sum_groups(float x) {
  u32x2_t r = swap16(x);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = swap32(x);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max_groups(float x) {
  u32x2_t r = swap16(x);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = swap32(x);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 2^x by the hardware v_exp_f32 (about 1 ulp; results below 2^-126 may flush
// to zero, which a softmax weight that small can take).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Inverse RoPE frequencies, float32, computed by the host (nearest float32 to
// theta^(-2i/D)) and passed by value so every kernel sees identical bits.
struct RopeFreqs {
  float inv[64];
};

// sin and cos of the fp32 RoPE angle ``ang``: the angle is reduced by a
// double-precision multiple of 2*pi (two-part constant) to one revolution and
// passed to the hardware v_sin_f32 / v_cos_f32, which take revolutions.
// Absolute error against the exact values at the fp32 angle is below 2e-7 for
// every RoPE angle up to position 2^17 (7e-8 for sincosf), at a fraction of
// sincosf's cost and registers for large angles.
__device__ __forceinline__ void angle_sincos(float ang, float* sn, float* cs) {
  constexpr double kInv2Pi = 0.15915494309189533577;
  constexpr double k2PiHi = 6.283185307179586232;   // double nearest 2*pi
  constexpr double k2PiLo = 2.4492935982947064e-16;  // 2*pi minus k2PiHi
  const double a = (double)ang;
  const double turns = rint(a * kInv2Pi);
  const float rev = (float)((fma(-turns, k2PiHi, a) - turns * k2PiLo) * kInv2Pi);
  *sn = __builtin_amdgcn_sinf(rev);
  *cs = __builtin_amdgcn_cosf(rev);
}

// RMSNorm with weight w, then the interleaved-pair rotation at position pos,
// applied in place to the fp32 values x of a row fragment (row = lane % 16,
// values x[ch*EPC + j] at column ch*4*EPC + g*EPC + j).
template <class T, int D>
__device__ __forceinline__ void norm_rope_row(float (&x)[D / 4], const float* __restrict__ w, float eps,
                                              int pos, const RopeFreqs& rf, int g) {
  constexpr int EPC = T::EPC;
  constexpr int NCH = D / (4 * EPC);
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < D / 4; ++k) ss += x[k] * x[k];
  ss = wave_sum_groups(ss);
  const float rs = 1.0f / sqrtf(ss / (float)D + eps);
  const float fpos = (float)pos;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
    for (int j = 0; j < EPC; j += 2) {
      const int col = ch * 4 * EPC + g * EPC + j;
      // frequency index col / 2 = ch*2*EPC + g*EPC/2 + j/2, selected by lane group
      const int f0 = ch * 2 * EPC + j / 2;
      const float inv = sel4(g, rf.inv[f0], rf.inv[f0 + EPC / 2], rf.inv[f0 + EPC], rf.inv[f0 + 3 * EPC / 2]);
      const float ang = fpos * inv;
      float sn, cs;
      angle_sincos(ang, &sn, &cs);
      const float y0 = x[ch * EPC + j] * rs * w[col];
      const float y1 = x[ch * EPC + j + 1] * rs * w[col + 1];
      x[ch * EPC + j] = y0 * cs - y1 * sn;
      x[ch * EPC + j + 1] = y1 * cs + y0 * sn;
    }
  }
}

// norm_rope_row with the weight and the inverse frequencies (inv[i] for the
// pair at columns 2i, 2i + 1) read per lane from arrays (LDS copies): the same
// arithmetic in the same order, so the same bits.
template <class T, int D>
__device__ __forceinline__ void norm_rope_row_lds(float (&x)[D / 4], const float* w, const float* inv, float eps,
                                                  int pos, int g) {
  constexpr int EPC = T::EPC;
  constexpr int NCH = D / (4 * EPC);
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < D / 4; ++k) ss += x[k] * x[k];
  ss = wave_sum_groups(ss);
  const float rs = 1.0f / sqrtf(ss / (float)D + eps);
  const float fpos = (float)pos;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
    for (int j = 0; j < EPC; j += 2) {
      const int col = ch * 4 * EPC + g * EPC + j;
      float sn, cs;
      angle_sincos(fpos * inv[col >> 1], &sn, &cs);
      const float y0 = x[ch * EPC + j] * rs * w[col];
      const float y1 = x[ch * EPC + j + 1] * rs * w[col + 1];
      x[ch * EPC + j] = y0 * cs - y1 * sn;
      x[ch * EPC + j + 1] = y1 * cs + y0 * sn;
    }
  }
}

template <class T>
__device__ __forceinline__ void store4(typename T::storage* p, const f32x4_t& v, float scale);

template <>
__device__ __forceinline__ void store4<Bf16>(uint16_t* p, const f32x4_t& v, float scale) {
  u32x2_t w;
  w[0] = f32_to_bf16_bits(v[0] * scale) | (f32_to_bf16_bits(v[1] * scale) << 16);
  w[1] = f32_to_bf16_bits(v[2] * scale) | (f32_to_bf16_bits(v[3] * scale) << 16);
  *(u32x2_t*)p = w;
}

template <>
__device__ __forceinline__ void store4<F32>(float* p, const f32x4_t& v, float scale) {
  *(f32x4_t*)p = v * scale;
}

template <>
__device__ __forceinline__ void store4<E4m3>(uint8_t* p, const f32x4_t& v, float scale) {
  *(uint32_t*)p = f32x4_to_e4m3(v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale);
}

// Exclusive prefix sum over a 1024-thread block; returns the block total in *total.
// Every thread of the block must call it (it synchronizes the block).
__device__ inline int block_exclusive_scan(int x, int* total) {
  __shared__ int wave_tot[16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wave_tot[wv] = inc;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    int t = wave_tot[w];
    if (w < wv) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - x;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

__device__ __forceinline__ int wave_in_block() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

}  // namespace fm
