// Bidirectional self-attention within each draft block for gfx950 (flashmap
// 0.1.0 wheel: sglang/model.py ``_denoise`` -> ``block_self_attention``;
// vllm/model.py ``_dit``; modeling_flashmap.py ``FlashMapLayer``).
//
// One wavefront per (block, head, 16-slot query tile); a block holds up to 64
// slots (four tiles).  q and k are RMS-normed and rotated at the slots'
// positions in registers, S^T = K Q^T leaves each lane one query row with four
// keys per key tile, the softmax over the block's keys reduces across the key
// tiles and the four lane groups, and O^T = V^T P^T takes P straight from the
// score layout (V moved to column layout by a selection-matrix MFMA).

#include "fm_internal.h"

namespace fm {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// RMSNorm of a slot's q and k fragments (weights wq, wk), then the
// interleaved-pair rotation of both at the slot's position.  q and k turn by
// the same angles, so each sine and cosine is evaluated once for the two;
// every element sees the same operations as one row through norm_rope_row.
template <class T, int D>
__device__ __forceinline__ void norm_rope_qk(float (&q)[D / 4], float (&k)[D / 4], const float* __restrict__ wq,
                                             const float* __restrict__ wk, float eps, int pos, const RopeFreqs& rf,
                                             int g) {
  constexpr int EPC = T::EPC;
  constexpr int NCH = D / (4 * EPC);
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int i = 0; i < D / 4; ++i) {
    sq += q[i] * q[i];
    sk += k[i] * k[i];
  }
  sq = wave_sum_groups(sq);
  sk = wave_sum_groups(sk);
  const float rq = 1.0f / sqrtf(sq / (float)D + eps);
  const float rk = 1.0f / sqrtf(sk / (float)D + eps);
  const float fpos = (float)pos;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
    for (int j = 0; j < EPC; j += 2) {
      const int col = ch * 4 * EPC + g * EPC + j;
      const int f0 = ch * 2 * EPC + j / 2;  // frequency index col / 2, by lane group
      const float inv = sel4(g, rf.inv[f0], rf.inv[f0 + EPC / 2], rf.inv[f0 + EPC], rf.inv[f0 + 3 * EPC / 2]);
      float sn, cs;
      angle_sincos(fpos * inv, &sn, &cs);
      const int e = ch * EPC + j;
      const float q0 = q[e] * rq * wq[col], q1 = q[e + 1] * rq * wq[col + 1];
      const float k0 = k[e] * rk * wk[col], k1 = k[e + 1] * rk * wk[col + 1];
      q[e] = q0 * cs - q1 * sn;
      q[e + 1] = q1 * cs + q0 * sn;
      k[e] = k0 * cs - k1 * sn;
      k[e + 1] = k1 * cs + k0 * sn;
    }
  }
}

// --------------------------------------------------------- self-attention --

// One wavefront per (block, head, 16-slot query tile).  A block of K <= 64
// slots is NKT = 1, 2 or 4 key tiles of 16; the wave scores its query tile
// against every key tile, takes the exact softmax over all K keys (one max,
// one sum) and adds up the key tiles' weighted values.  With one key tile
// (K <= 16) this is the whole block in one wave.
template <class T, int D, int NKT>
__global__ __launch_bounds__(256) void self_attn_kernel(SelfArgs a) {
  typedef typename T::storage st;
  constexpr int EPC = T::EPC;
  constexpr int NCH = D / (4 * EPC);
  constexpr int NDT = D / 16;
  const int lane = lane_id(), g = lane >> 4, c = lane & 15;
  const int K = a.K;
  const int nqt = (K + 15) >> 4;  // query tiles of a block
  const int unit = blockIdx.x * 4 + wave_in_block();
  const int bh = unit / nqt;
  const int ft = unit - bh * nqt;  // this wave's query tile
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  if (b >= a.n_blocks) return;
  const int ctx = max(0, a.ctx_lens[b]);
  const int64_t slot_stride = (int64_t)3 * a.H * D;
  // row c of tile t: slot 16 t + c (clamped reads for slots past the block, zeroed)
  auto slot_base = [&](int t) -> const st* {
    const int i = 16 * t + c;
    return (const st*)a.qkv + ((int64_t)b * K + (i < K ? i : 0)) * slot_stride + (int64_t)h * D;
  };
  auto load_rows = [&](int t, int which, float (&x)[D / 4]) {
    const bool has = 16 * t + c < K;
    const st* p = slot_base(t) + (int64_t)which * a.H * D;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      u32x4_t v = load16(p + ch * 4 * EPC + g * EPC);
      if (!has) v = (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < EPC; ++j) x[ch * EPC + j] = chunk_elem<T>(v, j);
    }
  };

  // Query tile ft and key tile ft sit at the same positions: normed and
  // rotated together (one sine and cosine per pair for both).
  u32x4_t qop[NCH];
  f32x4_t s[NKT];
  {
    float qf[D / 4], kf[D / 4];
    load_rows(ft, 0, qf);
    load_rows(ft, 1, kf);
    norm_rope_qk<T, D>(qf, kf, a.q_norm_w, a.k_norm_w, a.eps, ctx + 16 * ft + c, a.rope, g);
    u32x4_t kop[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      qop[ch] = pack_chunk<T>(&qf[ch * EPC]);
      kop[ch] = pack_chunk<T>(&kf[ch * EPC]);
    }
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      s[kt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      if (kt == ft) {
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) mma_chunk<T>(s[kt], kop[ch], qop[ch]);
      }
    }
  }
  // The other key tiles, each normed and rotated at its own slots' positions.
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    if (kt == ft || kt >= nqt) continue;
    float kf[D / 4];
    load_rows(kt, 1, kf);
    norm_rope_row<T, D>(kf, a.k_norm_w, a.eps, ctx + 16 * kt + c, a.rope, g);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) mma_chunk<T>(s[kt], pack_chunk<T>(&kf[ch * EPC]), qop[ch]);
  }
  // lane (g, c): query row c against keys 16 kt + 4g .. 16 kt + 4g + 3
  float sv[NKT][4];
  float mx = kNegInf;
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[kt][i] = (16 * kt + 4 * g + i < K) ? s[kt][i] * a.qscale_log2 : kNegInf;
      mx = fmaxf(mx, sv[kt][i]);
    }
  mx = wave_max_groups(mx);
  f32x4_t p[NKT];
  float l = 0.f;
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[kt][i] = operand_value<T>(exp2f(sv[kt][i] - mx));
      l += p[kt][i];
    }
  l = wave_sum_groups(l);
  Selector<T> sel;
  sel.init(lane);
  const float inv = 1.0f / l;
  // MFMAs run with every lane active; only the stores are predicated.
  f32x4_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    if (kt >= nqt) continue;
    const bool has = 16 * kt + c < K;
    const st* vp = slot_base(kt) + (int64_t)2 * a.H * D;
    u32x4_t vr[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      vr[ch] = load16(vp + ch * 4 * EPC + g * EPC);
      if (!has) vr[ch] = (u32x4_t){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) mma_pv<T>(o[dt], sel.template transpose_tile<NCH>(vr, dt), p[kt]);
  }
  if (16 * ft + c < K) {
    st* orow = (st*)a.out + (((int64_t)b * K + 16 * ft + c) * a.H + h) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) store4<T>(orow + 16 * dt + 4 * g, o[dt], inv);
  }
}

template <class T, int D, int NKT>
hipError_t launch_self_tiles(const SelfArgs& a, hipStream_t s) {
  const int64_t units = (int64_t)a.n_blocks * a.H * ((a.K + 15) / 16);
  if (units <= 0) return hipSuccess;
  if (!grid_fits((units + 3) / 4, 256)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((self_attn_kernel<T, D, NKT>), dim3((unsigned)((units + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class T, int D>
hipError_t launch_self_typed(const SelfArgs& a, hipStream_t s) {
  if (a.K <= 16) return launch_self_tiles<T, D, 1>(a, s);
  if (a.K <= 32) return launch_self_tiles<T, D, 2>(a, s);
  return launch_self_tiles<T, D, 4>(a, s);
}

}  // namespace

hipError_t launch_self_attention(const SelfArgs& a, int dtype, int Dh, hipStream_t s) {
  if (dtype == 1) return Dh == 128 ? launch_self_typed<Bf16, 128>(a, s) : launch_self_typed<Bf16, 64>(a, s);
  return Dh == 128 ? launch_self_typed<F32, 128>(a, s) : launch_self_typed<F32, 64>(a, s);
}

}  // namespace fm
