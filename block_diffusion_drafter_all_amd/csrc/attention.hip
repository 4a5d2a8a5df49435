// Paged cross-attention (with its per-step plan and split merge) and block
// self-attention for gfx950.
//
// Cross-attention follows the draft step of the flashmap 0.1.0 wheel
// (sglang/model.py ``forward``, ``_paged_cross_attention``, ``rms_norm_rope``;
// vllm/model.py ``paged_cross_attention``): each request's draft rows attend,
// non-causally, to the keys/values at positions 0..ctx_len-1 of its paged
// context.  Work unit = (request, context split, head), one wavefront each:
//   - the unit's 16 query rows are RMS-normed and rotated in registers;
//   - 16-token tiles of K and V are read straight from the pages into MFMA
//     operand layout (16-byte loads, DEPTH tiles in flight per wave);
//   - S^T = K Q^T puts each lane on one query row with four keys, which is
//     exactly the operand layout of O^T = V^T P^T, so the online softmax and
//     its rescale stay in registers; V is moved to column layout by an MFMA
//     against a 0/1 selection matrix;
//   - a request split over several units writes (m, l, O) partials that a
//     second kernel merges in split order (deterministic).
// Self-attention (``block_self_attention``): one wavefront per (block, head)
// holds the whole 16-slot block.

#include "fm_internal.h"

namespace fm {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// ------------------------------------------------------------------- plan --

__global__ __launch_bounds__(1024) void plan_kernel(PlanArgs a) {
  __shared__ unsigned long long total_ctx;
  uint8_t* ws = a.ws;
  PlanHeader* hdr = (PlanHeader*)ws;
  int32_t* first_entry = (int32_t*)(ws + a.lay.first_entry);
  int32_t* n_splits = (int32_t*)(ws + a.lay.n_splits);
  int2* entries = (int2*)(ws + a.lay.entries);
  const int tid = threadIdx.x;
  if (tid == 0) total_ctx = 0;
  __syncthreads();
  unsigned long long mine = 0;
  for (int b = tid; b < a.bs; b += 1024) mine += (unsigned long long)max(0, a.ctx_lens[b]);
  atomicAdd(&total_ctx, mine);
  __syncthreads();
  const unsigned long long target = (unsigned long long)plan_target_entries(a.H);
  unsigned long long s64 = (total_ctx + target - 1) / target;
  if (s64 < (unsigned long long)a.min_split) s64 = (unsigned long long)a.min_split;
  s64 = (s64 + 15) & ~15ull;
  if (s64 > (1ull << 30)) s64 = 1ull << 30;
  const int S = (int)s64;
  int carry = 0;
  for (int base = 0; base < a.bs; base += 1024) {
    const int b = base + tid;
    int n = 0;
    if (b < a.bs) {
      const int ctx = max(0, a.ctx_lens[b]);
      n = max(1, (int)(((long long)ctx + S - 1) / S));
    }
    int block_total;
    const int first = carry + block_exclusive_scan(n, &block_total);
    if (b < a.bs) {
      first_entry[b] = first;
      n_splits[b] = n;
      for (int s = 0; s < n; ++s)
        if (first + s < a.lay.max_entries) entries[first + s] = make_int2(b, s);
    }
    carry += block_total;
  }
  if (tid == 0) {
    hdr->magic = kPlanMagic;
    hdr->error = carry > a.lay.max_entries ? 2 : 0;
    hdr->n_entries = min(carry, a.lay.max_entries);
    hdr->split_tokens = S;
    hdr->bs = a.bs;
    hdr->H = a.H;
    hdr->max_entries = a.lay.max_entries;
  }
}

// -------------------------------------------------------- cross-attention --

template <class T, int D>
struct KVTile {
  u32x4_t k[D / (4 * T::EPC)];
  u32x4_t v[D / (4 * T::EPC)];
  uint32_t mask;  // bit t: token t of the tile is a valid key
};

template <class T, int D, int DEPTH>
__global__ __launch_bounds__(256) void cross_attn_kernel(CrossArgs a) {
  typedef typename T::storage st;
  constexpr int EPC = T::EPC;
  constexpr int NCH = D / (4 * EPC);
  constexpr int NDT = D / 16;
  const int lane = lane_id(), g = lane >> 4, c = lane & 15;
  uint8_t* ws = a.ws;
  PlanHeader* hdr = (PlanHeader*)ws;
  if (hdr->magic != kPlanMagic || hdr->bs != a.bs || hdr->H != a.H) return;
  const int unit = blockIdx.x * 4 + wave_in_block();
  const int e = unit / a.H;
  const int h = unit - e * a.H;
  if (e >= hdr->n_entries) return;
  const int2 ent = ((const int2*)(ws + a.lay.entries))[e];
  const int b = ent.x, split = ent.y;
  const int S = hdr->split_tokens;
  const int nsplit = ((const int32_t*)(ws + a.lay.n_splits))[b];
  const int ctx0 = max(0, a.ctx_lens[b]);
  const int64_t cap = a.pt_stride << a.log2ps;
  const int ctx = (int64_t)ctx0 > cap ? (int)cap : ctx0;
  const int t0 = split * S;
  const int t1 = min(ctx, t0 + S);
  const int r0 = max(0, a.cu_q[b]);
  const int nq = max(0, min(min(a.cu_q[b + 1], a.total_q) - r0, kQRows));

  // Query prologue: RMSNorm + RoPE at position ctx_len + k, in registers.
  float qf[D / 4];
  if (c < nq) {
    const st* qrow = (const st*)a.q + ((int64_t)(r0 + c) * a.H + h) * D;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const u32x4_t v = load16(qrow + ch * 4 * EPC + g * EPC);
#pragma unroll
      for (int j = 0; j < EPC; ++j) qf[ch * EPC + j] = chunk_elem<T>(v, j);
    }
  } else {
#pragma unroll
    for (int k = 0; k < D / 4; ++k) qf[k] = 0.f;
  }
  norm_rope_row<T, D>(qf, a.q_norm_w, a.eps, ctx0 + c, a.rope, g);
  u32x4_t qop[NCH];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) qop[ch] = pack_chunk<T>(&qf[ch * EPC]);

  Selector<T> sel;
  sel.init(lane);

  const st* kbase = (const st*)a.pool.k + (int64_t)h * a.pool.head_stride;
  const st* vbase = (const st*)a.pool.v + (int64_t)h * a.pool.head_stride;
  const int32_t* pt_row = a.page_table + (int64_t)b * a.pt_stride;
  const int ps_mask = (1 << a.log2ps) - 1;

  // Page ids of 64 consecutive logical pages, one per lane.
  int wbase = t0 >> a.log2ps;
  auto load_window = [&](int base) -> int {
    const int64_t idx = (int64_t)base + lane;
    return idx < a.pt_stride ? pt_row[idx] : -1;
  };
  int pw = load_window(wbase);

  auto load_tile = [&](KVTile<T, D>& tl, int tb) {
    const int last = min(tb + 15, t1 - 1);
    if ((last >> a.log2ps) - wbase >= 64) {
      wbase = tb >> a.log2ps;
      pw = load_window(wbase);
    }
    const int tok = tb + c;
    const bool in_range = tok < t1;
    const int page = __shfl(pw, ((tok >> a.log2ps) - wbase) & 63);
    const bool ok = in_range && page >= 0 && (int64_t)page < a.pool.num_pages;
    if (in_range && !ok) atomicOr(&hdr->error, 1);
    const int64_t off =
        ok ? (int64_t)page * a.pool.page_stride + (int64_t)(tok & ps_mask) * a.pool.slot_stride : 0;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      tl.k[ch] = load16(kbase + off + ch * 4 * EPC + g * EPC);
      tl.v[ch] = load16(vbase + off + ch * 4 * EPC + g * EPC);
    }
    tl.mask = (uint32_t)(__ballot(ok) & 0xffffull);
  };

  f32x4_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;  // running max of this lane's query row (log2 domain)
  float l_lane = 0.f;     // this lane's share of the running denominator

  auto compute_tile = [&](const KVTile<T, D>& tl) {
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) mma_chunk<T>(s, tl.k[ch], qop[ch]);
    float sv[4];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = (tl.mask >> (4 * g + i)) & 1u;
      sv[i] = valid ? s[i] * a.qscale_log2 : kNegInf;
      mx = fmaxf(mx, sv[i]);
    }
    mx = wave_max_groups(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    f32x4_t p;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = operand_value<T>(exp2f(sv[i] - m_use));
      psum += p[i];
    }
    l_lane = l_lane * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      o[dt] *= alpha;
      const f32x4_t vt = sel.template transpose_tile<NCH>(tl.v, dt);
      mma_pv<T>(o[dt], vt, p);
    }
  };

  const int n_tiles = t1 > t0 ? (t1 - t0 + 15) >> 4 : 0;
  KVTile<T, D> buf[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d)
    if (d < n_tiles) load_tile(buf[d], t0 + 16 * d);
  for (int it = 0; it < n_tiles; it += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int i = it + d;
      if (i < n_tiles) {
        const int pf = i + DEPTH - 1;
        if (pf < n_tiles) load_tile(buf[(d + DEPTH - 1) % DEPTH], t0 + 16 * pf);
        compute_tile(buf[d]);
      }
    }
  }

  const float l_row = wave_sum_groups(l_lane);
  if (nsplit <= 1) {
    const float inv = l_row > 0.f ? 1.0f / l_row : 0.f;
    if (c < nq) {
      st* orow = (st*)a.out + ((int64_t)(r0 + c) * a.H + h) * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) store4<T>(orow + 16 * dt + 4 * g, o[dt], inv);
    }
  } else {
    const int64_t prow = ((int64_t)e * a.H + h) * kQRows + c;
    float* po = (float*)(ws + a.lay.partial_o) + prow * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *(f32x4_t*)(po + 16 * dt + 4 * g) = o[dt];
    if (g == 0) {
      float* pml = (float*)(ws + a.lay.partial_ml) + prow * 2;
      pml[0] = m_run;
      pml[1] = l_row;
    }
  }
}

// Merge of a split request: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// summed in split order.  One wavefront per (request, head).
template <class T, int D>
__global__ __launch_bounds__(256) void merge_kernel(CrossArgs a) {
  typedef typename T::storage st;
  constexpr int NPL = D / 4;  // columns per lane
  const int lane = lane_id(), g = lane >> 4, row = lane & 15;
  const uint8_t* ws = a.ws;
  const PlanHeader* hdr = (const PlanHeader*)ws;
  if (hdr->magic != kPlanMagic || hdr->bs != a.bs || hdr->H != a.H) return;
  const int unit = blockIdx.x * 4 + wave_in_block();
  const int b = unit / a.H;
  const int h = unit - b * a.H;
  if (b >= a.bs) return;
  const int nsplit = ((const int32_t*)(ws + a.lay.n_splits))[b];
  if (nsplit <= 1) return;
  const int first = ((const int32_t*)(ws + a.lay.first_entry))[b];
  const int r0 = max(0, a.cu_q[b]);
  const int nq = max(0, min(min(a.cu_q[b + 1], a.total_q) - r0, kQRows));
  const float* pml = (const float*)(ws + a.lay.partial_ml);
  const float* po = (const float*)(ws + a.lay.partial_o);
  float M = kNegInf;
  for (int s = 0; s < nsplit && first + s < hdr->n_entries; ++s)
    M = fmaxf(M, pml[(((int64_t)(first + s) * a.H + h) * kQRows + row) * 2]);
  float acc[NPL];
#pragma unroll
  for (int k = 0; k < NPL; ++k) acc[k] = 0.f;
  float L = 0.f;
  if (M != kNegInf) {
    for (int s = 0; s < nsplit && first + s < hdr->n_entries; ++s) {
      const int64_t prow = ((int64_t)(first + s) * a.H + h) * kQRows + row;
      const float wgt = exp2f(pml[prow * 2] - M);
      L += wgt * pml[prow * 2 + 1];
      const float* src = po + prow * D + g * NPL;
#pragma unroll
      for (int k = 0; k < NPL; k += 4) {
        const f32x4_t v = *(const f32x4_t*)(src + k);
        acc[k] += wgt * v[0];
        acc[k + 1] += wgt * v[1];
        acc[k + 2] += wgt * v[2];
        acc[k + 3] += wgt * v[3];
      }
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  if (row < nq) {
    st* orow = (st*)a.out + ((int64_t)(r0 + row) * a.H + h) * D + g * NPL;
#pragma unroll
    for (int k = 0; k < NPL; k += 4) {
      const f32x4_t v = {acc[k], acc[k + 1], acc[k + 2], acc[k + 3]};
      store4<T>(orow + k, v, inv);
    }
  }
}

// --------------------------------------------------------- self-attention --

template <class T, int D>
__global__ __launch_bounds__(256) void self_attn_kernel(SelfArgs a) {
  typedef typename T::storage st;
  constexpr int EPC = T::EPC;
  constexpr int NCH = D / (4 * EPC);
  constexpr int NDT = D / 16;
  const int lane = lane_id(), g = lane >> 4, c = lane & 15;
  const int unit = blockIdx.x * 4 + wave_in_block();
  const int b = unit / a.H;
  const int h = unit - b * a.H;
  if (b >= a.n_blocks) return;
  const int K = a.K;
  const int ctx = max(0, a.ctx_lens[b]);
  const bool has = c < K;
  const int64_t slot_stride = (int64_t)3 * a.H * D;
  const st* base = (const st*)a.qkv + ((int64_t)b * K + (has ? c : 0)) * slot_stride + (int64_t)h * D;

  float qf[D / 4], kf[D / 4];
  u32x4_t vr[NCH];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const int col = ch * 4 * EPC + g * EPC;
    u32x4_t vq = load16(base + col);
    u32x4_t vk = load16(base + (int64_t)a.H * D + col);
    vr[ch] = load16(base + (int64_t)2 * a.H * D + col);
    if (!has) {
      vq = (u32x4_t){0u, 0u, 0u, 0u};
      vk = vq;
      vr[ch] = vq;
    }
#pragma unroll
    for (int j = 0; j < EPC; ++j) {
      qf[ch * EPC + j] = chunk_elem<T>(vq, j);
      kf[ch * EPC + j] = chunk_elem<T>(vk, j);
    }
  }
  norm_rope_row<T, D>(qf, a.q_norm_w, a.eps, ctx + c, a.rope, g);
  norm_rope_row<T, D>(kf, a.k_norm_w, a.eps, ctx + c, a.rope, g);
  u32x4_t qop[NCH], kop[NCH];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    qop[ch] = pack_chunk<T>(&qf[ch * EPC]);
    kop[ch] = pack_chunk<T>(&kf[ch * EPC]);
  }
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) mma_chunk<T>(s, kop[ch], qop[ch]);
  // lane (g, c): query row c against keys 4g .. 4g+3
  float sv[4];
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sv[i] = (4 * g + i < K) ? s[i] * a.qscale_log2 : kNegInf;
    mx = fmaxf(mx, sv[i]);
  }
  mx = wave_max_groups(mx);
  f32x4_t p;
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = operand_value<T>(exp2f(sv[i] - mx));
    l += p[i];
  }
  l = wave_sum_groups(l);
  Selector<T> sel;
  sel.init(lane);
  const float inv = 1.0f / l;
  // MFMAs run with every lane active; only the stores are predicated.
  f32x4_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    o[dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    mma_pv<T>(o[dt], sel.template transpose_tile<NCH>(vr, dt), p);
  }
  if (has) {
    st* orow = (st*)a.out + (((int64_t)b * K + c) * a.H + h) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) store4<T>(orow + 16 * dt + 4 * g, o[dt], inv);
  }
}

template <class T, int D>
hipError_t launch_cross_typed(const CrossArgs& a, hipStream_t s) {
  const int64_t units = (int64_t)a.lay.max_entries * a.H;
  if (units > 0) {
    const unsigned grid = (unsigned)((units + 3) / 4);
    hipLaunchKernelGGL((cross_attn_kernel<T, D, 3>), dim3(grid), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t merges = (int64_t)a.bs * a.H;
  if (merges > 0) {
    const unsigned grid = (unsigned)((merges + 3) / 4);
    hipLaunchKernelGGL((merge_kernel<T, D>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <class T, int D>
hipError_t launch_self_typed(const SelfArgs& a, hipStream_t s) {
  const int64_t units = (int64_t)a.n_blocks * a.H;
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL((self_attn_kernel<T, D>), dim3((unsigned)((units + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cross_attention(const CrossArgs& a, int dtype, int Dh, hipStream_t s) {
  if (dtype == 1) return Dh == 128 ? launch_cross_typed<Bf16, 128>(a, s) : launch_cross_typed<Bf16, 64>(a, s);
  return Dh == 128 ? launch_cross_typed<F32, 128>(a, s) : launch_cross_typed<F32, 64>(a, s);
}

hipError_t launch_self_attention(const SelfArgs& a, int dtype, int Dh, hipStream_t s) {
  if (dtype == 1) return Dh == 128 ? launch_self_typed<Bf16, 128>(a, s) : launch_self_typed<Bf16, 64>(a, s);
  return Dh == 128 ? launch_self_typed<F32, 128>(a, s) : launch_self_typed<F32, 64>(a, s);
}

}  // namespace fm
