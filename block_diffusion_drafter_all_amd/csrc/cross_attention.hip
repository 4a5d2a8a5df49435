// Paged cross-attention for gfx950: the per-step plan, the streaming
// attention kernel and the merge of pairs cut between waves.
//
// What is computed (flashmap 0.1.0 wheel: sglang/model.py ``forward``,
// ``_paged_cross_attention``, ``rms_norm_rope``; vllm/model.py
// ``paged_cross_attention``): each request's draft rows, RMS-normed and
// rotated at positions ctx_len + (k mod 16), attend non-causally to the
// keys/values at positions 0..ctx_len-1 of the request's paged context.  A
// request holds one draft block of 16 rows or, in tree drafting, up to four
// candidate blocks side by side, which share one read of its context: each
// 16-row block is one MFMA fragment (NQF fragments per request).
//
// How.  The work is the stream of 16-token K/V tiles of every (request, head)
// pair.  The plan cuts it into one equal contiguous range per resident
// wavefront; each wave streams its range with DEPTH tiles in flight and never
// restarts its load pipeline at a pair boundary: the loader walks on to the
// next pair and carries that pair's query rows along with its first tile.
//   - with pages of at least 16 tokens (one page per tile) K/V tiles arrive
//     in a per-wave LDS ring by direct buffer->LDS loads of whole rows
//     (nontemporal), chunks XOR-swizzled so the operand reads hit every bank;
//     with smaller pages they are read straight into MFMA operand layout
//     (16-byte loads into a register ring).  Page ids are read one tile ahead:
//     one scalar load of the page-table entry for pages of >= 16 tokens, else
//     from a per-wave LDS window of the request's page row; either way waiting
//     for one never waits for K/V loads in flight;
//   - S^T = K Q^T leaves each lane one query row and four keys, which is the
//     B-operand layout of O^T = V^T P^T, so the online softmax and its rescale
//     stay in registers; V reaches column layout through gfx950's LDS
//     transpose reads (bf16 and e4m3 tiles in LDS) or, in the register ring,
//     by an MFMA against a 0/1 selection matrix;
//   - a pair that lies inside one wave's range is written final; a pair cut by
//     range boundaries leaves (m, l, O) partials, and the last of its waves to
//     finish adds them up in wave order in the kernel's tail (deterministic).

#include <type_traits>

#include "fm_internal.h"

namespace fm {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;  // lazy online-softmax rescale: p stays <= 2^8 between rescales
constexpr int kWin = 512;  // page ids cached per wave

#ifndef FM_CROSS_DEPTH_BF16
#define FM_CROSS_DEPTH_BF16 3  // 16-token K/V tiles per wave in the load/compute ring (bf16)
#endif
#ifndef FM_CROSS_DEPTH_F32
#define FM_CROSS_DEPTH_F32 2
#endif
#ifndef FM_CROSS_LDS_KV
#define FM_CROSS_LDS_KV 1  // pages of >= 16 tokens: K/V tiles stream through LDS (whole-line, nontemporal loads)
#endif
#ifndef FM_CROSS_LDS_KV_MAXQF
#define FM_CROSS_LDS_KV_MAXQF 4  // ... for kernels of at most this many query fragments (every count: with the
                                  // bf16 V tile read transposed from LDS, four fragments gain too)
#endif
#ifndef FM_CROSS_DEPTH_LDS
#define FM_CROSS_DEPTH_LDS 2  // tiles in flight per wave through LDS (the loads hold no registers)
#endif

// s_waitcnt with vmcnt(n) only (expcnt and lgkmcnt left at their maxima).
constexpr int wait_vm_only(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kLoadNT = 2;  // nt in the buffer instructions' cache-policy operand: streamed once, not kept

// Slot flags.
// Tile flags, kept above the 16 key-mask bits of a stream slot's word.
constexpr uint32_t kStart = 1u << 16;  // first tile of a segment: reset the softmax state, take the query rows
constexpr uint32_t kEnd = 2u << 16;    // last tile of a segment: write the output or a partial
constexpr uint32_t kWhole = 4u << 16;  // the segment is the whole (request, head) pair: final output
constexpr uint32_t kPart1 = 8u << 16;  // partial goes to the wave's second partial slot
constexpr uint32_t kKeyMask = 0xFFFFu;

__device__ __forceinline__ int64_t shfl_up_i64(int64_t x, int d) {
  const int lo = __shfl_up((int)(uint32_t)(uint64_t)x, d);
  const int hi = __shfl_up((int)(uint32_t)((uint64_t)x >> 32), d);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Exclusive prefix sum of int64 over a 1024-thread block (all threads call it).
__device__ int64_t block_exclusive_scan_i64(int64_t x, int64_t* total) {
  __shared__ int64_t wave_tot[16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int64_t inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = shfl_up_i64(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wave_tot[wv] = inc;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    const int64_t t = wave_tot[w];
    if (w < wv) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - x;
}

__device__ __forceinline__ int tiles_of(int ctx) { return (max(ctx, 0) + 15) >> 4; }

// Partials cross waves on different XCDs, whose L2s are not coherent with one
// another.  They are written and read with the device-scope cache bit (sc1),
// which writes through and reads past the non-coherent cache levels, so no
// cache-wide write-back or invalidate is needed; the counter increment is
// ordered after a wave's partial stores by waiting for all of them to be
// acknowledged.  Buffer instructions also drop anything outside the partials.
constexpr int kDeviceScope = 16;         // sc1 in the buffer instructions' cache-policy operand
constexpr int kRsrcWord3 = 0x00020000;   // raw 32-bit buffer on gfx9-family targets
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t partials_rsrc(const CrossArgs& a) {
  return __builtin_amdgcn_make_buffer_rsrc(a.ws + a.lay.partial_ml, 0, (int)(a.lay.total - a.lay.partial_ml),
                                           kRsrcWord3);
}
__device__ __forceinline__ void wait_stores_acknowledged() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------------------------- plan --

// First tile of wave w's share of G tiles over NW waves, shares weighted by
// the XCD each wave runs on (share_start(w = NW) = G).  Workgroups go
// round-robin over the 8 XCDs, so wave w (4 per workgroup) runs on XCD
// (w / 4) mod 8.  The weights are inputs: the cut depends only on them and
// on the lengths, and so do the results.
//
// The share is floor(G wb / wt), wb the weight of waves 0 .. w-1 and wt that
// of all NW.  With G = Q wt + R it is Q wb + floor(R wb / wt).  Both
// quotients come from doubles (R wb < wt^2 < 2^46 is exact; G below 2^52),
// each at most one off its floor, which one product settles: no 64-bit
// integer division.
struct ShareSplit {
  int64_t Q, R, wt;
};

__device__ __forceinline__ int64_t floor_div_checked(int64_t num, int64_t den) {  // num >= 0, den > 0
  int64_t f = (int64_t)((double)num / (double)den);
  if (f * den > num) --f;
  else if ((f + 1) * den <= num) ++f;
  return f;
}

__device__ __forceinline__ int64_t weight_before(int v, const int32_t* W) {  // total weight of waves 0 .. v-1
  int64_t sum8 = 0;
#pragma unroll
  for (int x = 0; x < kXcds; ++x) sum8 += W[x];
  const int64_t blk = v >> 2, part = v & 3;  // whole workgroups before v, and v's own waves before it
  const int64_t turns = blk / kXcds, rem = blk % kXcds;
  int64_t acc = 4 * turns * sum8;
#pragma unroll
  for (int x = 0; x < kXcds; ++x) acc += x < rem ? 4 * (int64_t)W[x] : 0;
  return acc + part * W[rem];
}

__device__ __forceinline__ int64_t share_start(const ShareSplit& sp, int w, const int32_t* W) {
  const int64_t wb = weight_before(w, W);
  return sp.Q * wb + floor_div_checked(sp.R * wb, sp.wt);
}

// Batches up to this many requests keep each request's length and first
// tile in LDS, so the plan's searches and lookups never wait on memory.
constexpr int kPlanLdsRequests = 2048;
constexpr int kPlanMaxGroups = 64;

// kLds: bs <= kPlanLdsRequests.  Then every workgroup of the grid builds the
// request tables and the wave shares in its own LDS, and the workgroups split
// the wave and pair records between them.  Otherwise one workgroup, which
// reads the request tables back from the workspace.
template <bool kLds>
__global__ __launch_bounds__(1024) void plan_kernel(PlanArgs a) {
  uint8_t* ws = a.ws;
  PlanHeader* hdr = (PlanHeader*)ws;
  int64_t* pair_off = (int64_t*)(ws + a.lay.pair_off);
  WaveRec* rec = (WaveRec*)(ws + a.lay.wave_rec);
  PairRec* prec = (PairRec*)(ws + a.lay.pair_rec);
  int32_t* cnt = (int32_t*)(ws + a.lay.merge_cnt);
  __shared__ int64_t starts[kMaxPlanWaves + 1];
  __shared__ int64_t lds_off[kLds ? kPlanLdsRequests + 1 : 1];
  __shared__ int32_t lds_ctx[kLds ? kPlanLdsRequests : 1];
  const int64_t* off = kLds ? lds_off : pair_off;  // first tile of request b's pairs in the stream
  auto ctx_of = [&](int b) -> int { return kLds ? lds_ctx[b] : max(0, a.ctx_lens[b]); };
  const int tid = threadIdx.x;
  const bool lead = blockIdx.x == 0;  // writes the workspace's request table and header
  int64_t carry = 0;
  for (int base = 0; base < a.bs; base += 1024) {
    const int b = base + tid;
    const int ctx = b < a.bs ? max(0, a.ctx_lens[b]) : 0;
    int64_t tot;
    const int64_t ex = block_exclusive_scan_i64((int64_t)tiles_of(ctx) * a.H, &tot);
    if (b < a.bs) {
      if (lead) pair_off[b] = carry + ex;
      if constexpr (kLds) {
        lds_off[b] = carry + ex;
        lds_ctx[b] = ctx;
      }
    }
    carry += tot;
  }
  if (tid == 0) {
    if (lead) pair_off[a.bs] = carry;
    if constexpr (kLds) lds_off[a.bs] = carry;
  }
  const int64_t G = carry;
  const int NW = a.lay.n_waves;
  ShareSplit sp;
  sp.wt = weight_before(NW, a.xcd_w);
  sp.Q = floor_div_checked(G, sp.wt);
  sp.R = G - sp.Q * sp.wt;
  for (int w = tid; w <= NW; w += 1024) starts[w] = share_start(sp, w, a.xcd_w);
  __syncthreads();
  const int first = blockIdx.x * 1024 + tid, stride = gridDim.x * 1024;
  for (int w = first; w < NW; w += stride) {
    const int64_t g0 = starts[w], g1 = starts[w + 1];
    WaveRec r{};
    r.start = g0;
    if (g1 > g0) {
      // the request whose pairs hold tile g0: the largest b with off[b] <= g0
      int lo = 0, hi = a.bs - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= g0) lo = mid;
        else hi = mid - 1;
      }
      const int ctx = ctx_of(lo);
      const int T = tiles_of(ctx);
      const int64_t rel = g0 - off[lo];  // < H * T
      r.b = lo;
      if (rel <= INT32_MAX) {  // 32-bit division where it fits
        r.h = (int)rel / T;
        r.k = (int)rel - r.h * T;
      } else {
        r.h = (int)(rel / T);
        r.k = (int)(rel % T);
      }
      r.count = (int)(g1 - g0);
      r.ctx = ctx;
    }
    rec[w] = r;
    cnt[w] = 0;
  }
  // Each pair's first and last wave (the last wave whose range starts at or
  // before its first and last tile), and how many waves hold a part of it.
  // The shares are near-proportional (XCD weights within 1 : 4), so the
  // proportional guess is a few waves off at most: a short walk from it, and
  // a bisection of what is left if the walk runs long.
  auto wave_of = [&](int64_t x) -> int {
    int w = (int)min((int64_t)NW - 1, (int64_t)((double)x * NW / (double)G));
    for (int step = 0; step < 4; ++step) {
      if (starts[w] > x) --w;
      else if (w + 1 < NW && starts[w + 1] <= x) ++w;
      else return w;
    }
    int lo = 0, hi = NW - 1;
    if (starts[w] > x) hi = w - 1;
    else lo = w;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (starts[mid] <= x) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  const uint32_t pairs = (uint32_t)a.bs * (uint32_t)a.H;  // < 2^31 (checked by the host), so i never wraps
  for (uint32_t i = first; i < pairs; i += stride) {
    const int b = (int)(i / (uint32_t)a.H), h = (int)(i - (uint32_t)b * a.H);
    const int T = tiles_of(ctx_of(b));
    PairRec pr{};
    if (T > 0) {
      const int64_t P = off[b] + (int64_t)h * T;
      pr.w0 = wave_of(P);
      pr.w1 = wave_of(P + T - 1);
      pr.slot0 = starts[pr.w0] < P ? 1 : 0;
      for (int u = pr.w0; u <= pr.w1; ++u) pr.parts += starts[u + 1] > starts[u] ? 1 : 0;
    }
    prec[i] = pr;
  }
  if (lead && tid == 0) {
    hdr->magic = kPlanMagic;
    hdr->error = 0;
    hdr->n_waves = NW;
    hdr->bs = a.bs;
    hdr->H = a.H;
    hdr->nqf = a.lay.nqf;
    hdr->total_tiles = G;
    hdr->Dh = a.Dh;
    hdr->dtype = a.dtype;
  }
}

// Pool type code of a kernel instantiation (the fm_dtype value of the call).
template <class T, class PT>
__device__ constexpr int pool_type_code() {
  return std::is_same<PT, E4m3>::value ? 2 : (std::is_same<T, Bf16>::value ? 1 : 0);
}

// Whether the plan in the workspace was made for this call's sizes and pool
// type.  The layout past the header depends on all of them, so a call with any
// other value must neither read the plan's records nor write its own queries
// over them.
template <class T, class PT, int D, int NQF>
__device__ __forceinline__ bool plan_matches(const PlanHeader& ph, const CrossArgs& a) {
  return (ph.magic == kPlanMagic) & (ph.bs == a.bs) & (ph.H == a.H) & (ph.n_waves == a.lay.n_waves) &
         (ph.nqf == NQF) & (ph.Dh == D) & (ph.dtype == pool_type_code<T, PT>());
}

// ----------------------------------------------------------- query rows --

// q^ = RoPE(RMSNorm(q; q_norm_w, eps)) at position ctx_len + (k mod 16) for
// query row k of request b, stored as [b][k][h][:] for k < 16 NQF in the
// pool's storage type (rows past the request's count are zero), ready to be
// loaded as MFMA operands.  Over an e4m3 pool (sglang/model.py
// ``_paged_cross_attention_fp8``) the rows of one (request, head) share one
// scale, their largest magnitude / 448 (at least 1e-12 / 448), or the fixed
// per-tensor scale when one is given (vllm/model.py ``_dit``), and the stored
// e4m3 row is q^ / scale, rounded once from fp32; the scale goes to q_scale.
// A request with an empty context gets its zero output rows here instead.
// One wavefront per (request, head).  Launched for kernels of several query
// fragments (candidate blocks); the one-fragment kernel does the same work on
// its own rows (bf16 and fp32 rows: the same bits).
template <class T, class PT, int D, int NQF>
__global__ __launch_bounds__(256) void q_prologue_kernel(CrossArgs a) {
  typedef typename T::storage st;
  constexpr int EPC = T::EPC;
  constexpr int NCH = D / (4 * EPC);
  const int lane = lane_id(), g = lane >> 4, c = lane & 15;
  const int unit = blockIdx.x * 4 + wave_in_block();
  const int b = unit / a.H;
  const int h = unit - b * a.H;
  if (b >= a.bs) return;
  const int ctx0 = max(0, a.ctx_lens[b]);
  const int r0 = max(0, a.cu_q[b]);
  const int nq = max(0, min(min(a.cu_q[b + 1], a.total_q) - r0, kQRows * NQF));
  // A plan for other sizes keeps its records: no query row is written over them.
  const bool plan_ok = plan_matches<T, PT, D, NQF>(*(const PlanHeader*)a.ws, a);
  if constexpr (std::is_same<PT, E4m3>::value) {
    if (ctx0 == 0) {  // empty context: the output rows are zero
#pragma unroll
      for (int f = 0; f < NQF; ++f) {
        const int k = kQRows * f + c;
        if (k < nq) {
          st* orow = (st*)a.out + ((int64_t)(r0 + k) * a.H + h) * D;
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) *(u32x4_t*)(orow + ch * 4 * EPC + g * EPC) = (u32x4_t){0u, 0u, 0u, 0u};
        }
      }
      return;
    }
    if (!plan_ok) return;
    float qf[NQF][D / 4];
    float amax = 0.f;
#pragma unroll
    for (int f = 0; f < NQF; ++f) {
      const int k = kQRows * f + c;
      const bool has = k < nq;
      const st* qrow = (const st*)a.q + ((int64_t)(has ? r0 + k : 0) * a.H + h) * D;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const u32x4_t v = load16(qrow + ch * 4 * EPC + g * EPC);
#pragma unroll
        for (int j = 0; j < EPC; ++j) qf[f][ch * EPC + j] = has ? chunk_elem<T>(v, j) : 0.f;
      }
      norm_rope_row<T, D>(qf[f], a.q_norm_w, a.eps, ctx0 + c, a.rope, g);  // zero rows stay zero
#pragma unroll
      for (int j = 0; j < D / 4; ++j) amax = fmaxf(amax, fabsf(qf[f][j]));
    }
    float qs, r;
    if (a.q_static > 0.f) {
      qs = a.q_static;
      r = a.q_static_inv;
    } else {
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
      const float am = fmaxf(amax, 1e-12f);
      qs = am / 448.0f;
      r = 448.0f / am;
    }
    if (lane == 0) ((float*)(a.ws + a.lay.q_scale))[(int64_t)b * a.H + h] = qs;
#pragma unroll
    for (int f = 0; f < NQF; ++f) {
      const int k = kQRows * f + c;
      uint8_t* dst = (uint8_t*)(a.ws + a.lay.q_hat) + (((int64_t)b * kQRows * NQF + k) * a.H + h) * D;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {  // EPC (8) consecutive columns -> 8 codes
        const float* x = &qf[f][ch * EPC];
        const u32x2_t w = {f32x4_to_e4m3(x[0] * r, x[1] * r, x[2] * r, x[3] * r),
                           f32x4_to_e4m3(x[4] * r, x[5] * r, x[6] * r, x[7] * r)};
        *(u32x2_t*)(dst + ch * 4 * EPC + g * EPC) = w;
      }
    }
    return;
  }
#pragma unroll
  for (int f = 0; f < NQF; ++f) {
    const int k = kQRows * f + c;  // this lane's row of fragment f
    const bool has = k < nq;
    if (ctx0 == 0) {  // empty context: the output rows are zero
      if (has) {
        st* orow = (st*)a.out + ((int64_t)(r0 + k) * a.H + h) * D;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) *(u32x4_t*)(orow + ch * 4 * EPC + g * EPC) = (u32x4_t){0u, 0u, 0u, 0u};
      }
      continue;
    }
    if (!plan_ok) continue;
    float qf[D / 4];
    const st* qrow = (const st*)a.q + ((int64_t)(has ? r0 + k : 0) * a.H + h) * D;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const u32x4_t v = load16(qrow + ch * 4 * EPC + g * EPC);
#pragma unroll
      for (int j = 0; j < EPC; ++j) qf[ch * EPC + j] = has ? chunk_elem<T>(v, j) : 0.f;
    }
    norm_rope_row<T, D>(qf, a.q_norm_w, a.eps, ctx0 + c, a.rope, g);  // slot c of every candidate block
    st* dst = (st*)(a.ws + a.lay.q_hat) + (((int64_t)b * kQRows * NQF + k) * a.H + h) * D;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) *(u32x4_t*)(dst + ch * 4 * EPC + g * EPC) = pack_chunk<T>(&qf[ch * EPC]);
  }
}

// The output rows of every request with an empty context are zero: wave w
// writes those of requests w, w + n_waves, ... (the one-fragment kernels, which
// have no query prologue kernel).
template <class T, int D>
__device__ __forceinline__ void zero_empty_rows(const CrossArgs& a, int w) {
  typedef typename T::storage st;
  for (int b = w; b < a.bs; b += a.lay.n_waves) {
    if (sload_i32(a.ctx_lens + b) > 0) continue;
    const int r0 = max(0, sload_i32(a.cu_q + b));
    const int nq = max(0, min(min(sload_i32(a.cu_q + b + 1), a.total_q) - r0, kQRows));
    u32x4_t* o = (u32x4_t*)((st*)a.out + (int64_t)r0 * a.H * D);
    const int n16 = nq * a.H * D * (int)sizeof(st) / 16;
    for (int i = lane_id(); i < n16; i += 64) o[i] = (u32x4_t){0u, 0u, 0u, 0u};
  }
}

// The e4m3 query scale of one (request, head) whose 16 prepared rows the wave
// holds (x: this lane's values): the rows' largest magnitude / 448 (at least
// 1e-12 / 448), or the fixed per-tensor scale when one is given; r = 1 / qs.
struct QScale {
  float qs, r;
};
template <int N>
__device__ __forceinline__ QScale query_scale(const CrossArgs& a, const float (&x)[N]) {
  if (a.q_static > 0.f) return QScale{a.q_static, a.q_static_inv};
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < N; ++j) amax = fmaxf(amax, fabsf(x[j]));
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  const float am = fmaxf(amax, 1e-12f);
  return QScale{am / 448.0f, 448.0f / am};
}

// 16 consecutive columns x[0..15] times r as one chunk of e4m3 codes (nearest
// even, saturating at 448), column j in byte j.
__device__ __forceinline__ u32x4_t pack_e4m3_chunk(const float* x, float r) {
  u32x4_t v;
#pragma unroll
  for (int w = 0; w < 4; ++w) v[w] = f32x4_to_e4m3(x[4 * w] * r, x[4 * w + 1] * r, x[4 * w + 2] * r, x[4 * w + 3] * r);
  return v;
}

// -------------------------------------------------------- cross-attention --

// One K/V tile in the load ring.  With one query fragment, the pair's raw
// query rows ride along with its first tile (QN 16-byte chunks per lane, q),
// to be normed and rotated when that tile is computed; with more, the
// prepared rows are read then (q unused).  Which pair a tile belongs to is
// not stored: the compute side walks the same pair sequence as the loader.
template <class T, int D, int QN>
struct StreamSlot {
  u32x4_t k[D / (4 * T::EPC)];
  u32x4_t v[D / (4 * T::EPC)];
  u32x4_t q[QN > 0 ? QN : 1];
  uint32_t mf;  // bits 0-15: token t of the tile is a valid key; above: kStart, kEnd, kWhole, kPart1
};

// The type of the PV contraction's operands: an e4m3 pool's values enter it
// as bf16, which holds every e4m3 value exactly.
template <class T>
struct PvType {
  typedef T type;
};
template <>
struct PvType<E4m3> {
  typedef Bf16 type;
};

// The plan's record of the cut pair (b, h): its waves w0..w1, how many of
// them hold a part, and the partial slot of w0.
__device__ __forceinline__ PairRec pair_rec_of(const CrossArgs& a, int b, int h) {
  return ((const PairRec*)(a.ws + a.lay.pair_rec))[(int64_t)b * a.H + h];
}

// Counts this wave's partial of a cut pair in on the pair's counter (indexed
// by its first wave; this wave's partial stores must be acknowledged
// already) and returns the parts counted before it: the pair's last part
// sees pr.parts - 1.
__device__ __forceinline__ int count_in(const CrossArgs& a, const PairRec& pr) {
  int before = 0;
  if (lane_id() == 0)
    before = __hip_atomic_fetch_add((int32_t*)(a.ws + a.lay.merge_cnt) + pr.w0, 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
  return __shfl(before, 0);
}

// Combines the partials of the cut pair (b, h) in wave order, fragment by
// fragment,
//   O = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w,   M = max_w m_w,
// writes the output rows and re-arms the pair's counter for the next call.
// The parts are read kMergeBatch at a time: one round of loads (the waves'
// records with them) and one rescale per batch, so a pair cut over up to
// kMergeBatch waves costs one round trip.  Called by the wave that counted the
// last part in: every other part was acknowledged before it was counted.
// Lanes hold the same fragment of the rows as in the attention loop; COLS
// names the type whose column order (out_col) the fragments follow.
constexpr int kMergeBatch = 4;

template <class T, class COLS, int D, int NQF>
__device__ __forceinline__ void merge_pair(const CrossArgs& a, int b, int h, const PairRec& pr) {
  typedef typename T::storage st;
  constexpr int NDT = D / 16;
  const int lane = lane_id(), g = lane >> 4, c = lane & 15;
  const int w0 = pr.w0, w1 = pr.w1;
  const WaveRec* rec = (const WaveRec*)(a.ws + a.lay.wave_rec);
  const __amdgpu_buffer_rsrc_t prs = partials_rsrc(a);
  const uint32_t o_base = (uint32_t)(a.lay.partial_o - a.lay.partial_ml);
  const int r0 = max(0, sload_i32(a.cu_q + b));
  const int nq = max(0, min(min(sload_i32(a.cu_q + b + 1), a.total_q) - r0, kQRows * NQF));
  for (int f = 0; f < NQF; ++f) {
    float m_acc = kNegInf, l_acc = 0.f;
    f32x4_t acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    for (int base = w0; base <= w1; base += kMergeBatch) {
      bool ok[kMergeBatch];
      u32x2_t ml[kMergeBatch];
      u32x4_t ov[kMergeBatch][NDT];
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {  // past w1: a re-read of w1's part, not counted
        const int wv = min(base + j, w1);
        ok[j] = base + j <= w1 && rec[wv].count > 0;
        const uint32_t part = (uint32_t)((wv * 2 + (wv == w0 ? pr.slot0 : 0)) * NQF + f);
        ml[j] = __builtin_amdgcn_raw_buffer_load_b64(prs, (part * 64 + lane) * 8, 0, kDeviceScope);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          ov[j][dt] =
              __builtin_amdgcn_raw_buffer_load_b128(prs, o_base + ((part * NDT + dt) * 64 + lane) * 16, 0, kDeviceScope);
      }
      float m_new = m_acc;
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j)
        if (ok[j]) m_new = fmaxf(m_new, __uint_as_float(ml[j][0]));
      if (m_new == kNegInf) continue;  // nothing counted yet
      const float sa = m_acc == kNegInf ? 0.f : exp2_hw(m_acc - m_new);
      l_acc *= sa;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] *= sa;
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        const float m_w = __uint_as_float(ml[j][0]);
        const float sw = (ok[j] && m_w != kNegInf) ? exp2_hw(m_w - m_new) : 0.f;
        l_acc += __uint_as_float(ml[j][1]) * sw;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] += __builtin_bit_cast(f32x4_t, ov[j][dt]) * sw;
      }
      m_acc = m_new;
    }
    const float inv = l_acc > 0.f ? 1.0f / l_acc : 0.f;
    const int k = kQRows * f + c;
    if (k < nq) {
      st* orow = (st*)a.out + ((int64_t)(r0 + k) * a.H + h) * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) store4<T>(orow + out_col<COLS>(dt, g), acc[dt], inv * a.v_descale);
    }
  }
  if (lane == 0)
    __hip_atomic_store((int32_t*)(a.ws + a.lay.merge_cnt) + w0, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One K/V tile pair into this wave's LDS slot: NDMA direct-to-LDS loads of
// 1 KB per operand, lane offsets dma_off (the tile's row and chunk order),
// nontemporal; K at dst, V at dst + TILE_B.  The tile bases are wave-uniform.
template <int NDMA, int TILE_B>
__device__ __forceinline__ void tile_to_lds(const void* k, const void* v, uint8_t* dst, const uint32_t* dma_off) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)k, 0, 0x7fffffff, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)v, 0, 0x7fffffff, kRsrcWord3);
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(dst + i * 1024), 16, dma_off[i], 0, 0, kLoadNT);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)(dst + TILE_B + i * 1024), 16, dma_off[i], 0, 0, kLoadNT);
  }
}

// UNIFORM_PAGE: page_size >= 16, so the 16 keys of a tile share one page and
// the tile's base address is wave-uniform (scalar), with a per-lane offset that
// never changes.
// T: query/output rows; PT: the pool (T itself, or e4m3 under bf16 rows).
template <class T, class PT, int D, int DEPTH, bool UNIFORM_PAGE, int NQF, int OCC>
__global__ __launch_bounds__(256, OCC) void cross_attn_kernel(CrossArgs a) {
  typedef typename T::storage st;
  typedef typename PT::storage pst;
  typedef typename PvType<PT>::type PV;
  constexpr bool kFp8 = std::is_same<PT, E4m3>::value;
  // With one fragment the pair's raw query rows ride with its first tile and
  // the kernel norms and rotates them itself (q_prologue_kernel's work, fused);
  // with more, q_prologue_kernel prepares them and they are read when the
  // pair's first tile is computed.
  constexpr bool kQIn = NQF == 1;
  constexpr int EPC = PT::EPC;
  constexpr int NCH = D / (4 * EPC);
  constexpr int NDT = D / 16;
  constexpr int kQS = EPC / T::EPC;  // 16-byte chunks of raw query row per operand chunk
  typedef StreamSlot<PT, D, kQIn ? NCH * kQS : 0> Slot;
  const int lane = lane_id(), g = lane >> 4, c = lane & 15;
  const int wv = wave_in_block();
  uint8_t* ws = a.ws;
  PlanHeader* hdr = (PlanHeader*)ws;
  const int w = blockIdx.x * 4 + wv;
  if (w >= a.lay.n_waves) return;
  // the query norm weight, issued with the plan loads
  float qnw_reg[kQIn ? D / 64 : 1];
  if constexpr (kQIn) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) qnw_reg[i] = load_f32(a.q_norm_w + lane + 64 * i);
  }
  // The plan header and this wave's record, read together.
  // (No branch on the header before the record is read: the two loads issue
  // together and a mismatched plan simply leaves the wave no tiles.)
  const PlanHeader ph = *(const PlanHeader*)hdr;
  const WaveRec rec = ((const WaveRec*)(ws + a.lay.wave_rec))[w];
  if constexpr (kQIn) zero_empty_rows<T, D>(a, w);
  const bool plan_ok = plan_matches<T, PT, D, NQF>(ph, a);
  if (!plan_ok) {  // no plan for these sizes: nothing is computed, and the error word says so
    if (w == 0 && lane_id() == 0) atomicOr(&hdr->error, 4);
    return;
  }
  const int n_tiles = rec.count;
  if (n_tiles <= 0) return;
  const uint64_t t_start = a.wave_clock != nullptr ? __builtin_amdgcn_s_memrealtime() : 0;

  // Per-wave LDS window of page ids.
  __shared__ int32_t win_all[4][kWin];
  int32_t* win = win_all[wv];
  // Per-wave LDS copy of the query norm weight (D floats) and the inverse RoPE
  // frequencies (D / 2), read from LDS so that norming a pair's rows waits on
  // no vector-memory load behind the tiles in flight and holds no registers.
  __shared__ float qnw_all[4][kQIn ? D + D / 2 : 1];
  float* qnw = qnw_all[wv];
  if constexpr (kQIn) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) qnw[lane + 64 * i] = qnw_reg[i];
    if (lane == 0) {  // (a per-lane index into the kernel argument would cost scratch)
#pragma unroll
      for (int i = 0; i < D / 2; ++i) qnw[D + i] = a.rope.inv[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // K/V through LDS (pages of >= 16 tokens).  Each operand's tile is 16 rows of
  // kRowB contiguous bytes.  It arrives in kDma direct-to-LDS loads of 1 KB,
  // each reading whole rows (whole 128-byte lines, with the nontemporal hint):
  // lane l of load i fetches 16-byte chunk x ^ key(r) of row r, where
  // r, x = divmod(64 i + l, kCpr), into LDS chunk x of row r.  The MFMA
  // operand layout then reads chunk q = 4 ch + g of row c from LDS chunk
  // q ^ key(c): for each 16 lanes of one g the key spreads the 16 reads over
  // all 64 banks.  A ring of DEPTH slots per wave; loads hold no registers.
  constexpr bool LDS_KV = UNIFORM_PAGE && FM_CROSS_LDS_KV != 0 && NQF <= FM_CROSS_LDS_KV_MAXQF;
  constexpr int kRowB = D * (int)sizeof(pst);
  constexpr int kTileB = 16 * kRowB;
  constexpr int kCpr = kRowB / 16;                       // 16-byte chunks per row
  constexpr int kDma = kTileB / 1024;                    // loads per operand and tile
  constexpr int kKeyDiv = kCpr >= 16 ? 1 : 16 / kCpr;    // rows sharing one 256-byte bank window
  constexpr int kKeyMod = kCpr >= 16 ? 16 : kCpr;
  static_assert(!LDS_KV || (kTileB % 1024 == 0 && DEPTH >= 1 && DEPTH <= 3), "LDS ring shape");
  constexpr int kSlotB = LDS_KV ? 4 * 2 * kTileB : 16;   // one ring slot: 4 waves x (K, V)
  __shared__ __attribute__((aligned(1024))) uint8_t kv_ring0[kSlotB];
  __shared__ __attribute__((aligned(1024))) uint8_t kv_ring1[DEPTH > 1 ? kSlotB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t kv_ring2[DEPTH > 2 ? kSlotB : 16];
  auto ring_of = [&](auto dslot) -> uint8_t* {  // this wave's K tile of slot d (its V tile follows)
    constexpr int d = decltype(dslot)::value;
    uint8_t* base = d == 0 ? kv_ring0 : d == 1 ? kv_ring1 : kv_ring2;
    return base + wv * 2 * kTileB;
  };
  auto row_key = [](int r) { return (r / kKeyDiv) % kKeyMod; };
  uint32_t dma_off[LDS_KV ? kDma : 1];  // per lane, per load: byte offset inside the tile (slot stride aware)
  uint32_t lds_off[LDS_KV ? NCH : 1];   // per lane, per operand chunk: byte offset of its LDS chunk
  // A bf16 or e4m3 V tile is read in column layout by gfx950's transpose
  // reads, with no selection product.
  //  - bf16 (ds_read_b64_tr_b16): within each 16 lanes, lane i receives
  //    element i % 4 of the 8-byte pieces that lanes 4k + i / 4 (k = 0..3)
  //    address.  For column tile dt lane (g, c) addresses key 4g + c / 4,
  //    columns 16 dt + 4 (c % 4) .. +3, and receives V[4g .. 4g+3][16 dt + c].
  //  - e4m3 (ds_read_b64_tr_b8): lane i receives byte i % 8 of the pieces
  //    that lanes 2k + i / 8 (k = 0..7) address.  Read j serves column tiles
  //    j and j + NDT/2: lane (g, c) addresses key 4g + (c/2) % 4, columns
  //    16 dt' + 8 (c % 2) .. +7 with dt' = j for c < 8, else j + NDT/2, and
  //    receives V[4g .. 4g+3][16 j + c] in bytes 0-3 and the same keys of
  //    column 16 (j + NDT/2) + c in bytes 4-7.  Tiles NDT/2 apart differ in
  //    the top bit of the swizzled chunk, so the 32 pieces of a half-wave
  //    fall on 64 distinct banks.
  // The output columns then follow the plain order 16 dt + 4 g + i.
  constexpr bool kVtr = LDS_KV && !std::is_same<PT, F32>::value;
  typedef std::conditional_t<kVtr, Bf16, PT> OCols;  // the output column order
  constexpr int kVtrReads = kFp8 ? NDT / 2 : NDT;
  uint32_t vtr_off[kVtr ? kVtrReads : 1];
  if constexpr (kVtr && kFp8) {
    const int k = c >> 1, r = 4 * g + (k & 3);
#pragma unroll
    for (int j = 0; j < kVtrReads; ++j) {
      const int dtp = k < 4 ? j : j + NDT / 2;
      vtr_off[j] = (uint32_t)(kTileB + r * kRowB + ((dtp ^ row_key(r)) * 16) + 8 * (c & 1));
    }
  } else if constexpr (kVtr) {
    const int r = 4 * g + (c >> 2), q = c & 3;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      vtr_off[dt] = (uint32_t)(kTileB + r * kRowB + (((2 * dt + (q >> 1)) ^ row_key(r)) * 16) + 8 * (q & 1));
  }
  if constexpr (LDS_KV) {
    const uint32_t slot_b = a.slot_stride32 * (uint32_t)sizeof(pst);
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      const int u = 64 * i + lane, r = u / kCpr, x = u % kCpr;
      dma_off[i] = (uint32_t)r * slot_b + (uint32_t)((x ^ row_key(r)) * 16);
    }
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) lds_off[ch] = (uint32_t)((c * kCpr + ((4 * ch + g) ^ row_key(c))) * 16);
  }

  Selector<PT> sel;
  if constexpr (!kVtr) sel.init(lane);
  const int ps_mask = (1 << a.log2ps) - 1;
  const pst* kpool = (const pst*)a.pool.k;
  const pst* vpool = (const pst*)a.pool.v;

  // ---- loader state (wave-uniform) ----
  int lb = rec.b, lh = rec.h, lk = rec.k;
  int lctx = rec.ctx, lT = tiles_of(rec.ctx);
  bool exhausted = false;  // set only if the lengths changed after the plan was made
  bool seg_first = true, seg_from0 = (lk == 0);
  int wreq = -1, wbase = 0;
  auto fill_window = [&](int b, int base) {
    wreq = b;
    wbase = base;
    const int32_t* row = a.page_table + (int64_t)b * a.pt_stride;
    // every load issued before the first wait (clamped indices, masked after)
    int32_t v[kWin / 64];
#pragma unroll
    for (int k = 0; k < kWin / 64; ++k) v[k] = load_i32(row + min((int64_t)base + lane + 64 * k, a.pt_stride - 1));
#pragma unroll
    for (int k = 0; k < kWin / 64; ++k) win[lane + 64 * k] = (int64_t)base + lane + 64 * k < a.pt_stride ? v[k] : -1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  int64_t kv_last = 0;  // per-lane element offset of the last real tile (a safe re-read)
  uint64_t tile_base = 0;  // UNIFORM_PAGE: wave-uniform element offset of the tile (kept for re-reads)
  // Wave-uniform per-request and per-pair parts of the addresses: the
  // request's page-table row and the head's offset in the pool.
  const int32_t* prow = a.page_table + (int64_t)lb * a.pt_stride;
  uint64_t hoff = (uint64_t)(uint32_t)lh * a.head_stride32;
  // UNIFORM_PAGE: this lane's constant offset inside a tile (slot c, column group g)
  const uint32_t lane_off_b = (uint32_t)(((int64_t)c * a.pool.slot_stride + g * EPC) * (int64_t)sizeof(pst));
  bool bad_page = false;

  // Move to the next (request, head) pair with tiles once the current one is done.
  auto advance_if_done = [&]() {
    if (lk < lT || exhausted) return;
    ++lh;
    lk = 0;
    seg_first = false;
    seg_from0 = true;
    if (lh == a.H) {
      lh = 0;
      do {
        if (lb + 1 >= a.bs) {
          exhausted = true;
          break;
        }
        ++lb;
        lctx = max(0, sload_i32(a.ctx_lens + lb));
        lT = tiles_of(lctx);
      } while (lT == 0);
      prow = a.page_table + (int64_t)lb * a.pt_stride;
    }
    hoff = (uint64_t)(uint32_t)lh * a.head_stride32;
    exhausted = exhausted || lT == 0;
  };
  auto window_covers = [&](int tb) -> bool {
    const int first_page = tb >> a.log2ps;
    const int last_page = min(tb + 15, lctx - 1) >> a.log2ps;
    return wreq == lb && first_page >= wbase && last_page - wbase < kWin;
  };
  // Page id of the next tile, read one tile ahead so the read has completed
  // by the time that tile's loads are issued: from the window (per lane), or
  // with one page per tile straight from the page table through the scalar
  // cache (an index past the row reads as -1, a bad page).
  int pg_next = 0;
  bool pg_have = false;
  auto prefetch_page = [&]() {
    pg_have = false;
    if (exhausted || lk >= lT) return;
    const int tb = lk << 4;
    if constexpr (UNIFORM_PAGE) {
      const int idx = tb >> a.log2ps;
      pg_next = idx < a.pt_stride32 ? sload_i32(prow + idx) : -1;
      pg_have = true;
    } else {
      if (!window_covers(tb)) return;
      pg_next = win[((min(tb + c, lctx - 1) >> a.log2ps) - wbase) & (kWin - 1)];
      pg_have = true;
    }
  };

  auto load_slot = [&](Slot& s, int j, auto dslot) {
    int64_t off = kv_last;
    bool ok = false, bad = false;
    uint32_t flags = 0;
    uint32_t keys = 0;  // UNIFORM_PAGE: the tile's valid keys, in scalar registers
    if (j < n_tiles && !exhausted) {
      const bool last_of_pair = lk == lT - 1;
      flags = (lk == 0 || j == 0) ? kStart : 0;
      if (last_of_pair || j == n_tiles - 1)
        flags |= kEnd | ((seg_from0 && last_of_pair) ? kWhole : 0) | (seg_first ? 0 : kPart1);
      const int tb = lk << 4;
      if constexpr (UNIFORM_PAGE) {
        // one page per tile: scalar tile base; the lanes' slots c are in the page
        int pu;
        if (pg_have) {
          pu = pg_next;
        } else {
          const int idx = tb >> a.log2ps;
          pu = idx < a.pt_stride32 ? sload_i32(prow + idx) : -1;
        }
        const bool page_ok = (uint32_t)pu < (uint32_t)a.num_pages32;  // also rules out pu < 0
        keys = page_ok ? (kKeyMask >> (16 - min(16, lctx - tb))) : 0u;  // tb < lctx: at least one key
        bad_page |= !page_ok;
        tile_base = hoff + (page_ok ? (uint64_t)(uint32_t)pu * a.page_stride32 +
                                          (uint64_t)(uint32_t)(tb & ps_mask) * a.slot_stride32
                                    : 0);
      } else {
        const int tok = tb + c;
        const int tok_c = min(tok, lctx - 1);
        int page;
        if (pg_have) {
          page = pg_next;
        } else {
          if (!window_covers(tb))
            // the whole request's page row when it fits (every head's pair reuses it)
            fill_window(lb, ((lctx - 1) >> a.log2ps) < kWin ? 0 : (tb >> a.log2ps));
          page = win[((tok_c >> a.log2ps) - wbase) & (kWin - 1)];
        }
        const bool page_ok = page >= 0 && (int64_t)page < a.pool.num_pages;
        ok = tok < lctx && page_ok;
        bad = tok < lctx && !page_ok;
        off = (int64_t)lh * a.pool.head_stride +
              (page_ok ? (int64_t)page * a.pool.page_stride + (int64_t)(tok_c & ps_mask) * a.pool.slot_stride : 0);
        kv_last = off;
      }
      if (kQIn && (flags & kStart)) {
        // this pair's raw query rows ride along with its first tile: lane (g, c)
        // takes row c's columns ch*4*EPC + g*EPC .. +EPC-1 (the operand layout);
        // a row past the request's count reads row 0 and is zeroed when computed
        const int r0 = max(0, sload_i32(a.cu_q + lb));
        const int nq = min(sload_i32(a.cu_q + lb + 1), a.total_q) - r0;
        const st* qrow = (const st*)a.q + ((int64_t)(c < nq ? r0 + c : 0) * a.H + lh) * D;
#pragma unroll
        for (int i = 0; i < NCH * kQS; ++i) s.q[i] = load16(qrow + (i / kQS) * 4 * EPC + g * EPC + (i % kQS) * T::EPC);
      }
      ++lk;
      if (j + 1 < n_tiles) {
        advance_if_done();
        prefetch_page();
      }
    }
    if constexpr (LDS_KV) {
      tile_to_lds<kDma, kTileB>(kpool + tile_base, vpool + tile_base, ring_of(dslot), dma_off);
    } else if (UNIFORM_PAGE) {
      // scalar tile base + 32-bit per-lane byte offset (the SGPR-base addressing form)
      const char* kt = (const char*)(kpool + tile_base);
      const char* vt = (const char*)(vpool + tile_base);
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        s.k[ch] = load16_stream(kt + (lane_off_b + ch * 64u));
        s.v[ch] = load16_stream(vt + (lane_off_b + ch * 64u));
      }
    } else {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        s.k[ch] = load16_stream(kpool + off + ch * 4 * EPC + g * EPC);
        s.v[ch] = load16_stream(vpool + off + ch * 4 * EPC + g * EPC);
      }
    }
    if constexpr (UNIFORM_PAGE) {
      s.mf = flags | keys;
    } else {
      s.mf = flags | (uint32_t)(__ballot(ok) & 0xffffull);
      bad_page |= __ballot(bad) != 0;
    }
  };

  // ---- compute state (per query fragment f) ----
  u32x4_t qop[NQF][NCH];
  f32x4_t o[NQF][NDT];
  float m_run[NQF];   // running max of this lane's query row (log2 domain)
  float l_lane[NQF];  // this lane's share of the running denominator
  int cut_b[2] = {-1, -1}, cut_h[2] = {0, 0};  // pairs this wave left partials of
  float score_scale = a.qscale_log2;  // softmax scale * log2(e), times the pair's query scale over e4m3
  // ---- compute-side pair cursor: the pair of the slot being computed ----
  // The wave's first tile belongs to its record's pair; every later kStart
  // is the next pair with tiles, in the order the loader takes them.
  int cb = rec.b, chh = rec.h, cr0 = 0, cnq = 0;
  bool c_fresh = true;
  auto c_rows = [&]() {
    cr0 = max(0, sload_i32(a.cu_q + cb));
    cnq = max(0, min(min(sload_i32(a.cu_q + cb + 1), a.total_q) - cr0, kQRows * NQF));
  };
  c_rows();
  auto c_next_pair = [&]() {
    if (++chh < a.H) return;
    chh = 0;
    do {
      ++cb;
    } while (cb < a.bs - 1 && tiles_of(sload_i32(a.ctx_lens + cb)) == 0);
    c_rows();
  };
#pragma unroll
  for (int f = 0; f < NQF; ++f) {
    m_run[f] = kNegInf;
    l_lane[f] = 0.f;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) qop[f][ch] = (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[f][dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  }

  auto compute_slot = [&](const Slot& s, auto dslot) {
    // The tile's K and V: from the slot's registers, or from its LDS slot once
    // its loads have landed (the DEPTH - 1 later tiles' loads may still be in
    // flight; any later query-row or partial loads only make the wait stricter).
    u32x4_t kk[NCH], vv[NCH];
    if constexpr (LDS_KV) {
      __builtin_amdgcn_s_waitcnt(wait_vm_only((DEPTH - 1) * 2 * kDma));
      const uint8_t* src = ring_of(dslot);
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        kk[ch] = *(const u32x4_t*)(src + lds_off[ch]);
        if constexpr (!kVtr) vv[ch] = *(const u32x4_t*)(src + kTileB + lds_off[ch]);
      }
    } else {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        kk[ch] = s.k[ch];
        vv[ch] = s.v[ch];
      }
    }
    const uint32_t sflags = s.mf & ~kKeyMask;
    if (sflags & kStart) {
      if (!c_fresh) c_next_pair();
      c_fresh = false;
      if constexpr (kQIn) {
        // q^ = RoPE(RMSNorm(q)) at position ctx_len + c, as q_prologue_kernel
        // makes it, from the raw rows (zero past the request's rows)
        float qf[D / 4];
#pragma unroll
        for (int i = 0; i < NCH * kQS; ++i)
#pragma unroll
          for (int j = 0; j < T::EPC; ++j) qf[i * T::EPC + j] = c < cnq ? chunk_elem<T>(s.q[i], j) : 0.f;
        norm_rope_row_lds<PT, D>(qf, qnw, qnw + D, a.eps, max(0, sload_i32(a.ctx_lens + cb)) + c, g);
        if constexpr (kFp8) {
          const QScale qsc = query_scale(a, qf);
          score_scale = a.qscale_log2 * qsc.qs;
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) qop[0][ch] = pack_e4m3_chunk(&qf[ch * EPC], qsc.r);
        } else {
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) qop[0][ch] = pack_chunk<PT>(&qf[ch * EPC]);
        }
      } else {  // every fragment's prepared rows, read now
        if (kFp8)
          score_scale = a.qscale_log2 * sload_f32((const float*)(ws + a.lay.q_scale) + (int64_t)cb * a.H + chh);
        const pst* qrow = (const pst*)(ws + a.lay.q_hat) + (((int64_t)cb * kQRows * NQF + c) * a.H + chh) * D;
#pragma unroll
        for (int f = 0; f < NQF; ++f)
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch)
            qop[f][ch] = load16(qrow + (int64_t)f * kQRows * a.H * D + ch * 4 * EPC + g * EPC);
        // Wait here, on the pair's first tile only: left to the compiler, the
        // wait for these loads lands after the branch, on every tile, and
        // drains the whole load ring each time.
        wait_all_vector_loads();
      }
      // O and l restart through the rescale below: its factor is 0 while the
      // running max is -inf
#pragma unroll
      for (int f = 0; f < NQF; ++f) m_run[f] = kNegInf;
    }
    const bool start = (sflags & kStart) != 0;
    const uint32_t smask = s.mf & kKeyMask;
    // The fragments' scores, maxima, rescales and weights run phase by phase
    // across fragments, with one wave-uniform branch for every rescale, so
    // their independent MFMA, reduction and exp chains can interleave.
    f32x4_t p[NQF];
    float sv[NQF][4];
    {
      f32x4_t sc[NQF];
#pragma unroll
      for (int f = 0; f < NQF; ++f) {
        sc[f] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        if constexpr (kFp8 && NCH == 2) {  // head_dim 128 over e4m3: the whole contraction in one MFMA
          mma_two_chunks_e4m3(sc[f], kk[0], kk[1], qop[f][0], qop[f][1]);
        } else {
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) mma_chunk<PT>(sc[f], kk[ch], qop[f][ch]);
        }
      }
      // scale and key mask in one fma: the bias is 0 for a key of the
      // context (fma(s, scale, 0) is the rounded product) and -inf past it
      float bias[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) bias[i] = ((smask >> (4 * g + i)) & 1u) ? 0.f : kNegInf;
#pragma unroll
      for (int f = 0; f < NQF; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[f][i] = fmaf(sc[f][i], score_scale, bias[i]);
    }
    // Lazy rescale: the reference max moves only when a row's max exceeds it
    // by more than kRescaleSlack (log2 units), so p <= 2^slack and O, l are
    // rarely rescaled; O / l is the same quotient.  A pair's first tile always
    // moves it, which also clears O and l (the factor is 0 while the
    // reference max is -inf).  A row's max exceeds its reference max exactly
    // when one of its lanes' own maxima does, so the lanes' maxima and one
    // ballot decide whether any row moves; the rows' maxima (a reduction over
    // the four lane groups) are taken only then.
    float mx[NQF];
#pragma unroll
    for (int f = 0; f < NQF; ++f) mx[f] = fmaxf(fmaxf(sv[f][0], sv[f][1]), fmaxf(sv[f][2], sv[f][3]));
    bool any_move = start;
#pragma unroll
    for (int f = 0; f < NQF; ++f) any_move |= mx[f] > m_run[f] + kRescaleSlack;
    if (__ballot(any_move) != 0) {
      bool move[NQF];
#pragma unroll
      for (int f = 0; f < NQF; ++f) {
        mx[f] = wave_max_groups(mx[f]);
        move[f] = start || mx[f] > m_run[f] + kRescaleSlack;
      }
#pragma unroll
      for (int f = 0; f < NQF; ++f) {
        const float m_new = move[f] ? mx[f] : m_run[f];
        const float alpha = (m_run[f] == kNegInf) ? 0.f : exp2_hw(m_run[f] - m_new);
        if (move[f]) {
          l_lane[f] *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[f][dt] *= alpha;
          m_run[f] = m_new;
        }
      }
    }
    // bf16 weights: rounded two at a time by one packed conversion, which is
    // also the PV operand; the sum takes the rounded values in key order
    constexpr bool kPacked = std::is_same<PV, Bf16>::value;
    u32x2_t pk[kPacked ? NQF : 1];
#pragma unroll
    for (int f = 0; f < NQF; ++f) {
      const float m_use = (m_run[f] == kNegInf) ? 0.f : m_run[f];
      float psum = 0.f;
      if constexpr (kPacked) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = exp2_hw(sv[f][i] - m_use);
        pk[f] = (u32x2_t){pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3])};
        const float r[4] = {__uint_as_float(pk[f][0] << 16), __uint_as_float(pk[f][0] & 0xffff0000u),
                            __uint_as_float(pk[f][1] << 16), __uint_as_float(pk[f][1] & 0xffff0000u)};
#pragma unroll
        for (int i = 0; i < 4; ++i) psum += r[i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[f][i] = operand_value<PV>(exp2_hw(sv[f][i] - m_use));
          psum += p[f][i];
        }
      }
      l_lane[f] += psum;
    }
    // V moved to column layout once per tile, shared by every fragment
    if constexpr (kVtr && kFp8) {
      typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
      typedef __attribute__((address_space(3))) i32x2_t* lds_i32x2;
      const uint8_t* src = ring_of(dslot);
#pragma unroll
      for (int j = 0; j < kVtrReads; ++j) {
        const i32x2_t raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2)(src + vtr_off[j]));
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const i16x4_t vt = e4m3x4_to_bf16x4((uint32_t)raw[half]);
          const int dt = j + half * (NDT / 2);
#pragma unroll
          for (int f = 0; f < NQF; ++f)
            o[f][dt] =
                __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, __builtin_bit_cast(i16x4_t, pk[f]), o[f][dt], 0, 0, 0);
        }
      }
    } else if constexpr (kVtr) {
      typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4;
      const uint8_t* src = ring_of(dslot);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const i16x4_t vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(src + vtr_off[dt]));
#pragma unroll
        for (int f = 0; f < NQF; ++f)
          o[f][dt] =
              __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, __builtin_bit_cast(i16x4_t, pk[f]), o[f][dt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const auto vt = sel.template transpose_tile<NCH>(vv, dt);
#pragma unroll
        for (int f = 0; f < NQF; ++f) {
          if constexpr (kPacked) mma_pv_packed(o[f][dt], vt, pk[f]);
          else mma_pv<PV>(o[f][dt], vt, p[f]);
        }
      }
    }
    if (sflags & kEnd) {
      if (sflags & kWhole) {
#pragma unroll
        for (int f = 0; f < NQF; ++f) {
          const float l_row = wave_sum_groups(l_lane[f]);
          const float inv = l_row > 0.f ? 1.0f / l_row : 0.f;
          const int k = kQRows * f + c;
          if (k < cnq) {
            st* orow = (st*)a.out + ((int64_t)(cr0 + k) * a.H + chh) * D;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) store4<T>(orow + out_col<OCols>(dt, g), o[f][dt], inv * a.v_descale);
          }
        }
      } else {
        const int slot = (sflags & kPart1) ? 1 : 0;
        const __amdgpu_buffer_rsrc_t prs = partials_rsrc(a);
        const uint32_t o_base = (uint32_t)(a.lay.partial_o - a.lay.partial_ml);
#pragma unroll
        for (int f = 0; f < NQF; ++f) {
          const float l_row = wave_sum_groups(l_lane[f]);
          const uint32_t part = (uint32_t)((w * 2 + slot) * NQF + f);
          const u32x2_t ml = {__float_as_uint(m_run[f]), __float_as_uint(l_row)};
          __builtin_amdgcn_raw_buffer_store_b64(ml, prs, (part * 64 + lane) * 8, 0, kDeviceScope);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o[f][dt]), prs,
                                                   o_base + ((part * NDT + dt) * 64 + lane) * 16, 0, kDeviceScope);
        }
        cut_b[slot] = cb;
        cut_h[slot] = chh;
      }
    }
  };

  // Every slot index is loaded unconditionally (indices past the range
  // re-read the last tile, a cache hit, and are fully masked with no flags),
  // so the loop body is straight-line and DEPTH-1 tiles stay in flight.
  Slot buf[DEPTH];
  typedef std::integral_constant<int, 0> S0;
  typedef std::integral_constant<int, 1> S1;
  typedef std::integral_constant<int, 2> S2;
  static_assert(DEPTH >= 1 && DEPTH <= 3, "ring depth");
  if constexpr (DEPTH >= 2) load_slot(buf[0], 0, S0());
  if constexpr (DEPTH == 3) load_slot(buf[1], 1, S1());
  for (int it = 0; it < n_tiles; it += DEPTH) {
    if constexpr (DEPTH == 1) {
      load_slot(buf[0], it, S0());
      compute_slot(buf[0], S0());
    } else if constexpr (DEPTH == 3) {
      load_slot(buf[2], it + 2, S2());
      compute_slot(buf[0], S0());
      load_slot(buf[0], it + 3, S0());
      compute_slot(buf[1], S1());
      load_slot(buf[1], it + 4, S1());
      compute_slot(buf[2], S2());
    } else {
      load_slot(buf[1], it + 1, S1());
      compute_slot(buf[0], S0());
      load_slot(buf[0], it + 2, S0());
      compute_slot(buf[1], S1());
    }
  }
  if (a.wave_clock != nullptr) {  // a timed call: this wave's clock over its tile loop
    const uint64_t t_loop = __builtin_amdgcn_s_memrealtime();
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if (lane == 0) {
      uint64_t* r = a.wave_clock + 4 * (int64_t)w;
      r[0] = t_start;
      r[1] = t_loop;
      r[2] = xcc & 0xF;
      r[3] = (uint64_t)n_tiles;
    }
  }
  const int err = (bad_page ? 1 : 0) | (exhausted ? 2 : 0);
  if (err && lane == 0) atomicOr(&hdr->error, err);
  // The pairs this wave cut: the last of each pair's waves to get here merges it.
  // (The pairs' records are read while the partial stores are acknowledged.)
  if (cut_b[0] >= 0 || cut_b[1] >= 0) {
    PairRec pr[2];
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (cut_b[k] >= 0) pr[k] = pair_rec_of(a, cut_b[k], cut_h[k]);
    wait_stores_acknowledged();  // this wave's partials before their counts
    int before[2] = {-1, -1};
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (cut_b[k] >= 0) before[k] = count_in(a, pr[k]);
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (cut_b[k] >= 0 && before[k] == pr[k].parts - 1) merge_pair<T, OCols, D, NQF>(a, cut_b[k], cut_h[k], pr[k]);
  }
}

template <class T, class PT, int D, int DEPTH, bool UNIFORM_PAGE, int NQF, int OCC>
hipError_t launch_cross_paged(const CrossArgs& a, hipStream_t s) {
  const int64_t pairs = (int64_t)a.bs * a.H;
  if (!grid_fits((pairs + 3) / 4, 256) || !grid_fits((a.lay.n_waves + 3) / 4, 256)) return hipErrorInvalidConfiguration;
  if constexpr (NQF > 1) {  // one fragment: the attention kernel prepares its query rows itself
    hipLaunchKernelGGL((q_prologue_kernel<T, PT, D, NQF>), dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned grid = (unsigned)((a.lay.n_waves + 3) / 4);
  hipLaunchKernelGGL((cross_attn_kernel<T, PT, D, DEPTH, UNIFORM_PAGE, NQF, OCC>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class T, class PT, int D, int DEPTH, int NQF, int OCC>
hipError_t launch_cross_typed(const CrossArgs& a, hipStream_t s) {
  // page_size >= 16 keeps each 16-key tile inside one page; there the K/V
  // tiles of kernels with few query fragments stream through LDS
  constexpr bool kLds = FM_CROSS_LDS_KV != 0 && NQF <= FM_CROSS_LDS_KV_MAXQF;
  if (a.log2ps >= 4) return launch_cross_paged<T, PT, D, kLds ? FM_CROSS_DEPTH_LDS : DEPTH, true, NQF, OCC>(a, s);
  return launch_cross_paged<T, PT, D, DEPTH, false, NQF, OCC>(a, s);
}

#ifndef FM_CROSS_DEPTH_Q2
#define FM_CROSS_DEPTH_Q2 3  // tiles in flight with two query fragments per request (bf16)
#endif
#ifndef FM_CROSS_DEPTH_Q4
#define FM_CROSS_DEPTH_Q4 2  // ... with four (their accumulators fill the AGPRs)
#endif
// e4m3 tiles: two waves per SIMD, each with two tiles in flight.
#ifndef FM_CROSS_DEPTH_FP8
#define FM_CROSS_DEPTH_FP8 2
#endif
#ifndef FM_CROSS_DEPTH_FP8_Q2
#define FM_CROSS_DEPTH_FP8_Q2 2
#endif
#ifndef FM_CROSS_DEPTH_FP8_Q4
#define FM_CROSS_DEPTH_FP8_Q4 2
#endif

// Tiles in flight for one, two and four query fragments per request, each
// at the occupancy the plan was cut for.
template <class T, class PT, int D, int DTYPE, int DEPTH1, int DEPTH2, int DEPTH4>
hipError_t launch_cross_frags(const CrossArgs& a, hipStream_t s) {
  switch (a.lay.nqf) {
    case 1: return launch_cross_typed<T, PT, D, DEPTH1, 1, cross_occupancy(DTYPE)>(a, s);
    case 2: return launch_cross_typed<T, PT, D, DEPTH2, 2, cross_occupancy(DTYPE)>(a, s);
    default: return launch_cross_typed<T, PT, D, DEPTH4, 4, cross_occupancy(DTYPE)>(a, s);
  }
}

template <int D>
hipError_t launch_cross_dh(const CrossArgs& a, int dtype, hipStream_t s) {
  if (dtype == 1)
    return launch_cross_frags<Bf16, Bf16, D, 1, FM_CROSS_DEPTH_BF16, FM_CROSS_DEPTH_Q2, FM_CROSS_DEPTH_Q4>(a, s);
  if (dtype == 2)
    return launch_cross_frags<Bf16, E4m3, D, 2, FM_CROSS_DEPTH_FP8, FM_CROSS_DEPTH_FP8_Q2, FM_CROSS_DEPTH_FP8_Q4>(a, s);
  // fp32 rows, whose tiles take twice the registers, keep one tile in flight
  // with several candidate blocks
  return launch_cross_frags<F32, F32, D, 0, FM_CROSS_DEPTH_F32, 1, 1>(a, s);
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  if (a.bs <= kPlanLdsRequests) {  // a workgroup per 1024 pairs or waves, at most kPlanMaxGroups
    const int64_t work = max((int64_t)a.lay.n_waves, (int64_t)a.bs * a.H);
    const int groups = (int)min((int64_t)kPlanMaxGroups, max((int64_t)1, (work + 1023) / 1024));
    hipLaunchKernelGGL(plan_kernel<true>, dim3(groups), dim3(1024), 0, s, a);
  } else
    hipLaunchKernelGGL(plan_kernel<false>, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cross_attention(const CrossArgs& a, int dtype, int Dh, hipStream_t s) {
  return Dh == 128 ? launch_cross_dh<128>(a, dtype, s) : launch_cross_dh<64>(a, dtype, s);
}

}  // namespace fm
