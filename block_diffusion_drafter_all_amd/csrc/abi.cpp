// extern "C" entry points of libfm (declared in include/fm.h): host-side
// argument validation, the RoPE frequency table, workspace layout, launches.
// No entry point allocates, frees or synchronizes.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/fm.h"
#include "fm_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return FM_OK;
}

int from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  if (e == hipErrorInvalidConfiguration)  // a launcher's own grid check, before anything was enqueued
    return fail(FM_E_UNSUPPORTED, "%s: the sizes need a launch grid of 2^32 or more work-items", what);
  return fail(FM_E_HIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2_exact(int64_t x) {
  int r = 0;
  while ((int64_t(1) << r) < x) ++r;
  return r;
}

// Bytes of one pool element.
size_t pool_elem_size(fm_dtype dt) { return dt == FM_F32 ? 4 : (dt == FM_BF16 ? 2 : 1); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Inverse RoPE frequencies: the float32 nearest to theta^(-2i/D), i < D/2,
// evaluated in double precision and rounded once.
fm::RopeFreqs rope_freqs(float theta, int Dh) {
  fm::RopeFreqs r{};
  for (int i = 0; i < Dh / 2; ++i) r.inv[i] = (float)std::pow((double)theta, -(2.0 * i) / (double)Dh);
  return r;
}

int check_common(const char* fn, fm_dtype dt, int32_t H, int32_t Dh, float eps, float theta) {
  if (dt != FM_F32 && dt != FM_BF16 && dt != FM_BF16_E4M3)
    return fail(FM_E_UNSUPPORTED, "%s: dtype %d is not FM_F32, FM_BF16 or FM_BF16_E4M3", fn, (int)dt);
  if (H < 1) return fail(FM_E_INVALID, "%s: H = %d must be >= 1", fn, H);
  if (Dh != 64 && Dh != 128) return fail(FM_E_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", fn, Dh);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(FM_E_INVALID, "%s: eps must be finite and >= 0", fn);
  if (!(theta > 0.f) || !std::isfinite(theta)) return fail(FM_E_INVALID, "%s: rope_theta must be finite and > 0", fn);
  return FM_OK;
}

int check_pool(const char* fn, const fm_kv_pool& p, fm_dtype dt, int idx, int64_t* elems_per16) {
  const int64_t q = (int64_t)(16 / pool_elem_size(dt));
  *elems_per16 = q;
  if (p.k == nullptr || p.v == nullptr) return fail(FM_E_INVALID, "%s: pool %d has a null k or v pointer", fn, idx);
  if (!aligned16(p.k) || !aligned16(p.v)) return fail(FM_E_INVALID, "%s: pool %d k/v not 16-byte aligned", fn, idx);
  if (p.num_pages < 1) return fail(FM_E_INVALID, "%s: pool %d has num_pages %lld < 1", fn, idx, (long long)p.num_pages);
  if (p.num_pages > INT32_MAX) return fail(FM_E_UNSUPPORTED, "%s: pool %d has more than 2^31-1 pages", fn, idx);
  if (p.page_stride < 0 || p.slot_stride < 0 || p.head_stride < 0)
    return fail(FM_E_INVALID, "%s: pool %d has a negative stride", fn, idx);
  if (p.page_stride % q || p.slot_stride % q || p.head_stride % q)
    return fail(FM_E_INVALID, "%s: pool %d strides must be multiples of 16 bytes", fn, idx);
  return FM_OK;
}

int check_ws(const char* fn, const void* ws, size_t ws_bytes, size_t need) {
  if (ws == nullptr) return fail(FM_E_WORKSPACE, "%s: workspace is null", fn);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(FM_E_WORKSPACE, "%s: workspace not 256-byte aligned", fn);
  if (ws_bytes < need)
    return fail(FM_E_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
  return FM_OK;
}

// Compute units of the current device; a device that cannot be queried (no
// GPU) is taken to have 256 CUs, MI355X's count.
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      (void)hipGetLastError();
      cus = 256;
    }
    cached[dev] = cus;
  }
  return cached[dev];
}

// Resident cross-attention wavefronts for a pool type: CUs x 4 SIMDs x the
// waves per SIMD that type's kernel keeps.
int plan_waves(fm_dtype dt) {
  return std::min(device_cus() * 4 * fm::cross_occupancy((int)dt), fm::kMaxPlanWaves);
}

fm::PoolDesc to_desc(const fm_kv_pool& p) {
  fm::PoolDesc d;
  d.k = reinterpret_cast<uint64_t>(p.k);
  d.v = reinterpret_cast<uint64_t>(p.v);
  d.num_pages = p.num_pages;
  d.page_stride = p.page_stride;
  d.slot_stride = p.slot_stride;
  d.head_stride = p.head_stride;
  return d;
}

}  // namespace

extern "C" {

const char* fm_last_error(void) { return g_last_error.c_str(); }

const char* fm_version(void) { return "fm 0.1.0 (gfx950)"; }

size_t fm_write_context_kv_workspace_size(int64_t n_rows) { return fm::write_layout(n_rows).total; }

}  // extern "C"

namespace {

// The write of fm_write_context_kv and fm_write_context_kv_noalloc: with
// ``use_scratch`` the workspace is the static per-device array (ws ignored).
int write_context_kv(const char* fn, bool use_scratch, const void* x, int64_t n_rows, int32_t d_in, fm_dtype dt,
                     const void* w_kv, const float* k_norm_w, const int32_t* row_req, const int32_t* row_pos,
                     const int32_t* commit_lens, int32_t window, const int32_t* page_table, int64_t pt_stride,
                     int32_t page_size, int32_t bs, const fm_kv_pool* pools, int32_t L, int32_t H, int32_t Dh,
                     float eps, float rope_theta, const float* kv_scales, int32_t* out_slots, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  if (n_rows < 0) return fail(FM_E_INVALID, "%s: n_rows %lld < 0", fn, (long long)n_rows);
  if (use_scratch && n_rows > fm::kWriteScratchRows)
    return fail(FM_E_UNSUPPORTED, "%s: n_rows %lld above the %lld rows its static workspace serves", fn,
                (long long)n_rows, (long long)fm::kWriteScratchRows);
  if (n_rows == 0) return ok();
  if (int s = check_common(fn, dt, H, Dh, eps, rope_theta)) return s;
  if (!x || !w_kv || !k_norm_w || !row_req || !row_pos || !page_table || !pools)
    return fail(FM_E_INVALID, "%s: a required pointer is null", fn);
  if (!aligned16(x) || !aligned16(w_kv)) return fail(FM_E_INVALID, "%s: x and w_kv must be 16-byte aligned", fn);
  if (d_in < 64 || d_in % 64) return fail(FM_E_UNSUPPORTED, "%s: d_in %d must be a positive multiple of 64", fn, d_in);
  if (L < 1 || L > fm::kMaxLayers) return fail(FM_E_UNSUPPORTED, "%s: L = %d not in [1, %d]", fn, L, fm::kMaxLayers);
  if (!is_pow2(page_size) || page_size > 4096)
    return fail(FM_E_UNSUPPORTED, "%s: page_size %d is not a power of two in [1, 4096]", fn, page_size);
  if (pt_stride < 1) return fail(FM_E_INVALID, "%s: pt_stride %lld < 1", fn, (long long)pt_stride);
  if (bs < 1) return fail(FM_E_INVALID, "%s: bs %d < 1", fn, bs);
  if (commit_lens != nullptr && window < 1) return fail(FM_E_INVALID, "%s: commit_lens given with window %d", fn, window);
  if (n_rows > 65535LL * 64) return fail(FM_E_UNSUPPORTED, "%s: n_rows %lld above %lld", fn, (long long)n_rows, 65535LL * 64);
  if ((int64_t)L * 2 * H > INT32_MAX) return fail(FM_E_UNSUPPORTED, "%s: L*2*H too large", fn);
  int64_t min_pages = INT64_MAX;
  for (int l = 0; l < L; ++l) {
    int64_t q;
    if (int s = check_pool(fn, pools[l], dt, l, &q)) return s;
    min_pages = pools[l].num_pages < min_pages ? pools[l].num_pages : min_pages;
  }
  if (out_slots != nullptr && min_pages * (int64_t)page_size > INT32_MAX)
    return fail(FM_E_UNSUPPORTED, "%s: slots do not fit out_slots' int32", fn);
  if (kv_scales != nullptr) {
    if (dt != FM_BF16_E4M3) return fail(FM_E_INVALID, "%s: kv_scales apply to an e4m3 pool only", fn);
    for (int i = 0; i < 2 * L; ++i)
      if (!(kv_scales[i] > 0.f) || !std::isfinite(kv_scales[i]) || !std::isfinite(1.0 / kv_scales[i]))
        return fail(FM_E_INVALID, "%s: kv_scales[%d] must be finite and > 0", fn, i);
  }
  if (use_scratch) {
    uint8_t* sp = nullptr;
    size_t sb = 0;
    const hipError_t e = fm::write_scratch(&sp, &sb);
    if (e != hipSuccess)
      return fail(FM_E_HIP, "%s: no device address for the static workspace: %s", fn, hipGetErrorString(e));
    ws = sp;
    ws_bytes = sb;
  }
  if (int s = check_ws(fn, ws, ws_bytes, fm::write_layout(n_rows).total)) return s;

  fm::WritePrepArgs p{};
  p.row_req = row_req;
  p.row_pos = row_pos;
  p.commit_lens = commit_lens;
  p.window = commit_lens ? window : 0;
  p.bs = bs;
  p.n_rows = n_rows;
  p.page_table = page_table;
  p.pt_stride = pt_stride;
  p.log2ps = log2_exact(page_size);
  p.min_pages = min_pages;
  p.out_slots = out_slots;
  p.ws = static_cast<uint8_t*>(ws);
  p.lay = fm::write_layout(n_rows);

  fm::WriteGemmArgs g{};
  g.x = x;
  g.w = w_kv;
  g.k_norm_w = k_norm_w;
  g.d_in = d_in;
  g.L = L;
  g.H = H;
  g.eps = eps;
  g.ws = p.ws;
  g.lay = p.lay;
  for (int l = 0; l < L; ++l) {
    g.pools[l] = to_desc(pools[l]);
    for (int kv = 0; kv < 2; ++kv) g.inv_scale[l][kv] = kv_scales ? (float)(1.0 / kv_scales[2 * l + kv]) : 1.0f;
  }
  g.rope = rope_freqs(rope_theta, Dh);
  return from_hip(fm::launch_write(p, g, (int)dt, Dh, n_rows, stream), fn);
}

}  // namespace

extern "C" {

int fm_write_context_kv(const void* x, int64_t n_rows, int32_t d_in, fm_dtype dt, const void* w_kv,
                        const float* k_norm_w, const int32_t* row_req, const int32_t* row_pos,
                        const int32_t* commit_lens, int32_t window, const int32_t* page_table, int64_t pt_stride,
                        int32_t page_size, int32_t bs, const fm_kv_pool* pools, int32_t L, int32_t H, int32_t Dh,
                        float eps, float rope_theta, const float* kv_scales, int32_t* out_slots, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  return write_context_kv("fm_write_context_kv", false, x, n_rows, d_in, dt, w_kv, k_norm_w, row_req, row_pos,
                          commit_lens, window, page_table, pt_stride, page_size, bs, pools, L, H, Dh, eps,
                          rope_theta, kv_scales, out_slots, ws, ws_bytes, stream);
}

static_assert(FM_WRITE_NOALLOC_MAX_ROWS == fm::kWriteScratchRows, "fm.h states the static workspace's row limit");

int fm_write_context_kv_noalloc(const void* x, int64_t n_rows, int32_t d_in, fm_dtype dt, const void* w_kv,
                                const float* k_norm_w, const int32_t* row_req, const int32_t* row_pos,
                                const int32_t* commit_lens, int32_t window, const int32_t* page_table,
                                int64_t pt_stride, int32_t page_size, int32_t bs, const fm_kv_pool* pools, int32_t L,
                                int32_t H, int32_t Dh, float eps, float rope_theta, const float* kv_scales,
                                int32_t* out_slots, hipStream_t stream) {
  return write_context_kv("fm_write_context_kv_noalloc", true, x, n_rows, d_in, dt, w_kv, k_norm_w, row_req,
                          row_pos, commit_lens, window, page_table, pt_stride, page_size, bs, pools, L, H, Dh, eps,
                          rope_theta, kv_scales, out_slots, nullptr, 0, stream);
}

size_t fm_context_rows_workspace_size(int64_t n_hidden, int64_t n_anchor, int32_t d_hidden, int32_t d_target,
                                      int32_t dim) {
  // each width matters only when its rows exist (anchors alone pass d_hidden = 0)
  if (n_hidden < 0 || n_anchor < 0 || dim < 1 || (n_hidden == 0 && n_anchor == 0)) return 0;
  if ((n_hidden > 0 && d_hidden < 1) || (n_anchor > 0 && d_target < 1)) return 0;
  return fm::ctx_rows_layout(n_hidden, n_anchor, d_hidden, d_target, dim).total;
}

int fm_context_rows(const void* hidden, int64_t n_hidden, int32_t d_hidden, const void* w_fc,
                    const float* hidden_norm_w, const int32_t* anchor_ids, int64_t n_anchor, const void* embedding,
                    int64_t vocab, int32_t d_target, const void* w_anchor_proj, const void* b_anchor_proj,
                    const float* anchor_norm_w, int32_t dim, const int32_t* commit_lens, int32_t window, int32_t bs,
                    float eps, void* rows, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "fm_context_rows";
  if (n_hidden < 0 || n_anchor < 0) return fail(FM_E_INVALID, "%s: n_hidden and n_anchor must be >= 0", fn);
  if (n_hidden == 0 && n_anchor == 0) return ok();
  if (!rows) return fail(FM_E_INVALID, "%s: rows is null", fn);
  if (dim < 1024 || dim % 1024 || dim > 8192)
    return fail(FM_E_UNSUPPORTED, "%s: dim %d must be a multiple of 1024 in [1024, 8192]", fn, dim);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(FM_E_INVALID, "%s: eps must be finite and >= 0", fn);
  if (!aligned16(rows)) return fail(FM_E_INVALID, "%s: rows must be 16-byte aligned", fn);
  if (n_hidden > 0) {
    if (!hidden || !w_fc || !hidden_norm_w) return fail(FM_E_INVALID, "%s: a hidden-row pointer is null", fn);
    if (d_hidden < 64 || d_hidden % 64)
      return fail(FM_E_UNSUPPORTED, "%s: d_hidden %d must be a positive multiple of 64", fn, d_hidden);
    if (!aligned16(hidden) || !aligned16(w_fc) || !aligned16(hidden_norm_w))
      return fail(FM_E_INVALID, "%s: hidden, w_fc and hidden_norm_w must be 16-byte aligned", fn);
    if (commit_lens != nullptr && (window < 1 || bs < 1 || (int64_t)bs * window > n_hidden))
      return fail(FM_E_INVALID, "%s: commit_lens needs window >= 1 and bs >= 1 with bs * window <= n_hidden", fn);
  }
  if (n_anchor > 0) {
    if (!anchor_ids || !embedding || !w_anchor_proj || !b_anchor_proj || !anchor_norm_w)
      return fail(FM_E_INVALID, "%s: an anchor-row pointer is null", fn);
    if (d_target < 64 || d_target % 64)
      return fail(FM_E_UNSUPPORTED, "%s: d_target %d must be a positive multiple of 64", fn, d_target);
    if (vocab < 1) return fail(FM_E_INVALID, "%s: vocab %lld < 1", fn, (long long)vocab);
    if (!aligned16(embedding) || !aligned16(w_anchor_proj) || !aligned16(b_anchor_proj) || !aligned16(anchor_norm_w))
      return fail(FM_E_INVALID, "%s: embedding, w_anchor_proj, b_anchor_proj, anchor_norm_w must be 16-byte aligned",
                  fn);
  }
  if (n_hidden + n_anchor > INT32_MAX) return fail(FM_E_UNSUPPORTED, "%s: too many rows", fn);
  const fm::CtxRowsLayout lay = fm::ctx_rows_layout(n_hidden, n_anchor, d_hidden, d_target, dim);
  if (int s = check_ws(fn, ws, ws_bytes, lay.total)) return s;
  fm::CtxRowsArgs a{};
  a.hidden = hidden;
  a.n_hidden = n_hidden;
  a.d_hidden = d_hidden;
  a.w_fc = w_fc;
  a.hidden_norm_w = hidden_norm_w;
  a.anchor_ids = anchor_ids;
  a.n_anchor = n_anchor;
  a.embedding = embedding;
  a.vocab = vocab;
  a.d_target = d_target;
  a.w_anchor = w_anchor_proj;
  a.b_anchor = b_anchor_proj;
  a.anchor_norm_w = anchor_norm_w;
  a.dim = dim;
  a.commit_lens = commit_lens;
  a.window = commit_lens ? window : 0;
  a.bs = commit_lens ? bs : 0;
  a.eps = eps;
  a.rows = rows;
  a.ws = static_cast<uint8_t*>(ws);
  a.lay = lay;
  return from_hip(fm::launch_context_rows(a, stream), fn);
}

int fm_ada_layer_norm(const float* h, int64_t rows, int32_t dim, const float* scale, const float* shift, float eps,
                      void* out, hipStream_t stream) {
  const char* fn = "fm_ada_layer_norm";
  if (rows < 0) return fail(FM_E_INVALID, "%s: rows %lld < 0", fn, (long long)rows);
  if (rows == 0) return ok();
  if (!h || !scale || !shift || !out) return fail(FM_E_INVALID, "%s: a required pointer is null", fn);
  if (dim < 1024 || dim % 1024 || dim > 8192)
    return fail(FM_E_UNSUPPORTED, "%s: dim %d must be a multiple of 1024 in [1024, 8192]", fn, dim);
  if (!aligned16(h) || !aligned16(scale) || !aligned16(shift) || !aligned16(out))
    return fail(FM_E_INVALID, "%s: pointers must be 16-byte aligned", fn);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(FM_E_INVALID, "%s: eps must be finite and >= 0", fn);
  if (rows > INT32_MAX) return fail(FM_E_UNSUPPORTED, "%s: rows above 2^31-1", fn);
  fm::AdaLnArgs a{h, rows, dim, scale, shift, eps, out};
  return from_hip(fm::launch_ada_layer_norm(a, stream), fn);
}

size_t fm_linear_workspace_size(int64_t M, int32_t N, int32_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  const int splits = fm::linear_splits(M, N, K);
  if (splits == 1) return 0;
  if ((double)splits * (double)M * (double)N * 4.0 > 0x1p62) return SIZE_MAX;  // no such buffer exists
  return (size_t)splits * (size_t)M * (size_t)N * 4;
}

int fm_linear(const void* x, int64_t M, int32_t K, const void* w, int32_t N, const void* bias,
              fm_linear_epilogue epilogue, const float* gate, void* out, void* ws, size_t ws_bytes,
              hipStream_t stream) {
  const char* fn = "fm_linear";
  if (M < 0) return fail(FM_E_INVALID, "%s: M %lld < 0", fn, (long long)M);
  if (M == 0) return ok();
  if (!x || !w || !out) return fail(FM_E_INVALID, "%s: x, w and out are required", fn);
  if ((int)epilogue < 0 || (int)epilogue > 3) return fail(FM_E_UNSUPPORTED, "%s: epilogue %d", fn, (int)epilogue);
  if (epilogue == FM_LINEAR_RESIDUAL && !gate) return fail(FM_E_INVALID, "%s: the residual epilogue needs gate", fn);
  if (K < 64 || K % 64) return fail(FM_E_UNSUPPORTED, "%s: K %d must be a positive multiple of 64", fn, K);
  if (N < 1024 || N % 1024) return fail(FM_E_UNSUPPORTED, "%s: N %d must be a positive multiple of 1024", fn, N);
  if (!aligned16(x) || !aligned16(w) || !aligned16(out) || (bias && !aligned16(bias)) || (gate && !aligned16(gate)))
    return fail(FM_E_INVALID, "%s: pointers must be 16-byte aligned", fn);
  if (M > INT32_MAX) return fail(FM_E_UNSUPPORTED, "%s: M above 2^31-1", fn);
  const int splits = fm::linear_splits(M, N, K);
  const size_t need = fm_linear_workspace_size(M, N, K);
  if (need > 0) {
    if (int s = check_ws(fn, ws, ws_bytes, need)) return s;
  }
  fm::LinearArgs a{};
  a.x = x;
  a.w = w;
  a.bias = bias;
  a.gate = gate;
  a.out = out;
  a.part = static_cast<float*>(ws);
  a.M = M;
  a.K = K;
  a.N = N;
  a.splits = splits;
  a.epilogue = (int)epilogue;
  return from_hip(fm::launch_linear(a, stream), fn);
}

size_t fm_cross_attention_workspace_size(int32_t bs, int32_t H, int32_t Dh, int32_t max_q, fm_dtype dt) {
  const int nqf = fm::q_frags(max_q);
  if (bs < 0 || H < 1 || (Dh != 64 && Dh != 128) || nqf == 0) return 0;
  if (dt != FM_F32 && dt != FM_BF16 && dt != FM_BF16_E4M3) return 0;
  return fm::plan_layout(bs, H, Dh, plan_waves(dt), nqf).total;
}

}  // extern "C"

namespace {

// Waves on odd XCDs take ~10% longer per tile than waves on even ones on the
// MI355X parts measured (per-wave clocks over one call, K/V through LDS), so
// the default plan weights the shares 1045 : 955 for even : odd XCDs, over
// every pool type.  fm_plan_cross_attention_weighted takes measured weights.
constexpr int32_t kXcdSkew = 45;

int plan_cross_attention(const char* fn, const int32_t* ctx_lens, int32_t bs, int32_t H, int32_t Dh, int32_t max_q,
                         fm_dtype dt, const int32_t* xcd_weights, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dt != FM_F32 && dt != FM_BF16 && dt != FM_BF16_E4M3)
    return fail(FM_E_UNSUPPORTED, "%s: dtype %d is not FM_F32, FM_BF16 or FM_BF16_E4M3", fn, (int)dt);
  if (bs < 0) return fail(FM_E_INVALID, "%s: bs %d < 0", fn, bs);
  if (H < 1) return fail(FM_E_INVALID, "%s: H = %d must be >= 1", fn, H);
  if (Dh != 64 && Dh != 128) return fail(FM_E_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", fn, Dh);
  if (max_q < 0) return fail(FM_E_INVALID, "%s: max_q %d < 0", fn, max_q);
  if (max_q > fm::kQRows * fm::kMaxQFrags)
    return fail(FM_E_UNSUPPORTED, "%s: max_q %d above %d query rows per request", fn, max_q,
                fm::kQRows * fm::kMaxQFrags);
  if (bs > 0 && !ctx_lens) return fail(FM_E_INVALID, "%s: ctx_lens is null", fn);
  if ((int64_t)bs * H > INT32_MAX) return fail(FM_E_UNSUPPORTED, "%s: bs * H too large", fn);
  const fm::PlanLayout lay = fm::plan_layout(bs, H, Dh, plan_waves(dt), fm::q_frags(max_q));
  if (int s = check_ws(fn, ws, ws_bytes, lay.total)) return s;
  fm::PlanArgs a{};
  a.ctx_lens = ctx_lens;
  a.bs = bs;
  a.H = H;
  a.Dh = Dh;
  a.dtype = (int32_t)dt;
  for (int x = 0; x < fm::kXcds; ++x) {
    if (xcd_weights == nullptr) {
      a.xcd_w[x] = x % 2 == 0 ? 1000 + kXcdSkew : 1000 - kXcdSkew;
    } else {
      if (xcd_weights[x] < fm::kXcdWeightMin || xcd_weights[x] > fm::kXcdWeightMax)
        return fail(FM_E_INVALID, "%s: xcd_weights[%d] = %d outside [%d, %d]", fn, x, xcd_weights[x],
                    fm::kXcdWeightMin, fm::kXcdWeightMax);
      a.xcd_w[x] = xcd_weights[x];
    }
  }
  a.ws = static_cast<uint8_t*>(ws);
  a.lay = lay;
  return from_hip(fm::launch_plan(a, stream), fn);
}

}  // namespace

extern "C" {

int fm_plan_cross_attention(const int32_t* ctx_lens, int32_t bs, int32_t H, int32_t Dh, int32_t max_q, fm_dtype dt,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  return plan_cross_attention("fm_plan_cross_attention", ctx_lens, bs, H, Dh, max_q, dt, nullptr, ws, ws_bytes,
                              stream);
}

int fm_plan_cross_attention_weighted(const int32_t* ctx_lens, int32_t bs, int32_t H, int32_t Dh, int32_t max_q,
                                     fm_dtype dt, const int32_t* xcd_weights, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  const char* fn = "fm_plan_cross_attention_weighted";
  if (!xcd_weights) return fail(FM_E_INVALID, "%s: xcd_weights is null", fn);
  return plan_cross_attention(fn, ctx_lens, bs, H, Dh, max_q, dt, xcd_weights, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// The call of fm_paged_cross_attention and fm_paged_cross_attention_timed
// (wave_clock: null, or wave_clock_len records of 4 words).
int paged_cross_attention(const char* fn, const void* q, fm_dtype dt, int64_t total_q, const float* q_norm_w,
                          const fm_kv_pool* pool, const int32_t* page_table, int64_t pt_stride, int32_t page_size,
                          const int32_t* ctx_lens, const int32_t* cu_seqlens_q, int32_t max_q, int32_t bs, int32_t H,
                          int32_t Dh, float softmax_scale, float rope_theta, float eps, const float* fp8_scales,
                          void* out, void* ws, size_t ws_bytes, uint64_t* wave_clock, int64_t wave_clock_len,
                          hipStream_t stream) {
  if (total_q < 0 || bs < 0) return fail(FM_E_INVALID, "%s: total_q and bs must be >= 0", fn);
  if (total_q == 0 || bs == 0) return ok();
  if (int s = check_common(fn, dt, H, Dh, eps, rope_theta)) return s;
  if (!q || !q_norm_w || !pool || !page_table || !ctx_lens || !cu_seqlens_q || !out)
    return fail(FM_E_INVALID, "%s: a required pointer is null", fn);
  if (!aligned16(q) || !aligned16(out)) return fail(FM_E_INVALID, "%s: q and out must be 16-byte aligned", fn);
  if (!is_pow2(page_size) || page_size > 4096)
    return fail(FM_E_UNSUPPORTED, "%s: page_size %d is not a power of two in [1, 4096]", fn, page_size);
  if (pt_stride < 1) return fail(FM_E_INVALID, "%s: pt_stride %lld < 1", fn, (long long)pt_stride);
  if (!std::isfinite(softmax_scale)) return fail(FM_E_INVALID, "%s: softmax_scale must be finite", fn);
  if (total_q > INT32_MAX) return fail(FM_E_UNSUPPORTED, "%s: total_q above 2^31-1", fn);
  int64_t q16;
  if (int s = check_pool(fn, *pool, dt, 0, &q16)) return s;
  if (max_q < 0) return fail(FM_E_INVALID, "%s: max_q %d < 0", fn, max_q);
  const int nqf = fm::q_frags(max_q);
  if (nqf == 0)
    return fail(FM_E_UNSUPPORTED, "%s: max_q %d above %d query rows per request", fn, max_q,
                fm::kQRows * fm::kMaxQFrags);
  float q_static = 0.f, k_descale = 1.f, v_descale = 1.f;
  if (fp8_scales != nullptr) {
    if (dt != FM_BF16_E4M3) return fail(FM_E_INVALID, "%s: fp8_scales apply to an e4m3 pool only", fn);
    q_static = fp8_scales[0];
    k_descale = fp8_scales[1];
    v_descale = fp8_scales[2];
    if (!(q_static >= 0.f) || !std::isfinite(q_static) || (q_static > 0.f && !std::isfinite(1.0 / q_static)))
      return fail(FM_E_INVALID, "%s: fp8_scales[0] (query scale) must be 0 or finite and > 0", fn);
    if (!(k_descale > 0.f) || !std::isfinite(k_descale) || !(v_descale > 0.f) || !std::isfinite(v_descale))
      return fail(FM_E_INVALID, "%s: fp8_scales[1..2] (key, value descales) must be finite and > 0", fn);
  }
  const fm::PlanLayout lay = fm::plan_layout(bs, H, Dh, plan_waves(dt), nqf);
  if (int s = check_ws(fn, ws, ws_bytes, lay.total)) return s;
  if (wave_clock != nullptr && wave_clock_len < lay.n_waves)
    return fail(FM_E_INVALID, "%s: %lld wave records for %d waves", fn, (long long)wave_clock_len, lay.n_waves);
  fm::CrossArgs a{};
  a.wave_clock = wave_clock;
  a.q = q;
  a.out = out;
  a.q_norm_w = q_norm_w;
  if (pool->page_stride > UINT32_MAX || pool->slot_stride > UINT32_MAX || pool->head_stride > UINT32_MAX)
    return fail(FM_E_UNSUPPORTED, "%s: pool strides must be below 2^32 elements", fn);
  a.pool = to_desc(*pool);
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.log2ps = log2_exact(page_size);
  a.page_stride32 = (uint32_t)pool->page_stride;
  a.slot_stride32 = (uint32_t)pool->slot_stride;
  a.head_stride32 = (uint32_t)pool->head_stride;
  a.num_pages32 = (int32_t)std::min<int64_t>(pool->num_pages, INT32_MAX);  // page ids are int32
  a.pt_stride32 = (int32_t)std::min<int64_t>(pt_stride, INT32_MAX);
  a.ctx_lens = ctx_lens;
  a.cu_q = cu_seqlens_q;
  a.bs = bs;
  a.H = H;
  a.total_q = (int32_t)total_q;
  a.qscale_log2 = (float)((double)softmax_scale * (double)k_descale * 1.4426950408889634074);
  a.eps = eps;
  a.q_static = q_static;
  a.q_static_inv = q_static > 0.f ? (float)(1.0 / q_static) : 0.f;
  a.v_descale = v_descale;
  a.ws = static_cast<uint8_t*>(ws);
  a.lay = lay;
  a.rope = rope_freqs(rope_theta, Dh);
  return from_hip(fm::launch_cross_attention(a, (int)dt, Dh, stream), fn);
}

}  // namespace

extern "C" {

int fm_paged_cross_attention(const void* q, fm_dtype dt, int64_t total_q, const float* q_norm_w,
                             const fm_kv_pool* pool, const int32_t* page_table, int64_t pt_stride, int32_t page_size,
                             const int32_t* ctx_lens, const int32_t* cu_seqlens_q, int32_t max_q, int32_t bs,
                             int32_t H, int32_t Dh, float softmax_scale, float rope_theta, float eps,
                             const float* fp8_scales, void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return paged_cross_attention("fm_paged_cross_attention", q, dt, total_q, q_norm_w, pool, page_table, pt_stride,
                               page_size, ctx_lens, cu_seqlens_q, max_q, bs, H, Dh, softmax_scale, rope_theta, eps,
                               fp8_scales, out, ws, ws_bytes, nullptr, 0, stream);
}

int fm_paged_cross_attention_timed(const void* q, fm_dtype dt, int64_t total_q, const float* q_norm_w,
                                   const fm_kv_pool* pool, const int32_t* page_table, int64_t pt_stride,
                                   int32_t page_size, const int32_t* ctx_lens, const int32_t* cu_seqlens_q,
                                   int32_t max_q, int32_t bs, int32_t H, int32_t Dh, float softmax_scale,
                                   float rope_theta, float eps, const float* fp8_scales, void* out, void* ws,
                                   size_t ws_bytes, uint64_t* wave_clock, int64_t wave_clock_len, hipStream_t stream) {
  const char* fn = "fm_paged_cross_attention_timed";
  if (wave_clock == nullptr) return fail(FM_E_INVALID, "%s: wave_clock is null", fn);
  return paged_cross_attention(fn, q, dt, total_q, q_norm_w, pool, page_table, pt_stride, page_size, ctx_lens,
                               cu_seqlens_q, max_q, bs, H, Dh, softmax_scale, rope_theta, eps, fp8_scales, out, ws,
                               ws_bytes, wave_clock, wave_clock_len, stream);
}

int fm_block_self_attention(const void* qkv, fm_dtype dt, int32_t n_blocks, int32_t K, const float* q_norm_w,
                            const float* k_norm_w, const int32_t* ctx_lens, int32_t H, int32_t Dh,
                            float softmax_scale, float rope_theta, float eps, void* out, hipStream_t stream) {
  const char* fn = "fm_block_self_attention";
  if (n_blocks < 0) return fail(FM_E_INVALID, "%s: n_blocks %d < 0", fn, n_blocks);
  if (n_blocks == 0) return ok();
  if (int s = check_common(fn, dt, H, Dh, eps, rope_theta)) return s;
  if (dt == FM_BF16_E4M3)
    return fail(FM_E_UNSUPPORTED, "%s: the block's own q, k, v are activations: use FM_BF16", fn);
  if (K < 1 || K > 64) return fail(FM_E_UNSUPPORTED, "%s: block size %d not in [1, 64]", fn, K);
  if (!qkv || !q_norm_w || !k_norm_w || !ctx_lens || !out)
    return fail(FM_E_INVALID, "%s: a required pointer is null", fn);
  if (!aligned16(qkv) || !aligned16(out)) return fail(FM_E_INVALID, "%s: qkv and out must be 16-byte aligned", fn);
  if (!std::isfinite(softmax_scale)) return fail(FM_E_INVALID, "%s: softmax_scale must be finite", fn);
  if ((int64_t)n_blocks * H * ((K + 15) / 16) > INT32_MAX)
    return fail(FM_E_UNSUPPORTED, "%s: n_blocks * H * query tiles too large", fn);
  fm::SelfArgs a{};
  a.qkv = qkv;
  a.out = out;
  a.q_norm_w = q_norm_w;
  a.k_norm_w = k_norm_w;
  a.ctx_lens = ctx_lens;
  a.n_blocks = n_blocks;
  a.K = K;
  a.H = H;
  a.qscale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  a.eps = eps;
  a.rope = rope_freqs(rope_theta, Dh);
  return from_hip(fm::launch_self_attention(a, dt == FM_BF16 ? 1 : 0, Dh, stream), fn);
}

}  // extern "C"
