/*
 * fm.h - C ABI of the FlashMap draft-step attention path on MI355X (gfx950).
 *
 * The draft step of the FlashMap block drafter (flashmap 0.1.0 wheel:
 * sglang/model.py ``forward`` / ``_denoise``, vllm/model.py ``forward`` /
 * ``_dit``, modeling_flashmap.py ``draft``) runs, for every DiT layer:
 *   0. the rows that write takes: committed target positions through fc and
 *      hidden_norm, anchors through anchor_proj and anchor_norm
 *                                             -> fm_context_rows
 *   1. the context/anchor K/V write: one GEMM over every layer's context K/V
 *      weight, RMS k-norm, interleaved-pair RoPE and a paged scatter that skips
 *      uncommitted verify columns            -> fm_write_context_kv
 *   2. paged cross-attention of each request's draft rows onto its context
 *      positions 0..p                         -> fm_plan_cross_attention (once
 *      per step) + fm_paged_cross_attention (once per layer)
 *   3. bidirectional self-attention within each draft block
 *                                             -> fm_block_self_attention
 *   around them, the rest of each DiT block: time-modulated LayerNorms,
 *   projections with gated residuals, the GELU MLP
 *                                             -> fm_ada_layer_norm, fm_linear
 *
 * Conventions shared by every entry point
 *   - Pointers named as DEVICE pointers are device memory owned by the caller;
 *     the library never allocates, frees or keeps them.  Host pointers are read
 *     during the call only.
 *   - Every call is asynchronous on ``stream`` and never synchronizes with the
 *     host: it validates its host-side arguments, enqueues its kernels and
 *     returns.  Calls with all sizes zero enqueue nothing and return FM_OK.
 *   - Failures return a negative fm_status and leave a message for
 *     fm_last_error(); nothing is enqueued then.  FM_E_HIP means a launch
 *     failed after validation.
 *   - Element strides are in elements, not bytes.  Every head row (head_dim
 *     values) is contiguous and 16-byte aligned.
 *   - Device-side index checks: a page-table entry outside [0, num_pages), a
 *     position whose page index is past the page-table row, or a request index
 *     outside [0, bs) never produces an access outside the buffers; the row or
 *     token it names is skipped and bit 0 of the workspace's error word (the
 *     int32 at byte offset 4 of ``ws``) is set.  Such inputs are caller errors.
 *   - Not thread-safe on one workspace: calls that share ``ws`` must be ordered
 *     on one stream.
 */
#ifndef FM_H
#define FM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fm_status {
  FM_OK = 0,
  FM_E_INVALID = -1,     /* a null required pointer, a negative size, inconsistent sizes */
  FM_E_UNSUPPORTED = -2, /* a shape or type the library does not implement, or sizes whose launch grid
                            would reach 2^32 work-items */
  FM_E_WORKSPACE = -3,   /* workspace null, misaligned or smaller than required */
  FM_E_HIP = -4          /* a HIP launch failed */
} fm_status;

/* Storage type of the activations and of the KV pool.  FM_F32 and FM_BF16:
 * one type for both.  FM_BF16_E4M3: bf16 activations over an OCP float8 e4m3
 * ("e4m3fn") pool written with scale 1 (sglang/model.py ``_kv_write`` with
 * ``kv_norm_rope_write_fp8``, ``_paged_cross_attention_fp8``); the write
 * rounds each key/value to nearest-even e4m3, saturating at +-448, and
 * cross-attention quantizes the query per (request, head) as documented
 * there.  Block self-attention reads no pool and takes FM_F32 or FM_BF16. */
typedef enum fm_dtype { FM_F32 = 0, FM_BF16 = 1, FM_BF16_E4M3 = 2 } fm_dtype;

/* One layer's paged KV pool (vllm/model.py ``cache_layout``: page, head and
 * slot strides with head_dim contiguous; sglang's pool is page_size 1).
 * Key of slot ``s`` of page ``p`` for head ``h``: k + p*page_stride +
 * s*slot_stride + h*head_stride, head_dim contiguous elements; the value is at
 * the same offset from v.  Element type = the call's pool type (fp32, bf16 or
 * e4m3 for FM_F32, FM_BF16, FM_BF16_E4M3); strides count elements.
 * All strides and the byte addresses of k and v must be multiples of 16 bytes;
 * fm_paged_cross_attention also takes each stride below 2^32 elements
 * (FM_E_UNSUPPORTED otherwise). */
typedef struct fm_kv_pool {
  void* k;               /* DEVICE */
  void* v;               /* DEVICE */
  int64_t num_pages;     /* pages in this pool; page ids must lie in [0, num_pages) */
  int64_t page_stride;
  int64_t slot_stride;
  int64_t head_stride;
} fm_kv_pool;

/* Message of the last failure on the calling thread ("" if none). */
const char* fm_last_error(void);

/* Library version string. */
const char* fm_version(void);

/* ---------------------------------------------------------------- write -- */

/* Workspace bytes fm_write_context_kv needs for n_rows rows. */
size_t fm_write_context_kv_workspace_size(int64_t n_rows);

/*
 * Context/anchor K/V write of every layer (sglang/model.py
 * ``write_target_hidden_kv``, ``_write_context``, ``_kv_write``; vllm/model.py
 * ``_prologue``, ``_write``; modeling_flashmap.py ``project_kv``).
 *
 *   y_r = W_kv x_r                    one GEMM over all layers, fp32 accumulate
 *   for layer l, head h:
 *     k = RoPE(RMSNorm(y_r[l,k,h,:]; k_norm_w[l], eps), pos_r)   interleaved pairs
 *     v = y_r[l,v,h,:]                                           (no norm, no RoPE)
 *     slot = page_table[req_r][pos_r / page_size]*page_size + pos_r % page_size
 *     pools[l].k[slot, h, :] = k ;  pools[l].v[slot, h, :] = v  (rounded once)
 *
 * x          DEVICE [n_rows, d_in], row-major, the activation type of dt
 *            (bf16 for FM_BF16_E4M3; w_kv likewise).
 * w_kv       DEVICE [L*2*H*Dh, d_in] row-major: rows ordered (layer, {k, v},
 *            head, dim), i.e. the concatenation [k_proj_0; v_proj_0; k_proj_1; ...].
 * k_norm_w   DEVICE fp32 [L, Dh]: each layer's key RMSNorm weight.
 * row_req    DEVICE int32 [n_rows]: request (page-table row) of each row.
 * row_pos    DEVICE int32 [n_rows]: position of each row; a negative position
 *            skips the row.
 * commit_lens, window
 *            Optional verify-window rule (``commit_lens`` DEVICE int32 [bs], or
 *            NULL).  When given, rows [0, bs*window) are bs verify windows of
 *            ``window`` columns, request-major, and column j of request b is
 *            written only if j < commit_lens[b]; rows from bs*window on (the
 *            anchors) follow row_pos alone.
 * page_table DEVICE int32 [bs, pt_stride]: physical page of each logical page.
 * page_size  a power of two in [1, 4096].
 * pools      HOST array [L]; L <= 16.
 * H, Dh      heads and head dim; Dh in {64, 128}.  d_in a multiple of 64.
 * eps        RMSNorm epsilon;  rope_theta  RoPE base.
 * kv_scales  HOST float [L][2] (key scale, value scale of each layer) or NULL
 *            (all 1).  e4m3 pools only (FM_E_INVALID otherwise): the pool
 *            receives e4m3(k / k_scale) and e4m3(v / v_scale), as vLLM's
 *            calibrated fp8 caches do (vllm/model.py ``write_context_kv`` with
 *            ``kv_scales``); every scale finite and > 0.
 * out_slots  DEVICE int32 [n_rows] or NULL: slot written by each row, -1 if skipped.
 * ws         DEVICE workspace of fm_write_context_kv_workspace_size(n_rows)
 *            bytes, 256-byte aligned; its contents need no initialisation.
 * Rows that are written must name distinct slots.  Skipped rows cost no GEMM
 * work and touch no pool byte.
 */
int fm_write_context_kv(const void* x, int64_t n_rows, int32_t d_in, fm_dtype dt,
                        const void* w_kv, const float* k_norm_w,
                        const int32_t* row_req, const int32_t* row_pos,
                        const int32_t* commit_lens, int32_t window,
                        const int32_t* page_table, int64_t pt_stride, int32_t page_size,
                        int32_t bs, const fm_kv_pool* pools, int32_t L, int32_t H, int32_t Dh,
                        float eps, float rope_theta, const float* kv_scales, int32_t* out_slots,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/* Rows fm_write_context_kv_noalloc serves (its static workspace's size). */
#define FM_WRITE_NOALLOC_MAX_ROWS 65536

/*
 * fm_write_context_kv without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, computation and results
 * as fm_write_context_kv (the same kernels); the workspace is instead a static
 * device array of about 1 MB that the library holds on every GPU it runs on
 * until the process ends.  The entry point allocates and frees nothing.
 *
 * n_rows must not exceed FM_WRITE_NOALLOC_MAX_ROWS (FM_E_UNSUPPORTED
 * otherwise, nothing enqueued).  The array's device address is looked up on a
 * device's first call (FM_E_HIP if that fails).  Every call on one GPU shares
 * that GPU's array: calls that may overlap on one GPU (different streams, or
 * host threads without ordering) race and must be serialized by the caller.
 * The array needs no initialisation: each call rewrites what it reads.
 */
int fm_write_context_kv_noalloc(const void* x, int64_t n_rows, int32_t d_in, fm_dtype dt,
                                const void* w_kv, const float* k_norm_w,
                                const int32_t* row_req, const int32_t* row_pos,
                                const int32_t* commit_lens, int32_t window,
                                const int32_t* page_table, int64_t pt_stride, int32_t page_size,
                                int32_t bs, const fm_kv_pool* pools, int32_t L, int32_t H, int32_t Dh,
                                float eps, float rope_theta, const float* kv_scales, int32_t* out_slots,
                                hipStream_t stream);

/* ------------------------------------------------------- context rows -- */

/* Workspace bytes fm_context_rows needs (0 for invalid sizes or no rows).  A
 * width counts only when its rows exist: anchors alone pass d_hidden = 0. */
size_t fm_context_rows_workspace_size(int64_t n_hidden, int64_t n_anchor, int32_t d_hidden, int32_t d_target,
                                      int32_t dim);

/*
 * The rows fm_write_context_kv projects (sglang/model.py ``_write_context``,
 * ``_anchor_kv_impl``; vllm/model.py ``combine_hidden_states``,
 * ``precompute_and_store_context_kv``, ``_prologue``;
 * modeling_flashmap.py ``fc``, ``hidden_norm``, ``anchor_proj``, ``anchor_norm``):
 *
 *   rows[r]            = RMSNorm(W_fc hidden[r]; hidden_norm_w, eps)            r < n_hidden
 *   rows[n_hidden + a] = RMSNorm(W_ap embedding[anchor_ids[a]] + b_ap; anchor_norm_w, eps)
 *
 * fp32 accumulation, each row rounded once to bf16.  Hidden rows the commit
 * rule skips are neither computed nor written (their rows are left as they
 * were); it is the rule of fm_write_context_kv, so passing ``rows`` as its x
 * (with the anchors as its last n_anchor rows) writes the same context.
 *
 * hidden       DEVICE bf16 [n_hidden, d_hidden]: the target's hidden states of
 *              the chosen layers, concatenated per row (d_hidden = n_aux *
 *              target hidden size), a multiple of 64.
 * w_fc         DEVICE bf16 [dim, d_hidden] (``fc``, no bias).
 * hidden_norm_w, anchor_norm_w   DEVICE fp32 [dim].
 * anchor_ids   DEVICE int32 [n_anchor]: anchor tokens; an id outside [0, vocab)
 *              reads a clamped row and sets bit 0 of the workspace error word.
 * embedding    DEVICE bf16 [vocab, d_target] (the target's token embedding).
 * w_anchor_proj DEVICE bf16 [dim, d_target];  b_anchor_proj DEVICE bf16 [dim].
 * dim          DiT width, a multiple of 1024 in [1024, 8192].
 * commit_lens, window, bs  optional verify-window rule, as in
 *              fm_write_context_kv: rows [0, bs*window) are request-major
 *              windows and column j of request b is computed only if
 *              j < commit_lens[b] (NULL: every hidden row).
 * rows         DEVICE bf16 [n_hidden + n_anchor, dim].
 * ws           DEVICE workspace of fm_context_rows_workspace_size(...) bytes,
 *              256-byte aligned.
 * Every pointer 16-byte aligned.
 */
int fm_context_rows(const void* hidden, int64_t n_hidden, int32_t d_hidden, const void* w_fc,
                    const float* hidden_norm_w, const int32_t* anchor_ids, int64_t n_anchor, const void* embedding,
                    int64_t vocab, int32_t d_target, const void* w_anchor_proj, const void* b_anchor_proj,
                    const float* anchor_norm_w, int32_t dim, const int32_t* commit_lens, int32_t window, int32_t bs,
                    float eps, void* rows, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------- the DiT layer -- */

/*
 * The time-modulated LayerNorm of a DiT block (sglang/model.py ``_denoise``;
 * modeling_flashmap.py ``FlashMapAdaLayerNorm``):
 *   out[r] = LayerNorm(h[r]) * scale + shift      (no affine LayerNorm, eps)
 * h      DEVICE fp32 [rows, dim]: the residual stream.
 * scale  DEVICE fp32 [dim]: the step's 1 + scale;  shift  DEVICE fp32 [dim].
 * out    DEVICE bf16 [rows, dim]: the next projection's operand (rounded once).
 * dim    a multiple of 1024 in [1024, 8192].  Pointers 16-byte aligned.
 */
int fm_ada_layer_norm(const float* h, int64_t rows, int32_t dim, const float* scale, const float* shift, float eps,
                      void* out, hipStream_t stream);

/* Epilogues of fm_linear (y = x W^T + bias, fp32 accumulate). */
typedef enum fm_linear_epilogue {
  FM_LINEAR_BF16 = 0,        /* out bf16 [M, N] = y                           (qkv, q projections) */
  FM_LINEAR_GELU_BF16 = 1,   /* out bf16 [M, N] = gelu(y), exact erf GELU     (fc1) */
  FM_LINEAR_RESIDUAL = 2,    /* out fp32 [M, N] += gate * y                   (o_proj, fc2: gated residual) */
  FM_LINEAR_ASSIGN_F32 = 3   /* out fp32 [M, N] = y                           (x_embed) */
} fm_linear_epilogue;

/* Workspace bytes fm_linear needs for these sizes (0: none; SIZE_MAX: sizes
 * no buffer can serve, which fm_linear rejects). */
size_t fm_linear_workspace_size(int64_t M, int32_t N, int32_t K);

/*
 * A projection of the DiT block (sglang/model.py ``_denoise``: qkv, self and
 * cross ``o_proj``, cross ``q_proj``, ``fc1`` + GELU, ``fc2``; ``x_embed``),
 * y = x W^T + bias with the gated residual of ``hidden = hidden + gate * y``
 * folded in.  The contraction may be split into ranges whose fp32 partials
 * are summed in a fixed order (the result does not depend on scheduling).
 * x     DEVICE bf16 [M, K] row-major;  w  DEVICE bf16 [N, K] (nn.Linear layout).
 * bias  DEVICE bf16 [N] or NULL;  gate  DEVICE fp32 [N] (FM_LINEAR_RESIDUAL).
 * K a multiple of 64; N a multiple of 1024.  Pointers 16-byte aligned.
 * ws    DEVICE, fm_linear_workspace_size(M, N, K) bytes, 256-byte aligned (may
 *       be NULL when that is 0).
 */
int fm_linear(const void* x, int64_t M, int32_t K, const void* w, int32_t N, const void* bias,
              fm_linear_epilogue epilogue, const float* gate, void* out, void* ws, size_t ws_bytes,
              hipStream_t stream);

/* ------------------------------------------------------ cross-attention -- */

/* Workspace bytes for a cross-attention plan of bs requests with head dim Dh,
 * at most max_q query rows per request (max_q <= 64) and pool type dt on the
 * current device; 0 for an unsupported shape or type.  One workspace serves
 * every layer's call of a step. */
size_t fm_cross_attention_workspace_size(int32_t bs, int32_t H, int32_t Dh, int32_t max_q, fm_dtype dt);

/*
 * Tile schedule of paged cross-attention, computed once per draft step on the
 * device and reused by every layer's fm_paged_cross_attention (sglang/model.py
 * ``_cross_attention_schedule``: it depends only on shapes and lengths).
 *
 * The work of a call is the stream of 16-key tiles of every (request, head)
 * pair; the plan cuts it into contiguous ranges, one per resident wavefront
 * of the attention kernel, whatever the mix of context lengths.  Workgroups
 * run round-robin on the part's 8 XCDs (wave w on XCD (w / 4) mod 8), and a
 * range's length is proportional to its XCD's weight: by default 1045 for
 * even and 955 for odd XCDs (waves on odd XCDs stream ~10% slower per tile on
 * the parts measured).  fm_plan_cross_attention_weighted takes the 8 weights
 * instead.  The cut, and
 * so every result bit, depends only on the lengths and the weights.
 * ctx_lens  DEVICE int32 [bs]: keys per request, p + 1 (0 = empty context).
 * max_q     host bound on query rows per request: one draft block (16) or up
 *           to four candidate blocks side by side (<= 64), checked here.
 * dt        the pool type of the calls the plan serves: the number of
 *           resident waves, and so the cut, depends on it (two per SIMD over
 *           an e4m3 pool, one otherwise).
 * ws        DEVICE, fm_cross_attention_workspace_size(bs, H, Dh, max_q, dt)
 *           bytes, 256-byte aligned.
 */
int fm_plan_cross_attention(const int32_t* ctx_lens, int32_t bs, int32_t H, int32_t Dh, int32_t max_q,
                            fm_dtype dt, void* ws, size_t ws_bytes, hipStream_t stream);

/* fm_plan_cross_attention with the XCD weights given: xcd_weights HOST int32
 * [8], weight of the waves on XCD x (read during the call; each in
 * [500, 2000], FM_E_INVALID otherwise).  For parts whose XCDs stream at rates
 * other than the default's: weights proportional to each XCD's measured rate
 * (fm_paged_cross_attention_timed measures it) let every wave finish at the
 * same time. */
int fm_plan_cross_attention_weighted(const int32_t* ctx_lens, int32_t bs, int32_t H, int32_t Dh, int32_t max_q,
                                     fm_dtype dt, const int32_t* xcd_weights, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/*
 * Paged cross-attention (sglang/model.py ``_paged_cross_attention`` +
 * ``rms_norm_rope``; vllm/model.py ``paged_cross_attention``; modeling_flashmap.py
 * ``FlashMapAttention.forward`` with the ``draft`` positions).
 *
 * For request b, query row r in [cu_seqlens_q[b], cu_seqlens_q[b+1]) is draft
 * slot k = (r - cu_seqlens_q[b]) mod 16 at position ctx_lens[b] + k.  One
 * draft block has 16 rows; tree drafting puts a request's candidate blocks
 * side by side on the query axis, candidate-major, so that its context is
 * read once for all of them (sglang/model.py ``forward``, ``n_cand``):
 *   q^ = RoPE(RMSNorm(q[r,h,:]; q_norm_w, eps), ctx_lens[b] + k)
 *   out[r,h,:] = sum_t softmax_t(softmax_scale * q^.K_t) V_t,  t = 0..ctx_lens[b]-1
 * non-causal, one KV head per query head; keys/values are read through the
 * page table from ``pool``.  ctx_lens[b] = 0 gives out = 0.
 * Over an e4m3 pool (FM_BF16_E4M3; sglang/model.py ``_paged_cross_attention_fp8``)
 * q^ is first quantized per (request, head): s = max(max |q^|, 1e-12) / 448
 * over the request's rows and the head's channels, q8 = e4m3(q^ / s) (nearest,
 * ties to even, from fp32, saturating at +-448), and the scores use s * q8
 * (the softmax weights stay bf16; the e4m3 values enter the products exactly).
 * fp8_scales (HOST float[3] or NULL) = {q_scale, k_scale, v_scale} of vLLM's
 * per-tensor fp8 caches (vllm/model.py ``_dit``, ``paged_cross_attention``
 * descales): q_scale > 0 replaces s by that fixed scale (0 keeps the
 * per-(request, head) one); keys and values enter as k_scale and v_scale
 * times their codes.  NULL = {0, 1, 1}.  e4m3 pools only (FM_E_INVALID
 * otherwise); scales finite, k_scale and v_scale > 0.
 *
 * q, out      DEVICE [total_q, H, Dh] contiguous, the activation type of dt.
 * q_norm_w    DEVICE fp32 [Dh].
 * pool        HOST pointer to this layer's pool descriptor.
 * page_table  DEVICE int32 [bs, pt_stride].
 * ctx_lens, bs, H  as given to fm_plan_cross_attention, whose plan ``ws``
 *             must hold (same stream, earlier; lengths unchanged since).  A
 *             plan made for another bs, H, Dh, max_q fragment count or pool
 *             type (the plan header records each) computes nothing: only the
 *             zero rows of empty contexts are written, the plan's records are
 *             left as they were, and bit 2 of the error word is set.  If the
 *             lengths changed after the plan, the outputs are unspecified, no
 *             access leaves the buffers, and bit 1 of the error word is set
 *             when a wave's share runs past the last tile (not every change
 *             does that, so the bit is no proof that nothing changed); plan
 *             again.
 * cu_seqlens_q  DEVICE int32 [bs+1]: query rows of request b are
 *             [cu_seqlens_q[b], cu_seqlens_q[b+1]), at most max_q of them.
 * max_q       host bound on query rows per request (<= 64), the value the plan
 *             in ``ws`` was made with (a plan made with another value is a
 *             plan for other shapes, above); rows past it are not computed.
 * Dh in {64, 128}; page_size a power of two in [1, 4096].
 */
int fm_paged_cross_attention(const void* q, fm_dtype dt, int64_t total_q, const float* q_norm_w,
                             const fm_kv_pool* pool, const int32_t* page_table, int64_t pt_stride,
                             int32_t page_size, const int32_t* ctx_lens,
                             const int32_t* cu_seqlens_q, int32_t max_q, int32_t bs, int32_t H, int32_t Dh,
                             float softmax_scale, float rope_theta, float eps, const float* fp8_scales,
                             void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* fm_paged_cross_attention that also times its waves, to measure the XCDs'
 * rates for fm_plan_cross_attention_weighted on the part at hand: every wave
 * with tiles writes wave_clock[4 w .. 4 w + 3] (DEVICE uint64) = the start
 * and the end of its tile loop on the GPU's constant 100 MHz clock
 * (s_memrealtime), the XCD it ran on (0-7) and its tile count; waves without
 * tiles write nothing.  wave_clock_len is the number of records the array
 * holds, at least the plan's wave count (4 per CU, times 2 over an e4m3 pool;
 * at most 4096), FM_E_INVALID otherwise or if wave_clock is null.  The
 * results are those of fm_paged_cross_attention, bit for bit. */
int fm_paged_cross_attention_timed(const void* q, fm_dtype dt, int64_t total_q, const float* q_norm_w,
                                   const fm_kv_pool* pool, const int32_t* page_table, int64_t pt_stride,
                                   int32_t page_size, const int32_t* ctx_lens, const int32_t* cu_seqlens_q,
                                   int32_t max_q, int32_t bs, int32_t H, int32_t Dh, float softmax_scale,
                                   float rope_theta, float eps, const float* fp8_scales, void* out, void* ws,
                                   size_t ws_bytes, uint64_t* wave_clock, int64_t wave_clock_len,
                                   hipStream_t stream);

/* ------------------------------------------------------- self-attention -- */

/*
 * Bidirectional self-attention within each draft block (sglang/model.py
 * ``_denoise`` -> ``block_self_attention``; modeling_flashmap.py
 * ``FlashMapLayer`` self-attention over the block's slots).
 *
 * Slot i of block b sits at position ctx_lens[b] + i:
 *   q^_i = RoPE(RMSNorm(q_i; q_norm_w, eps)),  k^_i = RoPE(RMSNorm(k_i; k_norm_w, eps))
 *   out[b,i,h,:] = sum_j softmax_j(softmax_scale * q^_i.k^_j) v_j,  j = 0..K-1
 *
 * qkv   DEVICE [n_blocks, K, 3, H, Dh] contiguous ([q; k; v] per slot), dtype dt.
 * q_norm_w, k_norm_w  DEVICE fp32 [Dh].
 * ctx_lens  DEVICE int32 [n_blocks].
 * out   DEVICE [n_blocks, K, H, Dh] contiguous, dtype dt.
 * 1 <= K <= 64 (a draft block is 16 slots; larger blocks run one wavefront
 * per 16-slot query tile, each scoring all K keys); Dh in {64, 128}.
 */
int fm_block_self_attention(const void* qkv, fm_dtype dt, int32_t n_blocks, int32_t K,
                            const float* q_norm_w, const float* k_norm_w, const int32_t* ctx_lens,
                            int32_t H, int32_t Dh, float softmax_scale, float rope_theta, float eps,
                            void* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FM_H */
