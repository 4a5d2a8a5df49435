// Memory-system probes for the benchmark (include/fm_probe.h): a streaming
// read and a gather of exactly the tiles a paged cross-attention call reads.
// They fold what they read into a sink and compute nothing else.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fm_probe.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4_t* gptr_u32x4;

constexpr int kDepth = 4;       // 8 KB blocks in flight per wave (streaming read)
constexpr int kNT = 2;          // nt in the buffer instructions' cache-policy operand
constexpr int kBlock = 8192;    // bytes of one streaming-read block: eight 1 KB loads

// Nontemporal 16-byte load: streamed once, not kept (the hint the attention
// kernel's K/V loads carry; plain loads stream ~12% slower on MI355X).
__device__ __forceinline__ u32x4_t ld(const uint8_t* p) { return __builtin_nontemporal_load((gptr_u32x4)(p)); }

__device__ __forceinline__ void finish(uint32_t* sink, int64_t w, int lane, const u32x4_t& acc) {
  sink[w * 64 + lane] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Wave w reads blocks [w * per_wave, (w + 1) * per_wave) of 8 KB.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* buf, int64_t per_wave, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const uint8_t* base = buf + w * per_wave * kBlock + lane * 16;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (int64_t i = 0; i < per_wave; i += kDepth) {
    u32x4_t r[kDepth][8];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int64_t blk = i + d < per_wave ? i + d : per_wave - 1;  // past the share: re-read its last block
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) r[d][ch] = ld(base + blk * kBlock + ch * 1024);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the group issued before the first use
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) acc ^= r[d][ch];
  }
  finish(sink, w, lane, acc);
}

// Wave w reads tiles [n w / W, n (w + 1) / W) of the list, K and V of each,
// the way the attention kernel takes them: CH direct-to-LDS loads of 1 KB per
// operand and tile (whole lines, nontemporal) into a ring of two tiles per
// wave, each read back from LDS once its loads have landed.  With rec, lane 0
// of each wave records its start and end on the constant 100 MHz clock, its
// XCD and its tile count.
template <int CH>
__device__ __forceinline__ void gather_tile_to_lds(const uint8_t* k, const uint8_t* v, int64_t o, uint8_t* dst,
                                                   uint32_t lane_off) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k + o), 0, CH * 1024, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(v + o), 0, CH * 1024, 0x00020000);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(dst + i * 1024), 16, lane_off + i * 1024, 0, 0, kNT);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)(dst + (CH + i) * 1024), 16, lane_off + i * 1024, 0, 0,
                                             kNT);
  }
}

template <int CH>
__global__ __launch_bounds__(256) void tile_gather_kernel(const uint8_t* k, const uint8_t* v, const int64_t* off,
                                                          int64_t n_tiles, int n_waves, uint32_t* sink, uint64_t* rec) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[4 * 2 * CH * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[4 * 2 * CH * 1024];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int w = blockIdx.x * 4 + wv;
  if (w >= n_waves) return;
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  const int64_t t0 = n_tiles * w / n_waves, t1 = n_tiles * (w + 1) / n_waves;
  const int64_t* soff = off;
  uint8_t* s0 = ring0 + wv * 2 * CH * 1024;
  uint8_t* s1 = ring1 + wv * 2 * CH * 1024;
  const uint32_t lane_off = (uint32_t)lane * 16;
  auto tile = [&](int64_t t) -> int64_t {  // wave-uniform offset of tile t (past the share: its last tile again)
    return ((const __attribute__((address_space(4))) int64_t*)soff)[t < t1 ? t : t1 - 1];
  };
  constexpr int kWait = 2 * CH;  // the next tile's loads may stay in flight
  u32x4_t acc = {0u, 0u, 0u, 0u};
  auto drain = [&](const uint8_t* src) {
#pragma unroll
    for (int i = 0; i < 2 * CH; ++i) acc ^= *(const u32x4_t*)(src + i * 1024 + lane_off);
  };
  if (t1 > t0) gather_tile_to_lds<CH>(k, v, tile(t0), s0, lane_off);
  for (int64_t t = t0; t < t1; t += 2) {
    gather_tile_to_lds<CH>(k, v, tile(t + 1), s1, lane_off);
    __builtin_amdgcn_s_waitcnt((kWait & 15) | ((kWait >> 4) << 14) | 0x0F70);
    drain(s0);
    gather_tile_to_lds<CH>(k, v, tile(t + 2), s0, lane_off);
    __builtin_amdgcn_s_waitcnt((kWait & 15) | ((kWait >> 4) << 14) | 0x0F70);
    drain(s1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70 & 0xC07F);  // every load landed before the wave ends
  finish(sink, w, lane, acc);
  if (rec != nullptr && lane == 0) {
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    rec[4 * w] = t_start;
    rec[4 * w + 1] = t_end;
    rec[4 * w + 2] = xcc & 0xF;
    rec[4 * w + 3] = (uint64_t)(t1 - t0);
  }
}

int status_of(hipError_t e) { return e == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" {

int fm_probe_stream_read(const void* buf, size_t bytes, int32_t n_waves, uint32_t* sink, size_t* bytes_read,
                         hipStream_t stream) {
  if (!buf || !sink || !bytes_read || n_waves < 4 || n_waves % 4 || ((uintptr_t)buf & 15)) return -1;
  const int64_t per_wave = (int64_t)(bytes / (size_t)n_waves / kBlock);
  if (per_wave < 1) return -1;
  *bytes_read = (size_t)per_wave * kBlock * (size_t)n_waves;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)(n_waves / 4)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(buf), per_wave, sink);
  return status_of(hipGetLastError());
}

}  // extern "C"

namespace {

int tile_gather(const void* k, const void* v, const int64_t* tile_off, int64_t n_tiles, int32_t tile_bytes,
                int32_t n_waves, uint32_t* sink, uint64_t* rec, hipStream_t stream) {
  if (!k || !v || !tile_off || !sink || n_tiles < 1 || n_waves < 4 || n_waves % 4) return -1;
  if (tile_bytes < 1024 || tile_bytes > 8192 || tile_bytes % 1024) return -2;
  if (((uintptr_t)k & 15) || ((uintptr_t)v & 15)) return -1;
  const uint8_t* kb = static_cast<const uint8_t*>(k);
  const uint8_t* vb = static_cast<const uint8_t*>(v);
  const dim3 grid((unsigned)(n_waves / 4)), block(256);
  switch (tile_bytes / 1024) {
    case 1: hipLaunchKernelGGL(tile_gather_kernel<1>, grid, block, 0, stream, kb, vb, tile_off, n_tiles, n_waves, sink, rec); break;
    case 2: hipLaunchKernelGGL(tile_gather_kernel<2>, grid, block, 0, stream, kb, vb, tile_off, n_tiles, n_waves, sink, rec); break;
    case 4: hipLaunchKernelGGL(tile_gather_kernel<4>, grid, block, 0, stream, kb, vb, tile_off, n_tiles, n_waves, sink, rec); break;
    case 8: hipLaunchKernelGGL(tile_gather_kernel<8>, grid, block, 0, stream, kb, vb, tile_off, n_tiles, n_waves, sink, rec); break;
    default: return -2;  // 3, 5, 6, 7 KB tiles: not a tile size of a pool
  }
  return status_of(hipGetLastError());
}

}  // namespace

extern "C" {

int fm_probe_tile_gather(const void* k, const void* v, const int64_t* tile_off, int64_t n_tiles, int32_t tile_bytes,
                         int32_t n_waves, uint32_t* sink, hipStream_t stream) {
  return tile_gather(k, v, tile_off, n_tiles, tile_bytes, n_waves, sink, nullptr, stream);
}

int fm_probe_tile_gather_timed(const void* k, const void* v, const int64_t* tile_off, int64_t n_tiles,
                               int32_t tile_bytes, int32_t n_waves, uint32_t* sink, uint64_t* wave_rec,
                               hipStream_t stream) {
  if (!wave_rec) return -1;
  return tile_gather(k, v, tile_off, n_tiles, tile_bytes, n_waves, sink, wave_rec, stream);
}

}  // extern "C"
