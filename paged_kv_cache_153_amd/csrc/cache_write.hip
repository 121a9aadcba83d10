// cache_write.hip — slot-mapped K/V append and copy-on-write block copies.
//
// Decoding computes only the new token's K and V and appends them to the
// cache ([KVPA] "KV Cache与PagedAttention深度解析" §2.2; with paging, §5.3
// puts the row at offset t % block_size of the last block).  A slot names
// that place as block * BS + row; row i of key/value goes to
// kv[slot / BS, 0|1, :, slot % BS, :].  A sequence that writes into a block
// it shares first gets a whole-block copy ([NANO] zwxr.cn walkthrough §2.3,
// §5.5: copy-on-write); the copies are enqueued before the scatter.
//
// For f32 / f16 pools both kernels are pure 16-byte copies (bit-exact).  One
// thread moves one 16-byte chunk; consecutive threads take consecutive chunks
// of a row, so each wave reads and writes contiguous 1 KiB runs.  Slots and
// block ids are range-checked on the device: an out-of-range entry is
// skipped, never written through.
//
// INT8 pools ([KV2P] "KV Cache从原理到实战" §5.2: INT8 halves the cache, one
// scale per 128-element group): each (token, KV head) row of K and of V is
// quantised on its way in, symmetric, with its own float32 scale
// s = amax / 127 and codes rint(x / s) clamped to [-127, 127] (ties to even;
// an all-zero row gets s = 0 and zero codes).  Both divisions are IEEE
// float32 divisions, so the codes are exactly determined by the f16 inputs.
// A group of D/8 threads takes one row (8 values each) and finds amax with a
// butterfly over the group; copy-on-write copies move the scales too.
#include "device_common.h"
#include "kernels.h"

namespace pa {
namespace {

// Thread `first`, then every `stride`-th, over num_tokens * Hkv * CPR chunks
// (CPR = 16-byte chunks per row).
__device__ __forceinline__ void scatter_chunks(const u32x4_t* __restrict__ key,
                                               const u32x4_t* __restrict__ value,
                                               u32x4_t* __restrict__ kv,
                                               const int64_t* __restrict__ slots,
                                               int64_t num_tokens, int num_kv_heads, int cpr,
                                               int block_size, int64_t num_blocks,
                                               int64_t first, int64_t stride) {
  const int64_t per_token = (int64_t)num_kv_heads * cpr;
  const int64_t total = num_tokens * per_token;
  const int64_t head_chunks = (int64_t)block_size * cpr;
  const int64_t v_off = (int64_t)num_kv_heads * head_chunks;
  for (int64_t idx = first; idx < total; idx += stride) {
    const int64_t i = idx / per_token;
    const int64_t rem = idx - i * per_token;  // h * cpr + chunk
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_blocks * block_size) continue;
    const int64_t b = slot / block_size;
    const int64_t row = slot - b * block_size;
    const int64_t h = rem / cpr;
    const int64_t chunk = rem - h * cpr;
    const int64_t dst = (b * 2 * num_kv_heads + h) * head_chunks + row * cpr + chunk;
    kv[dst] = key[idx];
    kv[dst + v_off] = value[idx];
  }
}

__global__ __launch_bounds__(256) void cache_write_kernel(const u32x4_t* __restrict__ key,
                                                          const u32x4_t* __restrict__ value,
                                                          u32x4_t* __restrict__ kv,
                                                          const int64_t* __restrict__ slots,
                                                          int64_t num_tokens, int num_kv_heads,
                                                          int cpr, int block_size,
                                                          int64_t num_blocks) {
  scatter_chunks(key, value, kv, slots, num_tokens, num_kv_heads, cpr, block_size, num_blocks,
                 (int64_t)blockIdx.x * blockDim.x + threadIdx.x,
                 (int64_t)gridDim.x * blockDim.x);
}

// blockIdx.y = pair index; grid-stride over the block's chunks in x
__global__ __launch_bounds__(256) void copy_blocks_kernel(u32x4_t* __restrict__ kv,
                                                          const int32_t* __restrict__ pairs,
                                                          int64_t block_chunks,
                                                          int64_t num_blocks) {
  const int64_t src = pairs[2 * (int64_t)blockIdx.y];
  const int64_t dst = pairs[2 * (int64_t)blockIdx.y + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  const u32x4_t* from = kv + src * block_chunks;
  u32x4_t* to = kv + dst * block_chunks;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < block_chunks;
       k += (int64_t)gridDim.x * blockDim.x)
    to[k] = from[k];
}

// One row = (token i, head h, K|V); TPR threads per row, 8 f16 values each.
// Grid-stride over num_tokens * Hkv * 2 * TPR threads; TPR divides the
// stride, so a row's threads always run the same iteration together.
template <int TPR>
__device__ __forceinline__ void scatter_i8(const u32x4_t* __restrict__ key,
                                           const u32x4_t* __restrict__ value,
                                           u32x2_t* __restrict__ codes,
                                           float* __restrict__ scales,
                                           const int64_t* __restrict__ slots, int64_t num_tokens,
                                           int num_kv_heads, int block_size, int64_t num_blocks,
                                           int64_t first, int64_t stride) {
  const int64_t total = num_tokens * num_kv_heads * 2 * TPR;
  for (int64_t idx = first; idx < total; idx += stride) {
    const int c = (int)(idx % TPR);
    const int64_t row = idx / TPR;  // (i * Hkv + h) * 2 + kv
    const int kv = (int)(row & 1);
    const int64_t ih = row >> 1;    // i * Hkv + h
    const int64_t i = ih / num_kv_heads;
    const int64_t h = ih - i * num_kv_heads;
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_blocks * block_size) continue;  // uniform per row
    const half8_t x = __builtin_bit_cast(half8_t, (kv ? value : key)[ih * TPR + c]);
    float f[8];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f[e] = (float)x[e];
      amax = fmaxf(amax, fabsf(f[e]));
    }
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float sc = amax / 127.f;
    uint32_t w[2] = {0u, 0u};
    if (sc > 0.f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float q = rintf(f[e] / sc);
        q = fminf(fmaxf(q, -127.f), 127.f);
        w[e / 4] |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * (e % 4));
      }
    }
    const int64_t b = slot / block_size;
    const int64_t r = slot - b * block_size;
    const int64_t crow = ((b * 2 + kv) * num_kv_heads + h) * block_size + r;  // [NB, 2, Hkv, BS]
    const int64_t srow = ((b * num_kv_heads + h) * 2 + kv) * block_size + r;  // [NB, Hkv, 2, BS]
    codes[crow * TPR + c] = u32x2_t{w[0], w[1]};
    if (c == 0) scales[srow] = sc;
  }
}

template <int TPR>
__global__ __launch_bounds__(256) void cache_write_i8_kernel(const u32x4_t* __restrict__ key,
                                                             const u32x4_t* __restrict__ value,
                                                             u32x2_t* __restrict__ codes,
                                                             float* __restrict__ scales,
                                                             const int64_t* __restrict__ slots,
                                                             int64_t num_tokens,
                                                             int num_kv_heads, int block_size,
                                                             int64_t num_blocks) {
  scatter_i8<TPR>(key, value, codes, scales, slots, num_tokens, num_kv_heads, block_size,
                  num_blocks, (int64_t)blockIdx.x * blockDim.x + threadIdx.x,
                  (int64_t)gridDim.x * blockDim.x);
}

void copy_blocks(void* buf, const int32_t* cow_pairs, int64_t num_cow, int64_t block_chunks,
                 int64_t num_blocks, hipStream_t stream, int* rc) {
  const int64_t per_pair = (block_chunks + 255) / 256;
  const unsigned gx = (unsigned)(per_pair < 64 ? per_pair : 64);
  for (int64_t p0 = 0; p0 < num_cow && *rc == 0; p0 += 65535) {
    const unsigned gy = (unsigned)(num_cow - p0 < 65535 ? num_cow - p0 : 65535);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, gy), dim3(256), 0, stream,
                       reinterpret_cast<u32x4_t*>(buf), cow_pairs + 2 * p0, block_chunks,
                       num_blocks);
    if (hipGetLastError() != hipSuccess) *rc = 2;
  }
}

// Host -> device upload of a small page-locked buffer by a kernel that reads
// it over the bus (16-byte loads, then a 4-byte tail): the per-step tables
// reach the GPU without a copy-engine transfer and its hand-off to the
// compute queue.
__device__ __forceinline__ void stage_chunks(u32x4_t* __restrict__ dst,
                                             const u32x4_t* __restrict__ src, int64_t n16,
                                             int tail, int64_t first, int64_t stride,
                                             bool tail_block) {
  for (int64_t i = first; i < n16; i += stride) dst[i] = src[i];
  if (tail_block && (int)threadIdx.x < tail)
    reinterpret_cast<uint32_t*>(dst + n16)[threadIdx.x] =
        reinterpret_cast<const uint32_t*>(src + n16)[threadIdx.x];
}

__global__ __launch_bounds__(256) void stage_kernel(u32x4_t* __restrict__ dst,
                                                    const u32x4_t* __restrict__ src, int64_t n16,
                                                    int tail) {
  stage_chunks(dst, src, n16, tail, (int64_t)blockIdx.x * blockDim.x + threadIdx.x,
               (int64_t)gridDim.x * blockDim.x, blockIdx.x == 0);
}

// The upload and the K/V scatter in one launch: workgroups [0, stage_wgs)
// upload, the rest scatter (TPR = 0: byte copies of 16-byte chunks; 8 / 16:
// INT8 quantisation).  The two parts touch disjoint memory.
template <int TPR>
__global__ __launch_bounds__(256) void stage_write_kernel(
    u32x4_t* __restrict__ stage_dst, const u32x4_t* __restrict__ stage_src, int64_t n16,
    int tail, int stage_wgs, const u32x4_t* __restrict__ key, const u32x4_t* __restrict__ value,
    void* __restrict__ kv, float* __restrict__ scales, const int64_t* __restrict__ slots,
    int64_t num_tokens, int num_kv_heads, int cpr, int block_size, int64_t num_blocks) {
  if ((int)blockIdx.x < stage_wgs) {
    stage_chunks(stage_dst, stage_src, n16, tail, (int64_t)blockIdx.x * blockDim.x + threadIdx.x,
                 (int64_t)stage_wgs * blockDim.x, blockIdx.x == 0);
    return;
  }
  const int64_t first = (int64_t)(blockIdx.x - stage_wgs) * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)(gridDim.x - stage_wgs) * blockDim.x;
  if constexpr (TPR == 0)
    scatter_chunks(key, value, reinterpret_cast<u32x4_t*>(kv), slots, num_tokens, num_kv_heads,
                   cpr, block_size, num_blocks, first, stride);
  else
    scatter_i8<TPR>(key, value, reinterpret_cast<u32x2_t*>(kv), scales, slots, num_tokens,
                    num_kv_heads, block_size, num_blocks, first, stride);
}

}  // namespace

int launch_stage(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int tail = (int)((bytes % 16) / 4);
  int64_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 256) blocks = 256;
  hipLaunchKernelGGL(stage_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<u32x4_t*>(dst), reinterpret_cast<const u32x4_t*>(src), n16,
                     tail);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int launch_stage_write(void* stage_dst, const void* stage_src, int64_t stage_bytes,
                       const void* key, const void* value, void* kv, float* scales,
                       const int64_t* slots, int64_t num_tokens, const int32_t* cow_pairs,
                       int64_t num_cow, int64_t num_blocks, int num_kv_heads, int head_dim,
                       int block_size, int elem_bytes, hipStream_t stream) {
  int rc = 0;
  if (num_cow > 0) {  // copies go first, in a launch of their own
    copy_blocks(kv, cow_pairs, num_cow, 2LL * num_kv_heads * block_size * head_dim * elem_bytes / 16,
                num_blocks, stream, &rc);
    if (elem_bytes == 1)
      copy_blocks(scales, cow_pairs, num_cow, 2LL * num_kv_heads * block_size * 4 / 16,
                  num_blocks, stream, &rc);
    if (rc) return rc;
  }
  const int64_t n16 = stage_bytes / 16;
  const int tail = (int)((stage_bytes % 16) / 4);
  int64_t sw = (n16 + 255) / 256;
  sw = sw < 1 ? 1 : (sw > 64 ? 64 : sw);
  const int tpr = elem_bytes == 1 ? head_dim / 8 : 0;
  const int cpr = head_dim * elem_bytes / 16;
  const int64_t total = elem_bytes == 1 ? num_tokens * num_kv_heads * 2 * tpr
                                        : num_tokens * num_kv_heads * cpr;
  int64_t ww = (total + 255) / 256;
  ww = ww < 1 ? 1 : (ww > 65536 ? 65536 : ww);
  const dim3 grid((unsigned)(sw + ww));
  auto* sd = reinterpret_cast<u32x4_t*>(stage_dst);
  const auto* ss = reinterpret_cast<const u32x4_t*>(stage_src);
  const auto* k = reinterpret_cast<const u32x4_t*>(key);
  const auto* v = reinterpret_cast<const u32x4_t*>(value);
  if (tpr == 16)
    hipLaunchKernelGGL(stage_write_kernel<16>, grid, dim3(256), 0, stream, sd, ss, n16, tail,
                       (int)sw, k, v, kv, scales, slots, num_tokens, num_kv_heads, cpr,
                       block_size, num_blocks);
  else if (tpr == 8)
    hipLaunchKernelGGL(stage_write_kernel<8>, grid, dim3(256), 0, stream, sd, ss, n16, tail,
                       (int)sw, k, v, kv, scales, slots, num_tokens, num_kv_heads, cpr,
                       block_size, num_blocks);
  else if (tpr == 0)
    hipLaunchKernelGGL(stage_write_kernel<0>, grid, dim3(256), 0, stream, sd, ss, n16, tail,
                       (int)sw, k, v, kv, scales, slots, num_tokens, num_kv_heads, cpr,
                       block_size, num_blocks);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int launch_cache_write(const void* key, const void* value, void* kv, float* scales,
                       const int64_t* slots, int64_t num_tokens, const int32_t* cow_pairs,
                       int64_t num_cow, int64_t num_blocks, int num_kv_heads, int head_dim,
                       int block_size, int elem_bytes, hipStream_t stream) {
  int rc = 0;
  if (num_cow > 0) {
    copy_blocks(kv, cow_pairs, num_cow, 2LL * num_kv_heads * block_size * head_dim * elem_bytes / 16,
                num_blocks, stream, &rc);
    if (elem_bytes == 1)  // scale rows: 2 * Hkv * BS floats per block (a multiple of 16 bytes)
      copy_blocks(scales, cow_pairs, num_cow, 2LL * num_kv_heads * block_size * 4 / 16,
                  num_blocks, stream, &rc);
    if (rc) return rc;
  }
  if (num_tokens > 0 && elem_bytes == 1) {
    const int tpr = head_dim / 8;
    const int64_t total = num_tokens * num_kv_heads * 2 * tpr;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    const auto* k = reinterpret_cast<const u32x4_t*>(key);
    const auto* v = reinterpret_cast<const u32x4_t*>(value);
    auto* c = reinterpret_cast<u32x2_t*>(kv);
    if (tpr == 16)
      hipLaunchKernelGGL(cache_write_i8_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         k, v, c, scales, slots, num_tokens, num_kv_heads, block_size,
                         num_blocks);
    else if (tpr == 8)
      hipLaunchKernelGGL(cache_write_i8_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         k, v, c, scales, slots, num_tokens, num_kv_heads, block_size,
                         num_blocks);
    else
      return 1;
    return hipGetLastError() == hipSuccess ? 0 : 2;
  }
  const int cpr = head_dim * elem_bytes / 16;
  if (num_tokens > 0) {
    const int64_t total = num_tokens * num_kv_heads * cpr;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const u32x4_t*>(key),
                       reinterpret_cast<const u32x4_t*>(value), reinterpret_cast<u32x4_t*>(kv),
                       slots, num_tokens, num_kv_heads, cpr, block_size, num_blocks);
    if (hipGetLastError() != hipSuccess) return 2;
  }
  return 0;
}

}  // namespace pa
