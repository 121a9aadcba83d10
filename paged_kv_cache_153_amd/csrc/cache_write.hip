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
// Both kernels are pure 16-byte copies (bit-exact).  One thread moves one
// 16-byte chunk; consecutive threads take consecutive chunks of a row, so
// each wave reads and writes contiguous 1 KiB runs.  Slots and block ids are
// range-checked on the device: an out-of-range entry is skipped, never
// written through.
#include "device_common.h"
#include "kernels.h"

namespace pa {
namespace {

// grid-stride over num_tokens * Hkv * CPR chunks (CPR = 16-byte chunks per row)
__global__ __launch_bounds__(256) void cache_write_kernel(const u32x4_t* __restrict__ key,
                                                          const u32x4_t* __restrict__ value,
                                                          u32x4_t* __restrict__ kv,
                                                          const int64_t* __restrict__ slots,
                                                          int64_t num_tokens, int num_kv_heads,
                                                          int cpr, int block_size,
                                                          int64_t num_blocks) {
  const int64_t per_token = (int64_t)num_kv_heads * cpr;
  const int64_t total = num_tokens * per_token;
  const int64_t head_chunks = (int64_t)block_size * cpr;
  const int64_t v_off = (int64_t)num_kv_heads * head_chunks;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
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

}  // namespace

int launch_cache_write(const void* key, const void* value, void* kv, const int64_t* slots,
                       int64_t num_tokens, const int32_t* cow_pairs, int64_t num_cow,
                       int64_t num_blocks, int num_kv_heads, int head_dim, int block_size,
                       int elem_bytes, hipStream_t stream) {
  const int cpr = head_dim * elem_bytes / 16;
  if (num_cow > 0) {
    const int64_t block_chunks = 2LL * num_kv_heads * block_size * cpr;
    const int64_t per_pair = (block_chunks + 255) / 256;
    const unsigned gx = (unsigned)(per_pair < 64 ? per_pair : 64);
    for (int64_t p0 = 0; p0 < num_cow; p0 += 65535) {
      const unsigned gy = (unsigned)(num_cow - p0 < 65535 ? num_cow - p0 : 65535);
      hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, gy), dim3(256), 0, stream,
                         reinterpret_cast<u32x4_t*>(kv), cow_pairs + 2 * p0, block_chunks,
                         num_blocks);
      if (hipGetLastError() != hipSuccess) return 2;
    }
  }
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
