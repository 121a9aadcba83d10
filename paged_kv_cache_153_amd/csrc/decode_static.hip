// decode_static.hip — pa_decode_static: the decode with its split-context
// partials in a device array the library owns, for callers that cannot
// allocate device memory.
//
// pa_decode's balanced and partition schedules leave per-slice partials
// (m, l, normalised o) that the merge kernel combines; pa_decode takes the
// buffer for them from the caller.  Here the same kernels get it from
// `scratch`, a file-scope device array of kScratchBytes.  Each GPU holds its
// own copy (allocated when the library's code is loaded on that GPU, kept
// until the process ends), at an address the host learns once per device
// with hipGetSymbolAddress; the host never passes the array's name itself
// (in host code that is only a stand-in, not a device address).
//
// No clearing is needed: every partial the merge reads was written by the
// decode launch just before it on the same stream.  All calls on one GPU
// share the array, so calls that overlap on that GPU (other streams, other
// host threads) race; calls on one stream are ordered.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "../../include/pa.h"
#include "internal.h"

namespace pa {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// The current device's address of `scratch`, looked up on the first call on
// that device (with it current) and kept.
int scratch_address(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_HIP, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" {

size_t pa_decode_static_capacity(void) { return pa::kScratchBytes; }

int pa_decode_static(float* out, const void* query, const void* kv_cache, const float* kv_scales,
                     const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                     int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                     int max_blocks_per_seq, int max_context_len, int64_t num_blocks, float scale,
                     int sliding_window, int partition_size, int kernel, int dtype,
                     void* stream) {
  // the plan first (pa_decode's size query): nothing is enqueued unless the
  // partials fit the array
  size_t need = 0;
  int st = pa_decode(nullptr, query, kv_cache, kv_scales, block_tables, context_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     max_context_len, num_blocks, scale, sliding_window, partition_size, kernel,
                     nullptr, 0, &need, dtype, stream);
  if (st != PA_OK) return st;
  if (need > pa::kScratchBytes)
    return pa::fail(PA_ERR_WORKSPACE,
                    "pa_decode_static: this call's split partials need " + std::to_string(need) +
                        " bytes; the library's static scratch holds " +
                        std::to_string(pa::kScratchBytes) +
                        " (use pa_decode with a workspace, or larger partitions)");
  if (!out) return PA_OK;  // it fits
  void* ws = nullptr;
  if (need > 0 && (st = pa::scratch_address(&ws)) != PA_OK) return st;
  return pa_decode(out, query, kv_cache, kv_scales, block_tables, context_lens, num_seqs,
                   num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                   max_context_len, num_blocks, scale, sliding_window, partition_size, kernel, ws,
                   need > 0 ? pa::kScratchBytes : 0, nullptr, dtype, stream);
}

}  // extern "C"
