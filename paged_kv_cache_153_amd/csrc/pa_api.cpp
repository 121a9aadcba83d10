// pa_api.cpp — C ABI for the device calls: argument checks, partition
// choice, workspace sizing and kernel dispatch.
//
// The library allocates no device memory.  Split-context partials live in a
// caller-provided workspace whose size this file computes; every kernel is
// enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pa.h"
#include "internal.h"
#include "kernels.h"

namespace pa {

namespace {

thread_local std::string g_last_error;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool check_mode() {  // read on every call, so a caller can switch it at run time
  const char* e = std::getenv("PA_CHECK");
  return e && e[0] == '1';
}

// Schedule used when the caller passes partition_size 0 (measured on
// MI355X with 16 KiB-per-token MHA and 4 KiB-per-token GQA layers):
//  * single pass (-1) when one workgroup per (sequence, KV head) already fills
//    the chip (>= 1024 pairs) and contexts are moderate, or contexts are
//    short: no partials, no merge;
//  * pools read with cached loads (blocks shared by many sequences, e.g. a
//    common prefix): fixed partitions, so every sequence's first partition —
//    the shared prefix — is read by all workgroups at the same time and hits
//    in cache;
//  * otherwise the balanced schedule (-2): equal tile slices per workgroup
//    whatever the length mix (it needs S <= kBalancedMaxSeqs);
//  * fixed partitions are 512 tokens up to 4K contexts, 1024 up to 16K and
//    2048 beyond;
//  * under a sliding window that shortens the longest context, fixed
//    partitions of about a quarter of the window's span (256 to 2048).
int choose_partition(int num_seqs, int num_kv_heads, int max_context_len, int cached_kv,
                     bool windowed) {
  const long pairs = (long)num_seqs * num_kv_heads;
  if (max_context_len <= 512) return -1;
  if (pairs >= 1024 && max_context_len <= 8192) return -1;
  if (windowed) {
    // spans cut by a window are nearly equal: about four fixed partitions
    // per span (no straddling slices) measured faster than balanced slices
    int p = 256;
    while (p < 2048 && 2 * p <= max_context_len / 4) p *= 2;
    return p;
  }
  if (!cached_kv && num_seqs <= kBalancedMaxSeqs) return -2;
  if (max_context_len <= 4096) return 512;
  if (max_context_len <= 16384) return 1024;
  return 2048;
}

// Kernel family used when the caller passes PA_KERNEL_AUTO: the matrix-core
// kernel once the query group makes q.K^T a real [G x D] x [D x 16] product
// (G >= 4 measured faster: its VALU work per tile does not grow with G); the
// vector kernel for MHA / G = 2, where MFMA rows would be mostly padding.
int choose_kernel(int dtype, int group) {
  return (dtype != PA_F32 && group >= 4) ? PA_KERNEL_MFMA : PA_KERNEL_VALU;
}

struct Plan {
  int schedule = kScheduleSingle;
  int part_tokens = 0;
  int num_parts = 1;
  int workgroups = 0;  // balanced: grid size upper bound used for the workspace
  size_t ws_bytes = 0;
  size_t off_m = 0, off_l = 0, off_cut = 0;
};

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Compute units of the current device (cached per device id); 0 if unknown.
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

// At most this many 256-thread workgroups fit on one compute unit; the
// balanced workspace is sized for it so the size does not depend on which
// kernel variant is picked.
constexpr int kMaxWorkgroupsPerCU = 8;

// Balanced-schedule charge per (sequence, KV head) segment, in tiles: the
// fixed cost of starting and finishing a range (q and first-tile latency,
// the cross-wave merge).  Swept on the ragged GQA batch (64 seqs, lengths
// U[128, 8192]): f16 0 / 3 / 6 / 10 / 16 -> 190.0 / 184.1 / 182.9 / 181.8 /
// 183.4 us, INT8 0 / 6 / 10 / 16 -> 114.1 / 108.2 / 108.2 / 108.5 us.
constexpr int kSegCostF16 = 10;
constexpr int kSegCostI8 = 8;

Plan make_plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int max_tokens,
               int partition, int cus) {
  Plan p;
  if (partition == -1) {
    p.schedule = kScheduleSingle;
    p.num_parts = 1;
    p.part_tokens = (max_tokens + kTile - 1) / kTile * kTile + kTile;
    return p;
  }
  if (partition == -2) {
    p.schedule = kScheduleBalanced;
    p.num_parts = 1;
    p.part_tokens = (max_tokens + kTile - 1) / kTile * kTile + kTile;
    p.workgroups = cus * kMaxWorkgroupsPerCU;
    const int group = num_q_heads / num_kv_heads;
    const size_t slots = 2 * (size_t)p.workgroups * group;
    const size_t bytes_o = round_up(slots * head_dim * sizeof(float));
    const size_t bytes_ml = round_up(slots * sizeof(float));
    p.off_m = bytes_o;
    p.off_l = bytes_o + bytes_ml;
    p.off_cut = bytes_o + 2 * bytes_ml;
    p.ws_bytes = p.off_cut + round_up((size_t)p.workgroups * kCutInts * sizeof(int));
    return p;
  }
  p.schedule = kSchedulePartition;
  p.part_tokens = partition;
  p.num_parts = max_tokens <= 0 ? 1 : (max_tokens + partition - 1) / partition;
  const size_t rows = (size_t)num_seqs * num_q_heads * p.num_parts;
  const size_t bytes_o = round_up(rows * head_dim * sizeof(float));
  const size_t bytes_ml = round_up(rows * sizeof(float));
  p.off_m = bytes_o;
  p.off_l = bytes_o + bytes_ml;
  p.ws_bytes = bytes_o + 2 * bytes_ml;
  return p;
}

// PA_CHECK=1: copy index arrays to the host and validate them.
int check_decode_arrays(const int32_t* bt, const int32_t* cl, int num_seqs, int max_blocks,
                        int block_size, int max_context_len, int64_t num_blocks,
                        hipStream_t stream) {
  std::vector<int32_t> lens(num_seqs), table((size_t)num_seqs * max_blocks);
  if (hipStreamSynchronize(stream) != hipSuccess ||
      hipMemcpy(lens.data(), cl, lens.size() * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(table.data(), bt, table.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(PA_ERR_HIP, "PA_CHECK: copying tables to the host failed");
  for (int s = 0; s < num_seqs; ++s) {
    const int n = lens[s];
    if (n < 0 || n > max_context_len || (int64_t)n > (int64_t)max_blocks * block_size)
      return fail(PA_ERR_INVALID_ARG, "PA_CHECK: context_lens[" + std::to_string(s) +
                                          "] out of range");
    const int nb = (n + block_size - 1) / block_size;
    for (int i = 0; i < nb; ++i) {
      const int32_t b = table[(size_t)s * max_blocks + i];
      if (b < 0 || b >= num_blocks)
        return fail(PA_ERR_INVALID_ARG, "PA_CHECK: block_tables[" + std::to_string(s) + "," +
                                            std::to_string(i) + "] out of range");
    }
  }
  return PA_OK;
}

int check_write_arrays(const int64_t* slots, int64_t num_tokens, const int32_t* pairs,
                       int64_t num_cow, int64_t num_blocks, int block_size, hipStream_t stream) {
  std::vector<int64_t> sl(num_tokens);
  std::vector<int32_t> pr(2 * num_cow);
  if (hipStreamSynchronize(stream) != hipSuccess ||
      (num_tokens && hipMemcpy(sl.data(), slots, sl.size() * 8, hipMemcpyDefault)) ||
      (num_cow && hipMemcpy(pr.data(), pairs, pr.size() * 4, hipMemcpyDefault)))
    return fail(PA_ERR_HIP, "PA_CHECK: copying slots to the host failed");
  std::unordered_set<int64_t> seen;
  for (int64_t s : sl) {
    if (s < 0) continue;
    if (s >= num_blocks * block_size) return fail(PA_ERR_INVALID_ARG, "PA_CHECK: slot out of range");
    if (!seen.insert(s).second) return fail(PA_ERR_INVALID_ARG, "PA_CHECK: duplicate slot");
  }
  std::unordered_set<int32_t> srcs, dsts;
  for (int64_t k = 0; k < num_cow; ++k) {
    const int32_t a = pr[2 * k], b = pr[2 * k + 1];
    if (a < 0 || a >= num_blocks || b < 0 || b >= num_blocks || a == b)
      return fail(PA_ERR_INVALID_ARG, "PA_CHECK: bad copy pair");
    srcs.insert(a);
    if (!dsts.insert(b).second) return fail(PA_ERR_INVALID_ARG, "PA_CHECK: repeated destination");
  }
  for (int32_t b : dsts)
    if (srcs.count(b)) return fail(PA_ERR_INVALID_ARG, "PA_CHECK: a destination is also a source");
  return PA_OK;
}

int check_prefill_arrays(const int32_t* bt, const int32_t* cl, const int32_t* qstart,
                         int num_seqs, int total_queries, int max_query_len, int max_blocks,
                         int block_size, int64_t num_blocks, hipStream_t stream) {
  std::vector<int32_t> lens(num_seqs), qs(num_seqs + 1), table((size_t)num_seqs * max_blocks);
  if (hipStreamSynchronize(stream) != hipSuccess ||
      hipMemcpy(lens.data(), cl, lens.size() * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(qs.data(), qstart, qs.size() * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(table.data(), bt, table.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(PA_ERR_HIP, "PA_CHECK: copying prefill arrays to the host failed");
  if (qs[0] != 0 || qs[num_seqs] != total_queries)
    return fail(PA_ERR_INVALID_ARG, "PA_CHECK: query_start must run from 0 to total_queries");
  for (int s = 0; s < num_seqs; ++s) {
    const int t = qs[s + 1] - qs[s];
    if (t < 0 || t > max_query_len)
      return fail(PA_ERR_INVALID_ARG, "PA_CHECK: chunk length of sequence " + std::to_string(s) +
                                          " outside [0, max_query_len]");
    const int n = lens[s];
    if (n < 0 || (int64_t)n > (int64_t)max_blocks * block_size)
      return fail(PA_ERR_INVALID_ARG, "PA_CHECK: context_lens[" + std::to_string(s) +
                                          "] out of range");
    const int nb = (n + block_size - 1) / block_size;
    for (int i = 0; i < nb; ++i) {
      const int32_t b = table[(size_t)s * max_blocks + i];
      if (b < 0 || b >= num_blocks)
        return fail(PA_ERR_INVALID_ARG, "PA_CHECK: block_tables[" + std::to_string(s) + "," +
                                            std::to_string(i) + "] out of range");
    }
  }
  return PA_OK;
}

}  // namespace

int fail(int status, const std::string& message) {
  g_last_error = message;
  return status;
}
void clear_error() { g_last_error.clear(); }

}  // namespace pa

using pa::aligned16;
using pa::fail;

extern "C" {

const char* pa_strerror(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_OOM: return "out of KV cache blocks";
    case PA_ERR_NOT_FOUND: return "unknown sequence";
    case PA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* pa_last_error(void) { return pa::g_last_error.c_str(); }

const char* pa_version(void) { return "pa 0.1 gfx950"; }

namespace {
// Host-side checks shared by pa_cache_write and pa_stage_and_write; on
// success *eb is the element size.
int validate_write(const void* key, const void* value, void* kv_cache, float* kv_scales,
                   const int64_t* slot_mapping, int64_t num_tokens, const int32_t* cow_pairs,
                   int64_t num_cow, int64_t num_blocks, int num_kv_heads, int head_dim,
                   int block_size, int dtype, int* eb) {
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_I8)
    return fail(PA_ERR_UNSUPPORTED, "dtype");
  *eb = dtype == PA_F32 ? 4 : dtype == PA_F16 ? 2 : 1;
  if (num_tokens < 0 || num_cow < 0) return fail(PA_ERR_INVALID_ARG, "negative count");
  if (num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return fail(PA_ERR_INVALID_ARG, "sizes must be positive");
  if ((head_dim * *eb) % 16) return fail(PA_ERR_UNSUPPORTED, "head_dim * element size % 16 != 0");
  if (dtype == PA_I8) {
    if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "INT8 head_dim");
    if ((2LL * num_kv_heads * block_size * 4) % 16)
      return fail(PA_ERR_UNSUPPORTED, "INT8: num_kv_heads * block_size must be even");
    if (!kv_scales || !aligned16(kv_scales))
      return fail(PA_ERR_INVALID_ARG, "INT8 pool needs 16-byte aligned kv_scales");
  } else if (kv_scales) {
    return fail(PA_ERR_INVALID_ARG, "kv_scales is only for INT8 pools");
  }
  if (!kv_cache || !aligned16(kv_cache)) return fail(PA_ERR_INVALID_ARG, "kv_cache null/unaligned");
  if (num_tokens > 0 && (!key || !value || !slot_mapping || !aligned16(key) || !aligned16(value)))
    return fail(PA_ERR_INVALID_ARG, "key/value/slot_mapping null or unaligned");
  if (num_cow > 0 && !cow_pairs) return fail(PA_ERR_INVALID_ARG, "cow_pairs null");
  return PA_OK;
}

// The memory type of `p` as the GPU sees it: device, page-locked host, or
// neither (pageable host memory, a bad pointer).
hipMemoryType gpu_memory_type(const void* p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the lookup's error for the caller's next call
    return hipMemoryTypeUnregistered;
  }
  return at.type;
}
}  // namespace

int pa_cache_write(const void* key, const void* value, void* kv_cache, float* kv_scales,
                   const int64_t* slot_mapping, int64_t num_tokens, const int32_t* cow_pairs,
                   int64_t num_cow, int64_t num_blocks, int num_kv_heads, int head_dim,
                   int block_size, int dtype, void* stream_) {
  pa::clear_error();
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  int eb = 0;
  if (int st = validate_write(key, value, kv_cache, kv_scales, slot_mapping, num_tokens,
                              cow_pairs, num_cow, num_blocks, num_kv_heads, head_dim,
                              block_size, dtype, &eb))
    return st;
  if (num_tokens == 0 && num_cow == 0) return PA_OK;
  if (pa::check_mode()) {
    if (int st = pa::check_write_arrays(slot_mapping, num_tokens, cow_pairs, num_cow, num_blocks,
                                        block_size, stream))
      return st;
  }
  const int rc = pa::launch_cache_write(key, value, kv_cache, kv_scales, slot_mapping, num_tokens,
                                        cow_pairs, num_cow, num_blocks, num_kv_heads, head_dim,
                                        block_size, eb, stream);
  if (rc == 2) return fail(PA_ERR_HIP, hipGetErrorString(hipGetLastError()));
  return rc ? fail(PA_ERR_UNSUPPORTED, "cache write") : PA_OK;
}

int pa_stage_and_write(void* stage_dst, const void* stage_src, int64_t stage_bytes,
                       const void* key, const void* value, void* kv_cache, float* kv_scales,
                       const int64_t* slot_mapping, int64_t num_tokens,
                       const int32_t* cow_pairs, int64_t num_cow, int64_t num_blocks,
                       int num_kv_heads, int head_dim, int block_size, int dtype,
                       void* stream_) {
  pa::clear_error();
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  int eb = 0;
  if (int st = validate_write(key, value, kv_cache, kv_scales, slot_mapping, num_tokens,
                              cow_pairs, num_cow, num_blocks, num_kv_heads, head_dim,
                              block_size, dtype, &eb))
    return st;
  if (stage_bytes < 0 || stage_bytes % 4) return fail(PA_ERR_INVALID_ARG, "stage_bytes");
  if (stage_bytes > 0 && (!stage_dst || !stage_src || !aligned16(stage_dst) ||
                          !aligned16(stage_src)))
    return fail(PA_ERR_INVALID_ARG, "stage_dst/stage_src null or not 16-byte aligned");
  if (stage_bytes > 0 && gpu_memory_type(stage_src) != hipMemoryTypeHost)
    return fail(PA_ERR_INVALID_ARG, "stage_src is not page-locked host memory (hipHostMalloc)");
  // slots and pairs are read by the same launch that fills stage_dst: they
  // must come from elsewhere (device memory or page-locked host memory)
  auto inside_dst = [&](const void* p) {
    const char* c = static_cast<const char*>(p);
    const char* d = static_cast<const char*>(stage_dst);
    return stage_bytes > 0 && c >= d && c < d + stage_bytes;
  };
  auto gpu_readable = [&](const void* p) {
    const hipMemoryType t = gpu_memory_type(p);
    return t == hipMemoryTypeHost || t == hipMemoryTypeDevice;
  };
  if (num_tokens > 0 && (inside_dst(slot_mapping) || !gpu_readable(slot_mapping)))
    return fail(PA_ERR_INVALID_ARG,
                "slot_mapping must be device or page-locked host memory outside stage_dst");
  if (num_cow > 0 && (inside_dst(cow_pairs) || !gpu_readable(cow_pairs)))
    return fail(PA_ERR_INVALID_ARG,
                "cow_pairs must be device or page-locked host memory outside stage_dst");
  if (num_tokens == 0 && num_cow == 0 && stage_bytes == 0) return PA_OK;
  if (pa::check_mode()) {
    if (int st = pa::check_write_arrays(slot_mapping, num_tokens, cow_pairs, num_cow, num_blocks,
                                        block_size, stream))
      return st;
  }
  const int rc = pa::launch_stage_write(stage_dst, stage_src, stage_bytes, key, value, kv_cache,
                                        kv_scales, slot_mapping, num_tokens, cow_pairs, num_cow,
                                        num_blocks, num_kv_heads, head_dim, block_size, eb,
                                        stream);
  if (rc == 2) return fail(PA_ERR_HIP, hipGetErrorString(hipGetLastError()));
  return rc ? fail(PA_ERR_UNSUPPORTED, "cache write") : PA_OK;
}

int pa_stage_from_host(void* dst, const void* src, int64_t bytes, void* stream_) {
  pa::clear_error();
  if (bytes < 0) return fail(PA_ERR_INVALID_ARG, "negative size");
  if (bytes == 0) return PA_OK;
  if (!dst || !src) return fail(PA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(dst) || !aligned16(src) || bytes % 4)
    return fail(PA_ERR_INVALID_ARG, "dst/src must be 16-byte aligned and bytes a multiple of 4");
  // the kernel dereferences src on the GPU: it must be page-locked host memory
  if (gpu_memory_type(src) != hipMemoryTypeHost)
    return fail(PA_ERR_INVALID_ARG, "src is not page-locked host memory (hipHostMalloc)");
  const int rc = pa::launch_stage(dst, src, bytes, reinterpret_cast<hipStream_t>(stream_));
  return rc ? fail(PA_ERR_HIP, hipGetErrorString(hipGetLastError())) : PA_OK;
}

namespace {

// Resident workgroups per CU of the decode kernel a launch will use, cached
// per (kernel family, dtype, head_dim, block size, group, variant, device):
// the runtime's occupancy query would otherwise cost host time on every
// balanced-schedule call.  0 if the query fails (not cached).
int decode_occupancy(const pa::DecodeArgs& a, int use, int dtype, int head_dim, int block_size,
                     int group) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const uint64_t key = ((uint64_t)(unsigned)dev << 40) | ((uint64_t)(unsigned)use << 32) |
                       ((uint64_t)(unsigned)dtype << 24) | ((uint64_t)(unsigned)head_dim << 12) |
                       ((uint64_t)(unsigned)block_size << 6) | ((uint64_t)(unsigned)group << 2) |
                       (uint64_t)(a.variant & 3);
  static std::mutex mu;
  static std::unordered_map<uint64_t, int> cache;
  {
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int occ;
  if (dtype == PA_I8)
    occ = use == PA_KERNEL_MFMA ? pa::decode_mfma_i8_occupancy(a, head_dim, block_size, group)
                                : pa::decode_valu_i8_occupancy(a, head_dim, block_size, group);
  else
    occ = use == PA_KERNEL_MFMA ? pa::decode_mfma_occupancy(a, head_dim, block_size, group)
                                : pa::decode_valu_occupancy(a, dtype, head_dim, block_size, group);
  if (occ > 0) {
    std::lock_guard<std::mutex> lock(mu);
    cache[key] = occ;
  }
  return occ;
}

}  // namespace

int pa_decode(float* out, const void* query, const void* kv_cache, const float* kv_scales,
              const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads,
              int head_dim, int block_size, int max_blocks_per_seq, int max_context_len,
              int64_t num_blocks, float scale, int sliding_window, int partition_size, int kernel,
              void* workspace, size_t workspace_bytes, size_t* workspace_needed, int dtype,
              void* stream_) {
  pa::clear_error();
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  if (workspace_needed) *workspace_needed = 0;
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_I8)
    return fail(PA_ERR_UNSUPPORTED, "dtype");
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "sizes out of range");
  if (num_q_heads % num_kv_heads) return fail(PA_ERR_INVALID_ARG, "num_q_heads % num_kv_heads");
  if (sliding_window < 0) return fail(PA_ERR_INVALID_ARG, "sliding_window must be >= 0");
  const int group = num_q_heads / num_kv_heads;
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim");
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "block_size");
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PA_ERR_UNSUPPORTED, "group size");
  const int cached_kv = (kernel & PA_KV_CACHED) != 0;
  if (kernel & ~(0xFF | PA_KV_CACHED)) return fail(PA_ERR_INVALID_ARG, "kernel flags");
  kernel &= 0xFF;
  if (kernel < PA_KERNEL_AUTO || kernel > PA_KERNEL_MFMA) return fail(PA_ERR_INVALID_ARG, "kernel");
  if (kernel == PA_KERNEL_MFMA && (dtype == PA_F32 || group < 2))
    return fail(PA_ERR_UNSUPPORTED, "MFMA kernel needs f16 or INT8 and a query group of 2 or more");
  if (partition_size < -2 ||
      (partition_size > 0 && (partition_size % pa::kTile || partition_size % block_size)))
    return fail(PA_ERR_INVALID_ARG, "partition_size must be -2, -1, 0 or a multiple of 16 and "
                                    "block_size");
  const long long max_tokens_ll = (long long)max_blocks_per_seq * block_size;
  if (max_tokens_ll > (1LL << 30)) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq too large");
  const int max_tokens = (int)max_tokens_ll;
  int ctx = max_context_len < max_tokens ? max_context_len : max_tokens;
  // under a sliding window of W tokens a sequence's keys lie in at most
  // ceil(W/16) + 1 tiles: partitions and the schedule are sized for that span
  bool windowed = false;
  if (sliding_window > 0) {
    const long long span = ((long long)sliding_window + pa::kTile - 1) / pa::kTile * pa::kTile +
                           pa::kTile;
    if (span < ctx) {
      ctx = (int)span;
      windowed = true;
    }
  }
  int part = partition_size;
  if (part == 0) part = pa::choose_partition(num_seqs, num_kv_heads, ctx, cached_kv, windowed);
  // the balanced schedule keeps an int32 tile prefix of all sequences in LDS
  if (part == -2 && (num_seqs > pa::kBalancedMaxSeqs ||
                     (long long)num_seqs * ((max_tokens + pa::kTile - 1) / pa::kTile) >= (1LL << 31)))
    part = 2048;
  int cus = 0;
  if (part == -2) {
    cus = pa::device_cus();
    if (cus <= 0) return fail(PA_ERR_HIP, "cannot query the device's compute units");
  }
  const pa::Plan plan = pa::make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, ctx, part,
                                      cus);
  // the decode has one workgroup per (sequence, partition, KV head) unless
  // balanced; a merge after it has one per (sequence, query head)
  if ((plan.schedule != pa::kScheduleBalanced &&
       (long long)num_seqs * plan.num_parts * num_kv_heads > pa::kMaxGridWorkgroups) ||
      (plan.schedule != pa::kScheduleSingle &&
       (long long)num_seqs * num_q_heads > pa::kMaxGridWorkgroups))
    return fail(PA_ERR_INVALID_ARG, "grid too large: lower max_context_len or num_seqs, or use "
                                    "larger partitions");
  if (workspace_needed) *workspace_needed = plan.ws_bytes;
  if (!out) return PA_OK;  // size query
  if (num_seqs == 0) return PA_OK;
  if (!query || !kv_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "null device pointer");
  if (!aligned16(out) || !aligned16(query) || !aligned16(kv_cache))
    return fail(PA_ERR_INVALID_ARG, "out/query/kv_cache must be 16-byte aligned");
  if (dtype == PA_I8 ? (!kv_scales || !aligned16(kv_scales)) : kv_scales != nullptr)
    return fail(PA_ERR_INVALID_ARG, "kv_scales: 16-byte aligned for INT8 pools, NULL otherwise");
  if (plan.ws_bytes && (!workspace || workspace_bytes < plan.ws_bytes || !aligned16(workspace)))
    return fail(PA_ERR_WORKSPACE, "workspace of " + std::to_string(plan.ws_bytes) +
                                      " bytes (16-byte aligned) needed");
  if (pa::check_mode()) {
    if (int st = pa::check_decode_arrays(block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                         block_size, max_context_len, num_blocks, stream))
      return st;
  }
  pa::DecodeArgs a{};
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.ws_o = plan.ws_bytes ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_m = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.off_m) : nullptr;
  a.ws_l = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.off_l) : nullptr;
  a.ws_cut = plan.off_cut ? reinterpret_cast<int*>(ws + plan.off_cut) : nullptr;
  a.q = query;
  a.kv = kv_cache;
  a.kv_scales = kv_scales;
  a.bt = block_tables;
  a.cl = context_lens;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.max_tokens = max_tokens;
  a.num_parts = plan.num_parts;
  a.part_tokens = plan.part_tokens;
  a.schedule = plan.schedule;
  a.scale_log2 = scale * 1.4426950408889634f;
  // MFMA kernel: the register double buffer when K/V stream from HBM; one
  // tile per wave in flight at twice the occupancy when they are read through
  // the caches (shared blocks): measured faster in each case.
  a.variant = cached_kv ? 1 : 0;
  {  // PA_TUNE_VARIANT=0..2 overrides the choice (tuning experiments only)
    static const int forced = [] {
      const char* e = std::getenv("PA_TUNE_VARIANT");
      return e ? std::atoi(e) : -1;
    }();
    if (forced >= 0 && forced <= 2) a.variant = forced;
  }
  a.cached_kv = cached_kv;
  a.window = sliding_window;
  // Balanced schedule: what one (sequence, KV head) segment costs beyond its
  // tiles, in tiles of the kernel that runs (measured on ragged batches).
  a.seg_cost = dtype == PA_I8 ? pa::kSegCostI8 : pa::kSegCostF16;
  {  // PA_TUNE_SEGCOST overrides it (tuning experiments only)
    static const int forced = [] {
      const char* e = std::getenv("PA_TUNE_SEGCOST");
      return e ? std::atoi(e) : -1;
    }();
    if (forced >= 0 && forced <= 64) a.seg_cost = forced;
  }

  int use = kernel;
  if (use == PA_KERNEL_AUTO) use = pa::choose_kernel(dtype, group);
  if (plan.schedule == pa::kScheduleBalanced) {
    // as many workgroups as are resident at once: one wave of the grid
    const int occ = decode_occupancy(a, use, dtype, head_dim, block_size, group);
    if (occ <= 0) return fail(PA_ERR_HIP, "occupancy query failed");
    a.num_workgroups = std::min(plan.workgroups, cus * std::min(occ, pa::kMaxWorkgroupsPerCU));
  }
  int rc;
  if (dtype == PA_I8)
    rc = use == PA_KERNEL_MFMA ? pa::launch_decode_mfma_i8(a, head_dim, block_size, group, stream)
                               : pa::launch_decode_valu_i8(a, head_dim, block_size, group, stream);
  else
    rc = use == PA_KERNEL_MFMA
             ? pa::launch_decode_mfma(a, dtype, head_dim, block_size, group, 4, stream)
             : pa::launch_decode_valu(a, dtype, head_dim, block_size, group, 4, stream);
  if (rc == 1) return fail(PA_ERR_UNSUPPORTED, "no kernel for this shape");
  if (rc == 2) return fail(PA_ERR_HIP, hipGetErrorString(hipGetLastError()));
  if (plan.schedule != pa::kScheduleSingle) {
    rc = plan.schedule == pa::kScheduleBalanced ? pa::launch_merge_balanced(a, head_dim, stream)
                                                : pa::launch_merge(a, head_dim, stream);
    if (rc == 1) return fail(PA_ERR_UNSUPPORTED, "no merge kernel for this head_dim");
    if (rc == 2) return fail(PA_ERR_HIP, hipGetErrorString(hipGetLastError()));
  }
  return PA_OK;
}

int pa_prefill(float* out, const void* query, const void* kv_cache, const float* kv_scales,
               const int32_t* block_tables, const int32_t* context_lens,
               const int32_t* query_start, int num_seqs, int total_queries, int num_q_heads,
               int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
               int max_query_len, int64_t num_blocks, float scale, int sliding_window,
               int kernel, int dtype, void* stream_) {
  pa::clear_error();
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  if (dtype != PA_F16 && dtype != PA_I8)
    return fail(PA_ERR_UNSUPPORTED, "prefill needs an f16 or INT8 pool");
  if (num_seqs < 0 || total_queries < 0 || max_query_len < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "sizes out of range");
  if (num_q_heads % num_kv_heads) return fail(PA_ERR_INVALID_ARG, "num_q_heads % num_kv_heads");
  if (sliding_window < 0) return fail(PA_ERR_INVALID_ARG, "sliding_window must be >= 0");
  const int group = num_q_heads / num_kv_heads;
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim");
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "block_size");
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PA_ERR_UNSUPPORTED, "group size");
  if (kernel & ~(0xFF | PA_KV_CACHED)) return fail(PA_ERR_INVALID_ARG, "kernel flags");
  if ((kernel & 0xFF) != PA_KERNEL_AUTO && (kernel & 0xFF) != PA_KERNEL_MFMA)
    return fail(PA_ERR_UNSUPPORTED, "prefill runs on the matrix cores only");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PA_ERR_INVALID_ARG, "prefill scale must be positive and finite");
  const long long max_tokens_ll = (long long)max_blocks_per_seq * block_size;
  if (max_tokens_ll > (1LL << 30)) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq too large");
  // the kernels address a block in 32-bit byte offsets
  if ((long long)num_kv_heads * block_size * head_dim * 4 >= (1LL << 32))
    return fail(PA_ERR_UNSUPPORTED, "num_kv_heads too large for prefill");
  if (num_seqs == 0 || total_queries == 0 || max_query_len == 0) return PA_OK;
  if (!out || !query || !kv_cache || !block_tables || !context_lens || !query_start)
    return fail(PA_ERR_INVALID_ARG, "null device pointer");
  if (!aligned16(out) || !aligned16(query) || !aligned16(kv_cache))
    return fail(PA_ERR_INVALID_ARG, "out/query/kv_cache must be 16-byte aligned");
  if (dtype == PA_I8 ? (!kv_scales || !aligned16(kv_scales)) : kv_scales != nullptr)
    return fail(PA_ERR_INVALID_ARG, "kv_scales: 16-byte aligned for INT8 pools, NULL otherwise");
  if (pa::check_mode()) {
    if (int st = pa::check_prefill_arrays(block_tables, context_lens, query_start, num_seqs,
                                          total_queries, max_query_len, max_blocks_per_seq,
                                          block_size, num_blocks, stream))
      return st;
  }
  pa::PrefillArgs a{};
  a.out = out;
  a.q = query;
  a.kv = kv_cache;
  a.kv_scales = kv_scales;
  a.bt = block_tables;
  a.cl = context_lens;
  a.qstart = query_start;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.total_queries = total_queries;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.max_tokens = (int)max_tokens_ll;
  const long long cols = (long long)max_query_len * group;
  const int per_wg = dtype == PA_I8 ? pa::prefill_i8_columns_per_workgroup()
                                    : pa::prefill_columns_per_workgroup();
  a.qblocks = (int)((cols + per_wg - 1) / per_wg);
  if ((long long)num_seqs * a.qblocks * num_kv_heads > pa::kMaxGridWorkgroups)
    return fail(PA_ERR_INVALID_ARG, "grid too large");
  a.scale_log2 = scale * 1.4426950408889634f;
  a.window = sliding_window;
  const int rc = dtype == PA_I8 ? pa::launch_prefill_mfma_i8(a, head_dim, block_size, group, stream)
                                : pa::launch_prefill_mfma(a, head_dim, block_size, group, stream);
  if (rc == 1) return fail(PA_ERR_UNSUPPORTED, "no prefill kernel for this shape");
  if (rc == 2) return fail(PA_ERR_HIP, hipGetErrorString(hipGetLastError()));
  return PA_OK;
}

}  // extern "C"
