// stream_read.hip — HBM read-bandwidth probes used as the measured ceiling
// that decode bandwidth is compared with.  Built into libpa_probe.so, apart
// from libpa.so; not part of the attention library.
//
//  * pa_probe_read_linear: a grid-stride read of a buffer, 16 bytes per lane.
//  * pa_probe_read_tiles: reads 4 KiB tiles in the order given by a device
//    index array — the access pattern of a paged K or V tile at block 16,
//    head_dim 128, fp16; pa_probe_read_tiles_sized also reads 2 KiB tiles
//    (the same tile of an INT8 pool).
// Each reads either with plain loads or with non-temporal (streaming) loads,
// the two policies pa_decode can use for K/V.
// Both fold what they read into one value that is stored only if it matches
// an impossible constant, so the loads cannot be optimised away and nothing
// is written in practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u4 ld(const u4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT>
__global__ __launch_bounds__(256) void read_linear(const u4* __restrict__ p, size_t n16,
                                                   uint32_t* out) {
  uint32_t acc = 0;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x) {
    const u4 v = ld<NT>(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) out[0] = acc;
}

// TPT threads (16 bytes each) per tile: 256 / TPT tiles per load
// instruction of the 256-thread block, 8 load instructions in flight
template <bool NT, int TPT>
__global__ __launch_bounds__(256) void read_tiles(const u4* __restrict__ p,
                                                  const int32_t* __restrict__ idx, int per_wg,
                                                  int64_t num_tiles, uint32_t* out) {
  constexpr int TPL = 256 / TPT;
  uint32_t acc = 0;
  const int32_t* my = idx + (size_t)blockIdx.x * per_wg;
  const int sub = threadIdx.x / TPT;
  const int c = threadIdx.x % TPT;
  for (int t = 0; t < per_wg; t += 8 * TPL) {
    u4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = t + u * TPL + sub;
      int64_t tile = k < per_wg ? my[k] : 0;
      tile = tile < 0 || tile >= num_tiles ? 0 : tile;
      v[u] = ld<NT>(p + tile * TPT + c);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) out[0] = acc;
}

extern "C" {

// Reads `bytes` (a multiple of 16) from `buf` with `workgroups` x 256 threads;
// `streaming` != 0 uses non-temporal loads.
int pa_probe_read_linear(const void* buf, size_t bytes, int workgroups, int streaming,
                         uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes % 16 || workgroups <= 0) return -1;
  if (streaming)
    hipLaunchKernelGGL(read_linear<true>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       (const u4*)buf, bytes / 16, sink);
  else
    hipLaunchKernelGGL(read_linear<false>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       (const u4*)buf, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Reads the `tile_bytes` (2048 or 4096) tiles of `buf` listed in `tiles`
// ([num_listed] int32 on the device, each in [0, num_tiles)), `per_wg`
// consecutive entries per workgroup.
int pa_probe_read_tiles_sized(const void* buf, int64_t num_tiles, const int32_t* tiles,
                              int64_t num_listed, int per_wg, int tile_bytes, int streaming,
                              uint32_t* sink, void* stream) {
  if (!buf || !tiles || !sink || per_wg <= 0 || num_listed % per_wg) return -1;
  if (tile_bytes != 2048 && tile_bytes != 4096) return -1;
  const int64_t wgs = num_listed / per_wg;
  if (wgs <= 0 || wgs > INT32_MAX) return -1;
  const dim3 g((unsigned)wgs), b(256);
  hipStream_t st = (hipStream_t)stream;
  const u4* p = (const u4*)buf;
  if (tile_bytes == 4096) {
    if (streaming) hipLaunchKernelGGL((read_tiles<true, 256>), g, b, 0, st, p, tiles, per_wg, num_tiles, sink);
    else hipLaunchKernelGGL((read_tiles<false, 256>), g, b, 0, st, p, tiles, per_wg, num_tiles, sink);
  } else {
    if (streaming) hipLaunchKernelGGL((read_tiles<true, 128>), g, b, 0, st, p, tiles, per_wg, num_tiles, sink);
    else hipLaunchKernelGGL((read_tiles<false, 128>), g, b, 0, st, p, tiles, per_wg, num_tiles, sink);
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// 4 KiB tiles (see pa_probe_read_tiles_sized).
int pa_probe_read_tiles(const void* buf, int64_t num_tiles, const int32_t* tiles,
                        int64_t num_listed, int per_wg, int streaming, uint32_t* sink,
                        void* stream) {
  return pa_probe_read_tiles_sized(buf, num_tiles, tiles, num_listed, per_wg, 4096, streaming,
                                   sink, stream);
}

}  // extern "C"
