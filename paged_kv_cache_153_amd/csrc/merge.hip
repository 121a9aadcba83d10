// merge.hip — log-sum-exp merge of split-context partials (gfx950).
//
// The pages merge per-block results with the running max / running sum of
// the online softmax ([KVPA] "KV Cache与PagedAttention深度解析" §7.2; [NANO]
// zwxr.cn walkthrough §2.4, merging across blocks with decay factors).  The
// same algebra across partitions: with partition max m_p (log2 units), sum
// l_p and normalised output o_p,
//   M = max_p m_p,  w_p = l_p * exp2(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
// Partitions at or past ceil(n / P) were never written and are not read.
//
// One wave per (sequence, query head); lane j owns dims j, j+64, ...  The
// partition weights are computed once per wave: lane p reads (m_p, l_p) for
// p < 64 at a time and the wave reduces the max, then broadcasts each weight
// with readlane while all lanes stream o_p.
#include "device_common.h"
#include "kernels.h"

namespace pa {
namespace {

template <int D>
__global__ __launch_bounds__(64) void merge_kernel(DecodeArgs a) {
  constexpr int DPL = D / 64;  // dims per lane
  const int lane = threadIdx.x;
  const int row = blockIdx.x;  // s * Hq + h
  const int s = row / a.num_q_heads;
  int n = a.cl[s];
  n = n < 0 ? 0 : n;
  n = min(n, a.max_tokens);
  int np = (n + a.part_tokens - 1) / a.part_tokens;
  np = min(np, a.num_parts);
  float* out = a.out + (size_t)row * D;
  if (np == 0) {
#pragma unroll
    for (int k = 0; k < DPL; ++k) out[lane + 64 * k] = 0.f;
    return;
  }
  const size_t prow = (size_t)row * a.num_parts;
  // pass 1: global max over the live partitions
  float mx = kMaxInit;
  for (int p = lane; p < np; p += 64) mx = fmaxf(mx, a.ws_m[prow + p]);
  mx = cross_rows_max<1>(mx);
  // pass 2: weights and weighted sum
  float acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
  float wsum = 0.f;
  for (int p0 = 0; p0 < np; p0 += 64) {
    const int p = p0 + lane;
    float wl = 0.f;
    if (p < np) wl = a.ws_l[prow + p] * fast_exp2(a.ws_m[prow + p] - mx);
    wsum += wl;
    const int cnt = min(64, np - p0);
    for (int j = 0; j < cnt; ++j) {
      const float wj = __builtin_bit_cast(float, readlane(__builtin_bit_cast(int, wl), j));
      const float* o = a.ws_o + (prow + p0 + j) * D;
#pragma unroll
      for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wj, o[lane + 64 * k], acc[k]);
    }
  }
  wsum = cross_rows_sum<1>(wsum);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int k = 0; k < DPL; ++k) out[lane + 64 * k] = acc[k] * inv;
}

}  // namespace

int launch_merge(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  const unsigned grid = (unsigned)a.num_seqs * a.num_q_heads;
  if (grid == 0) return 0;
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(64), 0, stream, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(64), 0, stream, a);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // namespace pa
