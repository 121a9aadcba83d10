// merge.hip — log-sum-exp merge of split-context partials (gfx950).
//
// The pages merge per-block results with the running max / running sum of
// the online softmax ([KVPA] "KV Cache与PagedAttention深度解析" §7.2; [NANO]
// zwxr.cn walkthrough §2.4, merging across blocks with decay factors).  The
// same algebra across partitions: with partition max m_p (log2 units), sum
// l_p and normalised output o_p,
//   M = max_p m_p,  w_p = l_p * exp2(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
// Partitions at or past ceil(n / P) were never written and are not read; a
// sequence that fits one partition was finished by the decode kernel itself.
//
// One 256-thread workgroup per (sequence, query head).  D/4 threads cover
// one partition row with float4 loads (a 512-byte coalesced row at D = 128);
// the 256 / (D/4) thread groups take partitions round robin and each keeps
// a running (max, sum, weighted row) over its partitions, so every load a
// thread needs — m_p, l_p and its slice of o_p — is issued at once and the
// only dependent round trip is the context length.  The groups' states are
// combined through LDS with the same rescaling.
#include "decode_schedule.h"
#include "device_common.h"
#include "kernels.h"

namespace pa {
namespace {

constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(DecodeArgs a) {
  constexpr int TPR = D / 4;                  // threads per partition row
  constexpr int NG = kMergeThreads / TPR;     // partition groups
  __shared__ float s_o[NG][D];
  __shared__ float s_m[NG];
  __shared__ float s_l[NG];

  const int tid = threadIdx.x;
  const int row = blockIdx.x;  // s * Hq + h
  const int s = row / a.num_q_heads;
  int n = a.cl[s];
  n = n < 0 ? 0 : n;
  n = min(n, a.max_tokens);
  n = min(n, a.num_parts * a.part_tokens);
  const int np = (n + a.part_tokens - 1) / a.part_tokens;
  // 0 partitions: the decode kernel wrote zeros; 1: it wrote the output
  if (np <= 1) return;
  const size_t prow = (size_t)row * a.num_parts;

  const int grp = tid / TPR;
  const int c4 = (tid % TPR) * 4;
  float mx = kMaxInit, lsum = 0.f;
  float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
  for (int p = grp; p < np; p += NG) {
    const float mp = a.ws_m[prow + p];
    const float lp = a.ws_l[prow + p];
    const float4_t o = *reinterpret_cast<const float4_t*>(a.ws_o + (prow + p) * D + c4);
    const float m_new = fmaxf(mx, mp);
    const float keep = fast_exp2(mx - m_new);
    const float w = lp * fast_exp2(mp - m_new);
    lsum = fmaf(lsum, keep, w);
    acc = acc * keep + w * o;
    mx = m_new;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) s_o[grp][c4 + j] = acc[j];
  if (tid % TPR == 0) {
    s_m[grp] = mx;
    s_l[grp] = lsum;
  }
  __syncthreads();
  float* out = a.out + (size_t)row * D;
  for (int d = tid; d < D; d += kMergeThreads) {
    float big = s_m[0];
#pragma unroll
    for (int k = 1; k < NG; ++k) big = fmaxf(big, s_m[k]);
    float o = 0.f, wt = 0.f;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const float f = fast_exp2(s_m[k] - big);
      o = fmaf(s_o[k][d], f, o);
      wt = fmaf(s_l[k], f, wt);
    }
    out[d] = wt > 0.f ? o / wt : 0.f;
  }
}

// Balanced schedule: one workgroup per (sequence, KV head) merges the
// partials that the workgroups whose slices cut this segment left in their
// slots (slot 2w if the segment was workgroup w's first, 2w + 1 if its last),
// for all G query heads of the group.  It recomputes the slices from the
// context lengths exactly as the decode did.  A segment inside one slice was
// finished by the decode; an empty sequence gets zeros here.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_balanced_kernel(DecodeArgs a) {
  __shared__ int prefix[kBalancedMaxSeqs];
  build_tile_prefix(a, prefix);
  const int S = a.num_seqs, hkv = a.num_kv_heads, G = a.num_q_heads / hkv;
  const int s = blockIdx.x / hkv;
  const int g = blockIdx.x % hkv;
  const int before_tiles = s ? prefix[s - 1] : 0;
  const int nt = prefix[s] - before_tiles;
  float* out = a.out + ((size_t)s * a.num_q_heads + (size_t)g * G) * D;
  if (nt == 0) {
    for (int idx = threadIdx.x; idx < G * D; idx += kMergeThreads) out[idx] = 0.f;
    return;
  }
  const int64_t total = (int64_t)hkv * prefix[S - 1];
  const int64_t chunk = balanced_chunk(total, a.num_workgroups);
  const int64_t off = (int64_t)hkv * before_tiles + (int64_t)g * nt;
  const int64_t w_lo = off / chunk;
  const int64_t w_hi = (off + nt - 1) / chunk;
  if (w_lo == w_hi) return;
  for (int idx = threadIdx.x; idx < G * D; idx += kMergeThreads) {
    const int h = idx / D;
    const int d = idx % D;
    float mx = kMaxInit;
    for (int64_t w = w_lo; w <= w_hi; ++w) {
      const size_t slot = 2 * (size_t)w + (w * chunk >= off ? 0 : 1);
      mx = fmaxf(mx, a.ws_m[slot * G + h]);
    }
    float L = 0.f, O = 0.f;
    for (int64_t w = w_lo; w <= w_hi; ++w) {
      const size_t slot = 2 * (size_t)w + (w * chunk >= off ? 0 : 1);
      const float wgt = a.ws_l[slot * G + h] * fast_exp2(a.ws_m[slot * G + h] - mx);
      L += wgt;
      O = fmaf(wgt, a.ws_o[(slot * G + h) * D + d], O);
    }
    out[idx] = L > 0.f ? O / L : 0.f;
  }
}

}  // namespace

int launch_merge(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  const unsigned grid = (unsigned)a.num_seqs * a.num_q_heads;
  if (grid == 0) return 0;
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(kMergeThreads), 0, stream, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(kMergeThreads), 0, stream, a);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int launch_merge_balanced(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  const unsigned grid = (unsigned)a.num_seqs * a.num_kv_heads;
  if (grid == 0) return 0;
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_balanced_kernel<64>, dim3(grid), dim3(kMergeThreads), 0, stream, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL(merge_balanced_kernel<128>, dim3(grid), dim3(kMergeThreads), 0, stream, a);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // namespace pa
