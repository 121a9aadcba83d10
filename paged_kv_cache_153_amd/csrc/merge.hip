// merge.hip — log-sum-exp merge of split-context partials (gfx950).
//
// The pages merge per-block results with the running max / running sum of
// the online softmax ([KVPA] "KV Cache与PagedAttention深度解析" §7.2; [NANO]
// zwxr.cn walkthrough §2.4, merging across blocks with decay factors).  The
// same algebra across partitions: with partition max m_p (log2 units), sum
// l_p and normalised output o_p,
//   M = max_p m_p,  w_p = l_p * exp2(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
// Partitions past the last one that holds keys of the sequence were never
// written and are not read; a sequence whose keys fit one partition was
// finished by the decode kernel itself.
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

// Running log-sum-exp state of one thread over the partials it has visited:
// max m (log2 units), sum l and the weighted sum o of one float4 of the row.
struct Lse4 {
  float m = kMaxInit;
  float l = 0.f;
  float4_t o = float4_t{0.f, 0.f, 0.f, 0.f};

  __device__ __forceinline__ void push(float mp, float lp, const float4_t& op) {
    const float m_new = fmaxf(m, mp);
    const float keep = fast_exp2(m - m_new);
    const float w = lp * fast_exp2(mp - m_new);
    l = fmaf(l, keep, w);
    o = o * keep + w * op;
    m = m_new;
  }
};

// Threads are grouped D/4 to a row: group grp holds its partials' state for
// columns [c4, c4 + 4).  Combines the groups through LDS with the same
// rescaling and writes the normalised row (zero if nothing had weight).
template <int D>
__device__ __forceinline__ void combine_groups(const Lse4& st, int grp, int c4, float* out) {
  constexpr int TPR = D / 4;
  constexpr int NG = kMergeThreads / TPR;
  __shared__ float s_o[NG][D];
  __shared__ float s_m[NG];
  __shared__ float s_l[NG];
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) s_o[grp][c4 + j] = st.o[j];
  if (tid % TPR == 0) {
    s_m[grp] = st.m;
    s_l[grp] = st.l;
  }
  __syncthreads();
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

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(DecodeArgs a) {
  constexpr int TPR = D / 4;                  // threads per partition row
  constexpr int NG = kMergeThreads / TPR;     // partition groups
  const int tid = threadIdx.x;
  const int row = blockIdx.x;  // s * Hq + h
  const int s = row / a.num_q_heads;
  const int pt = a.part_tokens / kTile;
  const int np = (seq_span(a, s).nt + pt - 1) / pt;
  // 0 partitions: the decode kernel wrote zeros; 1: it wrote the output
  if (np <= 1) return;
  const size_t prow = (size_t)row * a.num_parts;
  const int grp = tid / TPR;
  const int c4 = (tid % TPR) * 4;
  Lse4 st;
  for (int p = grp; p < np; p += NG)
    st.push(a.ws_m[prow + p], a.ws_l[prow + p],
            *reinterpret_cast<const float4_t*>(a.ws_o + (prow + p) * D + c4));
  combine_groups<D>(st, grp, c4, a.out + (size_t)row * D);
}

// Sum of v over the workgroup, returned to every thread.
__device__ __forceinline__ int block_sum(int v, int* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int k = 0; k < kMergeThreads / 64; ++k) t += red[k];
  return t;
}

// Balanced schedule: one workgroup per (sequence, query head) row merges the
// partials that the workgroups whose slices cut the row's segment left in
// their slots (slot 2w if the segment's tiles start in workgroup w's slice,
// 2w + 1 if before it).  It locates the segment from two sums over the
// context lengths — the work units of the sequences before s and of all
// sequences — computed with the decode's own arithmetic.  A segment inside one slice was finished by
// the decode; an empty sequence gets zeros here.  Thread groups of D/4 take
// the slots round robin as in the partition merge.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_balanced_kernel(DecodeArgs a) {
  constexpr int TPR = D / 4;
  constexpr int NG = kMergeThreads / TPR;
  __shared__ int red[2][kMergeThreads / 64];
  const int S = a.num_seqs, hkv = a.num_kv_heads, G = a.num_q_heads / hkv;
  const int row = blockIdx.x;
  const int s = row / a.num_q_heads;
  const int h = row % a.num_q_heads;
  const int g = h / G;
  int before = 0, all = 0;
  for (int j = threadIdx.x; j < S; j += kMergeThreads) {
    const int t = seg_units(a, seq_span(a, j).nt);
    all += t;
    before += j < s ? t : 0;
  }
  before = block_sum(before, red[0]);
  all = block_sum(all, red[1]);
  const int nt = seq_span(a, s).nt;
  float* out = a.out + (size_t)row * D;
  if (nt == 0) {
    for (int d = threadIdx.x; d < D; d += kMergeThreads) out[d] = 0.f;
    return;
  }
  const int64_t total = (int64_t)hkv * all;
  const int64_t chunk = balanced_chunk(total, a.num_workgroups);
  const int64_t off = (int64_t)hkv * before + (int64_t)g * (nt + a.seg_cost) + a.seg_cost;
  const int64_t w_lo = off / chunk;
  const int64_t w_hi = (off + nt - 1) / chunk;
  if (w_lo == w_hi) return;
  const int grp = threadIdx.x / TPR;
  const int c4 = (threadIdx.x % TPR) * 4;
  const int hh = h % G;
  Lse4 st;
  for (int64_t w = w_lo + grp; w <= w_hi; w += NG) {
    const size_t idx = (2 * (size_t)w + (w * chunk >= off ? 0 : 1)) * G + hh;
    st.push(a.ws_m[idx], a.ws_l[idx], *reinterpret_cast<const float4_t*>(a.ws_o + idx * D + c4));
  }
  combine_groups<D>(st, grp, c4, out);
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
  const unsigned grid = (unsigned)a.num_seqs * a.num_q_heads;
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
