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

// Balanced schedule: one workgroup per decode workgroup w merges the
// segment that w recorded in its cut-list entry, if any: the segment's tiles
// were cut by slice boundaries, and the workgroups [w_lo, w_hi] left its
// partials (all G heads) in slot s_lo of w_lo and slot 2w of the others.
// Threads are grouped D/4 to a head row; each keeps the running
// log-sum-exp of its float4 over the contributors.  Empty sequences and
// segments inside one slice were finished by the decode kernel.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_balanced_kernel(DecodeArgs a) {
  constexpr int TPR = D / 4;
  const int* rec = a.ws_cut + (size_t)blockIdx.x * kCutInts;
  const int s = rec[0];
  if (s < 0) return;
  const int g = rec[1], w_lo = rec[2], w_hi = rec[3], slot_lo = rec[4];
  const int G = a.num_q_heads / a.num_kv_heads;
  const int hh = threadIdx.x / TPR;
  if (hh >= G) return;
  const int c4 = (threadIdx.x % TPR) * 4;
  Lse4 st;
  for (int w = w_lo; w <= w_hi; ++w) {
    const size_t idx = (size_t)(w == w_lo ? slot_lo : 2 * w) * G + hh;
    st.push(a.ws_m[idx], a.ws_l[idx], *reinterpret_cast<const float4_t*>(a.ws_o + idx * D + c4));
  }
  float* out = a.out + ((size_t)s * a.num_q_heads + g * G + hh) * D + c4;
  const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
  *reinterpret_cast<float4_t*>(out) = st.o * inv;
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
  const unsigned grid = (unsigned)a.num_workgroups;
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
