// prefill_common.h — what the f16 and INT8 prefill kernels share: the step
// and workgroup shape, the LDS layout of a converted K/V step tile, and the
// mapping of a workgroup to its (sequence, KV head, query block) with the
// keys it must cover.
//
// A chunk of T new tokens per sequence ([KV2P] "KV Cache从原理到实战" §5.4,
// chunked prefill) has its K/V in the cache; query i sits at position
// p = n - T + i and attends to keys t <= p (the causal mask of [INFRA]
// "大模型 (LLM) 推理加速核心技术解析" §2, aligned to the end of the
// context), under a sliding window of W tokens ([KV2P] §7.2) only to
// p - W < t <= p.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace pa {
namespace prefill {

// The softmax reference m of a column moves only when a score exceeds it by
// more than kSlack (log2 units), so most steps skip the cross-lane max and
// the rescale.  Weights are exp2(y - m + kPLog) <= 2^(kSlack + kPLog) = 2^15,
// inside fp16 range for the hi/lo split.
constexpr float kSlack = 8.f;
constexpr float kPLog = 7.f;
constexpr int kKeys = 32;   // keys per step: two 16-key MFMA tiles
constexpr int kBufs = 4;    // LDS buffers of raw step tiles
constexpr int kAhead = 3;   // steps in flight ahead of the one computed
constexpr int kCB = 2;      // 16-column blocks per wave

// Byte offset of 16-byte chunk c of row r in a 16-bit K step tile (rows of
// 2D bytes): chunks are XOR-swizzled by the row, so the 16 lanes that read
// one chunk of 16 different K rows hit distinct banks.
template <int D>
__device__ __forceinline__ uint32_t tile_off(int r, int c) {
  constexpr int CPR = D / 8;  // chunks per row
  return (uint32_t)(r * (2 * D) + ((c ^ (r & (CPR - 1))) << 4));
}

template <int D>
struct VRow;  // per-lane share of one 16-bit V row: 16 bytes (D=128) or 8 bytes (D=64)
template <>
struct VRow<128> {
  using type = u32x4_t;
};
template <>
struct VRow<64> {
  using type = u32x2_t;
};

// The work of one workgroup.
struct Work {
  int s, g, qb;     // sequence, KV head, query block
  int q0, T, n;     // first query row, chunk length, context length
  int wg_tok0;      // first chunk token of the workgroup's columns
  int wg_last;      // last one
  int wg_lo;        // first key any of its columns sees
  int st0, nsteps;  // key steps [st0, nsteps)
};

// Workgroups go to the 8 XCDs round robin.  Renumbered so that each XCD
// takes a contiguous range, every column block of one (sequence, KV head)
// runs on the XCD whose L2 holds that head's K/V; within a pair the latest
// tokens (the most keys) start first.  Returns false when the workgroup has
// no columns: an empty chunk, one that runs backwards or leaves
// [0, total_queries) (so a bad query_start entry can never address q or out
// outside their buffers), one longer than its context, or a query block past
// its end.
template <int G, int COLS>  // COLS: columns per workgroup
__device__ __forceinline__ bool workgroup_work(const PrefillArgs& a, Work& wk) {
  const unsigned nwg = gridDim.x, bid = blockIdx.x;
  const unsigned per = nwg / 8u, rem = nwg % 8u, xcd = bid % 8u;
  unsigned lid = xcd * per + (xcd < rem ? xcd : rem) + bid / 8u;
  wk.qb = a.qblocks - 1 - (int)(lid % (unsigned)a.qblocks);
  lid /= (unsigned)a.qblocks;
  wk.g = (int)(lid % (unsigned)a.num_kv_heads);
  wk.s = (int)(lid / (unsigned)a.num_kv_heads);
  wk.q0 = a.qstart[wk.s];
  const int q1 = a.qstart[wk.s + 1];
  if (wk.q0 < 0 || q1 <= wk.q0 || q1 > a.total_queries) return false;
  wk.T = q1 - wk.q0;
  int n = a.cl[wk.s];
  wk.n = n < 0 ? 0 : (n > a.max_tokens ? a.max_tokens : n);
  wk.wg_tok0 = wk.qb * (COLS / G);
  if (wk.T > wk.n || wk.wg_tok0 >= wk.T) return false;
  wk.wg_last = min(wk.T - 1, wk.wg_tok0 + COLS / G - 1);
  // keys: from the first window start of the columns (0 without a window)
  // to the last column's position; steps are absolute
  wk.wg_lo = a.window > 0 ? max(0, wk.n - wk.T + wk.wg_tok0 + 1 - a.window) : 0;
  wk.st0 = wk.wg_lo / kKeys;
  wk.nsteps = (wk.n - wk.T + wk.wg_last) / kKeys + 1;
  return true;
}

}  // namespace prefill
}  // namespace pa
