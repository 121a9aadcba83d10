// decode_schedule.h — how decode work is cut into workgroups.
//
// The unit of work is a 16-token tile of one (sequence, KV head).  Three
// schedules share the same per-range code (decode_range in the kernels):
//
//  * single:    one workgroup per (sequence, KV head), whole context;
//  * partition: one workgroup per (sequence, KV head, P-token partition);
//  * balanced:  W workgroups, each given an equal, contiguous slice of the
//               global work list ordered (sequence, KV head, tile), where a
//               (sequence, KV head) segment of nt > 0 tiles counts as
//               seg_cost + nt units: seg_cost units for what starting and
//               finishing a segment costs (loading q and the first tiles,
//               the cross-wave merge), then one unit per tile.  A workgroup
//               walks the segments its slice covers and computes the tiles
//               among its units; a segment it covers completely is finished
//               in place, a segment whose tiles a slice boundary cuts leaves
//               a partial (at most two per workgroup: the one whose first
//               tile lies in its slice, and its last) that the balanced
//               merge kernel combines; the workgroup whose slice start is
//               the first boundary inside a cut segment's tiles records it
//               for the merge, which then visits only the cut segments.
//               Every workgroup does the same amount of work whatever the
//               length distribution, which removes the tail that ragged
//               batches leave with the other schedules.
//
// A sequence's work is the tile span that holds its keys: tiles
// [t0, t0 + nt) with t0 = floor(lo / 16) and t0 + nt = ceil(n / 16), where
// lo is the first key (0, or n - W under a sliding window of W tokens).  The
// decode and the merge kernels derive spans, partitions and slices from the
// context lengths with the same integer arithmetic (seq_span), so they agree
// on every boundary without exchanging anything.
#pragma once

#include "decode_epilogue.h"
#include "device_common.h"
#include "kernels.h"

namespace pa {

__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int s) {
  int n = a.cl[s];
  n = n < 0 ? 0 : n;
  return min(n, a.max_tokens);
}

__device__ __forceinline__ int tiles_of(int n) { return (n + kTile - 1) / kTile; }

// Keys of one sequence: tokens [lo, n); the tiles [t0, t0 + nt) cover them.
struct Span {
  int lo;
  int n;
  int t0;
  int nt;
};

// The span is also cut to the tiles the launch covers (num_parts partitions
// of part_tokens; a context longer than the caller's bound loses its last
// tiles rather than reading past what the grid and the workspace hold).
__device__ __forceinline__ Span seq_span(const DecodeArgs& a, int s) {
  Span sp;
  sp.n = clamp_len(a, s);
  sp.lo = (a.window > 0 && sp.n > a.window) ? sp.n - a.window : 0;
  sp.t0 = sp.lo / kTile;
  const int covered = a.num_parts * (a.part_tokens / kTile);
  sp.nt = sp.n > 0 ? min(tiles_of(sp.n) - sp.t0, covered) : 0;
  return sp;
}

// Work units of one (sequence, KV head) segment in the balanced schedule.
__device__ __forceinline__ int seg_units(const DecodeArgs& a, int nt) {
  return nt > 0 ? nt + a.seg_cost : 0;
}

// Fills prefix[s] = sum_{s' <= s} units(s') for s < S (per KV head) with the
// whole workgroup; every thread sees the result after the final barrier.
// Scans in chunks of blockDim.x with a running carry.
__device__ inline void build_tile_prefix(const DecodeArgs& a, int* prefix) {
  const int nt = blockDim.x;
  int carry = 0;
  for (int base = 0; base < a.num_seqs; base += nt) {
    const int s = base + (int)threadIdx.x;
    if (s < a.num_seqs) prefix[s] = seg_units(a, seq_span(a, s).nt);
    __syncthreads();
    for (int off = 1; off < nt; off <<= 1) {  // inclusive Hillis-Steele scan
      int v = 0;
      if (s < a.num_seqs && (int)threadIdx.x >= off) v = prefix[s - off];
      __syncthreads();
      if (s < a.num_seqs) prefix[s] += v;
      __syncthreads();
    }
    if (s < a.num_seqs) prefix[s] += carry;
    const int last = min(a.num_seqs, base + nt) - 1;
    __syncthreads();
    carry = prefix[last];
    __syncthreads();
  }
}

// Smallest s with hkv * prefix[s] > t (the sequence holding global unit t).
__device__ __forceinline__ int owner_of(const int* prefix, int num_seqs, int hkv, int64_t t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)hkv * prefix[mid] > t) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// Slice of workgroup w: [w * chunk, min((w + 1) * chunk, total)).
__device__ __forceinline__ int64_t balanced_chunk(int64_t total, int workgroups) {
  const int64_t c = (total + workgroups - 1) / workgroups;
  return c > 0 ? c : 1;
}

}  // namespace pa

namespace pa {

// Maps this workgroup to its range(s) and calls
// range(s, g, lo, n, tile_begin, tile_end, sink) for each (absolute tile
// indices; keys are tokens [lo, n)); ranges are processed one after another
// by the whole workgroup (sm is reused in between).
template <int G, int D, int NW, typename RangeFn>
__device__ void run_schedule(const DecodeArgs& a, int* prefix, RangeFn&& range) {
  if (a.schedule == kScheduleBalanced) {
    build_tile_prefix(a, prefix);
    const int S = a.num_seqs, hkv = a.num_kv_heads, c = a.seg_cost;
    const int64_t total = (int64_t)hkv * prefix[S - 1];
    const int64_t chunk = balanced_chunk(total, a.num_workgroups);
    const int64_t t_start = (int64_t)blockIdx.x * chunk;
    const int64_t t1 = min(t_start + chunk, total);
    // Empty sequences own no units: workgroup w writes the zero outputs of
    // the empty sequences w, w + W, ...
    for (int s = blockIdx.x; s < S; s += gridDim.x)
      if (prefix[s] == (s ? prefix[s - 1] : 0))
        for (int g = 0; g < hkv; ++g) write_zero_output<G, D, NW>(a, s, g);
    // The segment whose tiles the boundary at t_start cuts, recorded for the
    // merge by the first boundary inside them (the workgroups [w_lo, w_hi]
    // that hold its tiles each left a partial; w_lo's slot is 2 w_lo when
    // the tiles start exactly at its slice, else 2 w_lo + 1)
    if (threadIdx.x == 0) {
      int rec[kCutInts] = {-1, 0, 0, 0, 0, 0, 0, 0};
      if (t_start > 0 && t_start < total) {
        const int s = owner_of(prefix, S, hkv, t_start);
        const int before_units = s ? prefix[s - 1] : 0;
        const int nu = prefix[s] - before_units;
        const int64_t before = (int64_t)hkv * before_units;
        const int g = (int)((t_start - before) / nu);
        const int64_t off = before + (int64_t)g * nu + c;
        const int nt = nu - c;
        const int64_t w_lo = off / chunk;
        if (off < t_start && t_start < off + nt && w_lo == (int64_t)blockIdx.x - 1) {
          rec[0] = s;
          rec[1] = g;
          rec[2] = (int)w_lo;
          rec[3] = (int)((off + nt - 1) / chunk);
          rec[4] = (int)(2 * w_lo + (w_lo * chunk >= off ? 0 : 1));
        }
      }
      int* dst = a.ws_cut + (size_t)blockIdx.x * kCutInts;
#pragma unroll
      for (int i = 0; i < kCutInts; ++i) dst[i] = rec[i];
    }
    int64_t t = t_start;
    while (t < t1) {
      const int s = owner_of(prefix, S, hkv, t);
      const int before_units = s ? prefix[s - 1] : 0;
      const int nu = prefix[s] - before_units;  // > 0: s owns unit t
      const int nt = nu - c;
      const int64_t before = (int64_t)hkv * before_units;
      const int g = (int)((t - before) / nu);
      const int64_t seg0 = before + (int64_t)g * nu;
      const int64_t off = seg0 + c;  // the segment's first tile unit
      const int ta = (int)(max(t, off) - off);
      const int tb = (int)(min(seg0 + nu, t1) - off);
      if (tb > ta) {
        Sink sink;
        if (ta == 0 && tb == nt) {
          sink = output_sink<G, D>(a, s, g);
        } else {  // slot 2w: the segment's tiles start in the slice, 2w + 1: before it
          const size_t slot = 2 * (size_t)blockIdx.x + (t_start >= off ? 0 : 1);
          sink = Sink{a.ws_o + slot * G * D, a.ws_m + slot * G, a.ws_l + slot * G, D, 1};
        }
        const Span sp = seq_span(a, s);
        range(s, g, sp.lo, sp.n, sp.t0 + ta, sp.t0 + tb, sink);
        __syncthreads();
      }
      t = seg0 + nu;
    }
    return;
  }
  int bid = blockIdx.x;
  const int g = bid % a.num_kv_heads;
  bid /= a.num_kv_heads;
  const int p = bid % a.num_parts;
  const int s = bid / a.num_parts;
  const Span sp = seq_span(a, s);
  const int pt = a.part_tokens / kTile;  // tiles per partition
  const int t_begin = p * pt;            // relative to the span
  if (t_begin >= sp.nt) {
    if (p == 0) write_zero_output<G, D, NW>(a, s, g);  // empty sequence
    return;
  }
  const int t_end = min(sp.nt, t_begin + pt);
  const int np = (sp.nt + pt - 1) / pt;
  Sink sink;
  if (a.schedule == kScheduleSingle || np == 1) {
    sink = output_sink<G, D>(a, s, g);
  } else {
    const size_t row0 = (size_t)s * a.num_q_heads + g * G;
    sink = Sink{a.ws_o + (row0 * a.num_parts + p) * D, a.ws_m + row0 * a.num_parts + p,
                a.ws_l + row0 * a.num_parts + p, (long)a.num_parts * D, a.num_parts};
  }
  range(s, g, sp.lo, sp.n, sp.t0 + t_begin, sp.t0 + t_end, sink);
}

}  // namespace pa
