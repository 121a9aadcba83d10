// decode_valu_i8.hip — paged decode attention over an INT8 KV cache on the
// vector ALUs (gfx950).
//
// The cache holds int8 codes with one float32 scale per (token, KV head) row
// of K and of V ([KV2P] "KV Cache从原理到实战" §5.2: INT8 halves the cache;
// one scale per 128-element group).  The attention is the same as over the
// dequantised values ([KVPA] "KV Cache与PagedAttention深度解析" §2.1, §4.3,
// §7.2): with k_t = sk_t * Kq_t and v_t = sv_t * Vq_t,
//   score_t = scale * sk_t * (q . Kq_t),   out = sum_t p_t sv_t Vq_t / sum_t p_t,
// so a row's scale multiplies its score, and its V scale multiplies its
// softmax weight; the codes enter the dot products as exact small integers.
//
// Work decomposition as in decode_valu.hip (workgroup = 4 waves over 16-token
// tiles, per-wave online softmax, LDS merge), with the lanes laid out for
// one-byte elements: 8 lanes per row, each holding D/8 codes (16 bytes at
// head_dim 128, 8 at 64), so one load instruction covers 8 whole rows.  Lane
// row r of a wave takes rows 2r and 2r + 1 of each tile, so the two scales it
// needs per tile and per K/V are adjacent (one 8-byte load each).  q is held
// in float32; codes are widened to float32 (exact) for the FMAs.
#include "decode_epilogue.h"
#include "decode_schedule.h"
#include "device_common.h"
#include "kernels.h"

namespace pa {
namespace {

typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr int kLanesPerRow = 8;
constexpr int kRowGroups = 64 / kLanesPerRow;     // 8 lane rows per wave
constexpr int kRowsPerLane = kTile / kRowGroups;  // 2 tile rows per lane row

// Signed byte k of w, widened to float (exact).
template <int K>
__device__ __forceinline__ float byte_f32(uint32_t w) {
  return (float)((int32_t)(w << (24 - 8 * K)) >> 24);
}

// The lane's codes of one row: 16 bytes (D = 128) or 8 bytes (D = 64).
template <int D>
struct Codes;
template <>
struct Codes<128> {
  using type = u32x4_t;
  static constexpr int kWords = 4;
  template <bool NT>
  static __device__ __forceinline__ type load(const void* base, uint32_t off) {
    return kv_load16<NT>(base, off);
  }
  static __device__ __forceinline__ type zero() { return type{0u, 0u, 0u, 0u}; }
};
template <>
struct Codes<64> {
  using type = u32x2_t;
  static constexpr int kWords = 2;
  template <bool NT>
  static __device__ __forceinline__ type load(const void* base, uint32_t off) {
    return kv_load8<NT>(base, off);
  }
  static __device__ __forceinline__ type zero() { return type{0u, 0u}; }
};

template <int D>
__device__ __forceinline__ void widen(const typename Codes<D>::type& c, float (&f)[D / 8]) {
#pragma unroll
  for (int wd = 0; wd < Codes<D>::kWords; ++wd) {
    f[4 * wd + 0] = byte_f32<0>(c[wd]);
    f[4 * wd + 1] = byte_f32<1>(c[wd]);
    f[4 * wd + 2] = byte_f32<2>(c[wd]);
    f[4 * wd + 3] = byte_f32<3>(c[wd]);
  }
}

template <int D, int BS, int G, int NW, bool NT>
__device__ __forceinline__ void decode_range(const DecodeArgs& a, DecodeSmem<G, D, NW>& sm, int s,
                                             int g, int lo, int n, int tile_begin, int tile_end,
                                             const Sink& sink) {
  constexpr int EPL = D / 8;  // codes per lane per row
  constexpr int BPT = BS >= kTile ? 1 : kTile / BS;
  static_assert(BPT <= 2, "a tile spans at most two blocks");
  using codes_t = typename Codes<D>::type;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r = lane / kLanesPerRow;
  const int c = lane % kLanesPerRow;
  const int Hq = a.num_q_heads;

  // ---- q chunk of each grouped head, widened to float32 --------------------
  float qf[G][EPL];
  {
    const half_t* qh = reinterpret_cast<const half_t*>(a.q) + ((size_t)s * Hq + g * G) * D +
                       c * EPL;
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int j = 0; j < EPL / 8; ++j) {
        const half8_t v = __builtin_bit_cast(half8_t, load16(qh + h * D + 8 * j));
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[h][8 * j + e] = (float)v[e];
      }
    }
  }

  // codes: [NB, 2, Hkv, BS, D] bytes; scales: [NB, Hkv, 2, BS] floats
  const size_t head_stride = (size_t)BS * D;
  const size_t block_stride = 2 * (size_t)a.num_kv_heads * head_stride;
  const size_t v_offset = (size_t)a.num_kv_heads * head_stride;
  const int8_t* kvh = reinterpret_cast<const int8_t*>(a.kv) + (size_t)g * head_stride;
  const size_t sblock_stride = 2 * (size_t)a.num_kv_heads * BS;
  const size_t sv_offset = BS;  // scales [NB, Hkv, 2, BS]: K then V of one head, one line
  const float* sch = a.kv_scales + (size_t)g * 2 * BS;
  const int32_t* bt_row = a.bt + (size_t)s * a.max_blocks;

  int ids[BPT];
  auto load_ids = [&](int k0) {
    const int tile = tile_begin + w + (k0 + lane) * NW;
#pragma unroll
    for (int jj = 0; jj < BPT; ++jj) {
      const int lb = BS >= kTile ? tile * kTile / BS : tile * BPT + jj;
      int v = 0;
      if (lb < a.max_blocks) {
        v = bt_row[lb];
        if (v < 0 || v >= a.num_blocks) v = 0;
      }
      ids[jj] = v;
    }
  };

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kMaxInit;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const float cs = a.scale_log2;

  struct Buf {
    codes_t k[kRowsPerLane], v[kRowsPerLane];
    u32x2_t sk, sv;  // scales of rows 2r, 2r + 1 (float bits)
  };
  Buf bA, bB;

  auto issue = [&](int tile, int k_it, Buf& b) {
    const int sel = k_it & 63;
    int blk[BPT];
#pragma unroll
    for (int jj = 0; jj < BPT; ++jj) blk[jj] = readlane(ids[jj], sel);
    const int row = kRowsPerLane * r;  // first of this lane's two rows
    if constexpr (BPT == 1) {
      const int row0 = BS > kTile ? (tile % (BS / kTile)) * kTile : 0;
      const int8_t* kb = kvh + (size_t)blk[0] * block_stride;
      const float* sb = sch + (size_t)blk[0] * sblock_stride;
#pragma unroll
      for (int i = 0; i < kRowsPerLane; ++i) {
        const uint32_t off = (uint32_t)((row0 + row + i) * D + c * EPL);
        b.k[i] = Codes<D>::template load<NT>(kb, off);
        b.v[i] = Codes<D>::template load<NT>(kb + v_offset, off);
      }
      const uint32_t soff = (uint32_t)(row0 + row) * 4u;
      b.sk = kv_load8<NT>(sb, soff);
      b.sv = kv_load8<NT>(sb + sv_offset, soff);
    } else {
      // 8-row blocks: lane rows 0-3 read the first block, 4-7 the second
      const int bk = row >= BS ? blk[BPT - 1] : blk[0];
      const int8_t* kb = kvh + (size_t)bk * block_stride;
      const float* sb = sch + (size_t)bk * sblock_stride;
#pragma unroll
      for (int i = 0; i < kRowsPerLane; ++i) {
        const uint32_t off = (uint32_t)(((row + i) % BS) * D + c * EPL);
        b.k[i] = Codes<D>::template load<NT>(kb, off);
        b.v[i] = Codes<D>::template load<NT>(kb + v_offset, off);
      }
      const uint32_t soff = (uint32_t)(row % BS) * 4u;
      b.sk = kv_load8<NT>(sb, soff);
      b.sv = kv_load8<NT>(sb + sv_offset, soff);
    }
  };

  auto compute = [&](int tile, Buf& b) {
    float y[kRowsPerLane][G];
    float svr[kRowsPerLane];
    // whole-vector casts: this compiler miscompiles a bit_cast of a single
    // vector element (it reads element 0)
    const float2_t skf = __builtin_bit_cast(float2_t, b.sk);
    const float2_t svf = __builtin_bit_cast(float2_t, b.sv);
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
      float kf[EPL];
      widen<D>(b.k[i], kf);
      const float sk = skf[i] * cs;
      svr[i] = svf[i];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d = fmaf(qf[h][e], kf[e], d);
        y[i][h] = group_sum<kLanesPerRow>(d) * sk;
      }
    }
    if ((tile + 1) * kTile > n || tile * kTile < lo) {  // partial tile: mask non-keys
#pragma unroll
      for (int i = 0; i < kRowsPerLane; ++i) {
        const int tok = tile * kTile + kRowsPerLane * r + i;
        if (tok >= n || tok < lo) {
#pragma unroll
          for (int h = 0; h < G; ++h) y[i][h] = -INFINITY;
          b.v[i] = Codes<D>::zero();
          svr[i] = 0.f;
        }
      }
    }
    float vf[kRowsPerLane][EPL];
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) widen<D>(b.v[i], vf[i]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float ym = y[0][h];
#pragma unroll
      for (int i = 1; i < kRowsPerLane; ++i) ym = fmaxf(ym, y[i][h]);
      const float m_new = fmaxf(m[h], ym);
      const float alpha = fast_exp2(m[h] - m_new);
      float pv[kRowsPerLane];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < kRowsPerLane; ++i) {
        pv[i] = fast_exp2(y[i][h] - m_new);
        ps += pv[i];
      }
      l[h] = fmaf(l[h], alpha, ps);
      if (wave_any(alpha != 1.f)) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
      }
#pragma unroll
      for (int i = 0; i < kRowsPerLane; ++i) {
        const float p = pv[i] * svr[i];  // the V row's scale rides on its weight
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vf[i][e], acc[h][e]);
      }
      m[h] = m_new;
    }
  };

  int tile = tile_begin + w;
  int k_it = 0;
  load_ids(0);
  if (tile < tile_end) issue(tile, 0, bA);
  while (tile < tile_end) {
    int nxt = tile + NW;
    if (nxt < tile_end) {
      if (((k_it + 1) & 63) == 0) load_ids(k_it + 1);
      issue(nxt, k_it + 1, bB);
    }
    compute(tile, bA);
    tile = nxt;
    ++k_it;
    if (tile >= tile_end) break;
    nxt = tile + NW;
    if (nxt < tile_end) {
      if (((k_it + 1) & 63) == 0) load_ids(k_it + 1);
      issue(nxt, k_it + 1, bA);
    }
    compute(tile, bB);
    tile = nxt;
    ++k_it;
  }

  // ---- merge the 8 lane rows of this wave, then the waves through LDS ------
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mw = cross_rows_max<kLanesPerRow>(m[h]);
    const float sc = fast_exp2(m[h] - mw);
    const float lw = cross_rows_sum<kLanesPerRow>(l[h] * sc);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = cross_rows_sum<kLanesPerRow>(acc[h][e] * sc);
    m[h] = mw;
    l[h] = lw;
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm.acc[w][h][c * EPL + e] = acc[h][e];
      if (c == 0) {
        sm.m[w][h] = m[h];
        sm.l[w][h] = l[h];
      }
    }
  }
  __syncthreads();
  finish_range<G, D, NW>(sm, sink);
}

template <int D, int BS, int G, int NW, bool NT>
__global__ __launch_bounds__(NW * 64) void decode_valu_i8_kernel(DecodeArgs a) {
  __shared__ DecodeSmem<G, D, NW> sm;
  __shared__ int prefix[kBalancedMaxSeqs];
  run_schedule<G, D, NW>(a, prefix, [&](int s, int g, int lo, int n, int ta, int tb,
                                         const Sink& sink) {
    decode_range<D, BS, G, NW, NT>(a, sm, s, g, lo, n, ta, tb, sink);
  });
}

unsigned grid_of(const DecodeArgs& a) {
  if (a.schedule == kScheduleBalanced) return (unsigned)a.num_workgroups;
  return (unsigned)a.num_seqs * a.num_parts * a.num_kv_heads;
}

// mode 0: launch; mode 1: report resident workgroups per CU in *occ
template <int D, int BS, int G, int NW>
int launch_one(const DecodeArgs& a, hipStream_t stream, int mode, int* occ) {
  if (mode == 1) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&decode_valu_i8_kernel<D, BS, G, NW, true>),
            NW * 64, 0) != hipSuccess)
      return 2;
    *occ = n;
    return 0;
  }
  const unsigned grid = grid_of(a);
  if (grid == 0) return 0;
  if (a.cached_kv)
    hipLaunchKernelGGL((decode_valu_i8_kernel<D, BS, G, NW, false>), dim3(grid), dim3(NW * 64),
                       0, stream, a);
  else
    hipLaunchKernelGGL((decode_valu_i8_kernel<D, BS, G, NW, true>), dim3(grid), dim3(NW * 64),
                       0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

template <int D, int BS, int NW>
int by_group(const DecodeArgs& a, int group, hipStream_t stream, int mode, int* occ) {
  switch (group) {
    case 1: return launch_one<D, BS, 1, NW>(a, stream, mode, occ);
    case 2: return launch_one<D, BS, 2, NW>(a, stream, mode, occ);
    case 4: return launch_one<D, BS, 4, NW>(a, stream, mode, occ);
    case 8: return launch_one<D, BS, 8, NW>(a, stream, mode, occ);
  }
  return 1;
}

template <int D, int NW>
int by_block(const DecodeArgs& a, int block_size, int group, hipStream_t stream, int mode,
             int* occ) {
  switch (block_size) {
    case 8: return by_group<D, 8, NW>(a, group, stream, mode, occ);
    case 16: return by_group<D, 16, NW>(a, group, stream, mode, occ);
    case 32: return by_group<D, 32, NW>(a, group, stream, mode, occ);
  }
  return 1;
}

int dispatch(const DecodeArgs& a, int head_dim, int block_size, int group, hipStream_t stream,
             int mode, int* occ) {
  if (head_dim == 64) return by_block<64, 4>(a, block_size, group, stream, mode, occ);
  if (head_dim == 128) return by_block<128, 4>(a, block_size, group, stream, mode, occ);
  return 1;
}

}  // namespace

int launch_decode_valu_i8(const DecodeArgs& a, int head_dim, int block_size, int group,
                          hipStream_t stream) {
  return dispatch(a, head_dim, block_size, group, stream, 0, nullptr);
}

int decode_valu_i8_occupancy(const DecodeArgs& a, int head_dim, int block_size, int group) {
  int occ = 0;
  return dispatch(a, head_dim, block_size, group, nullptr, 1, &occ) == 0 ? occ : 0;
}

}  // namespace pa
