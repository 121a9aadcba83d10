// decode_valu.hip — paged decode attention on the vector ALUs (gfx950).
//
// What it computes ([KVPA] "KV Cache与PagedAttention深度解析" §2.1 formula,
// §4.3 block-table addressing, §7.2 online softmax; [NANO] zwxr.cn
// walkthrough §2.4 kernel structure): for every sequence s and query head h,
// softmax(scale * q K^T) V over the context's tokens, where token t is row
// t % BS of physical block block_tables[s, t / BS] in a pool laid out
// [NB, 2, Hkv, BS, D].  Grouped heads ([KV2P] "KV Cache从原理到实战" §5.3):
// the G = Hq / Hkv query heads h = g*G .. g*G+G-1 read KV head g.
//
// Work decomposition (not from the pages; designed for CDNA4):
//  * One workgroup per (sequence, KV head, partition).  It serves all G query
//    heads of that KV head, so every K/V byte is read from HBM once.
//  * The workgroup's NW waves take the partition's 16-token tiles round
//    robin.  Each wave keeps its own online-softmax state and the waves merge
//    through LDS at the end, so the main loop has no barrier.
//  * Loads: a K (or V) tile of 16 rows is D*E bytes per row; lane (r, c)
//    of a wave reads the 16-byte chunk c of row r of each group of RPI rows,
//    so every load instruction covers RPI whole rows — contiguous bytes,
//    128-bit per lane.  The next tile's loads are issued before the current
//    tile is computed (register double buffer).
//  * q.k: each lane dots its chunk (v_dot2 for f16, FMA for f32) and the LPT
//    lanes of a row sum through DPP (quad permutes, half-row and row
//    mirrors), so every lane of the row holds the row's score.
//  * Softmax: each row of lanes keeps (m, l) for its own tokens in log2
//    units; no cross-row traffic inside the loop.  P.V accumulates in fp32
//    (v_fma_mix for f16 values).
//  * Block ids: lane j of a wave holds the physical id of the wave's j-th
//    tile (one vector load per 64 tiles); readlane moves it to an SGPR, so
//    the K/V address is an SGPR base plus a per-lane offset.
//  * Every block id read from the table is clamped into [0, NB), and rows at
//    or past the context length — or before a sliding window's first key
//    ([KV2P] §7.2) — are masked (score -inf, V zeroed), so the kernel never
//    reads outside the pool and never lets unused rows — even NaN ones —
//    reach the output.
#include "device_common.h"
#include "decode_epilogue.h"
#include "decode_schedule.h"
#include "kernels.h"

namespace pa {
namespace {

// One range: tiles [tile_begin, tile_end) of (sequence s, KV head g), whose
// keys are tokens [lo, n); the result goes to `sink`.
template <typename T, int D, int BS, int G, int NW, bool NT>
__device__ __forceinline__ void decode_range(const DecodeArgs& a, DecodeSmem<G, D, NW>& sm, int s,
                                             int g, int lo, int n, int tile_begin,
                                             int tile_end, const Sink& sink) {
  constexpr int E = DType<T>::kBytes;
  constexpr int EPL = 16 / E;        // elements per 16-byte chunk
  constexpr int LPT = D / EPL;       // lanes per token row
  constexpr int RPI = 64 / LPT;      // rows per load instruction
  constexpr int NI = kTile / RPI;    // load instructions per K (or V) tile
  constexpr int BPT = BS >= kTile ? 1 : kTile / BS;  // physical blocks per tile
  static_assert(LPT == 8 || LPT == 16 || LPT == 32, "unsupported row width");
  static_assert(RPI <= BS, "a load instruction must stay inside one block");

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r = lane / LPT;
  const int c = lane % LPT;
  const int Hq = a.num_q_heads;

  // ---- query chunk of each grouped head, held in registers ----------------
  const T* qbase = reinterpret_cast<const T*>(a.q) + ((size_t)s * Hq + g * G) * D + c * EPL;
  u32x4_t qraw[G];
#pragma unroll
  for (int h = 0; h < G; ++h) qraw[h] = load16(qbase + h * D);

  const size_t head_stride = (size_t)BS * D;                 // elements
  const size_t block_stride = 2 * (size_t)a.num_kv_heads * head_stride;
  const size_t v_offset = (size_t)a.num_kv_heads * head_stride;
  const T* kvh = reinterpret_cast<const T*>(a.kv) + (size_t)g * head_stride;
  const int32_t* bt_row = a.bt + (size_t)s * a.max_blocks;

  // ---- block ids of this wave's tiles: lane j <-> j-th tile of the window --
  int ids[BPT];
  auto load_ids = [&](int k0) {
    const int tile = tile_begin + w + (k0 + lane) * NW;
#pragma unroll
    for (int jj = 0; jj < BPT; ++jj) {
      const int lb = BS >= kTile ? tile * kTile / BS : tile * BPT + jj;
      int v = 0;
      // bounded by the table width only, so this load does not wait for
      // the context length; ids of tiles past the context are never used
      if (lb < a.max_blocks) {
        v = bt_row[lb];
        if (v < 0 || v >= a.num_blocks) v = 0;
      }
      ids[jj] = v;
    }
  };

  // ---- per-row online-softmax state --------------------------------------
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kMaxInit;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const float cs = a.scale_log2;

  u32x4_t kA[NI], vA[NI], kB[NI], vB[NI];

  auto issue = [&](int tile, int k_it, u32x4_t (&kr)[NI], u32x4_t (&vr)[NI]) {
    const int sel = k_it & 63;
    int blk[BPT];
#pragma unroll
    for (int jj = 0; jj < BPT; ++jj) blk[jj] = readlane(ids[jj], sel);
    const int row0 = BS > kTile ? (tile % (BS / kTile)) * kTile : 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int jj = BS >= kTile ? 0 : (i * RPI) / BS;
      const int row = BS >= kTile ? row0 + i * RPI + r : (i * RPI) % BS + r;
      const T* base = kvh + (size_t)blk[jj] * block_stride;   // wave-uniform
      const uint32_t off = (uint32_t)(row * D + c * EPL) * (uint32_t)sizeof(T);
      kr[i] = kv_load16<NT>(base, off);
      vr[i] = kv_load16<NT>(base + v_offset, off);
    }
  };

  auto compute = [&](int tile, u32x4_t (&kr)[NI], u32x4_t (&vr)[NI]) {
    float y[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d;
        if constexpr (E == 2) {
          const half8_t kq = __builtin_bit_cast(half8_t, kr[i]);
          const half8_t qq = __builtin_bit_cast(half8_t, qraw[h]);
          d = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            half2_t k2 = {kq[2 * j], kq[2 * j + 1]};
            half2_t q2 = {qq[2 * j], qq[2 * j + 1]};
            d = __builtin_amdgcn_fdot2(k2, q2, d, false);
          }
        } else {
          const float4_t kf = __builtin_bit_cast(float4_t, kr[i]);
          const float4_t qf = __builtin_bit_cast(float4_t, qraw[h]);
          d = kf[0] * qf[0];
          d = fmaf(kf[1], qf[1], d);
          d = fmaf(kf[2], qf[2], d);
          d = fmaf(kf[3], qf[3], d);
        }
        y[i][h] = group_sum<LPT>(d) * cs;
      }
    }
    if ((tile + 1) * kTile > n || tile * kTile < lo) {  // partial tile: mask non-keys
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int tok = tile * kTile + i * RPI + r;
        if (tok >= n || tok < lo) {
#pragma unroll
          for (int h = 0; h < G; ++h) y[i][h] = -INFINITY;
          vr[i] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float ym = y[0][h];
#pragma unroll
      for (int i = 1; i < NI; ++i) ym = fmaxf(ym, y[i][h]);
      const float m_new = fmaxf(m[h], ym);
      const float alpha = fast_exp2(m[h] - m_new);
      float pv[NI];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        pv[i] = fast_exp2(y[i][h] - m_new);
        ps += pv[i];
      }
      l[h] = fmaf(l[h], alpha, ps);
      if (wave_any(alpha != 1.f)) {  // the row's running max moved
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if constexpr (E == 2) {
          const half8_t vh = __builtin_bit_cast(half8_t, vr[i]);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pv[i], (float)vh[e], acc[h][e]);
        } else {
          const float4_t vf = __builtin_bit_cast(float4_t, vr[i]);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pv[i], vf[e], acc[h][e]);
        }
      }
      m[h] = m_new;
    }
  };

  // ---- main loop: two register buffers, loads one tile ahead --------------
  int tile = tile_begin + w;
  int k_it = 0;
  load_ids(0);
  if (tile < tile_end) issue(tile, 0, kA, vA);
  while (tile < tile_end) {
    int nxt = tile + NW;
    if (nxt < tile_end) {
      if (((k_it + 1) & 63) == 0) load_ids(k_it + 1);
      issue(nxt, k_it + 1, kB, vB);
    }
    compute(tile, kA, vA);
    tile = nxt;
    ++k_it;
    if (tile >= tile_end) break;
    nxt = tile + NW;
    if (nxt < tile_end) {
      if (((k_it + 1) & 63) == 0) load_ids(k_it + 1);
      issue(nxt, k_it + 1, kA, vA);
    }
    compute(tile, kB, vB);
    tile = nxt;
    ++k_it;
  }

  // ---- merge the RPI rows of this wave ------------------------------------
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mw = cross_rows_max<LPT>(m[h]);
    const float sc = fast_exp2(m[h] - mw);
    const float lw = cross_rows_sum<LPT>(l[h] * sc);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = cross_rows_sum<LPT>(acc[h][e] * sc);
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

template <typename T, int D, int BS, int G, int NW, bool NT>
__global__ __launch_bounds__(NW * 64) void decode_valu_kernel(DecodeArgs a) {
  __shared__ DecodeSmem<G, D, NW> sm;
  __shared__ int prefix[kBalancedMaxSeqs];
  run_schedule<G, D, NW>(a, prefix, [&](int s, int g, int lo, int n, int ta, int tb,
                                         const Sink& sink) {
    decode_range<T, D, BS, G, NW, NT>(a, sm, s, g, lo, n, ta, tb, sink);
  });
}

unsigned grid_of(const DecodeArgs& a) {
  if (a.schedule == kScheduleBalanced) return (unsigned)a.num_workgroups;
  return (unsigned)a.num_seqs * a.num_parts * a.num_kv_heads;
}

// mode 0: launch; mode 1: report resident workgroups per CU in *occ
template <typename T, int D, int BS, int G, int NW>
int launch_one(const DecodeArgs& a, hipStream_t stream, int mode, int* occ) {
  if (mode == 1) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&decode_valu_kernel<T, D, BS, G, NW, true>),
            NW * 64, 0) != hipSuccess)
      return 2;
    *occ = n;
    return 0;
  }
  const unsigned grid = grid_of(a);
  if (grid == 0) return 0;
  if (a.cached_kv)
    hipLaunchKernelGGL((decode_valu_kernel<T, D, BS, G, NW, false>), dim3(grid), dim3(NW * 64),
                       0, stream, a);
  else
    hipLaunchKernelGGL((decode_valu_kernel<T, D, BS, G, NW, true>), dim3(grid), dim3(NW * 64),
                       0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

template <typename T, int D, int BS, int NW>
int by_group(const DecodeArgs& a, int group, hipStream_t stream, int mode, int* occ) {
  switch (group) {
    case 1: return launch_one<T, D, BS, 1, NW>(a, stream, mode, occ);
    case 2: return launch_one<T, D, BS, 2, NW>(a, stream, mode, occ);
    case 4: return launch_one<T, D, BS, 4, NW>(a, stream, mode, occ);
    case 8: return launch_one<T, D, BS, 8, NW>(a, stream, mode, occ);
  }
  return 1;
}

template <typename T, int D, int NW>
int by_block(const DecodeArgs& a, int block_size, int group, hipStream_t stream, int mode,
             int* occ) {
  switch (block_size) {
    case 8: return by_group<T, D, 8, NW>(a, group, stream, mode, occ);
    case 16: return by_group<T, D, 16, NW>(a, group, stream, mode, occ);
    case 32: return by_group<T, D, 32, NW>(a, group, stream, mode, occ);
  }
  return 1;
}

template <typename T, int NW>
int by_dim(const DecodeArgs& a, int head_dim, int block_size, int group, hipStream_t stream,
           int mode, int* occ) {
  switch (head_dim) {
    case 64: return by_block<T, 64, NW>(a, block_size, group, stream, mode, occ);
    case 128: return by_block<T, 128, NW>(a, block_size, group, stream, mode, occ);
  }
  return 1;
}

int dispatch(const DecodeArgs& a, int dtype, int head_dim, int block_size, int group,
             hipStream_t stream, int mode, int* occ) {
  if (dtype == 0) return by_dim<float, 4>(a, head_dim, block_size, group, stream, mode, occ);
  if (dtype == 1) return by_dim<half_t, 4>(a, head_dim, block_size, group, stream, mode, occ);
  return 1;
}

}  // namespace

int launch_decode_valu(const DecodeArgs& a, int dtype, int head_dim, int block_size, int group,
                       int waves, hipStream_t stream) {
  if (waves != 4) return 1;
  return dispatch(a, dtype, head_dim, block_size, group, stream, 0, nullptr);
}

int decode_valu_occupancy(const DecodeArgs& a, int dtype, int head_dim, int block_size,
                          int group) {
  int occ = 0;
  return dispatch(a, dtype, head_dim, block_size, group, nullptr, 1, &occ) == 0 ? occ : 0;
}

}  // namespace pa
