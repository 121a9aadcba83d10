// decode_mfma.hip — paged decode attention on the matrix cores (gfx950, f16).
//
// Same computation and work decomposition as decode_valu.hip ([KVPA] "KV
// Cache与PagedAttention深度解析" §2.1, §4.3, §7.2; [NANO] zwxr.cn walkthrough
// §2.4): one workgroup per (sequence, KV head, partition), NW independent
// waves over 16-token tiles, online softmax per wave, LDS merge at the end.
// With grouped-query attention ([KV2P] "KV Cache从原理到实战" §5.3) the G query
// heads that share a KV head make q K^T a real [G x D] x [D x 16] product per
// tile, so the two contractions run as MFMA tiles with the G heads padded to
// 16 columns:
//
//  * S^T[t][h] = sum_d K[t][d] q[h][d] with v_mfma_f32_16x16x32_f16 over D/32
//    steps.  A = K (lane l: token l%16, eight consecutive d of the chunk
//    4j + l/16), B = q (lane l: head l%16, same d).  Each K load instruction
//    covers 64 contiguous bytes of all 16 rows of the tile.
//  * The C layout of that product (lane l: tokens 4*(l/16)+i of head l%16)
//    is exactly the B layout that v_mfma_f32_16x16x16f16 needs for P^T, so
//    O^T[d][h] += sum_t V^T[d][t] P^T[t][h] needs no lane shuffle.  Its A
//    operand (lane l: 4 consecutive tokens at one d) comes from V rows loaded
//    128-bit coalesced (lane l: row 4*(l/16)+i, 16-byte chunk l%16) and
//    paired with v_perm_b32; the MFMA row index m = l%16 then stands for
//    d = 8m + e in block e, a relabelling undone when the output is written.
//  * The softmax weights are split into fp16 hi + lo parts (two MFMAs per V
//    block) so P.V keeps about 22 significant bits; they are scaled by 2^15
//    first, so weights down to ~2e-9 of the running max stay normal fp16.
//    The sum l uses the same scaled weights, so the scale cancels in O / l.
//  * The running max per head needs one max across the four lane groups
//    (two butterfly steps); everything else stays in the lane.
#include "device_common.h"
#include "decode_epilogue.h"
#include "decode_schedule.h"
#include "kernels.h"

namespace pa {
namespace {

constexpr float kPScale = 32768.f;  // 2^15

template <int D>
struct VRow;  // per-lane share of one V row: 16 bytes (D=128) or 8 bytes (D=64)
template <>
struct VRow<128> {
  using type = u32x4_t;
  static __device__ __forceinline__ type load(const half_t* p) { return load16(p); }
  static __device__ __forceinline__ type zero() { return type{0u, 0u, 0u, 0u}; }
};
template <>
struct VRow<64> {
  using type = u32x2_t;
  static __device__ __forceinline__ type load(const half_t* p) {
    return *reinterpret_cast<const u32x2_t*>(p);
  }
  static __device__ __forceinline__ type zero() { return type{0u, 0u}; }
};

// DEPTH 2: the next tile's loads are issued before the current tile is
// computed (register double buffer, 2 waves per SIMD).  DEPTH 1: one tile
// per wave in flight and twice the waves per SIMD to hide the latency.
template <int D, int BS, int G, int NW, int DEPTH, bool NT>
__device__ __forceinline__ void decode_range(const DecodeArgs& a, DecodeSmem<G, D, NW>& sm, int s,
                                             int g, int lo, int n, int tile_begin,
                                             int tile_end, const Sink& sink) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(G >= 1 && G <= 16, "group");
  constexpr int KS = D / 32;                 // 16x16x32 steps for q.K
  constexpr int VH = D / 16;                 // halves of one V row per lane
  constexpr int NE = VH;                     // P.V blocks of 16 output rows
  constexpr int BPT = BS >= kTile ? 1 : kTile / BS;
  static_assert(BPT <= 2, "a tile spans at most two blocks");
  using vrow_t = typename VRow<D>::type;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int quad = lane >> 4;
  const int col = lane & 15;
  const int Hq = a.num_q_heads;

  // ---- q as the B operand of q.K: lane (quad, col) = head col, chunk 4j+quad
  half8_t qb[KS];
  {
    const half_t* qh = reinterpret_cast<const half_t*>(a.q) + ((size_t)s * Hq + g * G) * D;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      if (col < G)
        qb[j] = __builtin_bit_cast(half8_t, load16(qh + col * D + (4 * j + quad) * 8));
      else
        qb[j] = __builtin_bit_cast(half8_t, u32x4_t{0u, 0u, 0u, 0u});
    }
  }

  const size_t head_stride = (size_t)BS * D;
  const size_t block_stride = 2 * (size_t)a.num_kv_heads * head_stride;
  const size_t v_offset = (size_t)a.num_kv_heads * head_stride;
  const half_t* kvh = reinterpret_cast<const half_t*>(a.kv) + (size_t)g * head_stride;
  const int32_t* bt_row = a.bt + (size_t)s * a.max_blocks;

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

  float m = kMaxInit;  // running max of head `col` (same in all four quads)
  float l = 0.f;       // this lane's share of the (2^15-scaled) weight sum
  float4_t acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = float4_t{0.f, 0.f, 0.f, 0.f};
  const float cs = a.scale_log2;

  u32x4_t kA[KS], kB[KS];
  vrow_t vA[4], vB[4];

  auto issue = [&](int tile, int k_it, u32x4_t (&kr)[KS], vrow_t (&vr)[4]) {
    const int sel = k_it & 63;
    int blk[BPT];
#pragma unroll
    for (int jj = 0; jj < BPT; ++jj) blk[jj] = readlane(ids[jj], sel);
    const int row0 = BS > kTile ? (tile % (BS / kTile)) * kTile : 0;
    if constexpr (BPT == 1) {
      // one block: wave-uniform base, per-lane unsigned offsets
      const half_t* kb = kvh + (size_t)blk[0] * block_stride;
      const half_t* vb = kb + v_offset;
      const uint32_t krow = (uint32_t)(row0 + col) * (D * 2);
#pragma unroll
      for (int j = 0; j < KS; ++j) kr[j] = kv_load16<NT>(kb, krow + (4 * j + quad) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t off = (uint32_t)(row0 + 4 * quad + i) * (D * 2) + col * (VH * 2);
        if constexpr (D == 128)
          vr[i] = kv_load16<NT>(vb, off);
        else
          vr[i] = kv_load8<NT>(vb, off);
      }
    } else {
      // a tile spans two 8-row blocks: lanes pick their block
      const int bk = col >= BS ? blk[BPT - 1] : blk[0];
      const half_t* kb = kvh + (size_t)bk * block_stride;
      const uint32_t krow = (uint32_t)(col % BS) * (D * 2);
#pragma unroll
      for (int j = 0; j < KS; ++j) kr[j] = kv_load16<NT>(kb, krow + (4 * j + quad) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * quad + i;
        const half_t* vb = kvh + (size_t)(t >= BS ? blk[BPT - 1] : blk[0]) * block_stride +
                           v_offset;
        const uint32_t off = (uint32_t)(t % BS) * (D * 2) + col * (VH * 2);
        if constexpr (D == 128)
          vr[i] = kv_load16<NT>(vb, off);
        else
          vr[i] = kv_load8<NT>(vb, off);
      }
    }
  };

  auto compute = [&](int tile, u32x4_t (&kr)[KS], vrow_t (&vr)[4]) {
    float4_t sc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, kr[j]), qb[j], sc,
                                                   0, 0, 0);
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = sc[i] * cs;
    if ((tile + 1) * kTile > n || tile * kTile < lo) {  // partial tile: non-keys
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tile * kTile + 4 * quad + i;
        if (tok >= n || tok < lo) {
          y[i] = -INFINITY;
          vr[i] = VRow<D>::zero();
        }
      }
    }
    float ym = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
    ym = fmaxf(ym, __shfl_xor(ym, 16));
    ym = fmaxf(ym, __shfl_xor(ym, 32));
    const float m_new = fmaxf(m, ym);
    const float alpha = fast_exp2(m - m_new);
    // exp2 first, then an exact power-of-two scale: the max token weighs
    // exactly 2^15, so a lone token reproduces its V row bit for bit
    float pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pw[i] = col < G ? fast_exp2(y[i] - m_new) * kPScale : 0.f;
    l = fmaf(l, alpha, (pw[0] + pw[1]) + (pw[2] + pw[3]));
    // fp16 hi + lo split of the weights (B operand of P.V)
    const auto h01 = __builtin_amdgcn_cvt_pkrtz(pw[0], pw[1]);
    const auto h23 = __builtin_amdgcn_cvt_pkrtz(pw[2], pw[3]);
    const auto l01 = __builtin_amdgcn_cvt_pkrtz(pw[0] - (float)h01[0], pw[1] - (float)h01[1]);
    const auto l23 = __builtin_amdgcn_cvt_pkrtz(pw[2] - (float)h23[0], pw[3] - (float)h23[1]);
    const half4_t phi = __builtin_bit_cast(
        half4_t, u32x2_t{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)});
    const half4_t plo = __builtin_bit_cast(
        half4_t, u32x2_t{__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)});
    // rescale only when some head's running max moved (alpha == 1 otherwise)
    if (wave_any(alpha != 1.f)) {
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[e] *= alpha;
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      // A operand: tokens 4*quad .. 4*quad+3 of dim (chunk col, half e)
      const int wd = e >> 1;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t d0 = __builtin_amdgcn_perm(vr[1][wd], vr[0][wd], sel);
      const uint32_t d1 = __builtin_amdgcn_perm(vr[3][wd], vr[2][wd], sel);
      const half4_t av = __builtin_bit_cast(half4_t, u32x2_t{d0, d1});
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, phi, acc[e], 0, 0, 0);
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, plo, acc[e], 0, 0, 0);
    }
    m = m_new;
  };

  int tile = tile_begin + w;
  int k_it = 0;
  load_ids(0);
  if constexpr (DEPTH == 1) {
    for (; tile < tile_end; tile += NW, ++k_it) {
      if (k_it > 0 && (k_it & 63) == 0) load_ids(k_it);
      issue(tile, k_it, kA, vA);
      compute(tile, kA, vA);
    }
  } else {
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
  }

  // ---- wave totals, then the NW-wave merge through LDS --------------------
  float lt = l;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
  if (col < G) {
#pragma unroll
    for (int e = 0; e < NE; ++e) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.acc[w][col][VH * (4 * quad + i) + e] = acc[e][i];
    }
    if (quad == 0) {
      sm.m[w][col] = m;
      sm.l[w][col] = lt;
    }
  }
  __syncthreads();
  finish_range<G, D, NW>(sm, sink);
}

template <int D, int BS, int G, int NW, int DEPTH, bool NT>
__global__ __launch_bounds__(NW * 64, DEPTH == 1 ? 4 : 2) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ DecodeSmem<G, D, NW> sm;
  __shared__ int prefix[kBalancedMaxSeqs];
  run_schedule<G, D, NW>(a, prefix, [&](int s, int g, int lo, int n, int ta, int tb,
                                         const Sink& sink) {
    decode_range<D, BS, G, NW, DEPTH, NT>(a, sm, s, g, lo, n, ta, tb, sink);
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
    const void* fn =
        a.variant == 1 ? reinterpret_cast<const void*>(&decode_mfma_kernel<D, BS, G, NW, 1, true>)
                       : reinterpret_cast<const void*>(&decode_mfma_kernel<D, BS, G, NW, 2, true>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, NW * 64, 0) != hipSuccess) return 2;
    *occ = n;
    return 0;
  }
  const unsigned grid = grid_of(a);
  if (grid == 0) return 0;
  const dim3 g(grid), b(NW * 64);
  if (a.variant == 1 && a.cached_kv)
    hipLaunchKernelGGL((decode_mfma_kernel<D, BS, G, NW, 1, false>), g, b, 0, stream, a);
  else if (a.variant == 1)
    hipLaunchKernelGGL((decode_mfma_kernel<D, BS, G, NW, 1, true>), g, b, 0, stream, a);
  else if (a.cached_kv)
    hipLaunchKernelGGL((decode_mfma_kernel<D, BS, G, NW, 2, false>), g, b, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<D, BS, G, NW, 2, true>), g, b, 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

template <int D, int BS, int NW>
int by_group(const DecodeArgs& a, int group, hipStream_t stream, int mode, int* occ) {
  switch (group) {
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

int launch_decode_mfma(const DecodeArgs& a, int dtype, int head_dim, int block_size, int group,
                       int waves, hipStream_t stream) {
  if (dtype != 1 || waves != 4) return 1;
  return dispatch(a, head_dim, block_size, group, stream, 0, nullptr);
}

int decode_mfma_occupancy(const DecodeArgs& a, int head_dim, int block_size, int group) {
  int occ = 0;
  return dispatch(a, head_dim, block_size, group, nullptr, 1, &occ) == 0 ? occ : 0;
}

}  // namespace pa
