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
//    (two permlane swaps, no LDS traffic); everything else stays in the
//    lane.
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
  static __device__ __forceinline__ type zero() { return type{0u, 0u, 0u, 0u}; }
};
template <>
struct VRow<64> {
  using type = u32x2_t;
  static __device__ __forceinline__ type zero() { return type{0u, 0u}; }
};

// One 16-token tile in registers: K as the A operand of q.K (lane (quad,
// col): row col, 16-byte chunks 4j + quad) and four V rows (lane (quad, col):
// row 4*quad + i, chunk col).
template <int D>
struct MfmaTile {
  u32x4_t k[D / 32];
  typename VRow<D>::type v[4];
};

// Issues the loads of one tile.  kb0 / kb1 point at the K rows of the
// (block, KV head) that hold the tile's first / last eight tokens (the same
// block unless BS == 8); the V rows sit v_offset elements further; row0 is
// the tile's first row in its block (BS == 32: 0 or 16).
template <int D, int BS, bool NT>
__device__ __forceinline__ void load_tile(const half_t* kb0, const half_t* kb1, size_t v_offset,
                                          int row0, int quad, int col, MfmaTile<D>& t) {
  constexpr int KS = D / 32;
  constexpr int VH = D / 16;
  if constexpr (BS >= kTile) {
    const half_t* vb = kb0 + v_offset;
    const uint32_t krow = (uint32_t)(row0 + col) * (D * 2);
#pragma unroll
    for (int j = 0; j < KS; ++j) t.k[j] = kv_load16<NT>(kb0, krow + (4 * j + quad) * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = (uint32_t)(row0 + 4 * quad + i) * (D * 2) + col * (VH * 2);
      if constexpr (D == 128)
        t.v[i] = kv_load16<NT>(vb, off);
      else
        t.v[i] = kv_load8<NT>(vb, off);
    }
  } else {
    // a tile spans two 8-row blocks: lanes pick their block
    const half_t* kb = col >= BS ? kb1 : kb0;
    const uint32_t krow = (uint32_t)(col % BS) * (D * 2);
#pragma unroll
    for (int j = 0; j < KS; ++j) t.k[j] = kv_load16<NT>(kb, krow + (4 * j + quad) * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * quad + i;
      const half_t* vb = (r >= BS ? kb1 : kb0) + v_offset;
      const uint32_t off = (uint32_t)(r % BS) * (D * 2) + col * (VH * 2);
      if constexpr (D == 128)
        t.v[i] = kv_load16<NT>(vb, off);
      else
        t.v[i] = kv_load8<NT>(vb, off);
    }
  }
}

// Online-softmax state of one wave: running max m of head `col` (the same in
// all four quads), this lane's share l of the (2^15-scaled) weight sum, and
// O^T blocks acc[e] (lane (quad, col): d = VH*(4*quad + i) + e of head col).
template <int D>
struct MfmaState {
  float m;
  float l;
  float4_t acc[D / 16];
  __device__ __forceinline__ void reset() {
    m = kMaxInit;
    l = 0.f;
#pragma unroll
    for (int e = 0; e < D / 16; ++e) acc[e] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
};

// q of the G heads of (s, g) as the B operand of q.K: lane (quad, col) =
// head col, chunk 4j + quad.  The padding columns col >= G load head col % G
// (every lane loads, so the load count never depends on the lane): their
// scores are finite and get weight zero, so they reach no output.
template <int D, int G>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int s, int g, int quad, int col,
                                       half8_t (&qb)[D / 32]) {
  const half_t* qh = reinterpret_cast<const half_t*>(a.q) +
                     ((size_t)s * a.num_q_heads + g * G + col % G) * D;
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
    qb[j] = __builtin_bit_cast(half8_t, load16(qh + (4 * j + quad) * 8));
}

// Scores, online-softmax update and P.V of one tile (absolute tile index
// `tile` of a sequence whose keys are tokens [lo, n)).
template <int D, int G>
__device__ __forceinline__ void compute_tile(MfmaState<D>& st, const half8_t (&qb)[D / 32],
                                             MfmaTile<D>& t, int tile, int lo, int n, float cs,
                                             int quad, int col) {
  constexpr int KS = D / 32;
  constexpr int NE = D / 16;
  float4_t sc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KS; ++j)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, t.k[j]), qb[j], sc, 0,
                                                 0, 0);
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = sc[i] * cs;
  if ((tile + 1) * kTile > n || tile * kTile < lo) {  // partial tile: non-keys
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tile * kTile + 4 * quad + i;
      if (tok >= n || tok < lo) {
        y[i] = -INFINITY;
        t.v[i] = VRow<D>::zero();
      }
    }
  }
  const float ym = rows4_max(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])));
  const float m_new = fmaxf(st.m, ym);
  const float alpha = fast_exp2(st.m - m_new);
  // exp2 first, then an exact power-of-two scale: the max token weighs
  // exactly 2^15, so a lone token reproduces its V row bit for bit
  float pw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pw[i] = col < G ? fast_exp2(y[i] - m_new) * kPScale : 0.f;
  st.l = fmaf(st.l, alpha, (pw[0] + pw[1]) + (pw[2] + pw[3]));
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
    for (int e = 0; e < NE; ++e) st.acc[e] *= alpha;
  }
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    // A operand: tokens 4*quad .. 4*quad+3 of dim (chunk col, half e)
    const int wd = e >> 1;
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t d0 = __builtin_amdgcn_perm(t.v[1][wd], t.v[0][wd], sel);
    const uint32_t d1 = __builtin_amdgcn_perm(t.v[3][wd], t.v[2][wd], sel);
    const half4_t av = __builtin_bit_cast(half4_t, u32x2_t{d0, d1});
    st.acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, phi, st.acc[e], 0, 0, 0);
    st.acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, plo, st.acc[e], 0, 0, 0);
  }
  st.m = m_new;
}

// DEPTH 2: the next tile's loads are issued before the current tile is
// computed (register double buffer, 2 waves per SIMD).  DEPTH 1: one tile
// per wave in flight and twice the waves per SIMD to hide the latency.
template <int D, int BS, int G, int NW, int DEPTH, bool NT>
__device__ __forceinline__ void decode_range(const DecodeArgs& a, DecodeSmem<G, D, NW>& sm, int s,
                                             int g, int lo, int n, int tile_begin,
                                             int tile_end, const Sink& sink) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(G >= 1 && G <= 16, "group");
  constexpr int VH = D / 16;                 // halves of one V row per lane
  constexpr int NE = VH;                     // P.V blocks of 16 output rows
  constexpr int BPT = BS >= kTile ? 1 : kTile / BS;
  static_assert(BPT <= 2, "a tile spans at most two blocks");

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int quad = lane >> 4;
  const int col = lane & 15;

  half8_t qb[D / 32];
  load_q<D, G>(a, s, g, quad, col, qb);

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

  MfmaState<D> st;
  st.reset();
  const float cs = a.scale_log2;
  MfmaTile<D> tA, tB;

  auto issue = [&](int tile, int k_it, MfmaTile<D>& t) {
    const int sel = k_it & 63;
    const int b0 = readlane(ids[0], sel);
    const int b1 = readlane(ids[BPT - 1], sel);
    const int row0 = BS > kTile ? (tile % (BS / kTile)) * kTile : 0;
    load_tile<D, BS, NT>(kvh + (size_t)b0 * block_stride, kvh + (size_t)b1 * block_stride,
                         v_offset, row0, quad, col, t);
  };

  int tile = tile_begin + w;
  int k_it = 0;
  load_ids(0);
  if constexpr (DEPTH == 1) {
    for (; tile < tile_end; tile += NW, ++k_it) {
      if (k_it > 0 && (k_it & 63) == 0) load_ids(k_it);
      issue(tile, k_it, tA);
      compute_tile<D, G>(st, qb, tA, tile, lo, n, cs, quad, col);
    }
  } else {
    if (tile < tile_end) issue(tile, 0, tA);
    while (tile < tile_end) {
      int nxt = tile + NW;
      if (nxt < tile_end) {
        if (((k_it + 1) & 63) == 0) load_ids(k_it + 1);
        issue(nxt, k_it + 1, tB);
      }
      compute_tile<D, G>(st, qb, tA, tile, lo, n, cs, quad, col);
      tile = nxt;
      ++k_it;
      if (tile >= tile_end) break;
      nxt = tile + NW;
      if (nxt < tile_end) {
        if (((k_it + 1) & 63) == 0) load_ids(k_it + 1);
        issue(nxt, k_it + 1, tA);
      }
      compute_tile<D, G>(st, qb, tB, tile, lo, n, cs, quad, col);
      tile = nxt;
      ++k_it;
    }
  }

  // ---- wave totals, then the NW-wave merge through LDS --------------------
  float lt = st.l;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
  if (col < G) {
#pragma unroll
    for (int e = 0; e < NE; ++e) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.acc[w][col][VH * (4 * quad + i) + e] = st.acc[e][i];
    }
    if (quad == 0) {
      sm.m[w][col] = st.m;
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

// The register double buffer fits three workgroups per CU by its VGPRs;
// two measured faster (sliding-window 70B decode 51 vs 63 us, ragged GQA
// about 1%, the rest unchanged), so its launches reserve enough dynamic LDS
// that a third cannot be resident.  The one-tile variant is not capped.
constexpr int kDoubleBufferWorkgroupsPerCU = 2;
constexpr size_t kLdsPerCU = 160 * 1024;

template <int D, int G, int NW>
size_t lds_reserve(int variant) {
  if (variant == 1) return 0;
  const size_t fixed = sizeof(DecodeSmem<G, D, NW>) + sizeof(int) * kBalancedMaxSeqs;
  const size_t want = kLdsPerCU / (kDoubleBufferWorkgroupsPerCU + 1) + 256;
  return want > fixed ? want - fixed : 0;
}

// mode 0: launch; mode 1: report resident workgroups per CU in *occ
template <int D, int BS, int G, int NW>
int launch_one(const DecodeArgs& a, hipStream_t stream, int mode, int* occ) {
  const size_t dyn = lds_reserve<D, G, NW>(a.variant);
  if (mode == 1) {
    int n = 0;
    const void* fn =
        a.variant == 1 ? reinterpret_cast<const void*>(&decode_mfma_kernel<D, BS, G, NW, 1, true>)
                       : reinterpret_cast<const void*>(&decode_mfma_kernel<D, BS, G, NW, 2, true>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, NW * 64, dyn) != hipSuccess) return 2;
    *occ = n;
    return 0;
  }
  const unsigned grid = grid_of(a);
  if (grid == 0) return 0;
  const dim3 g(grid), b(NW * 64);
  if (a.variant == 1 && a.cached_kv)
    hipLaunchKernelGGL((decode_mfma_kernel<D, BS, G, NW, 1, false>), g, b, dyn, stream, a);
  else if (a.variant == 1)
    hipLaunchKernelGGL((decode_mfma_kernel<D, BS, G, NW, 1, true>), g, b, dyn, stream, a);
  else if (a.cached_kv)
    hipLaunchKernelGGL((decode_mfma_kernel<D, BS, G, NW, 2, false>), g, b, dyn, stream, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<D, BS, G, NW, 2, true>), g, b, dyn, stream, a);
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
