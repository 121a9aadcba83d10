// decode_mfma_i8.hip — paged decode attention over an INT8 KV cache on the
// matrix cores (gfx950), for grouped-query heads.
//
// The cache holds int8 codes with one float32 scale per (token, KV head) row
// of K and of V ([KV2P] "KV Cache从原理到实战" §5.2; [KV2P] §5.3 for the
// query groups).  Attention over the dequantised values ([KVPA] "KV
// Cache与PagedAttention深度解析" §2.1, §4.3, §7.2) is computed as
//   score_t = scale * sk_t * (q . Kq_t),   out = sum_t (p_t sv_t) Vq_t / sum_t p_t.
//
// Same work decomposition and tile flow as decode_mfma.hip; what changes:
//  * q.K^T: v_mfma_f32_16x16x32_f16 with the codes widened to fp16 exactly
//    (byte -> 1024 + u via v_perm, then one packed subtract).  The
//    contraction index is relabelled so that each lane's codes of a K row
//    are contiguous: step j, lane group quad, element e <-> d = quad*D/4 +
//    8j + e (q is loaded with the same map).  A lane reads D/4 contiguous
//    bytes of its row (two 16-byte loads at D = 128).
//  * The row scale of K multiplies the score; that of V multiplies the
//    softmax weight, so P.V runs on the codes themselves: V^T (codes widened
//    to bf16, exact for |code| <= 127) times P^T in bf16 hi + lo parts, each
//    rounded to nearest with v_cvt_pk_bf16_f32 (v_mfma_f32_16x16x16_bf16;
//    about 16 significant bits of each weight).
//    bf16's 8-bit exponent takes any weight * scale without the overflow an
//    fp16 weight would risk.
//  * The sum l keeps the weights without the V scales, in fp32.
#include "decode_epilogue.h"
#include "decode_schedule.h"
#include "device_common.h"
#include "i8_codes.h"
#include "kernels.h"

namespace pa {
namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));

template <int D>
struct VChunk;  // a lane's codes of one V row: 8 bytes (D = 128) or 4 (D = 64)
template <>
struct VChunk<128> {
  using type = u32x2_t;
  template <bool NT>
  static __device__ __forceinline__ type load(const void* base, uint32_t off) {
    return kv_load8<NT>(base, off);
  }
  static __device__ __forceinline__ type zero() { return type{0u, 0u}; }
  static __device__ __forceinline__ uint32_t word(const type& v, int i) { return v[i]; }
};
template <>
struct VChunk<64> {
  using type = uint32_t;
  template <bool NT>
  static __device__ __forceinline__ type load(const void* base, uint32_t off) {
    const uint32_t* p =
        reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(base) + off);
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
  }
  static __device__ __forceinline__ type zero() { return 0u; }
  static __device__ __forceinline__ uint32_t word(const type& v, int) { return v; }
};

template <int D>
struct KChunk;  // a lane's D/4 codes of one K row: 32 bytes (D = 128) or 16 (D = 64)
template <>
struct KChunk<128> {
  static constexpr int kLoads = 2;
};
template <>
struct KChunk<64> {
  static constexpr int kLoads = 1;
};

template <int D, int BS, int G, int NW, int DEPTH, bool NT>
__device__ __forceinline__ void decode_range(const DecodeArgs& a, DecodeSmem<G, D, NW>& sm, int s,
                                             int g, int lo, int n, int tile_begin, int tile_end,
                                             const Sink& sink) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int KS = D / 32;   // 16x16x32 steps for q.K
  constexpr int KL = KChunk<D>::kLoads;
  constexpr int VB = D / 16;   // codes of one V row per lane = P.V blocks
  constexpr int BPT = BS >= kTile ? 1 : kTile / BS;
  static_assert(BPT <= 2, "a tile spans at most two blocks");
  using vchunk_t = typename VChunk<D>::type;

  const int lane = threadIdx.x & 63;
  // the wave index is uniform: keeping it scalar keeps tile indices and
  // block-table reads scalar
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int quad = lane >> 4;
  const int col = lane & 15;
  const int Hq = a.num_q_heads;

  // ---- q as the B operand: lane (quad, col) = head col, d = quad*D/4 + 8j + e
  // (padding columns col >= G load head col % G: finite scores, zero weight)
  half8_t qb[KS];
  {
    const half_t* qh =
        reinterpret_cast<const half_t*>(a.q) + ((size_t)s * Hq + g * G + col % G) * D;
#pragma unroll
    for (int j = 0; j < KS; ++j)
      qb[j] = __builtin_bit_cast(half8_t, load16(qh + quad * (D / 4) + 8 * j));
  }

  const size_t head_stride = (size_t)BS * D;  // bytes
  const size_t block_stride = 2 * (size_t)a.num_kv_heads * head_stride;
  const size_t v_offset = (size_t)a.num_kv_heads * head_stride;
  const int8_t* kvh = reinterpret_cast<const int8_t*>(a.kv) + (size_t)g * head_stride;
  const size_t sblock_stride = 2 * (size_t)a.num_kv_heads * BS;  // floats
  const size_t sv_offset = BS;  // scales [NB, Hkv, 2, BS]: K then V of one head, one line
  const float* sch = a.kv_scales + (size_t)g * 2 * BS;
  const int32_t* bt_row = a.bt + (size_t)s * a.max_blocks;

  // Block ids are read with scalar loads one step before the tile's loads
  // are issued.  Look-ahead loads past the range re-read its last tile, so
  // every step issues the same vector loads and the compiler's wait counts
  // stay exact (a conditional load would force it to wait for all of them).
  auto fetch_ids = [&](int tile, int (&out)[BPT]) {
    if (tile >= tile_end) tile = tile_end - 1;
#pragma unroll
    for (int jj = 0; jj < BPT; ++jj) {
      const int lb = BS >= kTile ? tile * kTile / BS : tile * BPT + jj;
      const int v = lb < a.max_blocks ? load_uniform(bt_row + lb) : 0;
      out[jj] = (v < 0 || v >= a.num_blocks) ? 0 : v;
    }
  };

  float m = kMaxInit;  // running max of head `col` (same in all four quads)
  float l = 0.f;       // this lane's share of the weight sum
  float4_t acc[VB];
#pragma unroll
  for (int e = 0; e < VB; ++e) acc[e] = float4_t{0.f, 0.f, 0.f, 0.f};
  const float cs = a.scale_log2;

  struct Buf {
    u32x4_t k[KL];     // codes of K row `col`, bytes quad*D/4 ..
    vchunk_t v[4];     // codes of V rows 4*quad + i, bytes col*VB ..
    float sk, sv;      // scales of token 4*quad + (col & 3)
  };
  Buf buf[DEPTH];

  auto issue = [&](int tile, const int (&blk)[BPT], Buf& b) {
    if (tile >= tile_end) tile = tile_end - 1;  // look-ahead past the range
    const int row0 = BS > kTile ? (tile % (BS / kTile)) * kTile : 0;
    // K row `col`; V rows and scales of tokens 4*quad ..; blocks per lane
    // when a tile spans two 8-row blocks
    const int kb_id = BPT == 1 ? blk[0] : (col >= BS ? blk[BPT - 1] : blk[0]);
    const int vb_id = BPT == 1 ? blk[0] : (4 * quad >= BS ? blk[BPT - 1] : blk[0]);
    const int8_t* kb = kvh + (size_t)kb_id * block_stride;
    const int8_t* vb = kvh + (size_t)vb_id * block_stride + v_offset;
    const float* sb = sch + (size_t)vb_id * sblock_stride;
    const int krow = BPT == 1 ? row0 + col : col % BS;
    const int vrow = BPT == 1 ? row0 + 4 * quad : (4 * quad) % BS;
#pragma unroll
    for (int x = 0; x < KL; ++x)
      b.k[x] = kv_load16<NT>(kb, (uint32_t)(krow * D + quad * (D / 4) + 16 * x));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      b.v[i] = VChunk<D>::template load<NT>(vb, (uint32_t)((vrow + i) * D + col * VB));
    // one scale per lane: lanes 4k .. 4k+3 of a quad hold its four tokens
    const uint32_t soff = (uint32_t)(vrow + (col & 3)) * 4u;
    b.sk = __builtin_bit_cast(float, kv_load4<NT>(sb, soff));
    b.sv = __builtin_bit_cast(float, kv_load4<NT>(sb + sv_offset, soff));
  };

  auto compute = [&](int tile, Buf& b) {
    float4_t sc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < KL; ++x) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {  // 16 codes = two 8-element steps
        uint32_t h[4];
        codes_to_half(b.k[x][2 * jj], h[0], h[1]);
        codes_to_half(b.k[x][2 * jj + 1], h[2], h[3]);
        const half8_t ka = __builtin_bit_cast(half8_t, u32x4_t{h[0], h[1], h[2], h[3]});
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[2 * x + jj], sc, 0, 0, 0);
      }
    }
    // token 4*quad + i's scales come from lane i of each group of four
    // (quad_perm broadcast, fused into the multiply where it can be)
    const float skc = b.sk * cs;
    float y[4], svt[4];
    y[0] = sc[0] * quad_bcast<0>(skc);
    y[1] = sc[1] * quad_bcast<1>(skc);
    y[2] = sc[2] * quad_bcast<2>(skc);
    y[3] = sc[3] * quad_bcast<3>(skc);
    svt[0] = quad_bcast<0>(b.sv);
    svt[1] = quad_bcast<1>(b.sv);
    svt[2] = quad_bcast<2>(b.sv);
    svt[3] = quad_bcast<3>(b.sv);
    if ((tile + 1) * kTile > n || tile * kTile < lo) {  // partial tile: non-keys
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tile * kTile + 4 * quad + i;
        if (tok >= n || tok < lo) {  // codes are finite: a zero weight suffices
          y[i] = -INFINITY;
          svt[i] = 0.f;
        }
      }
    }
    // max across the four lane rows by permlane swaps: no LDS round trip, so
    // no wait on the scalar block-id loads in flight
    const float ym = rows4_max(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])));
    const float m_new = fmaxf(m, ym);
    const float alpha = fast_exp2(m - m_new);
    float pw[4], pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = col < G ? fast_exp2(y[i] - m_new) : 0.f;
      pv[i] = pw[i] * svt[i];
    }
    l = fmaf(l, alpha, (pw[0] + pw[1]) + (pw[2] + pw[3]));
    // bf16 hi + lo parts of the scaled weights (B operand of P.V)
    const uint32_t h01 = pack_bf16_rne(pv[0], pv[1]);
    const uint32_t h23 = pack_bf16_rne(pv[2], pv[3]);
    const uint32_t l01 =
        pack_bf16_rne(pv[0] - __builtin_bit_cast(float, h01 << 16),
                      pv[1] - __builtin_bit_cast(float, h01 & 0xFFFF0000u));
    const uint32_t l23 =
        pack_bf16_rne(pv[2] - __builtin_bit_cast(float, h23 << 16),
                      pv[3] - __builtin_bit_cast(float, h23 & 0xFFFF0000u));
    const short4_t phi = __builtin_bit_cast(short4_t, u32x2_t{h01, h23});
    const short4_t plo = __builtin_bit_cast(short4_t, u32x2_t{l01, l23});
    if (wave_any(alpha != 1.f)) {
#pragma unroll
      for (int e = 0; e < VB; ++e) acc[e] *= alpha;
    }
#pragma unroll
    for (int e = 0; e < VB; ++e) {
      // A operand: tokens 4*quad .. 4*quad+3 at d = VB*col + e, as bf16
      const int wd = e >> 2;
      float f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t word = VChunk<D>::word(b.v[i], wd);
        switch (e & 3) {
          case 0: f[i] = byte_f32<0>(word); break;
          case 1: f[i] = byte_f32<1>(word); break;
          case 2: f[i] = byte_f32<2>(word); break;
          default: f[i] = byte_f32<3>(word); break;
        }
      }
      const short4_t av =
          __builtin_bit_cast(short4_t, u32x2_t{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3])});
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, phi, acc[e], 0, 0, 0);
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, plo, acc[e], 0, 0, 0);
    }
    m = m_new;
  };

  // ---- main loop: DEPTH - 1 tiles in flight ahead of the one computed ------
  // buf[k] of an unrolled round of DEPTH steps holds the tile computed at
  // step k; each step first refills the buffer the previous step freed.
  int tile = tile_begin + w;
  if (tile < tile_end) {
    int nb[BPT];
#pragma unroll
    for (int k = 0; k < DEPTH - 1; ++k) {
      fetch_ids(tile + k * NW, nb);
      issue(tile + k * NW, nb, buf[k]);
    }
    fetch_ids(tile + (DEPTH - 1) * NW, nb);
    while (tile < tile_end) {
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) {
        const int ahead = tile + (DEPTH - 1) * NW;
        int cur[BPT];
#pragma unroll
        for (int jj = 0; jj < BPT; ++jj) cur[jj] = nb[jj];
        issue(ahead, cur, buf[(k + DEPTH - 1) % DEPTH]);
        fetch_ids(ahead + NW, nb);  // for the next step
        compute(tile, buf[k]);
        tile += NW;
        if (tile >= tile_end) break;
      }
    }
  }

  // ---- wave totals, then the NW-wave merge through LDS --------------------
  float lt = l;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
  if (col < G) {
#pragma unroll
    for (int e = 0; e < VB; ++e) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.acc[w][col][VB * (4 * quad + i) + e] = acc[e][i];
    }
    if (quad == 0) {
      sm.m[w][col] = m;
      sm.l[w][col] = lt;
    }
  }
  __syncthreads();
  finish_range<G, D, NW>(sm, sink);
}

template <int D, int BS, int G, int NW, int DEPTH, int OCC, bool NT>
__global__ __launch_bounds__(NW * 64, OCC) void decode_mfma_i8_kernel(DecodeArgs a) {
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

// Pipeline depth and waves per SIMD of each variant: 0 = one tile in flight
// ahead of the computed one at four waves per SIMD (streaming K/V; measured
// best: 70B-shaped layer 202 us, ragged GQA batch 118 us, against 203 / 128
// for two tiles ahead at three waves); 1 = no look-ahead at four waves
// (cached K/V); 2 = two tiles ahead at three waves (kept for tuning runs).
template <int D, int BS, int G, int NW, int DEPTH, int OCC>
int launch_variant(const DecodeArgs& a, hipStream_t stream, int mode, int* occ) {
  if (mode == 1) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&decode_mfma_i8_kernel<D, BS, G, NW, DEPTH, OCC, true>),
            NW * 64, 0) != hipSuccess)
      return 2;
    *occ = n;
    return 0;
  }
  const unsigned grid = grid_of(a);
  if (grid == 0) return 0;
  if (a.cached_kv)
    hipLaunchKernelGGL((decode_mfma_i8_kernel<D, BS, G, NW, DEPTH, OCC, false>), dim3(grid),
                       dim3(NW * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_mfma_i8_kernel<D, BS, G, NW, DEPTH, OCC, true>), dim3(grid),
                       dim3(NW * 64), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

template <int D, int BS, int G, int NW>
int launch_one(const DecodeArgs& a, hipStream_t stream, int mode, int* occ) {
  switch (a.variant) {
    case 1: return launch_variant<D, BS, G, NW, 1, 4>(a, stream, mode, occ);
    case 2: return launch_variant<D, BS, G, NW, 3, 3>(a, stream, mode, occ);
    // 8-row blocks need per-lane block addresses: more registers, three waves
    default: return launch_variant<D, BS, G, NW, 2, BS == 8 ? 3 : 4>(a, stream, mode, occ);
  }
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

int launch_decode_mfma_i8(const DecodeArgs& a, int head_dim, int block_size, int group,
                          hipStream_t stream) {
  return dispatch(a, head_dim, block_size, group, stream, 0, nullptr);
}

int decode_mfma_i8_occupancy(const DecodeArgs& a, int head_dim, int block_size, int group) {
  int occ = 0;
  return dispatch(a, head_dim, block_size, group, nullptr, 1, &occ) == 0 ? occ : 0;
}

}  // namespace pa
