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
#include "kernels.h"

namespace pa {
namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// bf16(a) | bf16(b) << 16, rounded to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, bf16x2_t));
}

// Four signed codes (one dword) -> two half2 words holding them exactly.
__device__ __forceinline__ void codes_to_half(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x80808080u;  // code + 128, as unsigned bytes
  // half bits 0x64uu = 1024 + uu; bytes 4..7 of the pair are the 0x64s
  const uint32_t l16 = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t h16 = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const half2_t bias = {(half_t)1152.f, (half_t)1152.f};
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, l16) - bias);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, h16) - bias);
}

// High 16 bits of two floats packed: bf16(a) | bf16(b) << 16 by truncation,
// exact for floats with at most 8 significant bits such as the codes.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a),
                               0x07060302u);
}

template <int K>
__device__ __forceinline__ float byte_f32(uint32_t w) {
  return (float)((int32_t)(w << (24 - 8 * K)) >> 24);
}

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
  const int w = threadIdx.x >> 6;
  const int quad = lane >> 4;
  const int col = lane & 15;
  const int Hq = a.num_q_heads;

  // ---- q as the B operand: lane (quad, col) = head col, d = quad*D/4 + 8j + e
  half8_t qb[KS];
  {
    const half_t* qh = reinterpret_cast<const half_t*>(a.q) + ((size_t)s * Hq + g * G) * D;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      if (col < G)
        qb[j] = __builtin_bit_cast(half8_t, load16(qh + col * D + quad * (D / 4) + 8 * j));
      else
        qb[j] = __builtin_bit_cast(half8_t, u32x4_t{0u, 0u, 0u, 0u});
    }
  }

  const size_t head_stride = (size_t)BS * D;  // bytes
  const size_t block_stride = 2 * (size_t)a.num_kv_heads * head_stride;
  const size_t v_offset = (size_t)a.num_kv_heads * head_stride;
  const int8_t* kvh = reinterpret_cast<const int8_t*>(a.kv) + (size_t)g * head_stride;
  const size_t sblock_stride = 2 * (size_t)a.num_kv_heads * BS;  // floats
  const size_t sv_offset = (size_t)a.num_kv_heads * BS;
  const float* sch = a.kv_scales + (size_t)g * BS;
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

  float m = kMaxInit;  // running max of head `col` (same in all four quads)
  float l = 0.f;       // this lane's share of the weight sum
  float4_t acc[VB];
#pragma unroll
  for (int e = 0; e < VB; ++e) acc[e] = float4_t{0.f, 0.f, 0.f, 0.f};
  const float cs = a.scale_log2;

  struct Buf {
    u32x4_t k[KL];     // codes of K row `col`, bytes quad*D/4 ..
    vchunk_t v[4];     // codes of V rows 4*quad + i, bytes col*VB ..
    u32x4_t sk, sv;    // scales of tokens 4*quad .. 4*quad + 3
  };
  Buf bA, bB;

  auto issue = [&](int tile, int k_it, Buf& b) {
    const int sel = k_it & 63;
    int blk[BPT];
#pragma unroll
    for (int jj = 0; jj < BPT; ++jj) blk[jj] = readlane(ids[jj], sel);
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
    b.sk = kv_load16<NT>(sb, (uint32_t)vrow * 4u);
    b.sv = kv_load16<NT>(sb + sv_offset, (uint32_t)vrow * 4u);
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
    // whole-vector casts: this compiler miscompiles a bit_cast of a single
    // vector element (it reads element 0)
    const float4_t skf = __builtin_bit_cast(float4_t, b.sk);
    const float4_t svf = __builtin_bit_cast(float4_t, b.sv);
    float y[4], svt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[i] = sc[i] * (skf[i] * cs);
      svt[i] = svf[i];
    }
    if ((tile + 1) * kTile > n || tile * kTile < lo) {  // partial tile: non-keys
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tile * kTile + 4 * quad + i;
        if (tok >= n || tok < lo) {
          y[i] = -INFINITY;
          b.v[i] = VChunk<D>::zero();
          svt[i] = 0.f;
        }
      }
    }
    float ym = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
    ym = fmaxf(ym, __shfl_xor(ym, 16));
    ym = fmaxf(ym, __shfl_xor(ym, 32));
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

  int tile = tile_begin + w;
  int k_it = 0;
  load_ids(0);
  if constexpr (DEPTH == 1) {
    for (; tile < tile_end; tile += NW, ++k_it) {
      if (k_it > 0 && (k_it & 63) == 0) load_ids(k_it);
      issue(tile, k_it, bA);
      compute(tile, bA);
    }
  } else {
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

template <int D, int BS, int G, int NW, int DEPTH, bool NT>
__global__ __launch_bounds__(NW * 64, DEPTH == 1 ? 4 : 2) void decode_mfma_i8_kernel(
    DecodeArgs a) {
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

template <int D, int BS, int G, int NW>
int launch_one(const DecodeArgs& a, hipStream_t stream, int mode, int* occ) {
  if (mode == 1) {
    int n = 0;
    const void* fn =
        a.variant == 1
            ? reinterpret_cast<const void*>(&decode_mfma_i8_kernel<D, BS, G, NW, 1, true>)
            : reinterpret_cast<const void*>(&decode_mfma_i8_kernel<D, BS, G, NW, 2, true>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, NW * 64, 0) != hipSuccess) return 2;
    *occ = n;
    return 0;
  }
  const unsigned grid = grid_of(a);
  if (grid == 0) return 0;
  const dim3 g(grid), b(NW * 64);
  if (a.variant == 1 && a.cached_kv)
    hipLaunchKernelGGL((decode_mfma_i8_kernel<D, BS, G, NW, 1, false>), g, b, 0, stream, a);
  else if (a.variant == 1)
    hipLaunchKernelGGL((decode_mfma_i8_kernel<D, BS, G, NW, 1, true>), g, b, 0, stream, a);
  else if (a.cached_kv)
    hipLaunchKernelGGL((decode_mfma_i8_kernel<D, BS, G, NW, 2, false>), g, b, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_mfma_i8_kernel<D, BS, G, NW, 2, true>), g, b, 0, stream, a);
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

int launch_decode_mfma_i8(const DecodeArgs& a, int head_dim, int block_size, int group,
                          hipStream_t stream) {
  return dispatch(a, head_dim, block_size, group, stream, 0, nullptr);
}

int decode_mfma_i8_occupancy(const DecodeArgs& a, int head_dim, int block_size, int group) {
  int occ = 0;
  return dispatch(a, head_dim, block_size, group, nullptr, 1, &occ) == 0 ? occ : 0;
}

}  // namespace pa
