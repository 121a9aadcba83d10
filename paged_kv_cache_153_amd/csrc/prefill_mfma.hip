// prefill_mfma.hip — causal attention of multi-token queries (a prefill chunk)
// over the paged KV cache, on the matrix cores (gfx950, f16).
//
// A chunk of T new tokens per sequence ([KV2P] "KV Cache从原理到实战" §5.4,
// chunked prefill) has its K/V written to the cache first; query i sits at
// position p = n - T + i and attends to the keys t <= p (the causal mask of
// [INFRA] "大模型 (LLM) 推理加速核心技术解析" §2, aligned to the end of the
// context).  Addressing is the paged one of the decode ([KVPA] "KV Cache与
// PagedAttention深度解析" §4.3): token t is row t % BS of block
// block_tables[s, t / BS].
//
// With T tokens the product q K^T is a real [T*G x D] x [D x 16] contraction
// per 16-key tile, so the 16 MFMA columns of one wave are 16 (query token,
// head) pairs of one KV head: column c is token c / G of the wave's block and
// head c % G of the group.  Each wave owns its columns outright: it walks the
// key tiles from 0 to the last one its latest token may see, keeps an online
// softmax per column, and writes its outputs itself (no cross-wave merge).
// The tile flow is the decode's matrix-core flow (decode_mfma.hip): K rows
// are the A operand of v_mfma_f32_16x16x32_f16, whose C layout is the B
// layout of v_mfma_f32_16x16x16f16 for P^T, and the weights go in as fp16
// hi + lo parts scaled by 2^15.  Block ids are read with scalar loads, and
// the next tile's loads are issued before the current one is computed, on
// every step (look-ahead past the end re-reads the last tile), so the
// compiler's wait counts keep them in flight.
#include "device_common.h"
#include "kernels.h"

namespace pa {
namespace {

constexpr float kPScale = 32768.f;  // 2^15
constexpr int kPrefillWaves = 4;    // waves (column blocks) per workgroup

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

template <int D, int BS, int G, int DEPTH, bool NT>
__global__ __launch_bounds__(kPrefillWaves * 64, 2) void prefill_mfma_kernel(PrefillArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int KS = D / 32;          // 16x16x32 steps for q.K
  constexpr int VH = D / 16;          // halves of one V row per lane
  constexpr int NE = VH;              // P.V blocks of 16 output rows
  constexpr int TPB = 16 / G;         // query tokens per column block
  constexpr int BPT = BS >= kTile ? 1 : kTile / BS;
  static_assert(BPT <= 2, "a tile spans at most two blocks");
  using vrow_t = typename VRow<D>::type;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int quad = lane >> 4;
  const int col = lane & 15;

  // ---- which sequence, KV head and column block ---------------------------
  int bid = blockIdx.x;
  const int g = bid % a.num_kv_heads;
  bid /= a.num_kv_heads;
  const int qb = bid % a.qblocks;
  const int s = bid / a.qblocks;
  const int q0 = a.qstart[s];
  const int T = a.qstart[s + 1] - q0;
  int n = a.cl[s];
  n = n < 0 ? 0 : (n > a.max_tokens ? a.max_tokens : n);
  const int cb = qb * kPrefillWaves + w;  // column block within the sequence
  const int i_first = cb * TPB;
  if (T <= 0 || T > n || i_first >= T) return;  // nothing for this wave
  const int i_last = min(T - 1, i_first + TPB - 1);
  const int tok = i_first + col / G;          // this lane's column: token, head
  const int hh = col % G;
  const bool col_valid = tok < T;
  // last key each column sees (-1 for columns past the chunk: they see none)
  const int p_col = col_valid ? n - T + tok : -1;
  const int p_max = n - T + i_last;           // wave-uniform
  const int p_min = i_first + TPB - 1 < T ? n - T + i_first : -1;
  const int tile_end = p_max / kTile + 1;

  // ---- q as the B operand: lane (quad, col) = column col, chunk 4j + quad ---
  half8_t qb_op[KS];
  {
    const half_t* qh =
        reinterpret_cast<const half_t*>(a.q) +
        ((size_t)(q0 + (col_valid ? tok : 0)) * a.num_q_heads + g * G + hh) * D;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      if (col_valid)
        qb_op[j] = __builtin_bit_cast(half8_t, load16(qh + (4 * j + quad) * 8));
      else
        qb_op[j] = __builtin_bit_cast(half8_t, u32x4_t{0u, 0u, 0u, 0u});
    }
  }

  const size_t head_stride = (size_t)BS * D;
  const size_t block_stride = 2 * (size_t)a.num_kv_heads * head_stride;
  const size_t v_offset = (size_t)a.num_kv_heads * head_stride;
  const half_t* kvh = reinterpret_cast<const half_t*>(a.kv) + (size_t)g * head_stride;
  const int32_t* bt_row = a.bt + (size_t)s * a.max_blocks;

  auto fetch_ids = [&](int tile, int (&out)[BPT]) {
    if (tile >= tile_end) tile = tile_end - 1;
#pragma unroll
    for (int jj = 0; jj < BPT; ++jj) {
      const int lb = BS >= kTile ? tile * kTile / BS : tile * BPT + jj;
      const int v = lb < a.max_blocks ? load_uniform(bt_row + lb) : 0;
      out[jj] = (v < 0 || v >= a.num_blocks) ? 0 : v;
    }
  };

  struct Buf {
    u32x4_t k[KS];
    vrow_t v[4];
  };
  Buf buf[DEPTH];

  auto issue = [&](int tile, const int (&blk)[BPT], Buf& b) {
    if (tile >= tile_end) tile = tile_end - 1;  // look-ahead past the range
    const int row0 = BS > kTile ? (tile % (BS / kTile)) * kTile : 0;
    const int kb_id = BPT == 1 ? blk[0] : (col >= BS ? blk[BPT - 1] : blk[0]);
    const half_t* kb = kvh + (size_t)kb_id * block_stride;
    const uint32_t krow = (uint32_t)(BPT == 1 ? row0 + col : col % BS) * (D * 2);
#pragma unroll
    for (int j = 0; j < KS; ++j) b.k[j] = kv_load16<NT>(kb, krow + (4 * j + quad) * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * quad + i;
      const int vb_id = BPT == 1 ? blk[0] : (t >= BS ? blk[BPT - 1] : blk[0]);
      const half_t* vb = kvh + (size_t)vb_id * block_stride + v_offset;
      const uint32_t off =
          (uint32_t)(BPT == 1 ? row0 + t : t % BS) * (D * 2) + col * (VH * 2);
      if constexpr (D == 128)
        b.v[i] = kv_load16<NT>(vb, off);
      else
        b.v[i] = kv_load8<NT>(vb, off);
    }
  };

  float m = kMaxInit;  // running max of column `col` (same in all four quads)
  float l = 0.f;
  float4_t acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = float4_t{0.f, 0.f, 0.f, 0.f};
  const float cs = a.scale_log2;

  auto compute = [&](int tile, Buf& b) {
    float4_t sc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, b.k[j]), qb_op[j],
                                                   sc, 0, 0, 0);
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = sc[i] * cs;
    if ((tile + 1) * kTile - 1 > p_min || (tile + 1) * kTile > n) {
      // the causal edge (or the end of the context) crosses this tile
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tile * kTile + 4 * quad + i;
        if (t > p_col) y[i] = -INFINITY;
        if (t >= n) b.v[i] = VRow<D>::zero();  // rows past the context: never weighed
      }
    }
    float ym = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
    ym = fmaxf(ym, __shfl_xor(ym, 16));
    ym = fmaxf(ym, __shfl_xor(ym, 32));
    const float m_new = fmaxf(m, ym);
    const float alpha = fast_exp2(m - m_new);
    float pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pw[i] = fast_exp2(y[i] - m_new) * kPScale;
    l = fmaf(l, alpha, (pw[0] + pw[1]) + (pw[2] + pw[3]));
    const auto h01 = __builtin_amdgcn_cvt_pkrtz(pw[0], pw[1]);
    const auto h23 = __builtin_amdgcn_cvt_pkrtz(pw[2], pw[3]);
    const auto l01 = __builtin_amdgcn_cvt_pkrtz(pw[0] - (float)h01[0], pw[1] - (float)h01[1]);
    const auto l23 = __builtin_amdgcn_cvt_pkrtz(pw[2] - (float)h23[0], pw[3] - (float)h23[1]);
    const half4_t phi = __builtin_bit_cast(
        half4_t, u32x2_t{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)});
    const half4_t plo = __builtin_bit_cast(
        half4_t, u32x2_t{__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)});
    if (wave_any(alpha != 1.f)) {
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[e] *= alpha;
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int wd = e >> 1;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t d0 = __builtin_amdgcn_perm(b.v[1][wd], b.v[0][wd], sel);
      const uint32_t d1 = __builtin_amdgcn_perm(b.v[3][wd], b.v[2][wd], sel);
      const half4_t av = __builtin_bit_cast(half4_t, u32x2_t{d0, d1});
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, phi, acc[e], 0, 0, 0);
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, plo, acc[e], 0, 0, 0);
    }
    m = m_new;
  };

  // ---- key tiles 0 .. tile_end - 1, DEPTH - 1 tiles in flight ahead ---------
  {
    int nb[BPT];
#pragma unroll
    for (int k = 0; k < DEPTH - 1; ++k) {
      fetch_ids(k, nb);
      issue(k, nb, buf[k]);
    }
    fetch_ids(DEPTH - 1, nb);
    int tile = 0;
    while (tile < tile_end) {
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) {
        int cur[BPT];
#pragma unroll
        for (int jj = 0; jj < BPT; ++jj) cur[jj] = nb[jj];
        issue(tile + DEPTH - 1, cur, buf[(k + DEPTH - 1) % DEPTH]);
        fetch_ids(tile + DEPTH, nb);
        compute(tile, buf[k]);
        ++tile;
        if (tile >= tile_end) break;
      }
    }
  }

  // ---- normalise and store: lane (quad, col) holds rows d = VH*(4 quad + i) + e
  float lt = l;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
  if (col_valid) {
    const float inv = 1.f / lt;
    float* o = a.out + ((size_t)(q0 + tok) * a.num_q_heads + g * G + hh) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < NE; ++e) o[VH * (4 * quad + i) + e] = acc[e][i] * inv;
    }
  }
}

template <int D, int BS, int G, int DEPTH>
int launch_depth(const PrefillArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)((size_t)a.num_seqs * a.qblocks * a.num_kv_heads);
  if (grid == 0) return 0;
  if (a.cached_kv)
    hipLaunchKernelGGL((prefill_mfma_kernel<D, BS, G, DEPTH, false>), dim3(grid),
                       dim3(kPrefillWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<D, BS, G, DEPTH, true>), dim3(grid),
                       dim3(kPrefillWaves * 64), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

template <int D, int BS, int G>
int launch_one(const PrefillArgs& a, hipStream_t stream) {
  switch (a.variant) {
    case 1: return launch_depth<D, BS, G, 2>(a, stream);
    case 2: return launch_depth<D, BS, G, 4>(a, stream);
    default: return launch_depth<D, BS, G, 3>(a, stream);
  }
}

template <int D, int BS>
int by_group(const PrefillArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_one<D, BS, 1>(a, stream);
    case 2: return launch_one<D, BS, 2>(a, stream);
    case 4: return launch_one<D, BS, 4>(a, stream);
    case 8: return launch_one<D, BS, 8>(a, stream);
  }
  return 1;
}

template <int D>
int by_block(const PrefillArgs& a, int block_size, int group, hipStream_t stream) {
  switch (block_size) {
    case 8: return by_group<D, 8>(a, group, stream);
    case 16: return by_group<D, 16>(a, group, stream);
    case 32: return by_group<D, 32>(a, group, stream);
  }
  return 1;
}

}  // namespace

int prefill_columns_per_workgroup() { return kPrefillWaves * 16; }

int launch_prefill_mfma(const PrefillArgs& a, int head_dim, int block_size, int group,
                        hipStream_t stream) {
  if (head_dim == 64) return by_block<64>(a, block_size, group, stream);
  if (head_dim == 128) return by_block<128>(a, block_size, group, stream);
  return 1;
}

}  // namespace pa
