// prefill_mfma.hip — causal attention of multi-token queries (a prefill chunk)
// over the paged KV cache, on the matrix cores (gfx950, f16).
//
// A chunk of T new tokens per sequence ([KV2P] "KV Cache从原理到实战" §5.4,
// chunked prefill) has its K/V written to the cache first; query i sits at
// position p = n - T + i and attends to the keys t <= p (the causal mask of
// [INFRA] "大模型 (LLM) 推理加速核心技术解析" §2, aligned to the end of the
// context); under a sliding window of W tokens ([KV2P] §7.2) only to
// p - W < t <= p.  Addressing is the paged one of the decode ([KVPA] "KV
// Cache与PagedAttention深度解析" §4.3): token t is row t % BS of block
// block_tables[s, t / BS].
//
// Columns are (query token, head) pairs of one KV head, head fastest; a wave
// owns CB = 2 blocks of 16 columns and a workgroup of four waves 128 columns
// of one (sequence, KV head).  The workgroup walks the keys in steps of 32:
// each step's K and V rows (32 x 2D bytes each) arrive by direct global->LDS
// loads (16 bytes per lane, no registers; block ids from scalar loads),
// issued three steps ahead into four LDS buffers, and every wave takes its
// matrix operands from there — the prefill reads each K/V row from L2 once
// per workgroup, not once per wave.  Per step and column block:
//   S^T = K q^T  two 16-key tiles x D/32 v_mfma_f32_16x16x32_f16 (K rows are
//                the A operand, q the B operand);
//   online softmax per column in log2 units, the causal mask only on steps
//                that cross the diagonal or the end of the context; the
//                reference value moves only when a score passes it by more
//                than 2^8, so most steps need no cross-lane max or rescale;
//   O^T += V^T P^T  one v_mfma_f32_16x16x32_f16 per 16 output rows and per
//                weight part: the C layout of the two S tiles gives each lane
//                keys 4q..4q+3 of both tiles, which is the B layout of a
//                32-deep contraction once the contraction index is relabelled
//                (k = 8q + j  ->  key 4q + j of tile j / 4); V is read with
//                the same relabelling, and the weights go in as fp16 hi + lo
//                parts, which keeps ~21 bits of each weight;
//   the weight sums as one more block whose V rows are all ones.
// q.K of step st + 1 is issued between the max and the exponentials of step
// st, so the matrix cores have work while the vector ALUs do the softmax;
// the softmax runs at raised wave priority (s_setprio) so that it overlaps
// the other wave's matrix products.
// LDS rows are 2D bytes.  K rows have their 16-byte chunks XOR-swizzled by
// the row, so that the 16 lanes that read one chunk of 16 different K rows
// hit distinct banks; V rows are plain, since the lanes of a quad read one V
// row whole (measured: an XOR swizzle by row there costs a two-way conflict).
#include "prefill_common.h"

#include <type_traits>

namespace pa {
namespace {

using prefill::kAhead;
using prefill::kBufs;
using prefill::kKeys;
using prefill::kPLog;
using prefill::kSlack;
using prefill::kWaves;
using prefill::tile_off;

template <int D, int BS, int G>
__global__ __launch_bounds__(kWaves * 64, 2) void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int CB = prefill::kCB;  // 16-column blocks per wave
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int KS = D / 32;                 // 16x16x32 steps of q.K
  constexpr int NE = D / 16;                 // P.V blocks of 16 output rows
  constexpr int VH = D / 16;                 // output row d = VH * r + e
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RPW = 64 / CPR;              // rows one wave loads per round
  constexpr int ROUNDS = kKeys / (kWaves * RPW);
  static_assert(ROUNDS >= 1 && BS % RPW == 0, "a wave's load rows lie in one block");
  constexpr int TILE = kKeys * 2 * D;        // bytes of one K or V step tile
  constexpr int COLS_W = 16 * CB;            // columns per wave
  constexpr int TOK_W = COLS_W / G;          // query tokens per wave
  using vrow_t = typename prefill::VRow<D>::type;

  // [buffer][K|V]: step st lives in buffer st % kBufs; its rows arrive by
  // direct global->LDS loads issued kAhead steps before it is used
  __shared__ __attribute__((aligned(16))) unsigned char lds[kBufs][2][TILE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int quad = lane >> 4;
  const int col = lane & 15;

  // ---- workgroup -> (sequence, KV head, query block) and its keys ----------
  prefill::Work wk;
  if (!prefill::workgroup_work<G>(a, wk)) return;  // the whole workgroup
  const int s = wk.s, g = wk.g, q0 = wk.q0, T = wk.T, n = wk.n;
  const int wg_tok0 = wk.wg_tok0, wg_lo = wk.wg_lo, st0 = wk.st0, nsteps = wk.nsteps;
  const int win = a.window;

  // this wave's columns: token w_tok0 + (16 cb + col) / G, head col % G
  const int w_tok0 = wg_tok0 + w * TOK_W;
  const int w_pmax = w_tok0 < T ? n - T + min(T - 1, w_tok0 + TOK_W - 1) : -1;
  const int w_pmin = w_tok0 + TOK_W - 1 < T ? n - T + w_tok0 : -1;
  // keys below the window start of the wave's last column need the mask
  const int w_lomax = win > 0 && w_pmax >= 0 ? max(0, w_pmax + 1 - win) : 0;
  const int hh = col % G;
  int tok[CB], p_col[CB], lo_col[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    tok[cb] = w_tok0 + (16 * cb + col) / G;
    p_col[cb] = tok[cb] < T ? n - T + tok[cb] : -1;  // last key the column sees
    lo_col[cb] = win > 0 ? max(0, p_col[cb] + 1 - win) : 0;  // and its first
  }

  // ---- q as the B operand: lane (quad, col), chunk 4j + quad of its row -----
  half8_t qop[CB][KS];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const bool ok = tok[cb] < T;
    const half_t* qh = reinterpret_cast<const half_t*>(a.q) +
                       ((size_t)(q0 + (ok ? tok[cb] : 0)) * a.num_q_heads + g * G + hh) * D;
#pragma unroll
    for (int j = 0; j < KS; ++j)
      qop[cb][j] = ok ? __builtin_bit_cast(half8_t, load16(qh + (4 * j + quad) * 8))
                      : __builtin_bit_cast(half8_t, u32x4_t{0u, 0u, 0u, 0u});
  }

  // ---- K/V step loads: wave w, round j loads rows (j * 4 + w) * RPW + lane / CPR
  const size_t head_bytes = (size_t)BS * D * 2;
  const size_t block_bytes = 2 * (size_t)a.num_kv_heads * head_bytes;
  const size_t v_bytes = (size_t)a.num_kv_heads * head_bytes;
  const char* kvg = reinterpret_cast<const char*>(a.kv) + (size_t)g * head_bytes;
  const int32_t* bt_row = a.bt + (size_t)s * a.max_blocks;
  const int lrow = lane / CPR;
  const int lch = lane % CPR;

  // Step sl goes to buffer (sl - st0) % kBufs.  Wave w's round j fills rows
  // (4 j + w) * RPW .. + RPW - 1 of the K and the V tile: lane l lands at
  // byte 16 l of that 1 KiB piece, i.e. row + l / CPR, physical chunk
  // l % CPR, so it loads logical chunk (l % CPR) ^ (row & (CPR - 1)).  Rows
  // past the context load row n - 1 instead, rows before the workgroup's
  // first key load row wg_lo (finite; their weights are 0): a piece's RPW
  // rows, clamped into [wg_lo, n - 1], still lie in one block, and rows no
  // column sees are never read.  Steps past the last re-read it, so every
  // step issues the same loads and the wait counts stay fixed.
  constexpr int LPS = 2 * ROUNDS;  // loads per lane per step
  int ids[ROUNDS];
  auto fetch_ids = [&](int sl) {
    const int sd = min(sl, nsteps - 1);
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j) {
      const int k0 = min(max(sd * kKeys + (j * kWaves + w) * RPW, wg_lo), n - 1);
      const int lb = k0 / BS;  // wave-uniform: the piece's rows share a block
      const int v = lb < a.max_blocks ? load_uniform(bt_row + lb) : 0;
      ids[j] = (v < 0 || v >= a.num_blocks) ? 0 : v;
    }
  };
  auto issue = [&](int sl, auto B) {
    constexpr int b = decltype(B)::value;
    const int sd = min(sl, nsteps - 1);
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j) {
      const int piece = j * kWaves + w;
      const int r = piece * RPW + lrow;
      const int key = min(max(sd * kKeys + r, wg_lo), n - 1);
      const int c = lch ^ (r & (CPR - 1));
      const char* src = kvg + (size_t)ids[j] * block_bytes + (key % BS) * (2 * D);
      load_lds16(src + c * 16, &lds[b][0][piece * 1024]);            // K: swizzled
      load_lds16(src + v_bytes + lch * 16, &lds[b][1][piece * 1024]);  // V: plain rows
    }
  };

  // acc: O^T blocks; acl: the weight sums, as one more block whose V rows
  // are all ones (the matrix cores add the weights, so numerator and
  // denominator sum the same rounded parts)
  float m[CB];
  float4_t acc[CB][NE], acl[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    m[cb] = kMaxInit;
    acl[cb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[cb][e] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  const half8_t ones = __builtin_bit_cast(
      half8_t, u32x4_t{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u});
  const float cs = a.scale_log2;  // > 0: the max is taken on the raw scores

  auto qk = [&](auto B, float4_t (&sc)[CB][2]) {
    constexpr int b = decltype(B)::value;
    const unsigned char* kt = lds[b][0];
    u32x4_t kr[2][KS];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < KS; ++j)
        kr[kk][j] =
            *reinterpret_cast<const u32x4_t*>(kt + tile_off<D>(16 * kk + col, 4 * j + quad));
    // 2 * CB independent accumulations, interleaved over the contraction
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) sc[cb][0] = sc[cb][1] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          sc[cb][kk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(half8_t, kr[kk][j]), qop[cb][j], sc[cb][kk], 0, 0, 0);
  };

  // softmax and P.V of step st; q.K of the next step (buffer Bn) is issued
  // between the max and the exponentials, so its matrix-core work overlaps
  // the vector work of this step
  auto softmax_pv = [&](int st, auto B, const float4_t (&sc)[CB][2], auto Bn,
                        float4_t (&sn)[CB][2]) {
    constexpr int b = decltype(B)::value;
    const unsigned char* vt = lds[b][1];
    // The wave takes issue priority for its vector work (V reads, max,
    // exponentials, weight split) and drops it before its P.V products: the
    // other wave of the SIMD is then usually in its matrix phase, whose
    // issued MFMAs keep running, so the two phases overlap more (measured
    // +3.5-5% on every head shape).  A wave's in-kernel priority, not a
    // queue priority.
    __builtin_amdgcn_s_setprio(1);
    // V rows 4 quad + i of both tiles, this lane's D/16 values of each
    vrow_t vr[8];
#pragma unroll
    for (int jv = 0; jv < 8; ++jv) {
      const int r = (jv >> 2) * 16 + 4 * quad + (jv & 3);
      if constexpr (D == 128)
        vr[jv] = *reinterpret_cast<const u32x4_t*>(vt + r * (2 * D) + col * 16);
      else
        vr[jv] = *reinterpret_cast<const u32x2_t*>(vt + r * (2 * D) + col * 8);
    }
    const bool edge = (st + 1) * kKeys - 1 > w_pmin || (st + 1) * kKeys > n ||
                      st * kKeys < w_lomax;
    float y[CB][8];  // raw scores; in log2 units they are cs * y
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) y[cb][4 * kk + i] = sc[cb][kk][i];
      if (edge) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int t = st * kKeys + (k >> 2) * 16 + 4 * quad + (k & 3);
          if (t > p_col[cb] || t < lo_col[cb]) y[cb][k] = -INFINITY;
        }
      }
      const float lm = cs * fmaxf(fmaxf(fmaxf(y[cb][0], y[cb][1]), fmaxf(y[cb][2], y[cb][3])),
                                  fmaxf(fmaxf(y[cb][4], y[cb][5]), fmaxf(y[cb][6], y[cb][7])));
      if (wave_any(lm > m[cb] + kSlack)) {
        // some column's reference must move: to the column's max, exactly
        const float m_new = fmaxf(m[cb], rows4_max(lm));
        const float alpha = fast_exp2(m[cb] - m_new);
        acl[cb] *= alpha;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[cb][e] *= alpha;
        m[cb] = m_new;
      }
    }
    qk(Bn, sn);
    half8_t phi[CB], plo[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const float off = kPLog - m[cb];
      float pw[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) pw[k] = fast_exp2(fmaf(y[cb][k], cs, off));
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const auto h = __builtin_amdgcn_cvt_pkrtz(pw[2 * k], pw[2 * k + 1]);
        const auto r = __builtin_amdgcn_cvt_pkrtz(fmaf((float)h[0], -1.f, pw[2 * k]),
                                                  fmaf((float)h[1], -1.f, pw[2 * k + 1]));
        hw[k] = __builtin_bit_cast(uint32_t, h);
        lw[k] = __builtin_bit_cast(uint32_t, r);
      }
      phi[cb] = __builtin_bit_cast(half8_t, u32x4_t{hw[0], hw[1], hw[2], hw[3]});
      plo[cb] = __builtin_bit_cast(half8_t, u32x4_t{lw[0], lw[1], lw[2], lw[3]});
    }
    __builtin_amdgcn_s_setprio(0);
    // P.V in pairs of output blocks: each accumulator's hi and lo products
    // are 2 * CB instructions apart
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      acl[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, phi[cb], acl[cb], 0, 0, 0);
#pragma unroll
    for (int e0 = 0; e0 < NE; e0 += 2) {
      half8_t av[2];
#pragma unroll
      for (int ee = 0; ee < 2; ++ee) {
        const int e = e0 + ee;
        const int wd = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        av[ee] = __builtin_bit_cast(
            half8_t, u32x4_t{__builtin_amdgcn_perm(vr[1][wd], vr[0][wd], sel),
                             __builtin_amdgcn_perm(vr[3][wd], vr[2][wd], sel),
                             __builtin_amdgcn_perm(vr[5][wd], vr[4][wd], sel),
                             __builtin_amdgcn_perm(vr[7][wd], vr[6][wd], sel)});
      }
#pragma unroll
      for (int ee = 0; ee < 2; ++ee)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[cb][e0 + ee] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[ee], phi[cb],
                                                                    acc[cb][e0 + ee], 0, 0, 0);
#pragma unroll
      for (int ee = 0; ee < 2; ++ee)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[cb][e0 + ee] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[ee], plo[cb],
                                                                    acc[cb][e0 + ee], 0, 0, 0);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      acl[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, plo[cb], acl[cb], 0, 0, 0);
    {  // K reads first, then each q.K product followed by vector work
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);
#pragma unroll
      for (int i = 0; i < 2 * KS * CB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }
  };

  // ---- steps st0 .. nsteps - 1 --------------------------------------------
  // Iteration st: wait until step st + 1 has landed (own loads, then the
  // barrier for everyone's), issue step st + kAhead into the buffer step
  // st - 1 used, then run q.K of step st + 1 on the matrix cores while the
  // softmax of step st runs on the vector ALUs, and P.V of step st.
  auto vm_wait = [](auto N) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(decltype(N)::value) : "memory");
  };
  auto barrier = []() { asm volatile("s_barrier" ::: "memory"); };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  fetch_ids(st0);
  issue(st0, I0{});
  fetch_ids(st0 + 1);
  issue(st0 + 1, I1{});
  fetch_ids(st0 + 2);
  issue(st0 + 2, I2{});
  fetch_ids(st0 + 3);
  vm_wait(std::integral_constant<int, 2 * LPS>{});
  barrier();
  float4_t sc[CB][2];
  if (w_pmax >= 0) qk(I0{}, sc);
  auto step = [&](int st, auto B) {
    constexpr int b = decltype(B)::value;
    vm_wait(std::integral_constant<int, LPS>{});
    barrier();
    issue(st + kAhead, std::integral_constant<int, (b + kAhead) % kBufs>{});
    fetch_ids(st + kAhead + 1);
    if (st * kKeys <= w_pmax) {
      float4_t sn[CB][2];
      softmax_pv(st, B, sc, std::integral_constant<int, (b + 1) % kBufs>{}, sn);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        sc[cb][0] = sn[cb][0];
        sc[cb][1] = sn[cb][1];
      }
    }
  };
  for (int st = st0; st < nsteps; st += kBufs) {  // fixed buffers in each trip
    step(st, I0{});
    if (st + 1 < nsteps) step(st + 1, I1{});
    if (st + 2 < nsteps) step(st + 2, I2{});
    if (st + 3 < nsteps) step(st + 3, I3{});
  }
  vm_wait(std::integral_constant<int, 0>{});  // no load may land after the exit

  // ---- normalise and store: lane (quad, col) holds d = VH * (4 quad + i) + e
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float lt = acl[cb][0];
    if (tok[cb] < T) {
      const float inv = 1.f / lt;
      float* o = a.out + ((size_t)(q0 + tok[cb]) * a.num_q_heads + g * G + hh) * D;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e4 = 0; e4 < NE / 4; ++e4)
          *reinterpret_cast<float4_t*>(o + VH * (4 * quad + i) + 4 * e4) =
              float4_t{acc[cb][4 * e4][i], acc[cb][4 * e4 + 1][i], acc[cb][4 * e4 + 2][i],
                       acc[cb][4 * e4 + 3][i]} * inv;
      }
    }
  }
}

template <int D, int BS, int G>
int launch_one(const PrefillArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)((size_t)a.num_seqs * a.qblocks * a.num_kv_heads);
  if (grid == 0) return 0;
  hipLaunchKernelGGL((prefill_mfma_kernel<D, BS, G>), dim3(grid), dim3(kWaves * 64), 0, stream,
                     a);
  return hipGetLastError() == hipSuccess ? 0 : 2;
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

int prefill_columns_per_workgroup() { return prefill::kColsWG; }

int launch_prefill_mfma(const PrefillArgs& a, int head_dim, int block_size, int group,
                        hipStream_t stream) {
  if (head_dim == 64) return by_block<64>(a, block_size, group, stream);
  if (head_dim == 128) return by_block<128>(a, block_size, group, stream);
  return 1;
}

}  // namespace pa
