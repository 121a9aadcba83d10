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
//                (k = 8q + j  ->  key 4q + j of tile j / 4); the V^T operand
//                (8 keys of one output row per lane) comes from the V rows in
//                LDS by transposing reads with the same relabelling, and the
//                weights go in as fp16 hi + lo parts, which keeps ~21 bits of
//                each weight;
//   the weight sums in fp32 on the vector ALUs, per lane, combined across
//                the four lane rows at the end (measured 1.6-2% faster than
//                one more matrix product per weight part on an all-ones
//                block).
// The step loop is software-pipelined by one step: q.K and the max of step
// st + 1 come before P.V of step st, and the exponentials and the weight
// split of step st + 1 are interleaved with those P.V products, so each
// wave feeds its SIMD's matrix core and vector ALU at the same time.
// LDS rows are 2D bytes, their 16-byte chunks XOR-swizzled by the row: in K
// so that the 16 lanes that read one chunk of 16 different K rows hit
// distinct banks, in V (by an even amount, keeping 32-byte pairs together)
// so that the 8 rows one half-wave's transposing read touches, 32 bytes of
// each, hit distinct banks.
#include "prefill_common.h"

#include <type_traits>

namespace pa {
namespace {

using prefill::kAhead;
using prefill::kBufs;
using prefill::kKeys;
using prefill::kPLog;
using prefill::kSlack;
using prefill::tile_off;

constexpr int kWaves = 4;                            // waves per workgroup
constexpr int kColsWG = kWaves * 16 * prefill::kCB;  // columns per workgroup

template <int D, int BS, int G>
__global__ __launch_bounds__(kWaves * 64, 2) void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int CB = prefill::kCB;  // 16-column blocks per wave
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int KS = D / 32;                 // 16x16x32 steps of q.K
  constexpr int NE = D / 16;                 // P.V blocks of 16 output rows
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RPW = 64 / CPR;              // rows one wave loads per round
  constexpr int ROUNDS = kKeys / (kWaves * RPW);
  static_assert(ROUNDS >= 1 && BS % RPW == 0, "a wave's load rows lie in one block");
  constexpr int TILE = kKeys * 2 * D;        // bytes of one K or V step tile
  constexpr int COLS_W = 16 * CB;            // columns per wave
  constexpr int TOK_W = COLS_W / G;          // query tokens per wave

  // [buffer][K|V]: step st lives in buffer st % kBufs; its rows arrive by
  // direct global->LDS loads issued kAhead steps before it is used
  __shared__ __attribute__((aligned(16))) unsigned char lds[kBufs][2][TILE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int quad = lane >> 4;
  const int col = lane & 15;

  // ---- workgroup -> (sequence, KV head, query block) and its keys ----------
  prefill::Work wk;
  if (!prefill::workgroup_work<G, kColsWG>(a, wk)) return;  // the whole workgroup
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
  // V chunk swizzle of row r: rows r and r' of one half-wave's transposing
  // read (r mod 8, or r / 2 mod 4 for D = 64, distinct) get distinct 32-byte
  // pairs of one 256-byte bank row
  auto vswz = [](int r) { return 2 * ((D == 64 ? r >> 1 : r) & (CPR / 2 - 1)); };

  // Step sl goes to buffer (sl - st0) % kBufs.  Wave w's round j fills rows
  // (4 j + w) * RPW .. + RPW - 1 of the K and the V tile: lane l lands at
  // byte 16 l of that 1 KiB piece, i.e. row + l / CPR, physical chunk
  // l % CPR, so it loads logical chunk (l % CPR) ^ (row & (CPR - 1)).  Rows
  // past the context load row n - 1 instead, rows before the workgroup's
  // first key load row wg_lo (finite; their weights are 0): a piece's RPW
  // rows, clamped into [wg_lo, n - 1], still lie in one block, and rows no
  // column sees are never read.  Steps past the last re-read it, so every
  // step issues the same loads and the wait counts stay fixed.  Most steps
  // lie wholly inside [wg_lo, n): their pieces need no clamping, and they
  // take one wave-uniform test instead of one per piece.  Keys are below
  // n <= max_blocks * BS, so a block index never passes the table's row.
  constexpr int LPS = 2 * ROUNDS;  // loads per lane per step
  auto inside = [&](int sd) { return sd * kKeys >= wg_lo && (sd + 1) * kKeys <= n; };
  uint32_t ids[ROUNDS];
  auto fetch_ids = [&](int sl) {
    const int sd = min(sl, nsteps - 1);
    const bool in = inside(sd);
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j) {
      const int k = sd * kKeys + (j * kWaves + w) * RPW;
      const int k0 = in ? k : min(max(k, wg_lo), n - 1);
      // wave-uniform: the piece's rows share a block
      const int v = load_uniform(bt_row + (uint32_t)k0 / BS);
      ids[j] = (uint32_t)v;  // checked against the pool where it is used
    }
  };
  // Lane offsets inside a piece whose rows are not clamped (most steps): the
  // piece's first row address is wave-uniform (scalar registers) and each
  // lane adds a fixed offset, so issuing a step takes no vector arithmetic.
  uint32_t koff[ROUNDS], voff[ROUNDS];
#pragma unroll
  for (int j = 0; j < ROUNDS; ++j) {
    const int r = (j * kWaves + w) * RPW + lrow;
    koff[j] = (uint32_t)(lrow * (2 * D) + ((lch ^ (r & (CPR - 1))) << 4));
    voff[j] = (uint32_t)(lrow * (2 * D) + ((lch ^ vswz(r)) << 4)) + (uint32_t)v_bytes;
  }
  const uint32_t blk_bytes = (uint32_t)block_bytes;  // < 2^32 for every supported shape
  // ids outside the pool read block 0 (32-bit scalar compare, at the use so
  // that the block-id loads are not waited for when they are issued)
  const uint32_t nb32 = (uint32_t)min(a.num_blocks, (int64_t)1 << 31);  // negative ids fail it
  auto issue = [&](int sl, auto B) {
    constexpr int b = decltype(B)::value;
    const int sd = min(sl, nsteps - 1);
    auto piece_base = [&](int j, int key) {
      const uint32_t id = ids[j] < nb32 ? ids[j] : 0u;
      return kvg + (uint64_t)id * blk_bytes + ((uint32_t)key % BS) * (2 * D);
    };
    if (inside(sd)) {
#pragma unroll
      for (int j = 0; j < ROUNDS; ++j) {
        const int piece = j * kWaves + w;
        const char* base = piece_base(j, sd * kKeys + piece * RPW);
        load_lds16(base + koff[j], &lds[b][0][piece * 1024]);  // K: swizzled
        load_lds16(base + voff[j], &lds[b][1][piece * 1024]);  // V: swizzled
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j) {
      const int piece = j * kWaves + w;
      const int kb = sd * kKeys + piece * RPW;  // the piece's first key
      if (kb >= wg_lo && kb + RPW <= n) {
        const char* base = piece_base(j, kb);
        load_lds16(base + koff[j], &lds[b][0][piece * 1024]);
        load_lds16(base + voff[j], &lds[b][1][piece * 1024]);
      } else {
        const int r = piece * RPW + lrow;
        const char* src = piece_base(j, min(max(sd * kKeys + r, wg_lo), n - 1));
        load_lds16(src + ((lch ^ (r & (CPR - 1))) << 4), &lds[b][0][piece * 1024]);
        load_lds16(src + v_bytes + ((lch ^ vswz(r)) << 4), &lds[b][1][piece * 1024]);
      }
    }
  };

  // acc: O^T blocks; the weight sums stay in fp32 per lane (the weights'
  // hi + lo parts differ from them by ~2^-22 relative)
  float m[CB];
  float4_t acc[CB][NE];
  float lsum[CB];  // this lane's share of its column's weight sum
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    m[cb] = kMaxInit;
    lsum[cb] = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[cb][e] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
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

  // V^T operand of output block e for the step in buffer B: lane (quad, col)
  // gets V[key][16 e + col] for the keys 4 quad + r of tile h (elements
  // 4 h + r); for that, lane (quad, 4 r + u) addresses V row 16 h + 4 quad + r
  // at d = 16 e + 4 u
  auto read_v = [&](auto B, half8_t (&av)[NE]) {
    constexpr int b = decltype(B)::value;
    const unsigned char* vt = lds[b][1];
    const int u = col & 3;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 16 * h + 4 * quad + (col >> 2);
      const unsigned char* vrow = vt + r * (2 * D) + (u & 1) * 8;
      const int sw = vswz(r);
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const half4_t t = lds_read_tr16(vrow + (((2 * e + (u >> 1)) ^ sw) << 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) av[e][4 * h + i] = t[i];
      }
    }
  };

  // Raw scores of step st (in log2 units they are cs * y), masked on the
  // steps that cross the diagonal, the end of the context or a window
  // start, and each lane's max in log2 units.
  auto scores = [&](int st, const float4_t (&sc)[CB][2], float (&y)[CB][8], float (&lm)[CB]) {
    const bool edge = (st + 1) * kKeys - 1 > w_pmin || (st + 1) * kKeys > n ||
                      st * kKeys < w_lomax;
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
      // scores are finite or -inf here (the mask replaces what no column sees)
      const float t = max3_nonan(max3_nonan(y[cb][0], y[cb][1], y[cb][2]),
                                 max3_nonan(y[cb][3], y[cb][4], y[cb][5]), y[cb][6]);
      lm[cb] = cs * max3_nonan(t, y[cb][7], y[cb][7]);
    }
  };

  // Moves the reference of a column block when some column's score passes
  // it by more than kSlack: to the columns' max rounded up to an integer, so
  // that the factor alpha = 2^(m_old - m_new) is a power of two.  Everything
  // summed so far is rescaled by alpha, and so are the weights P of the step
  // whose P.V products are still to come (exactly: a power of two, down to
  // fp16's subnormals).
  auto rescale = [&](const float (&lm)[CB], half8_t (*P)[CB]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      if (wave_any(lm[cb] > m[cb] + kSlack)) {
        const float m_new = ceilf(fmaxf(m[cb], rows4_max(lm[cb])));
        const float alpha = ldexpf(1.f, (int)fmaxf(m[cb] - m_new, -200.f));
        lsum[cb] *= alpha;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[cb][e] *= alpha;
        if (P) {
          const half_t ah = (half_t)alpha;
          P[0][cb] *= ah;
          P[1][cb] *= ah;
        }
        m[cb] = m_new;
      }
    }
  };

  // Weights exp2(cs y - m + kPLog) as fp16 hi + lo parts: P[0] hi, P[1] lo.
  auto weights = [&](const float (&y)[CB][8], half8_t (&P)[2][CB]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const float off = kPLog - m[cb];
      float pw[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) pw[k] = fast_exp2(fmaf(y[cb][k], cs, off));
      lsum[cb] += ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) split_f16(pw[2 * k], pw[2 * k + 1], hw[k], lw[k]);
      P[0][cb] = __builtin_bit_cast(half8_t, u32x4_t{hw[0], hw[1], hw[2], hw[3]});
      P[1][cb] = __builtin_bit_cast(half8_t, u32x4_t{lw[0], lw[1], lw[2], lw[3]});
    }
  };

  // P.V of one step: each accumulator's hi and lo products are 2 * CB
  // instructions apart.
  auto pv = [&](const half8_t (&av)[NE], const half8_t (&P)[2][CB]) {
#pragma unroll
    for (int e0 = 0; e0 < NE; e0 += 2) {
#pragma unroll
      for (int part = 0; part < 2; ++part)
#pragma unroll
        for (int ee = 0; ee < 2; ++ee)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[cb][e0 + ee] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                av[e0 + ee], P[part][cb], acc[cb][e0 + ee], 0, 0, 0);
    }
  };

  // ---- steps st0 .. nsteps - 1 --------------------------------------------
  // Software-pipelined by one step: iteration st waits until step st + 1
  // has landed (own loads, then the barrier for everyone's), issues step
  // st + kAhead into the buffer step st - 1 used, runs q.K of step st + 1
  // and its max (and, rarely, the rescale), and then P.V of step st on the
  // matrix cores interleaved with the exponentials and the weight split of
  // step st + 1 on the vector ALUs.  A wave's last step computes the scores
  // of the step after it too (all masked: weights 0, never used).
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
  // weights of even steps of a trip in pe, of odd ones in po
  half8_t pe[2][CB], po[2][CB];
  if (w_pmax >= 0) {
    float4_t s0[CB][2];
    float y[CB][8], lm[CB];
    qk(I0{}, s0);
    scores(st0, s0, y, lm);
    rescale(lm, nullptr);
    weights(y, pe);
  }
  auto step = [&](int st, auto B, half8_t (&pc)[2][CB], half8_t (&pn)[2][CB]) {
    constexpr int b = decltype(B)::value;
    vm_wait(std::integral_constant<int, LPS>{});
    barrier();
    issue(st + kAhead, std::integral_constant<int, (b + kAhead) % kBufs>{});
    fetch_ids(st + kAhead + 1);
    if (st * kKeys > w_pmax) return;  // the wave's columns end before this step
    float4_t sn[CB][2];
    float y[CB][8], lm[CB];
    qk(std::integral_constant<int, (b + 1) % kBufs>{}, sn);
    half8_t av[NE];
    read_v(B, av);  // after q.K: the V operand takes the K operand's registers
    scores(st + 1, sn, y, lm);
    rescale(lm, pc);
    pv(av, pc);
    weights(y, pn);
    // each P.V product followed by vector work of the next step
#pragma unroll
    for (int i = 0; i < 2 * NE * CB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
  };
  for (int st = st0; st < nsteps; st += kBufs) {  // fixed buffers in each trip
    step(st, I0{}, pe, po);
    if (st + 1 < nsteps) step(st + 1, I1{}, po, pe);
    if (st + 2 < nsteps) step(st + 2, I2{}, pe, po);
    if (st + 3 < nsteps) step(st + 3, I3{}, po, pe);
  }
  vm_wait(std::integral_constant<int, 0>{});  // no load may land after the exit

  // ---- normalise and store: lane (quad, col) holds d = 16 e + 4 quad + i
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float lt = rows4_sum(lsum[cb]);
    if (tok[cb] < T) {
      const float inv = 1.f / lt;
      float* o = a.out + ((size_t)(q0 + tok[cb]) * a.num_q_heads + g * G + hh) * D;
#pragma unroll
      for (int e = 0; e < NE; ++e)
        *reinterpret_cast<float4_t*>(o + 16 * e + 4 * quad) = acc[cb][e] * inv;
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

int prefill_columns_per_workgroup() { return kColsWG; }

int launch_prefill_mfma(const PrefillArgs& a, int head_dim, int block_size, int group,
                        hipStream_t stream) {
  if (head_dim == 64) return by_block<64>(a, block_size, group, stream);
  if (head_dim == 128) return by_block<128>(a, block_size, group, stream);
  return 1;
}

}  // namespace pa
