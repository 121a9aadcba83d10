// prefill_mfma_i8.hip — causal attention of multi-token queries (a prefill
// chunk) over an INT8 KV cache, on the matrix cores (gfx950).
//
// The cache holds int8 codes with one float32 scale per (token, KV head) row
// of K and of V ([KV2P] "KV Cache从原理到实战" §5.2); the chunk's rows were
// quantised by the cache write like any other.  Attention over the
// dequantised values, with the causal mask and sliding window of the f16
// prefill (prefill_common.h), is computed as
//   score_t = scale * sk_t * (q . Kq_t),  out = sum_t (p_t sv_t) Vq_t / sum_t p_t,
// the row scales applied outside the matrix products so that the codes
// enter them exactly.
//
// Work decomposition, step shape and softmax as in prefill_mfma.hip; what
// changes is how a step's K/V reach the matrix cores:
//  * raw step tiles: each step's K and V codes (32 rows x D bytes each) and
//    their 64 row scales arrive by direct global->LDS loads, issued five
//    steps ahead into four raw buffers (each wave loads 16 of the scales);
//  * conversion: once per workgroup, not per wave, the 256 threads widen the
//    codes of the step two ahead exactly — K to fp16 in the swizzled layout
//    of the f16 kernel's K tile, V to bf16 — into two K and three V buffers
//    (the V buffer also takes the step's scales), so the four waves share
//    the work;
//  * q.K^T: v_mfma_f32_16x16x32_f16 on the converted K, the K scale then
//    multiplies each score;
//  * P.V: the weights times the V scales, split into bf16 hi + lo parts
//    (~16 significant bits; bf16's exponent takes any weight * scale), with
//    v_mfma_f32_16x16x32_bf16 on the converted V codes;
//  * the weight sums stay in fp32 without the V scales.
// Per step: wait for the raw tile two ahead, one barrier, convert it, then
// the softmax and P.V of this step with q.K of the next interleaved.
#include "i8_codes.h"
#include "prefill_common.h"

#include <type_traits>

namespace pa {
namespace {

constexpr int kWaves = 4;                           // waves per workgroup
constexpr int kColsWG = kWaves * 16 * prefill::kCB;  // columns per workgroup

using prefill::kKeys;
using prefill::kPLog;
using prefill::kSlack;
using prefill::tile_off;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <int D>
struct RawTile {
  unsigned char kv[2 * kKeys * D];  // K codes [32][D], then V codes [32][D]
  // row scales: wave w's slot [64 w, 64 w + 16) holds entries 16 w .. 16 w + 15
  // (entry e < 32: K scale of row e; e >= 32: V scale of row e - 32); the
  // rest of each slot is filled by the slot's other lanes and never read
  float sc[kWaves * 64];
};

template <int D>
struct ConvertedV {
  unsigned char v[kKeys * 2 * D];  // bf16 rows
  float sc[2 * kKeys];             // K scales of the step's rows, then V scales
};

constexpr int kRawBufs = 4;  // raw buffers; steps are issued five ahead

template <int D, int BS, int G>
__global__ __launch_bounds__(kWaves * 64, 2) void prefill_mfma_i8_kernel(PrefillArgs a) {
  constexpr int CB = prefill::kCB;  // 16-column blocks per wave
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int KS = D / 32;            // 16x16x32 steps of q.K
  constexpr int NE = D / 16;            // P.V blocks of 16 output rows
  constexpr int VH = D / 16;            // output row d = VH * r + e
  constexpr int RCPR = D / 16;          // 16-byte chunks of a code row
  constexpr int RRPW = 64 / RCPR;       // code rows one 16-byte-per-lane load covers
  constexpr int PIECES = 2 * kKeys / RRPW;  // K pieces, then V pieces
  constexpr int ROUNDS = PIECES / kWaves;   // pieces per wave per step
  static_assert(ROUNDS >= 1 && PIECES % kWaves == 0, "pieces split evenly over the waves");
  static_assert(RRPW * D == 1024, "a piece is 1 KiB of the raw tile");
  constexpr int CTILE = kKeys * 2 * D;  // bytes of a converted K or V step tile
  constexpr int CPT = kKeys * D / (kWaves * 64);  // codes a thread converts per tile
  constexpr int COLS_W = 16 * CB;       // columns per wave
  constexpr int TOK_W = COLS_W / G;     // query tokens per wave
  using vrow_t = typename prefill::VRow<D>::type;

  // raw step tiles; converted K (fp16, swizzled) of two steps; converted V
  // (bf16, plain rows) of three steps, each with its step's 64 row scales
  __shared__ __attribute__((aligned(16))) RawTile<D> raw[kRawBufs];
  __shared__ __attribute__((aligned(16))) unsigned char cvk[2][CTILE];
  __shared__ __attribute__((aligned(16))) ConvertedV<D> cvv[3];

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

  // ---- raw step loads ------------------------------------------------------
  // Rows are clamped into [wg_lo, n - 1] (rows no column sees are never
  // read; their weights are 0).  Block ids are read per 8-row group of the
  // step with scalar loads, one step ahead: an 8-row group lies in one block
  // (block sizes 8, 16, 32), and so do its clamped rows.
  const size_t head_bytes = (size_t)BS * D;
  const size_t block_bytes = 2 * (size_t)a.num_kv_heads * head_bytes;
  const size_t v_bytes = (size_t)a.num_kv_heads * head_bytes;
  const char* kvg = reinterpret_cast<const char*>(a.kv) + (size_t)g * head_bytes;
  const float* scg = a.kv_scales + (size_t)g * 2 * BS;   // scales [NB, Hkv, 2, BS]
  const size_t sblock = 2 * (size_t)a.num_kv_heads * BS;  // floats per block
  const int32_t* bt_row = a.bt + (size_t)s * a.max_blocks;
  // Most steps lie wholly inside [wg_lo, n): they need no clamping, and
  // take one wave-uniform test instead of one per piece.  Keys are below
  // n <= max_blocks * BS, so a block index never passes the table's row.
  constexpr int LPS = ROUNDS + 1;  // loads per lane per step: pieces + scales
  uint32_t ids[kKeys / 8];
  auto clamp_key = [&](int k) { return min(max(k, wg_lo), n - 1); };
  auto inside = [&](int sd) { return sd * kKeys >= wg_lo && (sd + 1) * kKeys <= n; };
  // the block id of step row r (a select chain, not a dynamic register
  // index); ids outside the pool read block 0 (checked at the use, so that
  // the block-id loads are not waited for when they are issued)
  const uint32_t nb32 = (uint32_t)min(a.num_blocks, (int64_t)1 << 31);  // negative ids fail it
  auto id_of_row = [&](int r) {
    const int q = r >> 3;
    const uint32_t id = q == 0 ? ids[0] : q == 1 ? ids[1] : q == 2 ? ids[2] : ids[3];
    return id < nb32 ? id : 0u;
  };
  auto fetch_ids = [&](int sl) {
    const int sd = min(sl, nsteps - 1);
    const bool in = inside(sd);
#pragma unroll
    for (int j = 0; j < kKeys / 8; ++j) {
      const int k = sd * kKeys + 8 * j;
      const int v = load_uniform(bt_row + (uint32_t)(in ? k : clamp_key(k)) / BS);
      ids[j] = (uint32_t)v;  // checked against the pool where it is used
    }
  };
  // A piece of RRPW rows lies in one block when RRPW <= BS (both powers of
  // two, pieces aligned).  When none of its rows is clamped either (most
  // steps), its first row address is wave-uniform and each lane adds a fixed
  // offset; otherwise every lane finds its own row's block and clamped key.
  constexpr bool kPieceInBlock = RRPW <= BS;
  const uint32_t loff = (uint32_t)((lane / RCPR) * D + (lane % RCPR) * 16);
  const uint32_t blk_bytes = (uint32_t)block_bytes;  // < 2^32 for every supported shape
  auto issue = [&](int sl, int b) {
    const int sd = min(sl, nsteps - 1);
    const bool in = inside(sd);
    auto piece_src = [&](uint32_t id, bool is_v, int key) {
      return kvg + (uint64_t)id * blk_bytes + (is_v ? v_bytes : 0) + ((uint32_t)key % BS) * D;
    };
    if (kPieceInBlock && in) {
#pragma unroll
      for (int j = 0; j < ROUNDS; ++j) {
        const int piece = j * kWaves + w;
        const int r0 = (piece % (PIECES / 2)) * RRPW;
        load_lds16(piece_src(id_of_row(r0), piece >= PIECES / 2, sd * kKeys + r0) + loff,
                   &raw[b].kv[piece * 1024]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < ROUNDS; ++j) {
        const int piece = j * kWaves + w;
        const bool is_v = piece >= PIECES / 2;
        const int r0 = (piece % (PIECES / 2)) * RRPW;  // the piece's first row in the step
        const int kb = sd * kKeys + r0;
        if (kPieceInBlock && kb >= wg_lo && kb + RRPW <= n) {
          load_lds16(piece_src(id_of_row(r0), is_v, kb) + loff, &raw[b].kv[piece * 1024]);
        } else {
          const int r = r0 + lane / RCPR;  // row in the step
          load_lds16(piece_src(id_of_row(r), is_v, clamp_key(sd * kKeys + r)) +
                         (lane % RCPR) * 16,
                     &raw[b].kv[piece * 1024]);
        }
      }
    }
    // scales: wave w loads entries 16 w + (lane % 16)
    const int e = 16 * w + (lane & 15);
    const int r = e % kKeys;
    const int key = in ? sd * kKeys + r : clamp_key(sd * kKeys + r);
    const float* src =
        scg + (uint64_t)id_of_row(r) * sblock + (e >= kKeys ? BS : 0) + (uint32_t)key % BS;
    load_lds4(src, &raw[b].sc[64 * w]);
  };

  // ---- conversion of a raw step tile: thread t widens CPT codes of row
  // t / 8 of K and of V
  auto convert = [&](int rb, int kbuf, int vbuf) {
    const int t = threadIdx.x;
    const int row = t >> 3, sub = t & 7;
    const unsigned char* kr = &raw[rb].kv[row * D + sub * CPT];
    const unsigned char* vr = kr + kKeys * D;
    unsigned char* kc = cvk[kbuf];
    unsigned char* vc = cvv[vbuf].v;
    // the step's scales travel with its V: entry e (K rows, then V rows)
    // sits in wave e / 16's slot of the raw tile
    if (t < 2 * kKeys) cvv[vbuf].sc[t] = raw[rb].sc[64 * (t >> 4) + (t & 15)];
    if constexpr (CPT == 16) {
      const u32x4_t k4 = *reinterpret_cast<const u32x4_t*>(kr);
      const u32x4_t v4 = *reinterpret_cast<const u32x4_t*>(vr);
      uint32_t h[8], bb[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        codes_to_half(k4[i], h[2 * i], h[2 * i + 1]);
        codes_to_bf16(v4[i], bb[2 * i], bb[2 * i + 1]);
      }
      *reinterpret_cast<u32x4_t*>(kc + tile_off<D>(row, 2 * sub)) =
          u32x4_t{h[0], h[1], h[2], h[3]};
      *reinterpret_cast<u32x4_t*>(kc + tile_off<D>(row, 2 * sub + 1)) =
          u32x4_t{h[4], h[5], h[6], h[7]};
      *reinterpret_cast<u32x4_t*>(vc + row * (2 * D) + (2 * sub) * 16) =
          u32x4_t{bb[0], bb[1], bb[2], bb[3]};
      *reinterpret_cast<u32x4_t*>(vc + row * (2 * D) + (2 * sub + 1) * 16) =
          u32x4_t{bb[4], bb[5], bb[6], bb[7]};
    } else {
      const u32x2_t k2 = *reinterpret_cast<const u32x2_t*>(kr);
      const u32x2_t v2 = *reinterpret_cast<const u32x2_t*>(vr);
      uint32_t h[4], bb[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        codes_to_half(k2[i], h[2 * i], h[2 * i + 1]);
        codes_to_bf16(v2[i], bb[2 * i], bb[2 * i + 1]);
      }
      *reinterpret_cast<u32x4_t*>(kc + tile_off<D>(row, sub)) = u32x4_t{h[0], h[1], h[2], h[3]};
      *reinterpret_cast<u32x4_t*>(vc + row * (2 * D) + sub * 16) =
          u32x4_t{bb[0], bb[1], bb[2], bb[3]};
    }
  };

  float m[CB], l[CB];  // l: this lane's share of the column's weight sum
  float4_t acc[CB][NE];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    m[cb] = kMaxInit;
    l[cb] = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[cb][e] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float cs = a.scale_log2;  // > 0: the max is taken on the raw scores

  auto qk = [&](int kbuf, float4_t (&sc)[CB][2]) {
    const unsigned char* kt = cvk[kbuf];
    u32x4_t kr[2][KS];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < KS; ++j)
        kr[kk][j] =
            *reinterpret_cast<const u32x4_t*>(kt + tile_off<D>(16 * kk + col, 4 * j + quad));
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

  // softmax and P.V of step st (raw buffer RB for its scales, converted
  // buffer CV for its V); q.K of the next step (converted buffer CN) is
  // issued between the max and the exponentials
  auto softmax_pv = [&](int st, int vbuf, const float4_t (&sc)[CB][2], int knext,
                        float4_t (&sn)[CB][2]) {
    // vector work at raised issue priority, dropped before the P.V products
    // (a wave's in-kernel priority, as in the f16 kernel)
    __builtin_amdgcn_s_setprio(1);
    const unsigned char* vt = cvv[vbuf].v;
    vrow_t vr[8];
#pragma unroll
    for (int jv = 0; jv < 8; ++jv) {
      const int r = (jv >> 2) * 16 + 4 * quad + (jv & 3);
      if constexpr (D == 128)
        vr[jv] = *reinterpret_cast<const u32x4_t*>(vt + r * (2 * D) + col * 16);
      else
        vr[jv] = *reinterpret_cast<const u32x2_t*>(vt + r * (2 * D) + col * 8);
    }
    // this lane's keys 16 kk + 4 quad + i: their K and V scales
    float4_t sk[2], sv[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      sk[kk] = *reinterpret_cast<const float4_t*>(&cvv[vbuf].sc[16 * kk + 4 * quad]);
      sv[kk] = *reinterpret_cast<const float4_t*>(&cvv[vbuf].sc[kKeys + 16 * kk + 4 * quad]);
    }
    const bool edge = (st + 1) * kKeys - 1 > w_pmin || (st + 1) * kKeys > n ||
                      st * kKeys < w_lomax;
    float y[CB][8];  // scores sk * (q . codes); in log2 units cs * y
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) y[cb][4 * kk + i] = sc[cb][kk][i] * sk[kk][i];
      if (edge) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int t = st * kKeys + (k >> 2) * 16 + 4 * quad + (k & 3);
          if (t > p_col[cb] || t < lo_col[cb]) y[cb][k] = -INFINITY;
        }
      }
      // scores are finite or -inf here (codes and scales are finite)
      const float t = max3_nonan(max3_nonan(y[cb][0], y[cb][1], y[cb][2]),
                                 max3_nonan(y[cb][3], y[cb][4], y[cb][5]), y[cb][6]);
      const float lm = cs * max3_nonan(t, y[cb][7], y[cb][7]);
      if (wave_any(lm > m[cb] + kSlack)) {
        // some column's reference must move: to the column's max, exactly
        const float m_new = fmaxf(m[cb], rows4_max(lm));
        const float alpha = fast_exp2(m[cb] - m_new);
        l[cb] *= alpha;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[cb][e] *= alpha;
        m[cb] = m_new;
      }
    }
    qk(knext, sn);
    bf16x8_t phi[CB], plo[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const float off = kPLog - m[cb];
      float pv[8];
      float ls = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float pw = fast_exp2(fmaf(y[cb][k], cs, off));
        ls += pw;
        pv[k] = pw * sv[k >> 2][k & 3];
      }
      l[cb] += ls;
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        hw[k] = pack_bf16_rne(pv[2 * k], pv[2 * k + 1]);
        lw[k] = pack_bf16_rne(pv[2 * k] - __builtin_bit_cast(float, hw[k] << 16),
                              pv[2 * k + 1] - __builtin_bit_cast(float, hw[k] & 0xFFFF0000u));
      }
      phi[cb] = __builtin_bit_cast(bf16x8_t, u32x4_t{hw[0], hw[1], hw[2], hw[3]});
      plo[cb] = __builtin_bit_cast(bf16x8_t, u32x4_t{lw[0], lw[1], lw[2], lw[3]});
    }
    __builtin_amdgcn_s_setprio(0);
    // P.V: V^T (bf16 codes, relabelled contraction index as in the f16
    // kernel) times the weight parts
#pragma unroll
    for (int e0 = 0; e0 < NE; e0 += 2) {
      bf16x8_t av[2];
#pragma unroll
      for (int ee = 0; ee < 2; ++ee) {
        const int e = e0 + ee;
        const int wd = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        av[ee] = __builtin_bit_cast(
            bf16x8_t, u32x4_t{__builtin_amdgcn_perm(vr[1][wd], vr[0][wd], sel),
                              __builtin_amdgcn_perm(vr[3][wd], vr[2][wd], sel),
                              __builtin_amdgcn_perm(vr[5][wd], vr[4][wd], sel),
                              __builtin_amdgcn_perm(vr[7][wd], vr[6][wd], sel)});
      }
#pragma unroll
      for (int ee = 0; ee < 2; ++ee)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[cb][e0 + ee] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ee], phi[cb],
                                                                     acc[cb][e0 + ee], 0, 0, 0);
#pragma unroll
      for (int ee = 0; ee < 2; ++ee)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[cb][e0 + ee] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ee], plo[cb],
                                                                     acc[cb][e0 + ee], 0, 0, 0);
    }
  };

  // ---- steps st0 .. nsteps - 1 --------------------------------------------
  // Raw step tiles are issued five steps ahead into four buffers and
  // converted two steps ahead: iteration i (step st = st0 + i) waits until
  // raw step st + 2 has landed (own loads, then one barrier for everyone's;
  // the barrier also publishes step st + 1's conversion and ends everyone's
  // reads of iteration i - 1), issues raw step st + 5 into the buffer raw
  // step st + 1 left, converts raw step st + 2 (K into the buffer step st's
  // q.K used, V and scales into the one step st - 1's P.V used), and runs
  // the softmax and P.V of step st with q.K of step st + 1 interleaved.  K
  // conversions live two steps, V conversions three: one barrier per step.
  auto vm_wait = [](auto N) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(decltype(N)::value) : "memory");
  };
  auto barrier = []() { asm volatile("s_barrier" ::: "memory"); };
  auto lds_barrier = []() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  for (int j = 0; j < kRawBufs; ++j) {
    fetch_ids(st0 + j);
    issue(st0 + j, j);
  }
  fetch_ids(st0 + kRawBufs);
  vm_wait(std::integral_constant<int, 2 * LPS>{});  // raw steps st0, st0 + 1
  barrier();
  convert(0, 0, 0);
  convert(1, 1, 1);
  lds_barrier();  // both converted; raw buffers 0 and 1 free
  issue(st0 + kRawBufs, 0);
  fetch_ids(st0 + kRawBufs + 1);
  float4_t sc[CB][2];
  if (w_pmax >= 0) qk(0, sc);
  int v_cur = 0;  // (st - st0) % 3
  for (int st = st0; st < nsteps; ++st) {
    const int i = st - st0;
    const int v_conv = v_cur == 0 ? 2 : v_cur - 1;  // (i + 2) % 3
    vm_wait(std::integral_constant<int, 2 * LPS>{});  // raw step st + 2
    barrier();
    issue(st + kRawBufs + 1, (i + 1) & (kRawBufs - 1));
    fetch_ids(st + kRawBufs + 2);
    convert((i + 2) & (kRawBufs - 1), i & 1, v_conv);
    if (st * kKeys <= w_pmax) {
      float4_t sn[CB][2];
      softmax_pv(st, v_cur, sc, (i + 1) & 1, sn);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        sc[cb][0] = sn[cb][0];
        sc[cb][1] = sn[cb][1];
      }
    }
    v_cur = v_cur == 2 ? 0 : v_cur + 1;
  }
  vm_wait(std::integral_constant<int, 0>{});  // no load may land after the exit

  // ---- normalise and store: lane (quad, col) holds d = VH * (4 quad + i) + e
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float lt = rows4_sum(l[cb]);
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
  hipLaunchKernelGGL((prefill_mfma_i8_kernel<D, BS, G>), dim3(grid), dim3(kWaves * 64), 0,
                     stream, a);
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

int prefill_i8_columns_per_workgroup() { return kColsWG; }

int launch_prefill_mfma_i8(const PrefillArgs& a, int head_dim, int block_size, int group,
                           hipStream_t stream) {
  if (head_dim == 64) return by_block<64>(a, block_size, group, stream);
  if (head_dim == 128) return by_block<128>(a, block_size, group, stream);
  return 1;
}

}  // namespace pa
