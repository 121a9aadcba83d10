// decode_epilogue.h — end of a decode range, shared by the VALU and MFMA
// kernels: merge the waves' online-softmax states, then write either the
// output (the range was a whole sequence) or a partial (m, l, normalised o)
// for a merge kernel.
//
// The merge algebra is the pages' running-max / running-sum rescaling
// ([KVPA] "KV Cache与PagedAttention深度解析" §7.2; [NANO] zwxr.cn walkthrough
// §2.4) applied across waves: with wave states (m_i, l_i, O_i) in log2 units,
// M = max m_i, w_i = exp2(m_i - M), L = sum w_i l_i, out = sum w_i O_i / L.
//
// Partials are combined by a separate kernel rather than by the last
// workgroup to finish: making one workgroup's stores visible to another on a
// different XCD takes a device-scope fence, which writes back and invalidates
// that XCD's whole L2; thousands of workgroups doing so cost far more than
// one extra kernel boundary (measured: 7x slower split decode).
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace pa {

template <int G, int D, int NW>
struct DecodeSmem {
  float acc[NW][G][D];
  float m[NW][G];
  float l[NW][G];
};

// Where a range's result goes.  Head h of the group writes o[h * o_stride +
// d]; a partial (m != nullptr) also writes m[h * ml_stride] and l[...].
struct Sink {
  float* o;
  float* m;
  float* l;
  long o_stride;
  long ml_stride;
};

template <int G, int D>
__device__ __forceinline__ Sink output_sink(const DecodeArgs& a, int s, int g) {
  return Sink{a.out + ((size_t)s * a.num_q_heads + g * G) * D, nullptr, nullptr, D, 0};
}

// Zero output for an empty sequence.
template <int G, int D, int NW>
__device__ __forceinline__ void write_zero_output(const DecodeArgs& a, int s, int g) {
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64)
    a.out[((size_t)s * a.num_q_heads + g * G) * D + idx] = 0.f;
}

// All threads call this after every wave has stored its state in `sm` and a
// barrier has made it visible.
template <int G, int D, int NW>
__device__ void finish_range(const DecodeSmem<G, D, NW>& sm, const Sink& sink) {
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int h = idx / D;
    const int d = idx % D;
    float mx = sm.m[0][h];
#pragma unroll
    for (int k = 1; k < NW; ++k) mx = fmaxf(mx, sm.m[k][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const float wgt = fast_exp2(sm.m[k][h] - mx);
      L = fmaf(sm.l[k][h], wgt, L);
      O = fmaf(sm.acc[k][h][d], wgt, O);
    }
    sink.o[h * sink.o_stride + d] = L > 0.f ? O / L : 0.f;
    if (sink.m && d == 0) {
      sink.m[h * sink.ml_stride] = mx;
      sink.l[h * sink.ml_stride] = L;
    }
  }
}

}  // namespace pa
