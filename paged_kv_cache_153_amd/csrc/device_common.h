// device_common.h — small gfx950 device helpers shared by the kernels.
//
// Wave64 lane reductions use DPP row operations (quad permutes and row
// mirrors move data between lanes of one 16-lane row inside the VALU
// instruction itself); steps across rows use ds_swizzle / bpermute, which
// run on the LDS crossbar without touching LDS memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// log2(e): softmax weights are computed as exp2(z * scale * log2(e) - m).
constexpr float kLog2e = 1.4426950408889634f;
// Running-max start value: finite so that exp2(m_old - m_new) never sees
// (-inf) - (-inf).  Any real scaled score is far above it.
constexpr float kMaxInit = -1.0e30f;

// DPP controls (gfx9 encoding).
enum : int {
  kQuadSwap1 = 0xB1,    // quad_perm [1,0,3,2]: lane ^ 1
  kQuadSwap2 = 0x4E,    // quad_perm [2,3,0,1]: lane ^ 2
  kRowHalfMirror = 0x141,  // lane i <-> 7 - i inside each half row
  kRowMirror = 0x140,      // lane i <-> 15 - i inside each row
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over groups of N consecutive lanes (N in {1,2,4,8,16,32,64}); every lane
// of a group receives the group sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_mov<kQuadSwap1>(x);
  if constexpr (N >= 4) x += dpp_mov<kQuadSwap2>(x);
  if constexpr (N >= 8) x += dpp_mov<kRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_mov<kRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Butterfly over lanes that differ in the bits FROM..32 (FROM a power of two):
// combines the rows of a wave that hold the same columns.
template <int FROM>
__device__ __forceinline__ float cross_rows_max(float x) {
  if constexpr (FROM <= 1) x = fmaxf(x, __shfl_xor(x, 1));
  if constexpr (FROM <= 2) x = fmaxf(x, __shfl_xor(x, 2));
  if constexpr (FROM <= 4) x = fmaxf(x, __shfl_xor(x, 4));
  if constexpr (FROM <= 8) x = fmaxf(x, __shfl_xor(x, 8));
  if constexpr (FROM <= 16) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (FROM <= 32) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
template <int FROM>
__device__ __forceinline__ float cross_rows_sum(float x) {
  if constexpr (FROM <= 1) x += __shfl_xor(x, 1);
  if constexpr (FROM <= 2) x += __shfl_xor(x, 2);
  if constexpr (FROM <= 4) x += __shfl_xor(x, 4);
  if constexpr (FROM <= 8) x += __shfl_xor(x, 8);
  if constexpr (FROM <= 16) x += __shfl_xor(x, 16);
  if constexpr (FROM <= 32) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int readlane(int x, int lane) {
  return __builtin_amdgcn_readlane(x, lane);
}

// 16-byte global load: plain global_load_dwordx4.
__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Loads at a wave-uniform base plus a per-lane unsigned 32-bit byte offset,
// the shape the SGPR-base (saddr) form of global loads encodes directly.
__device__ __forceinline__ u32x4_t load16_at(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(base) + byte_off);
}
__device__ __forceinline__ u32x2_t load8_at(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const char*>(base) + byte_off);
}

// Streaming variants: every K/V byte is read once per call, so these carry
// the non-temporal hint (global_load ... nt) to keep them from displacing
// cached data.
__device__ __forceinline__ u32x4_t load16_nt(const void* base, uint32_t byte_off) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(base) + byte_off));
}
__device__ __forceinline__ u32x2_t load8_nt(const void* base, uint32_t byte_off) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const u32x2_t*>(reinterpret_cast<const char*>(base) + byte_off));
}

template <bool NT>
__device__ __forceinline__ u32x4_t kv_load16(const void* base, uint32_t byte_off) {
  if constexpr (NT) return load16_nt(base, byte_off);
  else return load16_at(base, byte_off);
}
template <bool NT>
__device__ __forceinline__ u32x2_t kv_load8(const void* base, uint32_t byte_off) {
  if constexpr (NT) return load8_nt(base, byte_off);
  else return load8_at(base, byte_off);
}

template <bool NT>
__device__ __forceinline__ uint32_t kv_load4(const void* base, uint32_t byte_off) {
  const uint32_t* p =
      reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(base) + byte_off);
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Lane I of every group of four lanes, broadcast to the group (DPP quad_perm).
template <int I>
__device__ __forceinline__ float quad_bcast(float x) {
  return dpp_mov<I | (I << 2) | (I << 4) | (I << 6)>(x);
}

// A wave-uniform int32 read through the scalar data cache (s_load_dword): for
// read-only data such as block tables.  Scalar loads complete on their own
// counter, so they never make the wave wait for its in-flight vector loads.
typedef const __attribute__((address_space(4))) int32_t const_i32;
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
  return *(const_i32*)(p);
}

// 16-byte global -> LDS load (global_load_lds_dwordx4): lane l's 16 bytes
// from `src` land at byte 16 l of the wave-uniform LDS address `dst`,
// without passing through registers; vmcnt tracks completion.  The builtin
// exists only for the device, hence the guard (the host pass compiles the
// kernel body too, and must still emit the launch stub).
__device__ __forceinline__ void load_lds16(const void* src, void* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
#endif
}
// The same with 4 bytes per lane (global_load_lds_dword): lane l's 4 bytes
// land at byte 4 l of `dst`.
__device__ __forceinline__ void load_lds4(const void* src, void* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
#endif
}

// v_max3_f32 as written: the max of three values that are never NaN (the
// plain fmaxf adds an operand-quieting op per input).
__device__ __forceinline__ float max3_nonan(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// The fp16 parts of two weights: hi = both rounded toward zero and packed
// (v_cvt_pkrtz), lo = what hi misses, p - hi in fp32 rounded to nearest fp16,
// packed the same way.  The lo part comes from one mixed-precision FMA per
// value (-hi * 1 + p with hi read as fp16, result written to one half):
// hi + lo keeps ~21 bits of each weight.
__device__ __forceinline__ void split_f16(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p0, p1));
  asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, -%1, 1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(lo)
      : "v"(hi), "v"(p0), "v"(p1));
}

// Transposing 8-byte LDS read (ds_read_b64_tr_b16).  In each group of 16
// lanes, the four 16-bit values that lanes 4r .. 4r + 3 address form row r
// of a 4 x 16 matrix, and lane i receives column i: element r of its result
// is value i % 4 of the piece that lane 4r + i / 4 addresses.  It turns rows
// stored in LDS into the per-lane columns a matrix-core operand needs.
__device__ __forceinline__ half4_t lds_read_tr16(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (__attribute__((address_space(3))) i16x4_t*)(p)));
#else
  return half4_t{};
#endif
}

// Max over the four lanes c, c + 16, c + 32, c + 48 (the four 16-lane
// rows), result in all four.  v_permlane32_swap exchanges the upper half of
// one register with the lower half of the other, v_permlane16_swap the odd
// rows of one with the even rows of the other: with both registers holding
// x, each lane ends up with the pair {x[i], x[i ^ 32]} (then {.., i ^ 16}),
// so one VALU op per stage replaces an LDS-routed shuffle.  Written as
// inline asm with both registers read-write: this compiler folds the
// builtin's second result into its first.  The s_nop covers the wait
// states a permlane needs after a VALU write of its operands.
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane16_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float rows4_max(float x) {
  float a = x, b = x;
  permlane32_swap(a, b);
  float c = fmaxf(a, b), d = c;
  permlane16_swap(c, d);
  return fmaxf(c, d);
}

// Sum over the same four lanes, result in all four.
__device__ __forceinline__ float rows4_sum(float x) {
  float a = x, b = x;
  permlane32_swap(a, b);
  float c = a + b, d = c;
  permlane16_swap(c, d);
  return c + d;
}

// True when any lane of the wave has `pred` set (wave-uniform).
__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}

template <typename T>
struct DType;
template <>
struct DType<float> {
  static constexpr int kBytes = 4;
};
template <>
struct DType<half_t> {
  static constexpr int kBytes = 2;
};

}  // namespace pa
