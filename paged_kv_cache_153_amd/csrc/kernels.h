// kernels.h — internal (C++) launch interface between the C ABI and the HIP
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Every decode kernel works on 16-token tiles of the context; partitions
// are whole tiles.
constexpr int kTile = 16;

struct DecodeArgs {
  float* out;               // [S, Hq, D] final output (single pass)
  float* ws_o;              // [S, Hq, NP, D] partition outputs (normalised)
  float* ws_m;              // [S, Hq, NP] partition max, log2 units
  float* ws_l;              // [S, Hq, NP] partition sum of exp2(y - m)
  const void* q;            // [S, Hq, D]
  const void* kv;           // [NB, 2, Hkv, BS, D]
  const int32_t* bt;        // [S, MB]
  const int32_t* cl;        // [S]
  int64_t num_blocks;       // NB
  int num_seqs;             // S
  int num_q_heads;          // Hq
  int num_kv_heads;         // Hkv
  int max_blocks;           // MB (row stride of bt)
  int max_tokens;           // MB * BS: context lengths are clamped to this
  int num_parts;            // NP
  int part_tokens;          // P (multiple of kTile and of BS); huge when single
  int single;               // 1: write `out` directly; 0: write ws_*
  float scale_log2;         // scale * log2(e)
  int variant;              // MFMA: 1 = one tile in flight per wave, 0 = two
};

// Each returns 0 on success, 1 if the (dtype, D, BS, G) combination has no
// instantiation, or 2 if the launch failed (hipGetLastError has the code).
int launch_decode_valu(const DecodeArgs& a, int dtype, int head_dim, int block_size, int group,
                       int waves, hipStream_t stream);
int launch_decode_mfma(const DecodeArgs& a, int dtype, int head_dim, int block_size, int group,
                       int waves, hipStream_t stream);
int launch_merge(const DecodeArgs& a, int head_dim, hipStream_t stream);
int launch_cache_write(const void* key, const void* value, void* kv, const int64_t* slots,
                       int64_t num_tokens, const int32_t* cow_pairs, int64_t num_cow,
                       int64_t num_blocks, int num_kv_heads, int head_dim, int block_size,
                       int elem_bytes, hipStream_t stream);

}  // namespace pa
