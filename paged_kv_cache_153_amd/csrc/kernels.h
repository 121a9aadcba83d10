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

// How decode work is cut into workgroups (see decode_schedule.h).
constexpr int kScheduleSingle = 0;     // one workgroup per (sequence, KV head)
constexpr int kSchedulePartition = 1;  // ... per (sequence, KV head, partition)
constexpr int kScheduleBalanced = 2;   // W workgroups, equal tile slices
// Sequences the balanced schedule handles: its tile prefix lives in LDS.
constexpr int kBalancedMaxSeqs = 1024;
// Workgroups one launch may have: a dispatch counts at most 2^32 - 1
// work-items, and every decode and prefill workgroup has 256.
constexpr long long kMaxGridWorkgroups = (1LL << 32) / 256 - 1;

struct DecodeArgs {
  float* out;               // [S, Hq, D] final output (single pass)
  float* ws_o;              // [S, Hq, NP, D] partition outputs (normalised)
  float* ws_m;              // [S, Hq, NP] partition max, log2 units
  float* ws_l;              // [S, Hq, NP] partition sum of exp2(y - m)
  int* ws_cut;              // balanced: per workgroup w, the segment whose tiles the
                            // boundary at the start of w's slice cuts first (kCutInts
                            // ints; s < 0: none)
  const void* q;            // [S, Hq, D]
  const void* kv;           // [NB, 2, Hkv, BS, D]
  const float* kv_scales;   // INT8 pool: [NB, Hkv, 2, BS] row scales; else null
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
  int schedule;             // kScheduleSingle / kSchedulePartition / kScheduleBalanced
  int num_workgroups;       // balanced: W workgroups (grid size)
  float scale_log2;         // scale * log2(e)
  int variant;              // MFMA: 1 = one tile in flight per wave, 0 = two
  int cached_kv;            // 1: plain K/V loads; 0: non-temporal (streaming) loads
  int window;               // > 0: attend to the last `window` tokens only; 0: all
  int seg_cost;             // balanced: tile-equivalents charged per (sequence, KV head)
};

// Balanced schedule: ints per workgroup in ws_cut: sequence, KV head, first
// and last contributing workgroup, slot of the first one (then padding).
constexpr int kCutInts = 8;

// Causal multi-token queries (a prefill chunk per sequence).
struct PrefillArgs {
  float* out;               // [total_q, Hq, D]
  const void* q;            // [total_q, Hq, D] f16
  const void* kv;           // [NB, 2, Hkv, BS, D] f16 (or int8 codes)
  const float* kv_scales;   // INT8 pool: [NB, Hkv, 2, BS] row scales; else null
  const int32_t* bt;        // [S, MB]
  const int32_t* cl;        // [S] context lengths, chunk included
  const int32_t* qstart;    // [S + 1] first query row of each sequence
  int64_t num_blocks;
  int num_seqs;
  int total_queries;        // rows of q and out: query_start entries are bounded by it
  int num_q_heads;
  int num_kv_heads;
  int max_blocks;
  int max_tokens;           // MB * BS
  int qblocks;              // workgroups per (sequence, KV head)
  float scale_log2;
  int window;               // > 0: a query sees the last `window` tokens up to itself
};
int prefill_columns_per_workgroup();     // f16 pools
int prefill_i8_columns_per_workgroup();  // INT8 pools
int launch_prefill_mfma(const PrefillArgs& a, int head_dim, int block_size, int group,
                        hipStream_t stream);
// INT8 pool (codes + row scales; query in f16).
int launch_prefill_mfma_i8(const PrefillArgs& a, int head_dim, int block_size, int group,
                           hipStream_t stream);

// Each returns 0 on success, 1 if the (dtype, D, BS, G) combination has no
// instantiation, or 2 if the launch failed (hipGetLastError has the code).
int launch_decode_valu(const DecodeArgs& a, int dtype, int head_dim, int block_size, int group,
                       int waves, hipStream_t stream);
int launch_decode_mfma(const DecodeArgs& a, int dtype, int head_dim, int block_size, int group,
                       int waves, hipStream_t stream);
// INT8 pool (codes + row scales; query in f16).
int launch_decode_valu_i8(const DecodeArgs& a, int head_dim, int block_size, int group,
                          hipStream_t stream);
int launch_decode_mfma_i8(const DecodeArgs& a, int head_dim, int block_size, int group,
                          hipStream_t stream);
int launch_merge(const DecodeArgs& a, int head_dim, hipStream_t stream);
int launch_merge_balanced(const DecodeArgs& a, int head_dim, hipStream_t stream);
// Resident workgroups per compute unit of the kernel a launch would pick
// (0 if none): sizes the balanced grid.
int decode_valu_occupancy(const DecodeArgs& a, int dtype, int head_dim, int block_size,
                          int group);
int decode_mfma_occupancy(const DecodeArgs& a, int head_dim, int block_size, int group);
int decode_valu_i8_occupancy(const DecodeArgs& a, int head_dim, int block_size, int group);
int decode_mfma_i8_occupancy(const DecodeArgs& a, int head_dim, int block_size, int group);
// elem_bytes 4 / 2: byte copies; 1: INT8 pool, f16 inputs quantised per
// row with their scales written to `scales` ([NB, Hkv, 2, BS] floats).
int launch_stage(void* dst, const void* src, int64_t bytes, hipStream_t stream);
int launch_stage_write(void* stage_dst, const void* stage_src, int64_t stage_bytes,
                       const void* key, const void* value, void* kv, float* scales,
                       const int64_t* slots, int64_t num_tokens, const int32_t* cow_pairs,
                       int64_t num_cow, int64_t num_blocks, int num_kv_heads, int head_dim,
                       int block_size, int elem_bytes, hipStream_t stream);
int launch_cache_write(const void* key, const void* value, void* kv, float* scales,
                       const int64_t* slots, int64_t num_tokens, const int32_t* cow_pairs,
                       int64_t num_cow, int64_t num_blocks, int num_kv_heads, int head_dim,
                       int block_size, int elem_bytes, hipStream_t stream);

}  // namespace pa
