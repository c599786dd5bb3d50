// Internal launcher declarations shared by the C-ABI shim and the kernels.
#pragma once

#include "../../include/pagedkv.h"
#include "pkv_common.h"

namespace pkv {

int launch_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                     void* k_cache, void* v_cache, int num_tokens, int num_kv_heads,
                     int row_bytes, int num_blocks, hipStream_t stream);

// One cache to quantise into: source rows, codes, per-(block, head) scales
// and optional per-(head, channel) factors.
struct QTargetArgs {
  const void* src;
  void* cache;
  float* scales;
  const float* chan;
};

// 8-bit append into one or two caches of the same code set (grid.y picks).
int launch_kv_append_q8(const QTargetArgs* targets, int num_targets, const int64_t* slot_mapping,
                        int num_tokens, int num_kv_heads, int head_dim, int num_blocks,
                        int src_dtype, int code_dtype, bool first_write, hipStream_t stream);

int launch_copy_blocks(void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                       const int32_t* src, const int32_t* dst, int n, int num_kv_heads,
                       int block_bytes, int num_blocks, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scales;   // 8-bit caches only: [num_blocks][num_kv_heads]
  const float* v_scales;   // 8-bit caches only
  const float* k_chan;     // 8-bit K only, may be NULL: [num_kv_heads][head_dim]
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale;
  void* out;
  float* o_part;           // [B*Hq][num_parts][D] when split
  float* ml_part;          // [B*Hq][num_parts][2] when split
  int num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks;
  int part_blocks, num_parts;
  int split;               // partial results go to the workspace (then merged)
  int window, sinks;       // sliding window (0 = off) and attention-sink tokens
  // full-precision sink tiles (q's dtype, [num_sink_tiles][Hkv][16][D]); when
  // set, positions < sinks are attended from them by the merge kernel and
  // the cache pass skips them
  const void* sink_k;
  const void* sink_v;
  const int32_t* sink_of_seq;
  int num_sink_tiles;
  int sink_tiles;
  int q_dtype, kv_dtype, v_dtype, out_dtype;   // kv_dtype is K's
};

// Partition plan: depends on dims only.
void plan_partitions(const pkv_decode_dims& d, int* part_blocks, int* num_parts);
size_t workspace_bytes_for(const pkv_decode_dims& d);

int launch_decode(const DecodeArgs& a, hipStream_t stream);

int launch_hbm_read(const void* buf, size_t bytes, uint32_t* sink, int sink_words,
                    hipStream_t stream);

}  // namespace pkv
