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

// 8-bit append into one or two caches of the same code set (grid.y picks);
// scale_mode is a pkv_scale_mode.
int launch_kv_append_q8(const QTargetArgs* targets, int num_targets, const int64_t* slot_mapping,
                        int num_tokens, int num_kv_heads, int head_dim, int num_blocks,
                        int src_dtype, int code_dtype, int scale_mode, hipStream_t stream);

int launch_copy_blocks(void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                       const int32_t* src, const int32_t* dst, int n, int num_kv_heads,
                       int block_bytes, int num_blocks, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scales;   // 8-bit K only: [num_blocks][num_kv_heads] (x 16 per token)
  const float* v_scales;   // 8-bit V only: likewise
  int k_tok, v_tok;        // 1: the scales are per (slot, head): [num_blocks][num_kv_heads][16]
  const float* k_chan;     // 8-bit K only, may be NULL: [num_kv_heads][head_dim]
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale;
  void* out;
  float* o_part;           // [B*Hq][part_stride][D] when split
  float* ml_part;          // [B*Hq][part_stride][2] when split
  int num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks;
  int part_blocks, num_parts;
  // workspace slots per row: num_parts for the per-sequence pass, then
  // group_num_parts for the shared-prefix pass
  int part_stride;
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
  // shared-prefix groups (num_groups = 0: none): sequences
  // [group_seq_start[g], group_seq_start[g+1]) share their first
  // group_blocks[g] table entries, which one pass reads once for all of them
  const int32_t* group_seq_start;
  const int32_t* group_blocks;
  int num_groups, group_max_seqs, group_max_blocks;
  int group_part_blocks, group_num_parts;   // split of a group's shared blocks
  int group_qchunks;                        // 64-row chunks of a group's queries
  // the step's append carried by the attention launch (new_slots NULL:
  // none): k_new, v_new [B][Hkv][D]; sequence b's token goes to slot
  // new_slots[b] of the caches, which are then also written
  const void* k_new;
  const void* v_new;
  const int64_t* new_slots;
  void* k_cache_rw;
  void* v_cache_rw;
  // workgroups of the group pass (0: none); they lead the combined launch
  // and write workspace slots [num_parts, part_stride) of their rows
  int group_wgs;
};

// A list of `natt` blocks uses min(ceil(natt / T), P) of P pieces, cut
// equally (T = the planned piece size): piece p covers entries [j0, j1).
struct SeqParts {
  int n, j0, j1;
  __device__ __forceinline__ SeqParts(int natt, int T, int P, int p) {
    n = natt > 0 ? min((natt + T - 1) / T, P) : 0;
    const int pb = n > 0 ? (natt + n - 1) / n : 0;
    j0 = p * pb;
    j1 = min(j0 + pb, natt);
  }
};

// (partition, KV head, sequence) of the k-th workgroup of the cache pass:
// the partition varies fastest, then the KV head.  (Workgroups go to the
// XCDs round robin, so with one partition an XCD takes one KV head of
// every sequence.  The sequence varying fastest instead, so that every XCD
// takes all heads, measured no faster on the 70B-shaped step and 7-10 us
// slower on the uneven Llama-3-8B and shared-prefix layers.)  The
// exception is an 8-bit cache with one partition and at most 8 KV heads:
// there the sequence varies fastest, so that one XCD reads every KV head
// of a block and each 64-byte line of per-(block, head) scales once, where
// eight XCDs would each fetch it for 4 bytes (70B-shaped fp8 step: 88.0 ->
// 86.9 us, HBM traffic 1.03 -> 1.00 of the algorithmic bytes).  With many
// KV heads a block's tiles are better read together, by consecutive
// workgroups, than the scale lines are shared (13B-shaped fp8 layer, 40
// KV heads: 109.5 -> 92.2 us per layer, and 52.4 -> 48.0 us with the
// shared-prefix pass).
struct Unit { int p, h, b; };
__device__ __forceinline__ Unit unit_of(const DecodeArgs& a, int k) {
  Unit u;
  u.p = k % a.num_parts;
  const int rest = k / a.num_parts;
  const bool eight_bit = a.kv_dtype == PKV_FP8_E4M3 || a.kv_dtype == PKV_INT8 ||
                         a.v_dtype == PKV_FP8_E4M3 || a.v_dtype == PKV_INT8;
  if (eight_bit && a.num_parts == 1 && a.num_kv_heads <= 8) {
    u.b = rest % a.num_seqs;
    u.h = rest / a.num_seqs;
    return u;
  }
  u.h = rest % a.num_kv_heads;
  u.b = rest / a.num_kv_heads;
  return u;
}

// One group as both passes see it, clamped so that they always agree on
// which blocks of which sequence the group pass covers.
struct PrefixGroup {
  int s0, nseq, nblk;   // first sequence, sequences covered, shared blocks
};

__device__ __forceinline__ PrefixGroup prefix_group(const DecodeArgs& a, int g) {
  PrefixGroup r;
  const int s0 = min(max(a.group_seq_start[g], 0), a.num_seqs);
  const int s1 = min(max(a.group_seq_start[g + 1], s0), a.num_seqs);
  r.s0 = s0;
  r.nseq = min(s1 - s0, a.group_max_seqs);
  r.nblk = r.nseq > 0 ? min(max(a.group_blocks[g], 0), a.group_max_blocks) : 0;
  return r;
}

// Leading blocks of sequence b that the group pass covers (0 outside every
// group): the last group starting at or before b, if b is among its
// covered sequences.
__device__ __forceinline__ int prefix_blocks_of_seq(const DecodeArgs& a, int b) {
  if (a.num_groups <= 0) return 0;
  int lo = 0, hi = a.num_groups;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.group_seq_start[mid] <= b) lo = mid; else hi = mid;
  }
  const PrefixGroup pg = prefix_group(a, lo);
  return (b >= pg.s0 && b < pg.s0 + pg.nseq) ? pg.nblk : 0;
}

// Partition plan: depends on dims only.
void plan_partitions(const pkv_decode_dims& d, int* part_blocks, int* num_parts);
// Shared-prefix plan (dims->prefix_groups > 0): blocks per piece, pieces,
// 64-row query chunks per group.
void plan_groups(const pkv_decode_dims& d, int* part_blocks, int* num_parts, int* qchunks);
size_t workspace_bytes_for(const pkv_decode_dims& d);

int launch_decode(const DecodeArgs& a, hipStream_t stream);

int launch_hbm_read(const void* buf, size_t bytes, uint32_t* sink, int sink_words,
                    hipStream_t stream);

// The attention launch's access pattern without its arithmetic (head_dim
// 128; K and V of one element width): sink has one word per workgroup.
int launch_paged_read_probe(const DecodeArgs& a, uint32_t* sink, hipStream_t stream);

}  // namespace pkv
