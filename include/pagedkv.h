/*
 * pagedkv — single-query decode attention over a paged KV cache (gfx950).
 *
 * The operations follow the source pages:
 *   - "KV Cache from first principles" (ldpk.cn/news/58971), 2.1: attention
 *     is softmax(q K^T * scale) V; 2.2: at a decode step the one new query
 *     attends to every cached position; 2.3: each step writes the new token's
 *     K and V at the current length, which then grows by one; 4.3: the kernel
 *     reads K and V through the block table from scattered places.
 *   - "The KV Cache memory ledger: PagedAttention and continuous batching"
 *     (gcssc.sfwss.com/posts/kv-cache-budget.html), 4: fixed 16-token blocks,
 *     a per-sequence block table, locate(seq, pos) = table[pos / 16] * 16 +
 *     pos % 16; prefix sharing points several tables at the same blocks;
 *     2: grouped-query attention (g query heads share one K/V head);
 *     7: 8-bit K/V with one scale per head, K (the more sensitive) in FP8
 *     with V in INT8 as a mixed form.
 *   - "KV Cache from first principles" 5.2: K has outlier channels, which
 *     per-channel factors absorb.
 *
 * Memory layout (all row-major, contiguous, device memory):
 *   k_cache, v_cache  [num_blocks][num_kv_heads][block_size=16][head_dim]
 *                     one (block, kv_head) tile is a contiguous 16*head_dim run
 *   block_tables      int32 [num_seqs][max_blocks_per_seq]; entries past
 *                     ceil(context_len / 16) are never read
 *   context_lens      int32 [num_seqs]: tokens to attend, the new one included
 *   q, out            [num_seqs][num_q_heads][head_dim]
 *   k_scales,v_scales fp32 [num_blocks][num_kv_heads] (8-bit caches only)
 *   k_channel_scales  fp32 [num_kv_heads][head_dim] (8-bit K, optional)
 *   slot_mapping      int64 [num_tokens]: flat slot = block * 16 + offset,
 *                     -1 = skip this token
 *   query head i reads KV head i / (num_q_heads / num_kv_heads).
 *
 * Ownership: the caller owns every buffer.  The library allocates nothing,
 * keeps no mutable global state, and every call is asynchronous on `stream`
 * (NULL = the default stream) with no host/device synchronisation inside.
 *
 * Errors: every call returns a pkv_status.  Arguments are checked on the host
 * before anything is launched, so a non-zero status means nothing ran.
 * Device-side faults surface at the caller's next synchronisation.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(PKV_BUILDING_LIBRARY)
#define PKV_API __attribute__((visibility("default")))
#else
#define PKV_API
#endif

#define PKV_VERSION 181  /* 1.8.1 */
#define PKV_BLOCK_SIZE 16
/* Device scratch held by pkv_paged_decode_attn_noalloc, per device. */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)

typedef enum {
  PKV_F32 = 0,
  PKV_F16 = 1,
  PKV_BF16 = 2,
  PKV_FP8_E4M3 = 3, /* OCP e4m3fn: bias 7, max 448, no inf, NaN = S.1111.111 */
  PKV_INT8 = 4      /* symmetric two's-complement codes -127..127 (-128 unused) */
} pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,      /* a required pointer is NULL */
  PKV_ERR_SHAPE = -2,     /* non-positive size, Hq % Hkv != 0, g not in {1,2,4,8},
                             head_dim not in {64,128}, block_size != 16,
                             negative window or sinks */
  PKV_ERR_DTYPE = -3,     /* unsupported dtype or dtype combination */
  PKV_ERR_WORKSPACE = -4, /* workspace missing or smaller than required */
  PKV_ERR_LAUNCH = -5,    /* the HIP runtime refused a launch */
  PKV_ERR_NO_BLOCKS = -6, /* block manager: not enough free blocks (nothing changed) */
  PKV_ERR_SEQUENCE = -7,  /* block manager: unknown or duplicate sequence id */
  PKV_ERR_SCRATCH = -8    /* pkv_paged_decode_attn_noalloc: the call's workspace would
                             exceed PKV_NOALLOC_SCRATCH_BYTES (nothing ran) */
} pkv_status;

typedef struct {
  int32_t num_seqs;            /* B */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hkv; Hq / Hkv in {1, 2, 4, 8} */
  int32_t head_dim;            /* D in {64, 128} */
  int32_t block_size;          /* must be 16 */
  int32_t num_blocks;          /* physical blocks in the pool (per cache) */
  int32_t max_blocks_per_seq;  /* row length of block_tables */
  int32_t q_dtype;             /* pkv_dtype */
  int32_t kv_dtype;            /* pkv_dtype (of K, where V may differ) */
  int32_t out_dtype;           /* pkv_dtype */
  int32_t partition_blocks;    /* blocks per context partition; 0 = automatic */
  int32_t window;              /* sliding window W: attend only the last W positions
                                  (0 = the whole context) */
  int32_t sinks;               /* with W > 0, also attend the first `sinks` positions */
  int32_t sink_tiles;          /* 1: positions < sinks come from full-precision side tiles
                                  (pkv_paged_decode_attn_quant only; 1 <= sinks <= 16,
                                  with or without a window); 0: from the cache */
  int32_t total_blocks;        /* optional hint, 0 = unknown: sum over the sequences of
                                  ceil(context_len / 16).  When the batch is much lighter
                                  than max_blocks_per_seq suggests, the split plan sizes
                                  its pieces from it; results do not depend on it */
  int32_t prefix_groups;       /* G >= 0 shared-prefix groups (the _prefix entry points
                                  only; 0 everywhere else) */
  int32_t prefix_max_seqs;     /* with G > 0: >= the sequence count of every group */
  int32_t prefix_max_blocks;   /* with G > 0: >= every group's shared block count,
                                  <= max_blocks_per_seq */
} pkv_decode_dims;

/*
 * Per-step append ("KV Cache from first principles" 2.3; "The KV Cache memory
 * ledger" 4, locate()).  For every t < num_tokens with slot_mapping[t] >= 0,
 * copies k_new[t][h][:] to k_cache[slot / 16][h][slot % 16][:] and v_new to
 * v_cache likewise, for every KV head h.  A bit-exact copy: no arithmetic.
 *   k_new, v_new: [num_tokens][num_kv_heads][head_dim] of `dtype`.
 *   Slots must be distinct (duplicates race).  Slots >= num_blocks * 16 are
 *   skipped like -1.  dtype: F32, F16 or BF16.  head_dim: any multiple of
 *   16 / sizeof(element) up to 1024 (the attention calls need 64 or 128).
 *   v_new and v_cache may both be NULL: K alone is written (a 16-bit K next
 *   to an 8-bit V, whose rows pkv_kv_append_quant writes).
 *   Does not touch context lengths: the caller advances them.
 */
PKV_API int pkv_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                  void* k_cache, void* v_cache, int32_t num_tokens, int32_t num_kv_heads,
                  int32_t head_dim, int32_t num_blocks, int32_t block_size, int32_t dtype,
                  hipStream_t stream);

typedef enum {
  PKV_SCALE_GIVEN = 0,       /* scales are set by the caller (e.g. calibrated) */
  PKV_SCALE_FIRST_WRITE = 1, /* a block's first token (offset 0) sets its scale */
  PKV_SCALE_PER_TOKEN = 2    /* one scale per (slot, head): scales are fp32
                                [NB][Hkv][16], and every token sets its own */
} pkv_scale_mode;

/*
 * FP8 append, quantising on write ("The KV Cache memory ledger" 7: 8-bit
 * K/V with one scale per head; "Why does KV Cache eat GPU memory?": FP8 KV
 * needs calibrated scales).  Caches hold e4m3fn codes [NB][Hkv][16][D];
 * k_scales, v_scales are fp32 [NB][Hkv] (device, read and, in first-write
 * mode, written).  k_new, v_new: [T][Hkv][D] of src_dtype (F32/F16/BF16).
 * For every t with 0 <= slot < NB*16, blk = slot/16, off = slot%16, head h:
 *   - PKV_SCALE_FIRST_WRITE and off == 0: scale[blk][h] = max_d |x| / 448 in
 *     fp32 (1.0 if that max is 0), set for all such tokens of the call before
 *     any token is quantised;
 *   - code = round-to-nearest-even(clamp(x / scale[blk][h], -448, 448)), the
 *     quotient a correctly rounded fp32 division; values beyond 448*scale
 *     saturate; NaN stays NaN.
 * head_dim must be a multiple of 16 (<= 1024).  Slots must be distinct.
 */
PKV_API int pkv_kv_append_fp8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                              void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                              int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              int32_t num_blocks, int32_t block_size, int32_t src_dtype,
                              int32_t scale_mode, hipStream_t stream);

/*
 * 8-bit append into ONE cache (K or V), quantising on write, for the fp8,
 * int8 and mixed (K fp8, V int8; K 16-bit, V 8-bit) layouts ("The KV Cache
 * memory ledger" 7; "KV Cache from first principles" 5.2: per-channel
 * factors for K, per-token scales).
 * cache: codes of cache_dtype (FP8_E4M3 or INT8) [NB][Hkv][16][D]; scales:
 * fp32 [NB][Hkv], or [NB][Hkv][16] with PKV_SCALE_PER_TOKEN (read and, in
 * first-write and per-token modes, written); channel_scales: NULL or fp32
 * [Hkv][D] (device).  x_new: [T][Hkv][D] of src_dtype.  With
 * QMAX = 448 (fp8) or 127 (int8), for every t with 0 <= slot < NB*16:
 *   - y = x / channel_scales[h][d] (correctly rounded fp32), or y = x;
 *   - PKV_SCALE_FIRST_WRITE and off == 0: scale[blk][h] = max_d |y| / QMAX
 *     (1.0 if that max is 0), set for all such tokens before any is quantised;
 *   - PKV_SCALE_PER_TOKEN: scale[blk][h][off] = max_d |y| / QMAX (1.0 if
 *     that max is 0) for every token, from its own row;
 *   - code = nearest code, ties to even, of clamp(y / scale, -QMAX, QMAX)
 *     (correctly rounded fp32 quotient); NaN stays NaN (fp8) or becomes 0
 *     (int8).
 * head_dim must be a multiple of 16 (<= 1024).  Slots must be distinct.
 */
PKV_API int pkv_kv_append_quant(const void* x_new, const int64_t* slot_mapping, void* cache,
                                float* scales, const float* channel_scales, int32_t num_tokens,
                                int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                int32_t block_size, int32_t src_dtype, int32_t cache_dtype,
                                int32_t scale_mode, hipStream_t stream);

/*
 * Bytes of workspace the decode attention calls need for `dims`; 0 when the
 * context is not split.  Depends only on `dims` (never on the device or on
 * context_lens), so a caller can size it once.  Returns 0 for invalid dims.
 * The workspace holds the partial results of the context pieces (per
 * query row: output, reference maximum and sum of each piece), which a
 * second kernel of the same call merges; calls sharing one workspace must
 * not overlap in time (one stream, or synchronised).
 */
PKV_API size_t pkv_decode_workspace_bytes(const pkv_decode_dims* dims);

/* Number of context partitions the attention call will use for `dims` (>= 1),
 * or a negative pkv_status for invalid dims. */
PKV_API int pkv_decode_num_partitions(const pkv_decode_dims* dims);

/*
 * Decode attention ("KV Cache from first principles" 2.1-2.2, 4.3; "The KV
 * Cache memory ledger" 2, 4).  For each sequence b and query head i, with
 * L = context_lens[b] and h = i / g:
 *   out[b][i][:] = sum_t softmax_t(scale * <q[b][i], K_t>) V_t,  t < L,
 * where K_t, V_t are read at locate(b, t).  With dims->window = W > 0 the
 * positions are restricted to t >= L - W plus t < dims->sinks ("KV Cache
 * from first principles" 5.3: sliding window and attention-sink tokens).
 * L = 0 gives a zero row.  Block
 * ids outside [0, num_blocks) and positions past max_blocks_per_seq * 16 are
 * ignored (the caller must not pass them).
 * Non-fp8 dtypes: q, caches and out all F32, or all F16, or all BF16.
 * Sums are fp32 and the scores exact products of the stored values; each
 * softmax weight enters the weighted sum of V with at least 11 significant
 * bits (about 22 for f16 and 16 for bf16 caches at head_dim 128 with 4 or
 * 8 query heads per KV head, where the products run on the matrix cores).
 * The output is rounded once (nearest-even).
 * workspace: device buffer of at least pkv_decode_workspace_bytes(dims)
 * bytes (may be NULL when that is 0), used only during this call.
 */
PKV_API int pkv_paged_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, float scale,
                          void* out, const pkv_decode_dims* dims, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_paged_decode_attn without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Arguments, results and errors
 * are those of pkv_paged_decode_attn; when the context is split, the
 * partial results go to a static device array of PKV_NOALLOC_SCRATCH_BYTES
 * that the library holds on every device it runs on (zero-filled when the
 * library is loaded, kept until the process ends) instead of a caller
 * workspace.  A call whose workspace (pkv_decode_workspace_bytes) would
 * exceed that returns PKV_ERR_SCRATCH and runs nothing.  The call allocates
 * nothing: the array's device address is looked up once per device, on
 * the first call that splits.  Every call on a device shares that device's
 * array and leaves its contents there, so calls on one device that may
 * overlap (two streams, two host threads) race and must be ordered by the
 * caller.
 */
PKV_API int pkv_paged_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* block_tables, const int32_t* context_lens,
                                          float scale, void* out, const pkv_decode_dims* dims,
                                          hipStream_t stream);

/*
 * FP8 variant ("The KV Cache memory ledger" 7: 8-bit K/V, one scale per head).
 * kv_dtype must be FP8_E4M3; q and out are F16, BF16 or F32.  The value of a
 * cached element is decode(code) * scale[block][kv_head].
 * Precision: the codes are widened exactly; the query (times K's channel
 * factors, where given) is multiplied by a power of two -- one per query
 * head at head_dim 128 with 4 or 8 query heads per KV head, one per KV
 * head's group of query heads otherwise -- chosen so that the largest
 * element of the head (group) lands in [2^14, 2^15), then rounded to f16
 * (nearest even); the scores undo the power of two.  So each query element
 * keeps 11 significant bits (an f32 query loses its 13 lowest); elements
 * more than 2^28 times smaller than that largest fall into f16's subnormal
 * range and keep fewer, and those more than 2^39 times smaller become 0.  Scores and sums are fp32; each
 * softmax weight enters the weighted sum of V with at least 11 significant
 * bits (about 22 at head_dim 128 with 4 or 8 query heads per KV head).
 * Weights are formed as (probability <= 256) * V's scale and held in f16,
 * so V's scales must stay below 255 (with scale = amax / 448: |V| below
 * about 114000); beyond that a weight can overflow.
 */
PKV_API int pkv_paged_decode_attn_fp8(const void* q, const void* k_cache, const void* v_cache,
                              const float* k_scales, const float* v_scales,
                              const int32_t* block_tables, const int32_t* context_lens,
                              float scale, void* out, const pkv_decode_dims* dims,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Arguments of the 8-bit decode entry point beyond those of the others. */
typedef struct {
  const float* k_scales;          /* fp32 [num_blocks][num_kv_heads], required */
  const float* v_scales;          /* fp32 [num_blocks][num_kv_heads], required */
  const float* k_channel_scales;  /* fp32 [num_kv_heads][head_dim], or NULL */
  int32_t v_dtype;                /* V's pkv_dtype (dims->kv_dtype is K's) */
  /* With dims->sink_tiles = 1: full-precision sink tiles, q's dtype,
   * [num_sink_tiles][num_kv_heads][16][head_dim]; sequence b's position
   * p < dims->sinks is read from tile sink_tiles_of_seq[b], offset p
   * (write it there with pkv_kv_append).  A tile id outside
   * [0, num_sink_tiles) leaves that sequence without sink tokens. */
  const void* k_sink;
  const void* v_sink;
  const int32_t* sink_tiles_of_seq;  /* int32 [num_seqs] */
  int32_t num_sink_tiles;
  /* 1: the scales are fp32 [num_blocks][num_kv_heads][16], one per (slot,
   * head) (written by pkv_kv_append_quant with PKV_SCALE_PER_TOKEN); 0: one
   * per (block, head) as above.  K and V choose independently. */
  int32_t k_scales_per_token;
  int32_t v_scales_per_token;
} pkv_quant_params;

/*
 * 8-bit variant with mixed formats, per-channel K factors and full-precision
 * sink tokens ("The KV Cache memory ledger" 7: K in FP8 with V in INT8, and
 * attention-sink tokens kept at their original precision; "KV Cache from
 * first principles" 5.2: per-channel factors for K's outlier channels).
 * dims->kv_dtype is K's format and p->v_dtype V's: (FP8_E4M3, FP8_E4M3) with
 * the q/out pairs of pkv_paged_decode_attn_fp8, or (FP8_E4M3, INT8) and
 * (INT8, INT8) with q and out both F16 or both BF16, or a 16-bit K with an
 * 8-bit V ("KV Cache from first principles" 5.2: quantise only V, keep K in
 * fp16): (F16 or BF16, FP8_E4M3 or INT8) with q and out of K's type, K read
 * as stored, k_scales and k_channel_scales NULL.  A cached 8-bit K element
 * is decode(code) * k_scales[block][h] * k_channel_scales[h][d] (the last
 * factor 1 when k_channel_scales is NULL), a V element decode(code) *
 * v_scales[block][h]; with per-token scales the scale is that of the
 * element's own slot, [block][h][offset].  int8 codes decode to their
 * integer value.  With
 * dims->sink_tiles = 1 the first dims->sinks positions are read as stored
 * from the side tiles (see pkv_quant_params); the attended positions are
 * those of pkv_paged_decode_attn, and the call always splits the context
 * (pkv_decode_workspace_bytes > 0).  Precision: as for
 * pkv_paged_decode_attn_fp8 (int8 codes are also widened exactly); the
 * side tiles are read as stored and attended in fp32.
 */
PKV_API int pkv_paged_decode_attn_quant(const void* q, const void* k_cache, const void* v_cache,
                                        const pkv_quant_params* p, const int32_t* block_tables,
                                        const int32_t* context_lens, float scale, void* out,
                                        const pkv_decode_dims* dims, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step in one launch: pkv_kv_append of each sequence's new token
 * followed by pkv_paged_decode_attn ("KV Cache from first principles" 2.2-2.3:
 * the new token's K and V are written at the current length, which then
 * counts it, and the new query attends to every cached position, its own
 * included).  Results and cache contents equal those of the two calls.
 *   k_new, v_new: [num_seqs][num_kv_heads][head_dim] of the caches' dtype:
 *     token b is sequence b's new token;
 *   slot_mapping: int64 [num_seqs], the slot of sequence b's position
 *     context_lens[b] - 1 (its last), or -1 for no new token; slots outside
 *     the pool are skipped.  A slot elsewhere in the sequence gives
 *     undefined results (its block may be read before it is written).
 * Caches F32, F16 or BF16 (q, caches and out of one type, as for
 * pkv_paged_decode_attn); no sink tiles or prefix groups.
 */
PKV_API int pkv_paged_decode_step(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                                  const void* q, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  float scale, void* out, const pkv_decode_dims* dims,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decode attention for batches whose sequences share prefix blocks ("The KV
 * Cache memory ledger" 4: prefix sharing points several block tables at the
 * same physical blocks; "Large-model inference KV Cache memory
 * optimisation" 3.1-3.3: shared blocks are stored once, whole blocks only).
 * The result is that of pkv_paged_decode_attn; only the order of the reads
 * changes: a group's shared blocks are read once and scored against the
 * queries of all its sequences together (a matrix product on the matrix
 * cores), the rest of each sequence as usual, and the two parts are merged
 * by log-sum-exp.  The shared part keeps the precision stated for
 * pkv_paged_decode_attn's matrix-core products: each softmax weight enters
 * the sum of V with about 22 (f16) or 16 (bf16) significant bits.
 *   group_seq_start: int32 device [G + 1], nondecreasing: group g is the
 *     sequences [group_seq_start[g], group_seq_start[g + 1]);
 *   group_prefix_blocks: int32 device [G]: every sequence of group g has the
 *     same first group_prefix_blocks[g] block-table entries (those of the
 *     group's first sequence are read), each a full block: 16 * that count
 *     <= context_lens[b] for every b of the group.
 * Sequences outside every group, and past dims->prefix_max_seqs in a group,
 * are attended as usual; counts are clamped to [0, dims->prefix_max_blocks].
 * Tables that break the sharing promise, or unsorted starts, give undefined
 * results but never out-of-bounds accesses.  dims->prefix_groups = G with
 * G * ceil(prefix_max_seqs * g / 64) <= 65535; window and sink tiles must be
 * off; q, caches and out all F16 or all BF16.  Always splits (workspace > 0).
 */
PKV_API int pkv_paged_decode_attn_prefix(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* group_seq_start,
                                         const int32_t* group_prefix_blocks,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         float scale, void* out, const pkv_decode_dims* dims,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/*
 * One decode step with an 8-bit cache in one launch: the quantise-on-write
 * append of each sequence's new token followed by pkv_paged_decode_attn_quant
 * ("KV Cache from first principles" 2.2-2.3: write the new token at the
 * current length, then attend to every position, its own included; "The KV
 * Cache memory ledger" 7: 8-bit K/V with scales; "KV Cache from first
 * principles" 5.2: per-token scales, or V alone quantised).
 *   k_new, v_new: [num_seqs][num_kv_heads][head_dim] of q's dtype: token b
 *     is sequence b's new token; slot_mapping: int64 [num_seqs], the slot of
 *     sequence b's position context_lens[b] - 1, or -1 for none (slots
 *     outside the pool are skipped; a slot elsewhere gives undefined
 *     results).
 *   p, dims, caches and the remaining arguments as for
 *     pkv_paged_decode_attn_quant, without sink tiles (dims->sink_tiles 0).
 * The new rows are written as pkv_kv_append_quant writes them with
 * PKV_SCALE_GIVEN (the block's scale in k_scales / v_scales is read) or,
 * for a cache with per-token scales, PKV_SCALE_PER_TOKEN (the token's slot
 * scale is written first); a 16-bit K is copied as pkv_kv_append copies it.
 * Codes, scales, output: those of the separate calls.
 */
PKV_API int pkv_paged_decode_step_quant(const void* k_new, const void* v_new,
                                        const int64_t* slot_mapping, const void* q, void* k_cache,
                                        void* v_cache, const pkv_quant_params* p,
                                        const int32_t* block_tables, const int32_t* context_lens,
                                        float scale, void* out, const pkv_decode_dims* dims,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step for a batch with shared-prefix groups, in one launch: the
 * append of pkv_paged_decode_step followed by pkv_paged_decode_attn_prefix
 * ("KV Cache from first principles" 2.2-2.3; "The KV Cache memory ledger"
 * 4).  Arguments are those two calls' together; caches, q and out all F16
 * or all BF16.  Each sequence's new token must lie past its group's shared
 * blocks (context_lens[b] - 1 >= 16 * group_prefix_blocks[g]: shared
 * blocks are full, and a token is never appended into a block other
 * sequences hold); otherwise the results are undefined (no out-of-bounds
 * access).  Results and cache contents equal those of the two calls.
 */
PKV_API int pkv_paged_decode_step_prefix(const void* k_new, const void* v_new,
                                         const int64_t* slot_mapping, const void* q, void* k_cache,
                                         void* v_cache, const int32_t* group_seq_start,
                                         const int32_t* group_prefix_blocks,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         float scale, void* out, const pkv_decode_dims* dims,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/*
 * pkv_paged_decode_attn_prefix for an 8-bit cache ("The KV Cache memory
 * ledger" 4 and 7: shared prefix blocks, and 8-bit K/V with one scale per
 * (block, head)).  K and V both FP8_E4M3 or both INT8 (p->v_dtype =
 * dims->kv_dtype) with one scale per (block, KV head) in p->k_scales and
 * p->v_scales; no channel factors, per-token scales or sink tiles
 * (p->k_channel_scales NULL, the per-token flags 0, dims->sink_tiles 0:
 * -3 / -2 otherwise); q and out both F16 or both BF16; head_dim 128 (-2
 * otherwise).  Groups as for pkv_paged_decode_attn_prefix.  The result is
 * that of pkv_paged_decode_attn_quant.  Precision: the sequences' own
 * blocks as stated for pkv_paged_decode_attn_fp8; in the shared part the
 * codes are widened to f16 exactly, the query is rounded to f16 after a
 * power-of-two rescale per query row (its largest element in [2^14, 2^15),
 * so 11 significant bits for each element within 2^28 of that one), and
 * each softmax weight times V's block scale enters the sum of V with about
 * 22 significant bits.  Always splits (workspace > 0).
 */
PKV_API int pkv_paged_decode_attn_quant_prefix(const void* q, const void* k_cache, const void* v_cache,
                                               const pkv_quant_params* p, const int32_t* group_seq_start,
                                               const int32_t* group_prefix_blocks,
                                               const int32_t* block_tables, const int32_t* context_lens,
                                               float scale, void* out, const pkv_decode_dims* dims,
                                               void* workspace, size_t workspace_bytes,
                                               hipStream_t stream);

/*
 * One decode step for an 8-bit cache with shared-prefix groups, in one
 * launch: the quantise-on-write append of pkv_paged_decode_step_quant
 * (given block scales) followed by pkv_paged_decode_attn_quant_prefix
 * ("KV Cache from first principles" 2.2-2.3; "The KV Cache memory ledger"
 * 4 and 7).  Arguments are those two calls' together, with the limits of
 * the latter; k_new and v_new are of q's dtype.  Each sequence's new token
 * must lie past its group's shared blocks, as for
 * pkv_paged_decode_step_prefix.  Codes and output equal those of the two
 * calls.
 */
PKV_API int pkv_paged_decode_step_quant_prefix(const void* k_new, const void* v_new,
                                               const int64_t* slot_mapping, const void* q, void* k_cache,
                                               void* v_cache, const pkv_quant_params* p,
                                               const int32_t* group_seq_start,
                                               const int32_t* group_prefix_blocks,
                                               const int32_t* block_tables, const int32_t* context_lens,
                                               float scale, void* out, const pkv_decode_dims* dims,
                                               void* workspace, size_t workspace_bytes,
                                               hipStream_t stream);

/*
 * Bandwidth reference ("KV Cache from first principles" 4.1: decode time is
 * set by the bytes moved).  Reads the first `bytes` (rounded down to a
 * multiple of 16) of device buffer `buf` once with 16-byte loads, using
 * `sink_words` workgroups: workgroup k reads the 16-byte words
 * [k * c, (k + 1) * c), c = ceil(words / sink_words), and XORs them into
 * sink[k] (device, caller-zeroed if the value matters).  The rate of this
 * call is what a read-only kernel achieves on the device.
 * Errors: NULL buf/sink with bytes >= 16, sink_words < 1 -> status.
 */
PKV_API int pkv_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t sink_words,
                               hipStream_t stream);

/*
 * The memory traffic of pkv_paged_decode_attn without its arithmetic, as a
 * bandwidth reference for that access pattern ("KV Cache from first
 * principles" 4.1, 4.3: decode is bound by the bytes it moves, fetched
 * through the block table from scattered places).  Same grid and
 * partition plan as the attention call for `dims`, the same per-wave
 * order of blocks, K tiles copied into LDS by non-temporal DMA and V tiles
 * read into registers one block ahead (non-temporal loads when the
 * attention call takes its matrix-core pass, head_dim 128 with 4 or 8
 * query heads per KV head; ordinary loads otherwise, as its vector pass
 * does); only the token rows that hold a token are fetched (all 16 but in
 * a sequence's last block).  Each workgroup folds what it read into
 * sink[(b * Hkv + h) * P + p]
 * (uint32 device array of num_seqs * num_kv_heads *
 * pkv_decode_num_partitions(dims) words, caller-zeroed if the value
 * matters).  head_dim 128; dims->kv_dtype is K's format and v_dtype V's,
 * each F16, BF16, FP8_E4M3 or INT8, V no wider than K (a 16-bit K with an
 * 8-bit V reads 2-byte K tiles and 1-byte V tiles, as the attention call
 * does; per-token scales are not read); no window, sink tiles or groups.
 * Computes nothing else.
 * Errors: head_dim != 128, a window, sink tiles or groups -> PKV_ERR_SHAPE;
 * a format outside that list or V wider than K -> PKV_ERR_DTYPE.
 */
PKV_API int pkv_paged_read_probe(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, const pkv_decode_dims* dims,
                                 int32_t v_dtype, uint32_t* sink, hipStream_t stream);

/*
 * Copy-on-write block copies ("Large-model inference KV Cache memory
 * optimisation" 3.2: copy a shared block before writing into it).  For every
 * i < num_pairs, block dst_blocks[i] of both caches receives a bit copy of
 * block src_blocks[i] (every KV head, all 16 slots), and for 8-bit caches
 * the scales k_scales/v_scales[dst][h] receive those of src (pass NULL scales
 * for other dtypes; a mixed fp8 K / int8 V pair passes either 8-bit dtype).  src_blocks, dst_blocks: int32 device arrays.  Destinations
 * must be distinct and not also sources in the same call; ids outside
 * [0, num_blocks) are skipped.  num_pairs <= 65535.
 */
PKV_API int pkv_copy_blocks(void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                            const int32_t* src_blocks, const int32_t* dst_blocks, int32_t num_pairs,
                            int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                            int32_t dtype, hipStream_t stream);

/*
 * Host block manager ("Large-model inference KV Cache memory optimisation"
 * 2.2-2.3 pool and recycling, 3.1-3.2 shared blocks, reference counts and
 * copy-on-write; "The KV Cache memory ledger" 4).  Host memory only; every
 * call is thread-safe (one internal lock; reference counts are atomic).
 *   create: `num_blocks` blocks of 16 tokens; free_order (may be NULL =
 *     0, 1, 2, ...) is the order in which fresh blocks are handed out; freed
 *     blocks are handed out again first, most recently freed first.
 *     Returns NULL for bad arguments.
 *   fork: `child` references every block of `parent` (the partial last one
 *     too) and has its length.
 *   append_slots: reserves the next position of each of seqs[0..n) (distinct)
 *     and writes its flat slot to slots_out[i].  A new block is taken when
 *     the position opens a block; when it falls in a partial last block that
 *     other sequences still reference, a fresh block replaces it and the pair
 *     (old, fresh) is written to copy_src/copy_dst (capacity >= n): run
 *     pkv_copy_blocks on those pairs before appending.  Fails with
 *     PKV_ERR_NO_BLOCKS, changing nothing, if the pool is short.
 *   free_sequence: drops one reference from each of its blocks; blocks at
 *     zero return to the pool.
 *   block_tables: rows of max_blocks int32 (padded with -1) and lengths for
 *     seqs[0..n), ready for pkv_paged_decode_attn after a copy to the device.
 */
typedef struct pkv_block_manager pkv_block_manager;
PKV_API pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size,
                                         const int32_t* free_order);
PKV_API void pkv_bm_destroy(pkv_block_manager* bm);
PKV_API int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq);
PKV_API int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);
PKV_API int pkv_bm_append_slots(pkv_block_manager* bm, const int64_t* seqs, int32_t n,
                                int64_t* slots_out, int32_t* copy_src, int32_t* copy_dst,
                                int32_t copy_capacity, int32_t* num_copies);
PKV_API int pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq);
PKV_API int pkv_bm_num_free(pkv_block_manager* bm);
PKV_API int pkv_bm_refcount(pkv_block_manager* bm, int32_t block);
PKV_API int pkv_bm_block_tables(pkv_block_manager* bm, const int64_t* seqs, int32_t n,
                                int32_t max_blocks, int32_t* tables_out, int32_t* lens_out);

/* Static text for a status code. */
PKV_API const char* pkv_status_string(int status);

/* PKV_VERSION of the built library. */
PKV_API int pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
