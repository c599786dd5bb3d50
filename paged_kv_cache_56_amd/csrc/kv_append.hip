// Per-step K/V append into the paged cache.
//
// "KV Cache from first principles" (ldpk.cn) 2.3: a decode step writes the
// new token's K and V at the current length.  "The KV Cache memory ledger"
// (gcssc.sfwss.com) 4: with paging that place is the flat slot
// block * 16 + offset, found through the block table (locate()).
//
// The work is a scatter of T * Hkv rows of head_dim elements into scattered
// 16-token tiles.  One thread moves 16 bytes; consecutive threads take
// consecutive 16-byte pieces of one (token, head) row, so both the read of
// k_new and the write into the tile are contiguous.  K and V are handled by
// the two halves of the grid's y dimension.  Bits are copied, never converted.
#include "pkv_internal.h"

namespace pkv {

__global__ void __launch_bounds__(256) kv_append_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, int num_tokens, int num_kv_heads, int chunks_per_row,
    int64_t num_slots) {
  const int64_t per_tensor = (int64_t)num_tokens * num_kv_heads * chunks_per_row;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= per_tensor) return;
  const bool is_v = blockIdx.y != 0;
  const int chunk = (int)(idx % chunks_per_row);
  const int64_t row = idx / chunks_per_row;  // t * Hkv + h
  const int h = (int)(row % num_kv_heads);
  const int64_t t = row / num_kv_heads;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / PKV_BLOCK_SIZE;
  const int64_t off = slot % PKV_BLOCK_SIZE;
  const int64_t dst_row = (blk * num_kv_heads + h) * PKV_BLOCK_SIZE + off;
  const uint4* src = is_v ? v_new : k_new;
  uint4* dst = is_v ? v_cache : k_cache;
  dst[dst_row * chunks_per_row + chunk] = src[idx];
}

// ---------------------------------------------------------------------------
// 8-bit append: quantise on write ("The KV Cache memory ledger" 7: 8-bit K/V
// with one scale per head, K in FP8 with V in INT8 as the mixed form; "Why
// does KV Cache eat GPU memory?": FP8 KV needs calibrated scales; "KV Cache
// from first principles" 5.2: per-channel factors for K's outlier channels).
// Scales are per (block, KV head), or per (slot, KV head) ("KV Cache from
// first principles" 5.2: per-token granularity).  With channel factors the
// source is first divided by its channel's factor.  In first-write mode the
// token that opens a block (offset 0) sets that block's scale to
// max|y| / QMAX of its own row; in per-token mode every token sets its own
// slot's scale that way.  The pass that sets scales runs before the one
// that quantises, so tokens of one call that land later in the same block
// already see it.  Codes are the
// nearest code (ties to even) of clamp(y / scale, +-QMAX), every quotient a
// correctly rounded fp32 division: for fp8 the hardware's round-to-nearest-
// even e4m3 (OCP) convert, for int8 rint (NaN gives 0).
//
// grid.y selects one of up to two (source, cache, scales, factors) targets:
// K and V in one launch, or a single cache.

struct QTarget {
  const void* src;       // [T][Hkv][D] of the source dtype
  uint8_t* cache;        // [NB][Hkv][16][D] codes
  float* scales;         // [NB][Hkv]
  const float* chan;     // [Hkv][D] or NULL
};
struct QTargets { QTarget t[2]; };

template <KV ST>
__device__ __forceinline__ float src_elem(const void* base, int64_t i) {
  if constexpr (ST == KV::F32) return ((const float*)base)[i];
  else if constexpr (ST == KV::F16) return (float)((const _Float16*)base)[i];
  else return __builtin_bit_cast(float, ((uint32_t)((const uint16_t*)base)[i]) << 16);
}

// Source element divided by its channel factor (if any).
template <KV ST>
__device__ __forceinline__ float scaled_src(const QTarget& q, int64_t row, int h, int d, int head_dim) {
  const float x = src_elem<ST>(q.src, row * head_dim + d);
  return q.chan ? x / q.chan[(int64_t)h * head_dim + d] : x;
}

// Index of the scale a token uses: per (block, head), or per (slot, head).
__device__ __forceinline__ int64_t scale_index(int64_t slot, int h, int num_kv_heads, int per_token) {
  const int64_t bh = (slot / PKV_BLOCK_SIZE) * num_kv_heads + h;
  return per_token ? bh * PKV_BLOCK_SIZE + slot % PKV_BLOCK_SIZE : bh;
}

template <KV ST, KV CT>
__global__ void __launch_bounds__(256) q8_first_write_scale_kernel(
    QTargets tg, const int64_t* __restrict__ slot_mapping, int num_tokens, int num_kv_heads,
    int head_dim, int64_t num_slots, int per_token) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // t * Hkv + h
  if (row >= (int64_t)num_tokens * num_kv_heads) return;
  const QTarget q = blockIdx.y ? tg.t[1] : tg.t[0];   // uniform: no indexed copy
  const int64_t t = row / num_kv_heads;
  const int h = (int)(row % num_kv_heads);
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots || (!per_token && slot % PKV_BLOCK_SIZE != 0)) return;
  float amax = 0.f;
  for (int d = 0; d < head_dim; ++d) amax = fmaxf(amax, fabsf(scaled_src<ST>(q, row, h, d, head_dim)));
  q.scales[scale_index(slot, h, num_kv_heads, per_token)] = amax > 0.f ? amax / qmax<CT>() : 1.0f;
}

template <KV ST, KV CT>
__global__ void __launch_bounds__(256) q8_quantize_append_kernel(
    QTargets tg, const int64_t* __restrict__ slot_mapping, int num_tokens, int num_kv_heads,
    int head_dim, int64_t num_slots, int per_token) {
  const int groups = head_dim / 16;                         // 16 elements per thread
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)num_tokens * num_kv_heads * groups) return;
  const QTarget q = blockIdx.y ? tg.t[1] : tg.t[0];   // uniform: no indexed copy
  const int gi = (int)(idx % groups);
  const int64_t row = idx / groups;                         // t * Hkv + h
  const int h = (int)(row % num_kv_heads);
  const int64_t t = row / num_kv_heads;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / PKV_BLOCK_SIZE, off = slot % PKV_BLOCK_SIZE;
  const float scale = q.scales[scale_index(slot, h, num_kv_heads, per_token)];
  constexpr float QM = qmax<CT>();
  uint32_t packed[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float v4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = scaled_src<ST>(q, row, h, gi * 16 + w * 4 + e, head_dim) / scale;
      v4[e] = v > QM ? QM : (v < -QM ? -QM : v);   // NaN passes through
    }
    packed[w] = encode_codes<CT, 4>(v4);
  }
  uint8_t* dst = q.cache + ((blk * num_kv_heads + h) * PKV_BLOCK_SIZE + off) * head_dim + gi * 16;
  *(uint4*)dst = make_uint4(packed[0], packed[1], packed[2], packed[3]);
}

int launch_kv_append_q8(const QTargetArgs* targets, int num_targets, const int64_t* slot_mapping,
                        int num_tokens, int num_kv_heads, int head_dim, int num_blocks,
                        int src_dtype, int code_dtype, int scale_mode, hipStream_t stream) {
  const bool first_write = scale_mode == PKV_SCALE_FIRST_WRITE;
  const int per_token = scale_mode == PKV_SCALE_PER_TOKEN ? 1 : 0;
  const int64_t rows = (int64_t)num_tokens * num_kv_heads;
  if (rows == 0) return PKV_OK;
  const int64_t slots = (int64_t)num_blocks * PKV_BLOCK_SIZE;
  const int64_t threads = rows * (head_dim / 16);
  if ((rows + 255) / 256 > 0x7FFFFFFF || (threads + 255) / 256 > 0x7FFFFFFF) return PKV_ERR_SHAPE;
  QTargets tg{};
  for (int i = 0; i < num_targets; ++i)
    tg.t[i] = QTarget{targets[i].src, (uint8_t*)targets[i].cache, targets[i].scales, targets[i].chan};
  const dim3 g1((unsigned)((rows + 255) / 256), num_targets);
  const dim3 g2((unsigned)((threads + 255) / 256), num_targets);
#define PKV_Q8_APPEND(ST, CT)                                                                     \
  do {                                                                                            \
    if (first_write || per_token)                                                                 \
      hipLaunchKernelGGL((q8_first_write_scale_kernel<ST, CT>), g1, dim3(256), 0, stream, tg,     \
                         slot_mapping, num_tokens, num_kv_heads, head_dim, slots, per_token);     \
    hipLaunchKernelGGL((q8_quantize_append_kernel<ST, CT>), g2, dim3(256), 0, stream, tg,        \
                       slot_mapping, num_tokens, num_kv_heads, head_dim, slots, per_token);       \
  } while (0)
#define PKV_Q8_SRC(CT)                                       \
  switch ((KV)src_dtype) {                                   \
    case KV::F32: PKV_Q8_APPEND(KV::F32, CT); break;         \
    case KV::F16: PKV_Q8_APPEND(KV::F16, CT); break;         \
    case KV::BF16: PKV_Q8_APPEND(KV::BF16, CT); break;       \
    default: return PKV_ERR_DTYPE;                           \
  }
  if ((KV)code_dtype == KV::FP8) {
    PKV_Q8_SRC(KV::FP8)
  } else if ((KV)code_dtype == KV::INT8) {
    PKV_Q8_SRC(KV::INT8)
  } else {
    return PKV_ERR_DTYPE;
  }
#undef PKV_Q8_SRC
#undef PKV_Q8_APPEND
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int launch_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                     void* k_cache, void* v_cache, int num_tokens, int num_kv_heads,
                     int row_bytes, int num_blocks, hipStream_t stream) {
  const int chunks = row_bytes / 16;
  const int64_t per_tensor = (int64_t)num_tokens * num_kv_heads * chunks;
  if (per_tensor == 0) return PKV_OK;
  const int threads = 256;
  const int64_t blocks = (per_tensor + threads - 1) / threads;
  if (blocks > 0x7FFFFFFF) return PKV_ERR_SHAPE;
  const unsigned tensors = v_cache ? 2 : 1;   // K and V, or K alone
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks, tensors), dim3(threads), 0, stream,
                     (const uint4*)k_new, (const uint4*)v_new, slot_mapping, (uint4*)k_cache,
                     (uint4*)v_cache, num_tokens, num_kv_heads, chunks,
                     (int64_t)num_blocks * PKV_BLOCK_SIZE);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // namespace pkv
