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
// FP8 append: quantise on write ("The KV Cache memory ledger" 7: 8-bit K/V
// with one scale per head; "Why does KV Cache eat GPU memory?": FP8 KV needs
// calibrated scales).  Scales are per (block, KV head).  In first-write mode
// the token that opens a block (offset 0) sets that block's scale to
// max|x| / 448 of its own row; the pass that does so runs before the one
// that quantises, so tokens of one call that land later in the same block
// already see it.  Codes are RNE(clamp(x / scale, +-448)) with the quotient
// a correctly rounded fp32 division and the conversion the hardware's
// round-to-nearest-even e4m3 (OCP) convert.

template <KV ST>
__device__ __forceinline__ float src_elem(const void* base, int64_t i) {
  if constexpr (ST == KV::F32) return ((const float*)base)[i];
  else if constexpr (ST == KV::F16) return (float)((const _Float16*)base)[i];
  else return __builtin_bit_cast(float, ((uint32_t)((const uint16_t*)base)[i]) << 16);
}

template <KV ST>
__global__ void __launch_bounds__(256) fp8_first_write_scale_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, float* __restrict__ k_scales,
    float* __restrict__ v_scales, int num_tokens, int num_kv_heads, int head_dim,
    int64_t num_slots) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // t * Hkv + h
  if (row >= (int64_t)num_tokens * num_kv_heads) return;
  const bool is_v = blockIdx.y != 0;
  const int64_t t = row / num_kv_heads;
  const int h = (int)(row % num_kv_heads);
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots || slot % PKV_BLOCK_SIZE != 0) return;
  const void* src = is_v ? v_new : k_new;
  float amax = 0.f;
  for (int d = 0; d < head_dim; ++d) amax = fmaxf(amax, fabsf(src_elem<ST>(src, row * head_dim + d)));
  float* scales = is_v ? v_scales : k_scales;
  scales[(slot / PKV_BLOCK_SIZE) * num_kv_heads + h] = amax > 0.f ? amax / 448.0f : 1.0f;
}

template <KV ST>
__global__ void __launch_bounds__(256) fp8_quantize_append_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const float* __restrict__ k_scales,
    const float* __restrict__ v_scales, int num_tokens, int num_kv_heads, int head_dim,
    int64_t num_slots) {
  const int groups = head_dim / 16;                         // 16 elements per thread
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)num_tokens * num_kv_heads * groups) return;
  const bool is_v = blockIdx.y != 0;
  const int gi = (int)(idx % groups);
  const int64_t row = idx / groups;                         // t * Hkv + h
  const int h = (int)(row % num_kv_heads);
  const int64_t t = row / num_kv_heads;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / PKV_BLOCK_SIZE, off = slot % PKV_BLOCK_SIZE;
  const float scale = (is_v ? v_scales : k_scales)[blk * num_kv_heads + h];
  const void* src = is_v ? v_new : k_new;
  uint32_t packed[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float q[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = src_elem<ST>(src, row * head_dim + gi * 16 + w * 4 + e) / scale;
      v = v > 448.0f ? 448.0f : (v < -448.0f ? -448.0f : v);   // NaN passes through
      q[e] = v;
    }
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], word, true);
    packed[w] = (uint32_t)word;
  }
  uint8_t* dst = (is_v ? v_cache : k_cache) +
                 ((blk * num_kv_heads + h) * PKV_BLOCK_SIZE + off) * head_dim + gi * 16;
  *(uint4*)dst = make_uint4(packed[0], packed[1], packed[2], packed[3]);
}

int launch_kv_append_fp8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                         void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                         int num_tokens, int num_kv_heads, int head_dim, int num_blocks,
                         int src_dtype, bool first_write, hipStream_t stream) {
  const int64_t rows = (int64_t)num_tokens * num_kv_heads;
  if (rows == 0) return PKV_OK;
  const int64_t slots = (int64_t)num_blocks * PKV_BLOCK_SIZE;
  const int64_t threads = rows * (head_dim / 16);
  if ((rows + 255) / 256 > 0x7FFFFFFF || (threads + 255) / 256 > 0x7FFFFFFF) return PKV_ERR_SHAPE;
  const dim3 g1((unsigned)((rows + 255) / 256), 2), g2((unsigned)((threads + 255) / 256), 2);
#define PKV_FP8_APPEND(ST)                                                                        \
  do {                                                                                            \
    if (first_write)                                                                              \
      hipLaunchKernelGGL(fp8_first_write_scale_kernel<ST>, g1, dim3(256), 0, stream, k_new,      \
                         v_new, slot_mapping, k_scales, v_scales, num_tokens, num_kv_heads,       \
                         head_dim, slots);                                                        \
    hipLaunchKernelGGL(fp8_quantize_append_kernel<ST>, g2, dim3(256), 0, stream, k_new, v_new,   \
                       slot_mapping, (uint8_t*)k_cache, (uint8_t*)v_cache, k_scales, v_scales,   \
                       num_tokens, num_kv_heads, head_dim, slots);                                \
  } while (0)
  switch ((KV)src_dtype) {
    case KV::F32: PKV_FP8_APPEND(KV::F32); break;
    case KV::F16: PKV_FP8_APPEND(KV::F16); break;
    case KV::BF16: PKV_FP8_APPEND(KV::BF16); break;
    default: return PKV_ERR_DTYPE;
  }
#undef PKV_FP8_APPEND
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
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks, 2), dim3(threads), 0, stream,
                     (const uint4*)k_new, (const uint4*)v_new, slot_mapping, (uint4*)k_cache,
                     (uint4*)v_cache, num_tokens, num_kv_heads, chunks,
                     (int64_t)num_blocks * PKV_BLOCK_SIZE);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // namespace pkv
