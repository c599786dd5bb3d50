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
