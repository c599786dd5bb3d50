// Block copies for copy-on-write ("Large-model inference KV Cache memory
// optimisation" (wmrh.cn) 3.2: a shared block is copied before a sequence
// writes into it).  Pair i copies the whole K and V tile run of block
// src[i] -- every KV head, all 16 slots -- onto block dst[i], and, for fp8
// caches, the per-(block, head) scales.  A bit copy: one thread per 16 bytes,
// grid (16-byte chunks of a block / 256, pairs, K|V).
#include "pkv_internal.h"

namespace pkv {

__global__ void __launch_bounds__(256) copy_blocks_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, float* __restrict__ k_scales,
    float* __restrict__ v_scales, const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
    int chunks_per_block, int num_kv_heads, int num_blocks) {
  const int pair = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int s = src[pair], d = dst[pair];
  if ((unsigned)s >= (unsigned)num_blocks || (unsigned)d >= (unsigned)num_blocks || s == d) return;
  uint4* cache = is_v ? v_cache : k_cache;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < chunks_per_block)
    cache[(int64_t)d * chunks_per_block + c] = cache[(int64_t)s * chunks_per_block + c];
  float* scales = is_v ? v_scales : k_scales;
  if (scales && blockIdx.x == 0 && threadIdx.x < num_kv_heads)
    scales[(int64_t)d * num_kv_heads + threadIdx.x] = scales[(int64_t)s * num_kv_heads + threadIdx.x];
}

int launch_copy_blocks(void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                       const int32_t* src, const int32_t* dst, int n, int num_kv_heads,
                       int block_bytes, int num_blocks, hipStream_t stream) {
  if (n == 0) return PKV_OK;
  const int chunks = block_bytes / 16;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((chunks + 255) / 256, n, 2), dim3(256), 0, stream,
                     (uint4*)k_cache, (uint4*)v_cache, k_scales, v_scales, src, dst, chunks,
                     num_kv_heads, num_blocks);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // namespace pkv
