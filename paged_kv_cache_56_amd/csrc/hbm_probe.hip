// Plain streaming read of a device buffer: the bandwidth reference for the
// decode kernels.  "KV Cache from first principles" (ldpk.cn) 4.1 argues
// that decode is bound by memory traffic, not arithmetic; this kernel is the
// other end of that argument -- it reads every byte once with 16-byte
// loads and does nothing else, so its rate is what HBM delivers to a kernel
// on this device.  Each workgroup folds what it read into one word (so no
// load can be dropped) and writes it to `sink`.
#include "pkv_internal.h"

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) hbm_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                       uint32_t* __restrict__ sink) {
  constexpr int UNROLL = 8;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    u32x4 x[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) x[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 x = src[i];
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  // fold the workgroup: any lane's value reaches the sink through the wave xor
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, acc);
}

int launch_hbm_read(const void* buf, size_t bytes, uint32_t* sink, int sink_words,
                    hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return PKV_OK;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(sink_words), dim3(256), 0, stream, (const u32x4*)buf,
                     n16, sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // namespace pkv
