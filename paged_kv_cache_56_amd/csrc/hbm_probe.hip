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

// Workgroup k reads the k-th of gridDim.x contiguous chunks, its 256
// threads 16 bytes apart, eight loads in flight per thread, non-temporal.
// Long contiguous chunks per workgroup stream faster on this chip than a
// grid-wide stride over the buffer (7.1 against 6.8 TB/s over 4 GiB at the
// best grid size of each form).
__global__ void __launch_bounds__(256) hbm_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                       uint32_t* __restrict__ sink) {
  constexpr int UNROLL = 8;
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  int64_t j = lo + threadIdx.x;
  uint32_t acc = 0;
  for (; j + (UNROLL - 1) * 256 < hi; j += UNROLL * 256) {
    u32x4 x[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) x[u] = __builtin_nontemporal_load(src + j + u * 256);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  for (; j < hi; j += 256) {
    const u32x4 x = src[j];
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

// ---------------------------------------------------------------------------
// The decode kernel's memory traffic without its arithmetic: the reference
// for how fast this access pattern can stream on the device.  Same grid
// (partition, KV head, sequence) and partition plan as the attention
// launch; in a workgroup wave w takes the blocks j0 + w, j0 + w + 4, ...;
// per block, K's (block, head) tile is copied into a two-slot per-wave LDS
// ring by non-temporal LDS DMA, 1 KiB per wave instruction, and V's tile
// is read into registers by non-temporal loads, four rows per wave
// instruction, one block ahead of the one being consumed; the table entry
// of the next block is read as a scalar load.  Only the token rows that
// hold a token are fetched (all 16 but in a sequence's last block).
// Consuming a block is reading the lane's 32 channels of K back from LDS
// and folding them and the V words of those rows into one word, which
// each wave adds to sink[workgroup].
// head_dim 128; K tiles of 16-bit (KEB = 2) or 8-bit (KEB = 1) elements,
// V tiles likewise (VEB), V no wider than K (a 16-bit K may go with an
// 8-bit V, as the attention call allows).  V's loads take the cache policy of the pass the attention launch runs for
// the same shape: non-temporal (NTV) for the matrix-core pass (4 or 8
// query heads per KV head), the default policy for the vector pass, whose
// V loads are ordinary (a repeated batch then finds part of V in the
// last-level cache).
template <int EB, int VEB, bool NTV>
__global__ void __launch_bounds__(256) paged_read_probe_kernel(DecodeArgs a, uint32_t* __restrict__ sink) {
  static_assert(VEB <= EB, "V is no wider than K");
  constexpr int D = 128, ROW_B = D * EB, TILE_B = 16 * ROW_B, NDMA = TILE_B / 1024;
  constexpr int VROW_B = D * VEB, VTILE_B = 16 * VROW_B;
  constexpr int KREADS = 2 * EB, VW = 2 * VEB, NW = 4, KR = 2;
  __shared__ __attribute__((aligned(16))) char ring[NW * KR * TILE_B];
  const Unit u = unit_of(a, blockIdx.x);
  const int p = u.p, h = u.h, b = u.b;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lq = lane & 15, lg = lane >> 4;
  int L = a.context_lens[b];
  L = L < 0 ? 0 : (L > a.max_blocks * 16 ? a.max_blocks * 16 : L);
  const SeqParts parts((L + 15) >> 4, a.part_blocks, a.num_parts, p);
  const int nunits = parts.j1 - parts.j0;
  const int n_my = w < nunits ? (nunits - w + NW - 1) / NW : 0;
  const __attribute__((address_space(4))) int32_t* table =
      (const __attribute__((address_space(4))) int32_t*)(a.block_tables + (int64_t)b * a.max_blocks);
  // (block, head) index of logical block j; a tile's offset is that times
  // the cache's tile bytes
  auto tile = [&](int j) __attribute__((always_inline)) {
    const int phys = table[j];
    return (int64_t)(((unsigned)phys < (unsigned)a.num_blocks) ? phys : 0) * a.num_kv_heads + h;
  };
  // the decode pass's LDS placement of K: HBM column x of row r at LDS
  // column x ^ f(r), so that a lane group's reads of one column of 16 rows
  // hit 16 bank groups
  uint32_t dma_off[NDMA], kaddr[KREADS];
  const uint32_t slot0 = lds_offset(ring) + (uint32_t)(w * KR * TILE_B);
#pragma unroll
  for (int n = 0; n < NDMA; ++n) {
    if constexpr (EB == 2) {
      const int r = n * 4 + lg;
      dma_off[n] = (uint32_t)(r * 256 + ((lq ^ r) & 15) * 16);
    } else {
      const int r = n * 8 + (lane >> 3);
      dma_off[n] = (uint32_t)(r * 128 + (((lane & 7) ^ (r >> 1)) & 7) * 16);
    }
  }
#pragma unroll
  for (int k = 0; k < KREADS; ++k) {
    if constexpr (EB == 2) kaddr[k] = slot0 + (uint32_t)(lq * 256 + (((lg * 4 + k) ^ lq) & 15) * 16);
    else kaddr[k] = slot0 + (uint32_t)(lq * 128 + (((lg * 2 + k) ^ (lq >> 1)) & 7) * 16);
  }
  typedef uint32_t VRow[4][VW];
  // rows of block j that hold a token: only those are fetched, as the
  // decode pass does
  auto rows_of = [&](int j) __attribute__((always_inline)) {
    const int n = L - j * 16;
    return n < 0 ? 0 : (n > 16 ? 16 : n);
  };
  auto issue = [&](int64_t bh, int sk, VRow& v, int nv) __attribute__((always_inline)) {
    const char* k = (const char*)a.k_cache + bh * TILE_B;
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      const int row = EB == 2 ? n * 4 + lg : n * 8 + (lane >> 3);   // as in dma_off
      if (nv >= 16 || row < nv) lds_dma16(k, dma_off[n], slot0 + sk * TILE_B + n * 1024);
    }
    const char* vsrc = (const char*)a.v_cache + bh * VTILE_B;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (nv < 16 && lg * 4 + i >= nv) {
#pragma unroll
        for (int q = 0; q < VW; ++q) v[i][q] = 0u;
        continue;
      }
      const uint32_t o = (uint32_t)((lg * 4 + i) * VROW_B + lq * 8 * VEB);
      if constexpr (VW == 4) {
        const u32x4_t x = NTV ? __builtin_nontemporal_load((const u32x4_t*)(vsrc + o))
                              : *(const u32x4_t*)(vsrc + o);
        v[i][0] = x[0]; v[i][1] = x[1]; v[i][2] = x[2]; v[i][3] = x[3];
      } else {
        const u32x2_t x = NTV ? __builtin_nontemporal_load((const u32x2_t*)(vsrc + o))
                              : *(const u32x2_t*)(vsrc + o);
        v[i][0] = x[0]; v[i][1] = x[1];
      }
    }
  };
  constexpr unsigned kWaitVm0 = 0x0F70;     // vmcnt(0), expcnt(7), lgkmcnt(15)
  uint32_t acc = 0;
  int64_t next = 0;
  VRow va, vb;
  if (n_my > 0) {
    issue(tile(parts.j0 + w), 0, va, rows_of(parts.j0 + w));
    if (n_my > 1) next = tile(parts.j0 + w + NW);
  }
  // step t: wait for everything (block t is the newest load in flight),
  // issue block t + 1 into the other ring slot and register set, consume t
  auto step = [&](int t, VRow& vcur, VRow& vnext) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    wait_vmcnt<0>();
    if (t + 1 < n_my) {
      issue(next, (t + 1) & 1, vnext, rows_of(parts.j0 + w + (t + 1) * NW));
      if (t + 2 < n_my) next = tile(parts.j0 + w + (t + 2) * NW);
    }
    uint32_t addr[KREADS];
#pragma unroll
    for (int k = 0; k < KREADS; ++k) addr[k] = kaddr[k] + (uint32_t)((t & 1) * TILE_B);
    u32x4_t kr[KREADS];
    lds_read16_wait<KREADS>(kr, addr);
    if (lq < rows_of(parts.j0 + w + t * NW))        // the lane's K row holds a token
#pragma unroll
      for (int k = 0; k < KREADS; ++k) acc ^= kr[k][0] ^ kr[k][1] ^ kr[k][2] ^ kr[k][3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < VW; ++k) acc ^= vcur[i][k];
  };
  int t = 0;
  for (; t + 1 < n_my; t += 2) {
    step(t, va, vb);
    step(t + 1, vb, va);
  }
  if (t < n_my) step(t, va, vb);
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d);
  if (lane == 0) atomicXor(sink + ((int64_t)b * a.num_kv_heads + h) * a.num_parts + p, acc);
}

int launch_paged_read_probe(const DecodeArgs& a, uint32_t* sink, hipStream_t stream) {
  const int64_t n = (int64_t)a.num_parts * a.num_kv_heads * a.num_seqs;
  if (n > 0x7FFFFFFF) return PKV_ERR_SHAPE;
  const dim3 grid((unsigned)n);
  const int g = a.num_kv_heads > 0 ? a.num_q_heads / a.num_kv_heads : 0;
  const bool matrix_core_pass = a.head_dim == 128 && (g == 4 || g == 8);
  auto width = [](int dt) { return dt == PKV_FP8_E4M3 || dt == PKV_INT8 ? 1 : 2; };
  const int keb = width(a.kv_dtype), veb = width(a.v_dtype);
  if (keb == 1 && veb == 1) {
    if (matrix_core_pass)
      hipLaunchKernelGGL((paged_read_probe_kernel<1, 1, true>), grid, dim3(256), 0, stream, a, sink);
    else
      hipLaunchKernelGGL((paged_read_probe_kernel<1, 1, false>), grid, dim3(256), 0, stream, a, sink);
  } else if (veb == 1) {
    if (matrix_core_pass)
      hipLaunchKernelGGL((paged_read_probe_kernel<2, 1, true>), grid, dim3(256), 0, stream, a, sink);
    else
      hipLaunchKernelGGL((paged_read_probe_kernel<2, 1, false>), grid, dim3(256), 0, stream, a, sink);
  } else if (keb == 2) {
    if (matrix_core_pass)
      hipLaunchKernelGGL((paged_read_probe_kernel<2, 2, true>), grid, dim3(256), 0, stream, a, sink);
    else
      hipLaunchKernelGGL((paged_read_probe_kernel<2, 2, false>), grid, dim3(256), 0, stream, a, sink);
  } else {
    return PKV_ERR_DTYPE;   // V wider than K
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // namespace pkv
