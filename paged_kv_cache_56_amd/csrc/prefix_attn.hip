// Shared-prefix pass of paged decode attention for gfx950: matrix cores.
//
// When several sequences share their first blocks ("The KV Cache memory
// ledger" 4: prefix sharing points several block tables at one physical
// block; "Large-model inference KV Cache memory optimisation" 3.1-3.3: such
// blocks are stored once), the per-sequence pass would read every shared
// tile once per sequence.  Here a workgroup reads each shared (block, KV
// head) tile once and scores it against the queries of every sequence of
// the group at the same time.  With n sequences and g query heads per KV
// head that is an (n*g x D) by (D x tokens) product followed by a
// (n*g x tokens) by (tokens x D) one: a real dense contraction, so it runs on
// v_mfma_f32_16x16x32_{f16,bf16}.  Its partial results (o, m, l per query
// row) go to the workspace next to those of the per-sequence pass, which
// skips the shared blocks, and the merge kernel combines both by log-sum-exp.
//
// Work split.  Grid = (piece p of the group's shared blocks, KV head h,
// group x 64-row chunk of its queries).  Query row r of a group is sequence
// s0 + r / g, query head h * g + r % g.  Each of the four waves owns 16 rows;
// the workgroup stages 32 tokens (two blocks) of K and V in LDS per step:
// K row-major, V transposed (column d holds the tokens), so that both
// products read 16-byte operands.
//
// Orientation.  Scores are computed transposed, S^T = K Q^T (A = K tile,
// B = Q^T), so the result leaves lane l with query l % 16 and tokens
// 4 * (l / 16) + 0..3 of each 16-token tile.  The output is computed
// transposed too, O^T = V^T P^T (A = V^T, B = P^T): P^T's B operand is then
// exactly those 8 tokens of query l % 16, taken as the lane's 8 contraction
// indices, and V^T's A operand reads the same 8 tokens for one channel
// (the transposed LDS tile stores them side by side).  The accumulator
// leaves lane l with query l % 16, so the softmax rescale stays in-lane.
//
// Precision.  q, K and V are read as stored; products accumulate in fp32.
// The probabilities are rounded once to the operand type (f16 or bf16) and
// the running sum adds the rounded values, so the result is an exact convex
// combination of V rows with weights off by at most half an ulp of that
// type.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <KV T> struct Mma;
template <> struct Mma<KV::F16> {
  static __device__ __forceinline__ f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  // probability -> operand bits (round to nearest even) and the rounded value
  static __device__ __forceinline__ uint32_t round(float p, float* back) {
    const _Float16 h = (_Float16)p;
    *back = (float)h;
    return __builtin_bit_cast(uint16_t, h);
  }
};
template <> struct Mma<KV::BF16> {
  static __device__ __forceinline__ f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t round(float p, float* back) {
    const uint32_t bits = f32_to_bf16_rne(p);
    *back = __builtin_bit_cast(float, bits << 16);
    return bits;
  }
};

// Column of token t (0..31 of a step) in the transposed V tile: lane group q
// contracts over tokens 4q..4q+3 of the first block and 16+4q..16+4q+3 of
// the second, stored at columns 8q..8q+7.
__device__ __forceinline__ int vt_col(int t) {
  return ((t & 15) >> 2) * 8 + (t >> 4) * 4 + (t & 3);
}

template <KV T, int D>
__global__ void __launch_bounds__(256) group_prefix_kernel(DecodeArgs a) {
  constexpr int KS = D + 8;            // K tile row stride in LDS (elements)
  constexpr int VS = 40;               // transposed V tile row stride (elements)
  constexpr int CH = D / 8;            // 16-byte chunks per token row
  constexpr int NL = 32 * CH / 256;    // chunks per thread per 32-token step
  constexpr int KK = D / 32;           // contraction steps over the head dimension
  constexpr int DT = D / 16;           // 16-channel output tiles
  static_assert(NL >= 1 && 32 * CH == 256 * NL, "whole chunks per thread");
  __shared__ __attribute__((aligned(16))) uint16_t ks[32 * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VS];

  const int qc = blockIdx.z % a.group_qchunks, g = blockIdx.z / a.group_qchunks;
  const int h = blockIdx.y, pp = blockIdx.x;
  const PrefixGroup pg = prefix_group(a, g);
  const int gq = a.num_q_heads / a.num_kv_heads;
  const int nrows = pg.nseq * gq;
  const int row0 = qc * 64;
  const SeqParts parts(pg.nblk, a.group_part_blocks, a.group_num_parts, pp);
  if (row0 >= nrows || parts.j0 >= parts.j1) return;   // uniform over the workgroup

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 15, lg = lane >> 4;
  const bool wave_on = row0 + w * 16 < nrows;          // uniform over the wave
  const int r = row0 + w * 16 + lq;
  const bool rv = r < nrows;
  const int b = pg.s0 + (rv ? r / gq : 0);
  const int head = h * gq + (rv ? r % gq : 0);
  const int L = rv ? max(a.context_lens[b], 0) : 0;

  // B operand of S^T = K Q^T: lane holds q[row lq][kk*32 + 8*lg .. +7]
  u32x4_t qf[KK];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)b * a.num_q_heads + head) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = rv ? *(const u32x4_t*)(qrow + kk * 32 + 8 * lg) : u32x4_t{0u, 0u, 0u, 0u};
  }

  const int32_t* table = a.block_tables + (int64_t)pg.s0 * a.max_blocks;
  auto block_ok = [&](int j) __attribute__((always_inline)) {
    return j < parts.j1 && (unsigned)table[j] < (unsigned)a.num_blocks;
  };

  // staging: chunk c = tid + 256*e is token c % 32, channels (c / 32)*8 .. +7
  u32x4_t kreg[NL], vreg[NL];
  auto load_step = [&](int j) __attribute__((always_inline)) {
    const int ph0 = table[j];
    const int ph1 = j + 1 < parts.j1 ? table[j + 1] : -1;
#pragma unroll
    for (int e = 0; e < NL; ++e) {
      const int c = tid + 256 * e, t = c & 31, col = c >> 5;
      const int ph = t < 16 ? ph0 : ph1;
      if ((unsigned)ph < (unsigned)a.num_blocks) {
        const int64_t off = (((int64_t)ph * a.num_kv_heads + h) * 16 + (t & 15)) * D + col * 8;
        kreg[e] = *(const u32x4_t*)((const uint16_t*)a.k_cache + off);
        vreg[e] = *(const u32x4_t*)((const uint16_t*)a.v_cache + off);
      } else {
        kreg[e] = u32x4_t{0u, 0u, 0u, 0u};   // missing block: zeros, never NaN
        vreg[e] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_step = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < NL; ++e) {
      const int c = tid + 256 * e, t = c & 31, col = c >> 5;
      *(u32x4_t*)&ks[t * KS + col * 8] = kreg[e];
      const int vc = vt_col(t);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        vt[(col * 8 + 2 * k) * VS + vc] = (uint16_t)(vreg[e][k] & 0xFFFFu);
        vt[(col * 8 + 2 * k + 1) * VS + vc] = (uint16_t)(vreg[e][k] >> 16);
      }
    }
  };

  float m = -INFINITY, l = 0.f;
  f32x4_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_step(parts.j0);
  for (int j = parts.j0; j < parts.j1; j += 2) {
    __syncthreads();                     // the previous step's LDS reads are done
    store_step();
    __syncthreads();
    if (j + 2 < parts.j1) load_step(j + 2);
    if (!wave_on) continue;

    // S^T tiles: lane holds (token 16*tt + 4*lg + i, query lq) in s[tt][i]
    f32x4_t s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      s[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4_t ka = *(const u32x4_t*)&ks[(tt * 16 + lq) * KS + kk * 32 + 8 * lg];
        s[tt] = Mma<T>::run(ka, qf[kk], s[tt]);
      }
    }
    const bool ok0 = block_ok(j), ok1 = block_ok(j + 1);
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = (j + tt) * 16 + 4 * lg + i;
        const bool ok = (tt == 0 ? ok0 : ok1) && pos < L;
        sv[tt * 4 + i] = ok ? s[tt][i] * a.scale : -INFINITY;   // log2 units
        mx = fmaxf(mx, sv[tt * 4 + i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);

    // B operand of O^T = V^T P^T: the lane's 8 tokens of query lq, rounded
    uint32_t pw[4];
    float ps = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float r0, r1;
      const float p0 = sv[2 * k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[2 * k] - mn);
      const float p1 = sv[2 * k + 1] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[2 * k + 1] - mn);
      pw[k] = Mma<T>::round(p0, &r0) | (Mma<T>::round(p1, &r1) << 16);
      ps += r0 + r1;
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l = l * alpha + ps;
    m = mn;
    const u32x4_t pb = {pw[0], pw[1], pw[2], pw[3]};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x4_t va = *(const u32x4_t*)&vt[(dt * 16 + lq) * VS + 8 * lg];
      acc[dt] = Mma<T>::run(va, pb, acc[dt] * alpha);
    }
  }

  // partial result of this piece: lane holds channels dt*16 + 4*lg + 0..3
  if (wave_on && rv) {
    const int64_t slot =
        ((int64_t)b * a.num_q_heads + head) * a.part_stride + a.num_parts + pp;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* o = a.o_part + slot * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *(f32x4_t*)(o + dt * 16 + 4 * lg) = acc[dt] * inv;
    if (lg == 0) {
      a.ml_part[slot * 2 + 0] = m;
      a.ml_part[slot * 2 + 1] = l;
    }
  }
}

template <KV T>
int launch_t(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.group_num_parts, a.num_kv_heads, a.num_groups * a.group_qchunks);
  if (a.head_dim == 128)
    hipLaunchKernelGGL((group_prefix_kernel<T, 128>), grid, dim3(256), 0, s, a);
  else if (a.head_dim == 64)
    hipLaunchKernelGGL((group_prefix_kernel<T, 64>), grid, dim3(256), 0, s, a);
  else
    return PKV_ERR_SHAPE;
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // namespace

void plan_groups(const pkv_decode_dims& d, int* part_blocks, int* num_parts, int* qchunks) {
  const int g = d.num_q_heads / d.num_kv_heads;
  *qchunks = (int)(((int64_t)d.prefix_max_seqs * g + 63) / 64);
  const int maxb = d.prefix_max_blocks < d.max_blocks_per_seq ? d.prefix_max_blocks
                                                              : d.max_blocks_per_seq;
  if (d.prefix_groups <= 0 || maxb <= 0) {
    *part_blocks = 1;
    *num_parts = 0;
    return;
  }
  // About 256 workgroups (one per CU) for the whole pass, never fewer than
  // 8 blocks per piece: each piece adds a partial result per query row.
  const int64_t units = (int64_t)d.prefix_groups * d.num_kv_heads * *qchunks;
  const int64_t want = units >= 256 ? 1 : (256 + units - 1) / units;
  int pb = (int)((maxb + want - 1) / want);
  if (pb < 8) pb = 8;
  if (pb > maxb) pb = maxb;
  *part_blocks = pb;
  *num_parts = (maxb + pb - 1) / pb;
}

int launch_group_prefix(const DecodeArgs& a, hipStream_t s) {
  if (a.num_groups <= 0 || a.group_num_parts <= 0) return PKV_OK;
  if (a.kv_dtype == (int)KV::F16) return launch_t<KV::F16>(a, s);
  if (a.kv_dtype == (int)KV::BF16) return launch_t<KV::BF16>(a, s);
  return PKV_ERR_DTYPE;
}

}  // namespace pkv
