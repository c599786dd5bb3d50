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
// Work split.  A workgroup takes (piece p of the group's shared blocks,
// KV head h, 64-row chunk of the group's queries).  Query row r of a group
// is sequence s0 + r / g, query head h * g + r % g.  Each of the four waves
// owns 16 rows; the workgroup stages 32 tokens (two blocks) of K and V in
// LDS per step: K row-major, V transposed (column d holds the tokens), so
// that both products read 16-byte operands.  These workgroups lead the
// launch of the per-sequence pass (decode_group_kernel): a piece is a chain
// of dependent memory round trips (descriptor, table, tiles, one step after
// another), which the other workgroups' streaming hides; pieces are long
// (32 blocks or more) so that few partial results are written and merged.
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
// Each probability exp2(s - m) (m: a reference at most 8 below the largest
// score so far, so they stay <= 256) enters P.V as its value rounded to the
// operand type plus the rounding remainder, itself rounded: about 22
// significant bits with f16 operands, 16 with bf16.  The running sum adds
// the fp32 probabilities.
//
// 8-bit caches ("The KV Cache memory ledger" 7: FP8 K/V with one scale per
// (block, head); e4m3 or int8 codes, K and V of one format).  The codes
// are widened to f16 exactly as a step is staged in LDS, and both products
// run on f16 operands.  The query is held in f16 after a power-of-two
// rescale per query row (its largest element lands in [2^14, 2^15)); the
// scores undo it together with the block's K scale, and each probability
// enters P.V times the block's V scale (the running sum adds the
// probabilities themselves).
#pragma once

#include "pkv_internal.h"

// Loads in flight per workgroup (32-token steps), and the split plan: about
// PKV_GROUP_WGS workgroups, pieces of at least PKV_GROUP_MIN_PB blocks.
#ifndef PKV_GROUP_PF
#define PKV_GROUP_PF 1
#endif
#ifndef PKV_GROUP_WGS
#define PKV_GROUP_WGS 256
#endif
#ifndef PKV_GROUP_MIN_PB
#define PKV_GROUP_MIN_PB 32
#endif

namespace pkv {

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

// LDS of one group workgroup: the K tile of a step, then the transposed V tile.
template <int D> struct GroupLds {
  static constexpr int KS = D + 8;     // K tile row stride (elements)
  static constexpr int VS = 40;        // transposed V tile row stride (elements)
  static constexpr int BYTES = (32 * KS + D * VS) * 2;
};

// 16 codes (one 16-byte chunk of an 8-bit tile row) -> 16 f16 values, two
// to a word, element 0 in the low half of word 0.  Exact: every e4m3 value
// and every integer of magnitude <= 128 is an f16 value.
template <KV T>
__device__ __forceinline__ void widen16(const u32x4_t& c, uint32_t (&h)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (T == KV::FP8) {
      h[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[k], 1.0f, false));
      h[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[k], 1.0f, true));
    } else {
      uint16_t e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        e[u] = __builtin_bit_cast(uint16_t, (_Float16)(int8_t)(uint8_t)(c[k] >> (8 * u)));
      h[2 * k] = e[0] | ((uint32_t)e[1] << 16);
      h[2 * k + 1] = e[2] | ((uint32_t)e[3] << 16);
    }
  }
}

// One workgroup of the group pass: piece pp of the shared blocks of group
// z / group_qchunks, KV head h, query chunk z % group_qchunks; smem holds
// at least GroupLds<D>::BYTES bytes.  T: the caches' element type (f16,
// bf16, or 8-bit codes with one scale per (block, KV head)); QT: the
// query's (T itself for 16-bit caches; f16 or bf16 for 8-bit ones).
template <KV T, KV QT, int D>
__device__ __forceinline__ void group_body(const DecodeArgs& a, int pp, int h, int z, char* smem) {
  constexpr bool Q8 = is_quantised<T>();
  static_assert(Q8 || QT == T, "a 16-bit cache takes a query of its own type");
  static_assert(QT == KV::F16 || QT == KV::BF16, "a 16-bit query");
  constexpr KV MT = Q8 ? KV::F16 : T;  // operand type of both products
  constexpr int EB = kv_bytes<T>::value;
  constexpr int EPC = 16 / EB;         // elements per 16-byte chunk
  constexpr int KS = GroupLds<D>::KS, VS = GroupLds<D>::VS;
  constexpr int CH = D / EPC;          // 16-byte chunks per token row
  constexpr int NL = 32 * CH / 256;    // chunks per thread per 32-token step
  constexpr int KK = D / 32;           // contraction steps over the head dimension
  constexpr int DT = D / 16;           // 16-channel output tiles
  static_assert(NL >= 1 && 32 * CH == 256 * NL, "whole chunks per thread");
  uint16_t* ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* vt = ks + 32 * KS;

  const int qc = z % a.group_qchunks, g = z / a.group_qchunks;
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
  // (8-bit caches: rescaled by 2^qexp into f16, and qinv = 2^-qexp)
  u32x4_t qf[KK];
  float qinv = 1.f;
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)b * a.num_q_heads + head) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = rv ? *(const u32x4_t*)(qrow + kk * 32 + 8 * lg) : u32x4_t{0u, 0u, 0u, 0u};
    if constexpr (Q8) {
      float f[KK][8];
      float mq = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f[kk][2 * k] = QT == KV::F16 ? f16lo(qf[kk][k]) : bf16lo(qf[kk][k]);
          f[kk][2 * k + 1] = QT == KV::F16 ? f16hi(qf[kk][k]) : bf16hi(qf[kk][k]);
          mq = fmaxf(mq, fmaxf(fabsf(f[kk][2 * k]), fabsf(f[kk][2 * k + 1])));
        }
      mq = across_rows<16, true>(mq);          // the row's four lane groups
      int ex;
      (void)__builtin_frexpf(mq, &ex);
      int qexp = mq > 0.f ? 15 - ex : 0;
      qexp = qexp > 100 ? 100 : (qexp < -100 ? -100 : qexp);
      qinv = __builtin_ldexpf(1.0f, -qexp);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          qf[kk][k] = pack_f16x2(__builtin_ldexpf(f[kk][2 * k], qexp), __builtin_ldexpf(f[kk][2 * k + 1], qexp));
    }
  }

  const int32_t* table = a.block_tables + (int64_t)pg.s0 * a.max_blocks;

  // Staging: chunk c = tid + 256*e is token c % 32, channels (c / 32)*8 .. +7
  // of a step: the 32 lanes that write one channel octet of the transposed
  // V tile then cover one LDS row, free of bank conflicts (a wave's load
  // still reads 32-byte runs of 32 token rows).  PF steps of loads are in flight in a register ring.  Loads
  // are never conditional (a missing block reads block 0, a step past the
  // end re-reads the last one) so the compiler's waits stay exact; missing
  // blocks turn into zeros when the ring slot is written to LDS.
  constexpr int PF = PKV_GROUP_PF;
  const int nsteps = (parts.j1 - parts.j0 + 1) >> 1;
  // A ring slot also carries its step's block validity (bit 0: first
  // block, bit 1: second), taken when its table entries are read, so that
  // no table read (a scalar load, counted with the LDS reads) sits in the
  // compute.
  // 8-bit caches: the step's two K and two V block scales travel with it
  // (scalar loads next to its table entries).
  struct StepScales { float k[2], v[2]; };
  u32x4_t kreg[PF][NL], vreg[PF][NL];
  int okb[PF];
  StepScales scb[PF];
  auto load_step = [&](int i, u32x4_t (&kr)[NL], u32x4_t (&vr)[NL], int& ok, StepScales& sc)
                       __attribute__((always_inline)) {
    const int j = parts.j0 + 2 * min(i, nsteps - 1);
    const int ph0 = table[j];
    const int ph1 = j + 1 < parts.j1 ? table[j + 1] : -1;
    ok = ((unsigned)ph0 < (unsigned)a.num_blocks ? 1 : 0) | ((unsigned)ph1 < (unsigned)a.num_blocks ? 2 : 0);
    if constexpr (Q8) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        int ph = u == 0 ? ph0 : ph1;
        ph = (unsigned)ph < (unsigned)a.num_blocks ? ph : 0;
        const int64_t si = (int64_t)ph * a.num_kv_heads + h;
        sc.k[u] = ((const __attribute__((address_space(4))) float*)a.k_scales)[si];
        sc.v[u] = ((const __attribute__((address_space(4))) float*)a.v_scales)[si];
      }
    }
#pragma unroll
    for (int e = 0; e < NL; ++e) {
      const int c = tid + 256 * e, t = c & 31, col = c >> 5;
      int ph = t < 16 ? ph0 : ph1;
      ph = (unsigned)ph < (unsigned)a.num_blocks ? ph : 0;
      const int64_t off = ((((int64_t)ph * a.num_kv_heads + h) * 16 + (t & 15)) * D + col * EPC) * EB;
      kr[e] = *(const u32x4_t*)((const char*)a.k_cache + off);
      vr[e] = *(const u32x4_t*)((const char*)a.v_cache + off);
    }
  };
  auto store_step = [&](int ok, const u32x4_t (&kr)[NL], const u32x4_t (&vr)[NL]) __attribute__((always_inline)) {
    const bool ok0 = ok & 1, ok1 = ok & 2;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < NL; ++e) {
      const int c = tid + 256 * e, t = c & 31, col = c >> 5;
      const bool ok = t < 16 ? ok0 : ok1;            // a missing block: zeros, never NaN
      const int vc = vt_col(t);
      if constexpr (!Q8) {
        *(u32x4_t*)&ks[t * KS + col * 8] = ok ? kr[e] : zero;
        const u32x4_t v = ok ? vr[e] : zero;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          vt[(col * 8 + 2 * k) * VS + vc] = (uint16_t)(v[k] & 0xFFFFu);
          vt[(col * 8 + 2 * k + 1) * VS + vc] = (uint16_t)(v[k] >> 16);
        }
      } else {
        // 16 codes: channels col * 16 .. + 15 of token t, widened to f16
        uint32_t hk[8], hv[8];
        widen16<T>(ok ? kr[e] : zero, hk);
        widen16<T>(ok ? vr[e] : zero, hv);
        *(u32x4_t*)&ks[t * KS + col * 16] = u32x4_t{hk[0], hk[1], hk[2], hk[3]};
        *(u32x4_t*)&ks[t * KS + col * 16 + 8] = u32x4_t{hk[4], hk[5], hk[6], hk[7]};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          vt[(col * 16 + 2 * k) * VS + vc] = (uint16_t)(hv[k] & 0xFFFFu);
          vt[(col * 16 + 2 * k + 1) * VS + vc] = (uint16_t)(hv[k] >> 16);
        }
      }
    }
  };

  // Online softmax with a lazily moved reference: probabilities are
  // exp2(s - m) with m shared by the four lanes of a query, and m moves
  // (one cross-lane max, one rescale of the sums) only when a score passes
  // it by more than 2^8 -- on the first scores, and rarely after.  A lane
  // keeps the sum of its own probabilities; the four are added at the end.
  constexpr float SLACK = 8.f;           // log2 units: probabilities stay <= 256
  float m = -INFINITY, l = 0.f;
  f32x4_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute_step = [&](int j, int ok, const StepScales& sc) __attribute__((always_inline)) {

    // S^T tiles: lane holds (token 16*tt + 4*lg + i, query lq) in s[tt][i]
    f32x4_t s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      s[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        s[tt] = Mma<MT>::run(*(const u32x4_t*)&ks[(tt * 16 + lq) * KS + kk * 32 + 8 * lg], qf[kk], s[tt]);
    }
    const bool ok0 = ok & 1, ok1 = ok & 2;
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float cs = a.scale;                                      // log2 units
      if constexpr (Q8) cs *= sc.k[tt] * qinv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = (j + tt) * 16 + 4 * lg + i;
        const bool ok = (tt == 0 ? ok0 : ok1) && pos < L;
        sv[tt * 4 + i] = ok ? s[tt][i] * cs : -INFINITY;
        mx = fmaxf(mx, sv[tt * 4 + i]);
      }
    }
    if (__builtin_amdgcn_ballot_w64(mx > m + SLACK)) {         // uniform over the wave
      mx = across_rows<16, true>(mx);   // the query's four lane groups
      const float mn = fmaxf(m, mx);
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      m = mn;
    }

    // B operands of O^T = V^T P^T: the lane's 8 tokens of query lq, each
    // probability as its value rounded to the operand type (hi) plus the
    // rounding remainder, rounded too (lo), in two products
    uint32_t pw[4], pr[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float r0, r1, e0, e1;
      const float p0 = sv[2 * k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[2 * k] - m);
      const float p1 = sv[2 * k + 1] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[2 * k + 1] - m);
      l += p0 + p1;
      // weights of P.V: tokens 2k, 2k + 1 of the lane's 8 lie in tile k / 2
      const float vsc = Q8 ? sc.v[k >> 1] : 1.f;
      const float w0 = p0 * vsc, w1 = p1 * vsc;
      pw[k] = Mma<MT>::round(w0, &r0) | (Mma<MT>::round(w1, &r1) << 16);
      pr[k] = Mma<MT>::round(w0 - r0, &e0) | (Mma<MT>::round(w1 - r1, &e1) << 16);
    }
    const u32x4_t pb = {pw[0], pw[1], pw[2], pw[3]};
    const u32x4_t pl = {pr[0], pr[1], pr[2], pr[3]};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x4_t va = *(const u32x4_t*)&vt[(dt * 16 + lq) * VS + 8 * lg];
      acc[dt] = Mma<MT>::run(va, pl, Mma<MT>::run(va, pb, acc[dt]));
    }
  };

  // step i uses ring slot i % PF and refills it with step i + PF
  auto step = [&](int i, u32x4_t (&kr)[NL], u32x4_t (&vr)[NL], int& okr, StepScales& scr)
                  __attribute__((always_inline)) {
    const int j = parts.j0 + 2 * i;
    const int ok = okr;
    const StepScales sc = scr;
    __syncthreads();                      // the previous step's LDS reads are done
    store_step(ok, kr, vr);
    __syncthreads();
    load_step(i + PF, kr, vr, okr, scr);
    if (wave_on) compute_step(j, ok, sc);
  };
#pragma unroll
  for (int s = 0; s < PF; ++s) load_step(s, kreg[s], vreg[s], okb[s], scb[s]);
  // whole rounds of PF steps carry no conditions, so every wait for a ring
  // slot leaves the PF - 1 younger slots in flight
  int i0 = 0;
  for (; i0 + PF <= nsteps; i0 += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) step(i0 + s, kreg[s], vreg[s], okb[s], scb[s]);
  }
#pragma unroll
  for (int s = 0; s < PF - 1; ++s)
    if (i0 + s < nsteps) step(i0 + s, kreg[s], vreg[s], okb[s], scb[s]);   // uniform over the workgroup

  // partial result of this piece: lane holds channels dt*16 + 4*lg + 0..3
  l = across_rows<16, false>(l);
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

}  // namespace pkv
