// Paged decode attention for gfx950 (CDNA4, wave64).  The per-sequence pass
// below does its arithmetic on the VALU; for head_dim 128 with 4 or 8 query
// heads per KV head the kernels run its matrix-core form instead
// (decode_mfma.h), and the shared-prefix group pass (group_prefix.h), which
// the per-sequence pass can carry in the same launch, also uses MFMA.
//
// What is computed ("KV Cache from first principles" 2.1-2.2 and 4.3; "The
// KV Cache memory ledger" 2 and 4): for every sequence b and query head i,
//   out[b][i] = softmax_t(scale * <q[b][i], K_t>) . V_t  over t < L_b,
// with K_t, V_t read through the block table (block table[t / 16], offset
// t % 16), and query head i reading KV head i / g.
//
// Decode is a matrix-vector product per KV head, bound by HBM: every K/V
// byte is used by only g query heads.  The kernel therefore streams each
// (block, kv_head) tile once from HBM and makes that one read serve all g
// query heads.  Scores use packed dot2 for f16/bf16 K (and for fp8 or int8
// K after widening it to f16, both exact -- int8 by SDWA converts; the query is held in f16 after a
// power-of-two rescale of the KV group that the scores undo), fp32 FMA for
// fp32 K.  P.V accumulates in fp32: for f16, fp8 and int8 V it is a dot2
// over pairs of tokens with the probabilities rounded once to f16 (relative
// error <= 2^-11 per weight); bf16 and fp32 V use fp32 FMA.
//
// 8-bit caches ("The KV Cache memory ledger" 7; "KV Cache from first
// principles" 5.2): K and V may use different code sets (K fp8 with V int8)
// of the same width, each with a scale per (block, KV head); K may also have
// one factor per (KV head, channel), which is folded into the query once:
// <q, k * c> = <q * c, k>.
//
// Work split.  Grid = (partition p, kv head h, sequence b); a workgroup of
// four waves owns the blocks [p*PB, (p+1)*PB) of (b, h); wave w takes every
// fourth step of them, a step being one block (two for 8-bit caches with 8
// query heads, whose tiles are small).  K tiles are copied by LDS DMA into
// a per-wave ring, each copy reading 1 KiB contiguously; V tiles are loaded
// straight into registers (see "Staging" below).  Inside a wave, lane l then
// takes token rows of group r = l / LPT of every tile and the column c =
// l % LPT of LW bytes (16; 8 for 8-bit caches with 8 query heads, so that a
// lane owns 8 channels and its accumulators fit two waves per SIMD), and
// keeps its slice of all g query vectors in registers for the whole
// partition.  At the end the token rows of a wave are combined with lane
// swaps (reduce-scatter), and the waves through LDS.
//
// Scores.  A lane's partial dot products (g heads x its tokens) are summed
// over the LPT lanes of its row with a DPP reduce-scatter: at every level a
// lane keeps half of its partial sums and adds its partner's matching half.
// Partners hold mirrored register orders (slot k of lane l holds quantity
// k ^ M(l), M built from the lane's level bits), so each level is a plain
// "s[k] += dpp(s[k + n/2])" with no selects.  After the reduce-scatter every
// score exists once per row, so the exponentials are not duplicated; an
// all-gather (the same exchange run backwards) then hands every lane the
// probabilities it needs for its V slice.
//
// Softmax.  Online softmax with a lazily moved reference maximum per head:
// probabilities are exp2(s - m_ref) and m_ref moves (rescaling the running
// sum and accumulator) only when a score exceeds it by more than 2^8, which
// after the first block is rare.  Every token row of every wave is its own
// stream; streams are merged by log-sum-exp at the end of the partition, and
// partitions by a second small kernel.
//
// Masking.  Positions >= L (the tail of the last block), and with a sliding
// window the positions outside it, get score -inf and a zeroed V operand, so
// poisoned slots never reach the sums (0 * NaN would).  Block ids outside
// the pool are treated as fully masked.  A window skips whole blocks: a
// partition walks only the attended blocks (sink blocks, then window blocks).
#include "pkv_internal.h"
#include "group_prefix.h"

#include <type_traits>
#include <utility>

namespace pkv {

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

template <KV KT, int D, int G>
struct Cfg {
  static constexpr int EB = kv_bytes<KT>::value;
  // Bytes a lane loads at a time.  16 in general; 8-bit caches serving 8
  // query heads load 8, so that a lane owns 8 channels as with 16-bit caches
  // (with 16 it would keep 16 channels x 8 heads of accumulators and query
  // and fall to one wave per SIMD).
  static constexpr int LW = (EB == 1 && G == 8) ? 8 : 16;
  static constexpr int NWD = LW / 4;                       // words per load
  static constexpr int E = LW / EB;                        // elements per load
  static constexpr int VPT = (D / E > 16) ? (D / E) / 16 : 1;  // loads per token per lane
  static constexpr int LPT = D / (E * VPT);                // lanes sharing one token
  static constexpr int R = 64 / LPT;                       // token rows per wave
  static constexpr int TPL = 16 / R;                       // tokens per lane per block
  static constexpr int NS = G * TPL;                       // score slots per lane
  static constexpr int LEVELS = ilog2(LPT);
  static constexpr int NRS = cmin(LEVELS, ilog2(NS));      // reduce-scatter levels
  static constexpr int NF = NS >> NRS;                     // slots left after it
  static constexpr int EL = E * VPT;                       // elements per lane per token
  static constexpr int NW = 4;                             // waves per workgroup
  static constexpr int NWT = NWD * VPT;                    // words per token per lane
  static constexpr int LPB = TPL * VPT;                    // loads per lane per tile
  static constexpr int TILE_B = 16 * D * EB;               // bytes of one (block, kv_head) tile
  static constexpr int NDMA = TILE_B / 1024;               // 1 KiB LDS DMA copies per tile
  // K tiles are staged in LDS, two slots per wave (deeper rings measured
  // slower); V tiles go straight to registers.
  static constexpr int KR = 2;
  // Blocks per step: a step of a wave waits for, issues and computes BPS
  // consecutive blocks.  Tiles of 8-bit caches with 8 query heads are small
  // (2 KiB at D = 128) and their kernels hold two waves per SIMD, so one
  // block per step would leave half the bytes in flight of a 16-bit step.
  static constexpr int BPS = (EB == 1 && G == 8) ? 2 : 1;
  static constexpr int KRING_B = NW * KR * BPS * TILE_B;
  // per-token scales of a ring tile's block: 16 K scales, then 16 V scales
  static constexpr int TOKS_B = 128;
  static constexpr int TOKRING_B = NW * KR * BPS * TOKS_B;
  static constexpr int RED_B = NW * G * (D + 2) * 4;       // end-of-partition combine
  static constexpr int SMEM_B = KRING_B + TOKRING_B > RED_B ? KRING_B + TOKRING_B : RED_B;
  static_assert(LPB * 64 * LW == TILE_B, "a tile is LPB wave-wide loads");
  static_assert(LW == 16 || NWT == 2, "8-byte loads: one per token");
  static_assert(LPT >= 1 && LPT <= 16 && (LPT & (LPT - 1)) == 0, "lanes per token");
  static_assert(TPL >= 1, "tokens per lane");
};

constexpr float kLazyMaxSlack = 8.0f;   // log2 units: probabilities stay <= 256

// Exchange of level KIND (0: c^8, 1: half mirror, 2: c^2, 3: c^1).
template <int KIND>
__device__ __forceinline__ float xlevel(float v) {
  if constexpr (KIND == 0) return dpp<DPP_ROW_ROR8>(v);
  else if constexpr (KIND == 1) return dpp<DPP_ROW_HALF_MIRROR>(v);
  else if constexpr (KIND == 2) return dpp<DPP_QUAD_XOR2>(v);
  else return dpp<DPP_QUAD_XOR1>(v);
}

// Lane bit that flips exactly across the partners of level KIND and across
// no other level's partners (solves m_k(F_j) = [k == j] for the flip sets
// F = {8}, {0,1,2}, {1}, {0} of the four exchanges).
template <int KIND, int LEVELS>
__device__ __forceinline__ int level_bit(int c) {
  const int b2 = LEVELS >= 3 ? (c >> 2) & 1 : 0;
  if constexpr (KIND == 0) return (c >> 3) & 1;
  else if constexpr (KIND == 1) return (c >> 2) & 1;
  else if constexpr (KIND == 2) return ((c >> 1) & 1) ^ b2;
  else return (c & 1) ^ b2;
}

// ---- per-dtype pieces ------------------------------------------------------
// The lane's slice of one query vector, kept in registers for the whole
// partition: packed 16-bit pairs when K is f16/bf16 (dot2 with K directly),
// packed f16 pairs when K is 8-bit (dot2 with K converted to f16), fp32 when
// K is fp32.
template <KV KT, int EL> struct QSlice { uint32_t w[EL / 2]; };
template <int EL> struct QSlice<KV::F32, EL> { float f[EL]; };

template <KV T>
__device__ __forceinline__ float load_elem_f32(const void* base, int64_t idx) {
  if constexpr (T == KV::F32) return ((const float*)base)[idx];
  else if constexpr (T == KV::F16) return (float)((const _Float16*)base)[idx];
  else return __builtin_bit_cast(float, ((uint32_t)((const uint16_t*)base)[idx]) << 16);
}

// The lane's slice of one query row as fp32: elements (v * LPT + c) * E + e
// for v < VPT, e < E (E consecutive elements per v, read 16 bytes at a time).
template <KV QT, int EL, int LPT, int E, int VPT>
__device__ __forceinline__ void q_slice_f32(const void* qrow, int c, float (&f)[EL]) {
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int e0 = (v * LPT + c) * E;
    if constexpr (QT == KV::F32) {
#pragma unroll
      for (int u = 0; u < E / 4; ++u) {
        const float4 x = *(const float4*)((const float*)qrow + e0 + 4 * u);
        f[v * E + 4 * u + 0] = x.x; f[v * E + 4 * u + 1] = x.y;
        f[v * E + 4 * u + 2] = x.z; f[v * E + 4 * u + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < E / 8; ++u) {
        const uint4 x = *(const uint4*)((const uint16_t*)qrow + e0 + 8 * u);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f[v * E + 8 * u + 2 * k] = QT == KV::F16 ? f16lo(w[k]) : bf16lo(w[k]);
          f[v * E + 8 * u + 2 * k + 1] = QT == KV::F16 ? f16hi(w[k]) : bf16hi(w[k]);
        }
      }
    }
  }
}

// q row (already offset to the lane's head) -> the lane's slice, for f16,
// bf16 and fp32 K (the query is read as stored).
template <KV KT, KV QT, int EL, int LPT, int E, int VPT>
__device__ __forceinline__ void load_q(QSlice<KT, EL>& qs, const void* qrow, int c) {
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int e0 = (v * LPT + c) * E;
    if constexpr (KT == KV::F16 || KT == KV::BF16) {
      static_assert(QT == KT, "16-bit caches take a query of the same type");
      const uint4 x = *(const uint4*)((const uint16_t*)qrow + e0);
      qs.w[v * 4 + 0] = x.x; qs.w[v * 4 + 1] = x.y; qs.w[v * 4 + 2] = x.z; qs.w[v * 4 + 3] = x.w;
    } else {
      static_assert(KT == KV::F32, "8-bit K packs its query with q8_pack");
#pragma unroll
      for (int e = 0; e < E; ++e) qs.f[v * E + e] = load_elem_f32<QT>(qrow, e0 + e);
    }
  }
}

// 8-bit K: the slice times K's channel factors `cf`, rescaled by 2^qexp and
// packed into f16 pairs.
template <KV KT, int EL>
__device__ __forceinline__ void q8_pack(QSlice<KT, EL>& qs, const float (&f)[EL], const float (&cf)[EL],
                                        int qexp) {
#pragma unroll
  for (int e = 0; e < EL; e += 2)
    qs.w[e / 2] = pack_f16x2(__builtin_ldexpf(f[e] * cf[e], qexp), __builtin_ldexpf(f[e + 1] * cf[e + 1], qexp));
}

// K/V words of one token for one lane: NWT dwords (VPT loads of 16 or 8 bytes).
template <int NWT> struct TokWords { uint32_t w[NWT]; };

template <int NWT>
__device__ __forceinline__ void words_of(const TokWords<NWT>& t, uint32_t (&w)[NWT]) {
#pragma unroll
  for (int k = 0; k < NWT; ++k) w[k] = t.w[k];
}

template <KV KT, int EL, int NWT>
__device__ __forceinline__ void to_f32(const TokWords<NWT>& t, float (&f)[EL]) {
  uint32_t w[NWT];
  words_of(t, w);
#pragma unroll
  for (int k = 0; k < NWT; ++k) {
    if constexpr (KT == KV::F32) {
      f[k] = __builtin_bit_cast(float, w[k]);
    } else if constexpr (KT == KV::F16) {
      f[2 * k] = f16lo(w[k]);
      f[2 * k + 1] = f16hi(w[k]);
    } else if constexpr (KT == KV::BF16) {
      f[2 * k] = bf16lo(w[k]);
      f[2 * k + 1] = bf16hi(w[k]);
    } else if constexpr (KT == KV::FP8) {
      const float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
      const float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
      f[4 * k + 0] = lo.x; f[4 * k + 1] = lo.y; f[4 * k + 2] = hi.x; f[4 * k + 3] = hi.y;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) f[4 * k + j] = (float)(int)(int8_t)(w[k] >> (8 * j));
    }
  }
}

// fp8 token words -> f16 pairs of adjacent elements (same token): EL / 2 words.
template <int EL, int NWT>
__device__ __forceinline__ void fp8_to_f16_pairs(const TokWords<NWT>& t, uint32_t (&h)[EL / 2]) {
  uint32_t w[NWT];
  words_of(t, w);
#pragma unroll
  for (int k = 0; k < NWT; ++k) {
    h[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[k], 1.0f, false));
    h[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[k], 1.0f, true));
  }
}

// int8 -> f16 pair, exactly (|x| <= 128 is an f16 integer): byte BL of `lo`
// and byte BH of `hi`, each sign-extended and converted by one SDWA convert
// that writes its half of the result (the second keeps the first's half).
#define PKV_CVT_I8_LO(B)                                                            \
  asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD "       \
      "src0_sel:BYTE_" #B : "=v"(r) : "v"(lo))
#define PKV_CVT_I8_HI(B)                                                            \
  asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE "  \
      "src0_sel:BYTE_" #B : "+v"(r) : "v"(hi))
template <int BL, int BH>
__device__ __forceinline__ uint32_t i8_pair_to_f16(uint32_t lo, uint32_t hi) {
  uint32_t r;
  if constexpr (BL == 0) PKV_CVT_I8_LO(0);
  else if constexpr (BL == 1) PKV_CVT_I8_LO(1);
  else if constexpr (BL == 2) PKV_CVT_I8_LO(2);
  else PKV_CVT_I8_LO(3);
  if constexpr (BH == 0) PKV_CVT_I8_HI(0);
  else if constexpr (BH == 1) PKV_CVT_I8_HI(1);
  else if constexpr (BH == 2) PKV_CVT_I8_HI(2);
  else PKV_CVT_I8_HI(3);
  return r;
}
#undef PKV_CVT_I8_LO
#undef PKV_CVT_I8_HI

// int8 token words -> f16 pairs of adjacent elements (same token): EL / 2 words.
template <int EL, int NWT>
__device__ __forceinline__ void int8_to_f16_pairs(const TokWords<NWT>& t, uint32_t (&h)[EL / 2]) {
  uint32_t w[NWT];
  words_of(t, w);
#pragma unroll
  for (int k = 0; k < NWT; ++k) {
    h[2 * k] = i8_pair_to_f16<0, 1>(w[k], w[k]);
    h[2 * k + 1] = i8_pair_to_f16<2, 3>(w[k], w[k]);
  }
}

// Partial <q_slice, K_slice> for one token.
template <KV KT, int EL, int NWT>
__device__ __forceinline__ float qk_partial(const QSlice<KT, EL>& qs, const TokWords<NWT>& t,
                                            const float (&kf)[EL], const uint32_t (&kh)[EL / 2]) {
  float s;
  if constexpr (KT == KV::F16 || is_quantised<KT>()) {
    uint32_t w[EL / 2];
    if constexpr (KT == KV::F16) words_of(t, w);
    else {
#pragma unroll
      for (int k = 0; k < EL / 2; ++k) w[k] = kh[k];
    }
    // three-operand form with an inline zero: no register to clear
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(s) : "v"(qs.w[0]), "v"(w[0]));
#pragma unroll
    for (int k = 1; k < EL / 2; ++k)
      s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qs.w[k]), __builtin_bit_cast(half2_t, w[k]),
                                 s, false);
  } else if constexpr (KT == KV::BF16) {
    uint32_t w[EL / 2];
    words_of(t, w);
    s = 0.f;
#pragma unroll
    for (int k = 0; k < EL / 2; ++k)
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, qs.w[k]),
                                          __builtin_bit_cast(bf162_t, w[k]), s, false);
  } else {
    s = 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) s = __builtin_fmaf(qs.f[e], kf[e], s);
  }
  return s;
}

// V of two tokens -> per element, an f16 pair (token 0, token 1) for dot2.
template <KV KT, int EL, int NWT>
__device__ __forceinline__ void v_token_pairs(const TokWords<NWT>& t0, const TokWords<NWT>& t1,
                                              uint32_t (&vp)[EL]) {
  uint32_t a[NWT], b[NWT];
  words_of(t0, a);
  words_of(t1, b);
#pragma unroll
  for (int k = 0; k < NWT; ++k) {
    if constexpr (KT == KV::F16) {
      // word k holds elements 2k, 2k+1 of each token
      vp[2 * k] = __builtin_amdgcn_perm(b[k], a[k], 0x05040100u);
      vp[2 * k + 1] = __builtin_amdgcn_perm(b[k], a[k], 0x07060302u);
    } else if constexpr (KT == KV::INT8) {
      // word k holds int8 elements 4k..4k+3: element j of both tokens
      vp[4 * k + 0] = i8_pair_to_f16<0, 0>(a[k], b[k]);
      vp[4 * k + 1] = i8_pair_to_f16<1, 1>(a[k], b[k]);
      vp[4 * k + 2] = i8_pair_to_f16<2, 2>(a[k], b[k]);
      vp[4 * k + 3] = i8_pair_to_f16<3, 3>(a[k], b[k]);
    } else {
      // word k holds fp8 elements 4k..4k+3: interleave bytes, then widen
      const uint32_t lo = __builtin_amdgcn_perm(b[k], a[k], 0x05010400u);
      const uint32_t hi = __builtin_amdgcn_perm(b[k], a[k], 0x07030602u);
      vp[4 * k + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false));
      vp[4 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true));
      vp[4 * k + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false));
      vp[4 * k + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true));
    }
  }
}

template <KV OT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float x) {
  if constexpr (OT == KV::F32) ((float*)out)[idx] = x;
  else if constexpr (OT == KV::F16) ((_Float16*)out)[idx] = (_Float16)x;
  else ((uint16_t*)out)[idx] = f32_to_bf16_rne(x);
}

__device__ __forceinline__ float exp2_safe_factor(float m_old, float m_new) {
  // factor that moves a sum referenced to m_old onto m_new (m_new >= m_old)
  return m_old == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_old - m_new);
}

// The blocks one sequence's query attends in the cache, as a compressed
// list: with a sliding window of W and S sink tokens ("KV Cache from first
// principles" 5.3) they are the sink blocks [0, nsb) then the window blocks
// [wb0, nblk); without a window, or when the two ranges touch, simply
// [0, nblk).  Position pos of block j is attended iff pos < L and (no
// window, or pos < se, or pos >= ws).  With full-precision sink tiles
// (`skip` = S > 0) the sinks are attended elsewhere: the cache serves only
// positions >= S (and inside the window).
struct SeqSpan {
  int L, nblk, natt, nsb, wb0, se, ws;
  bool windowed;
  __device__ __forceinline__ SeqSpan(int len, int max_blocks, int window, int sinks, int skip) {
    L = len < 0 ? 0 : (len > max_blocks * 16 ? max_blocks * 16 : len);
    nblk = (L + 15) >> 4;
    windowed = window > 0 && L > window;
    ws = windowed ? L - window : 0;
    se = windowed ? min(sinks, L) : 0;
    if (skip > 0) {                      // sinks come from their own tiles
      se = 0;
      ws = max(ws, min(skip, L));
      windowed = ws > 0;
    }
    if (se >= ws) windowed = false;      // sinks reach the window: everything
    nsb = 0;
    wb0 = 0;
    if (windowed) {
      nsb = (se + 15) >> 4;
      wb0 = ws >> 4;
      if (nsb >= wb0) { nsb = 0; wb0 = 0; }  // the ranges touch: one range
    }
    natt = nsb + nblk - wb0;
  }
  __device__ __forceinline__ int logical(int cidx) const { return cidx < nsb ? cidx : cidx - nsb + wb0; }
  // token rows of logical block j that hold a token: 16, but fewer in the
  // last block.  Rows past them are never fetched: their scores are masked
  // and their V rows zeroed whatever the staging holds there, so the
  // kernels read the bytes of the sequence's tokens and no more.
  __device__ __forceinline__ int rows(int j) const {
    const int n = L - j * 16;
    return n < 0 ? 0 : (n > 16 ? 16 : n);
  }
  // bit t set: token t of logical block j is attended
  __device__ __forceinline__ uint32_t valid_bits(int j) const {
    const int base = j * 16;
    const int nv = min(16, L - base);
    uint32_t m = nv >= 16 ? 0xFFFFu : (nv > 0 ? ((1u << nv) - 1u) : 0u);
    if (windowed) {
      const int lo = ws - base;                    // tokens >= lo are in the window
      const int hi = se - base;                    // tokens < hi are sinks
      const uint32_t win = lo <= 0 ? 0xFFFFu : (lo >= 16 ? 0u : (0xFFFFu & ~((1u << lo) - 1u)));
      const uint32_t snk = hi <= 0 ? 0u : (hi >= 16 ? 0xFFFFu : ((1u << hi) - 1u));
      m &= (win | snk);
    }
    return m;
  }
};

// ---- pieces both per-sequence passes share --------------------------------
// The step's append, when the call carries it ("KV Cache from first
// principles" 2.3: the new token's K and V are written at the current
// length before it is attended).  The partition holding the sequence's last
// attended block -- the new token's -- writes head h's new rows into the
// slot, and within it the wave that will read that block, so the write
// needs no barrier: the wave's read of the block is issued after a wait for
// all its memory operations (the per-step wait, or an explicit one when
// that block is the wave's first).  No other workgroup reads the block.
// Partition 0 writes when nothing is attended.  One wave: a K row and a V
// row, 16 bytes per lane.
//
// The copy comes in two halves, so that a caller can overlap its round trip
// with other loads: append_rows_load issues the load of the lane's 16 bytes
// and append_rows_store writes them.  In between the caller must not read
// the new token's block; the store is complete after the caller's next
// wait for all its memory operations.
struct PendingRow {
  u32x4_t x;
  u32x4_t* dst;   // null: the lane writes nothing
};
template <int D, int EB>
__device__ __forceinline__ PendingRow append_rows_load(const DecodeArgs& a, int b, int h, int lane, int64_t slot) {
  PendingRow r;
  r.dst = nullptr;
  constexpr int ROWC = D * EB / 16;   // 16-byte chunks of one row
  static_assert(2 * ROWC <= 64, "one wave copies a K row and a V row");
  if (slot >= 0 && slot < (int64_t)a.num_blocks * 16 && lane < 2 * ROWC) {
    const bool isv = lane >= ROWC;
    const int ch = isv ? lane - ROWC : lane;
    const int64_t src = ((int64_t)b * a.num_kv_heads + h) * ROWC + ch;
    const int64_t dst = (((slot >> 4) * a.num_kv_heads + h) * 16 + (slot & 15)) * ROWC + ch;
    r.x = reinterpret_cast<const u32x4_t*>(isv ? a.v_new : a.k_new)[src];
    r.dst = reinterpret_cast<u32x4_t*>(isv ? a.v_cache_rw : a.k_cache_rw) + dst;
  }
  return r;
}
__device__ __forceinline__ void append_rows_store(const PendingRow& r) {
  if (r.dst) *r.dst = r.x;
}
template <int D, int EB>
__device__ __forceinline__ void append_new_rows(const DecodeArgs& a, int b, int h, int lane, int64_t slot) {
  append_rows_store(append_rows_load<D, EB>(a, b, h, lane, slot));
}

// The step's append into a layout with an 8-bit cache: K (8-bit, or a
// 16-bit K, which is copied) and V (8-bit) of sequence b's new token, head
// h, written at its slot exactly as pkv_kv_append_quant (8-bit) and
// pkv_kv_append (16-bit) write them: y = x / channel factor (8-bit K, when
// given), then with per-token scales the slot's scale max|y| / QMAX (1 for
// a zero row) is written first, otherwise the block's given scale is read;
// codes are the nearest (ties to even) of clamp(y / scale, +-QMAX).  One
// wave: lanes 0..31 take K, 32..63 V, D / 32 consecutive elements each.
// The quantising append comes in two halves as well (see append_rows_load):
// append_q8_load issues the loads -- the lane's elements of the new row as
// stored and the block's given scale -- and append_q8_store does the rest
// (K's channel factors, when given, are read there).
template <KV QT, int D>
struct PendingQ8 {
  static constexpr int EPL = D / 32;                            // elements per lane
  static constexpr int RW = EPL * (QT == KV::F32 ? 4 : 2) / 4;  // their dwords: 1, 2 or 4
  uint32_t raw[RW];
  float given;        // the block's scale for the lane's half (one per block and head)
  bool on;            // the slot is in the pool (uniform over the wave)
};
template <KV KT, KV VT, KV QT, int D>
__device__ __forceinline__ PendingQ8<QT, D> append_q8_load(const DecodeArgs& a, int b, int h, int lane,
                                                           int64_t slot) {
  static_assert(is_quantised<VT>(), "an 8-bit V");
  using P = PendingQ8<QT, D>;
  constexpr int EPL = P::EPL, RW = P::RW;
  static_assert(EPL == 2 || EPL == 4, "head_dim 64 or 128");
  P r;
  r.on = slot >= 0 && slot < (int64_t)a.num_blocks * 16;
  r.given = 1.0f;
#pragma unroll
  for (int k = 0; k < RW; ++k) r.raw[k] = 0u;
  if (!r.on) return r;
  const bool isv = lane >= 32;
  const int e0 = (lane & 31) * EPL;
  const int64_t bh = (slot >> 4) * a.num_kv_heads + h;             // (block, head), uniform
  const int64_t src = ((int64_t)b * a.num_kv_heads + h) * D + e0;  // element of k_new / v_new
  const char* from = (const char*)(isv ? a.v_new : a.k_new) + src * (RW * 4 / EPL);
  if constexpr (RW == 1) {
    r.raw[0] = *(const uint32_t*)from;
  } else if constexpr (RW == 2) {
    const u32x2_t x = *(const u32x2_t*)from;
    r.raw[0] = x[0]; r.raw[1] = x[1];
  } else {
    const u32x4_t x = *(const u32x4_t*)from;
    r.raw[0] = x[0]; r.raw[1] = x[1]; r.raw[2] = x[2]; r.raw[3] = x[3];
  }
  // each half's given scale by a load of its own (uniform addresses), then
  // a choice of values: a choice of pointers per lane would put both in
  // per-lane scratch memory
  float gv = 1.0f, gk = 1.0f;
  if (!a.v_tok) gv = a.v_scales[bh];
  if constexpr (is_quantised<KT>()) {
    if (!a.k_tok) gk = a.k_scales[bh];
  }
  r.given = isv ? gv : gk;
  return r;
}

// Element e of the lane's loaded row, as fp32.
template <KV QT, int D>
__device__ __forceinline__ float pending_elem(const PendingQ8<QT, D>& r, int e) {
  if constexpr (QT == KV::F32) return __builtin_bit_cast(float, r.raw[e]);
  else {
    const uint32_t hbits = (r.raw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    if constexpr (QT == KV::F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)hbits);
    else return __builtin_bit_cast(float, hbits << 16);
  }
}

// The step's append into a layout with an 8-bit cache: K (8-bit, or a
// 16-bit K, which is copied) and V (8-bit) of sequence b's new token, head
// h, written at its slot exactly as pkv_kv_append_quant (8-bit) and
// pkv_kv_append (16-bit) write them: y = x / channel factor (8-bit K, when
// given), then with per-token scales the slot's scale max|y| / QMAX (1 for
// a zero row) is written first, otherwise the block's given scale is used;
// codes are the nearest (ties to even) of clamp(y / scale, +-QMAX).  One
// wave: lanes 0..31 take K, 32..63 V, D / 32 consecutive elements each.
template <KV KT, KV VT, KV QT, int D>
__device__ __forceinline__ void append_q8_store(const DecodeArgs& a, int h, int lane, int64_t slot,
                                                const PendingQ8<QT, D>& r) {
  constexpr int EPL = PendingQ8<QT, D>::EPL, RW = PendingQ8<QT, D>::RW;
  if (!r.on) return;                                                // uniform over the wave
  const bool isv = lane >= 32;
  const int e0 = (lane & 31) * EPL;
  const int64_t bh = (slot >> 4) * a.num_kv_heads + h;             // (block, head)
  const int64_t dst = (bh * 16 + (slot & 15)) * D + e0;            // element of the cache
  if constexpr (!is_quantised<KT>()) {
    static_assert(QT == KT, "a 16-bit K takes rows of its own type");
    if (!isv) {                                                     // K: a bit copy
      uint32_t* to = (uint32_t*)((uint16_t*)a.k_cache_rw + dst);
#pragma unroll
      for (int k = 0; k < RW; ++k) to[k] = r.raw[k];
    }
  }
  float y[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) y[e] = pending_elem<QT, D>(r, e);
  if constexpr (is_quantised<KT>()) {
    if (!isv && a.k_chan)
#pragma unroll
      for (int e = 0; e < EPL; ++e) y[e] = y[e] / a.k_chan[(int64_t)h * D + e0 + e];
  }
  // both flags read, then a bit picked: a select between the two fields'
  // addresses would put them in per-lane scratch memory
  const int tok_bits = (a.k_tok ? 1 : 0) | (a.v_tok ? 2 : 0);
  const bool tok = (tok_bits >> (isv ? 1 : 0)) & 1;
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(y[e]));
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));   // over the half
  auto write = [&](auto ct) __attribute__((always_inline)) {
    constexpr KV CT = decltype(ct)::value;
    constexpr float QM = qmax<CT>();
    float scale = r.given;
    if (tok) {
      scale = amax > 0.f ? amax / QM : 1.0f;
      float* scales = const_cast<float*>(isv ? a.v_scales : a.k_scales);
      if ((lane & 31) == 0) scales[bh * 16 + (slot & 15)] = scale;
    }
    float v[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float q = y[e] / scale;
      v[e] = q > QM ? QM : (q < -QM ? -QM : q);   // NaN passes through
    }
    const uint32_t codes = encode_codes<CT, EPL>(v);
    uint8_t* to = (uint8_t*)(isv ? a.v_cache_rw : a.k_cache_rw) + dst;
    if constexpr (EPL == 4) *(uint32_t*)to = codes;
    else *(uint16_t*)to = (uint16_t)codes;
  };
  if (isv) write(std::integral_constant<KV, VT>{});
  else if constexpr (is_quantised<KT>()) write(std::integral_constant<KV, KT>{});
}

template <KV KT, KV VT, KV QT, int D>
__device__ __forceinline__ void append_new_rows_q8(const DecodeArgs& a, int b, int h, int lane, int64_t slot) {
  append_q8_store<KT, VT, QT, D>(a, h, lane, slot, append_q8_load<KT, VT, QT, D>(a, b, h, lane, slot));
}

// The step's append for any cache layout (see append_new_rows and
// append_new_rows_q8), by one wave; slot = new_slots[b].
template <KV KT, KV VT, KV QT, int D>
__device__ __forceinline__ void append_step_rows(const DecodeArgs& a, int b, int h, int lane, int64_t slot) {
  if constexpr (is_quantised<VT>()) append_new_rows_q8<KT, VT, QT, D>(a, b, h, lane, slot);
  else append_new_rows<D, kv_bytes<KT>::value>(a, b, h, lane, slot);
}
// The same in two halves (append_rows_load / append_q8_load, then the
// matching store).
template <KV KT, KV VT, KV QT, int D>
__device__ __forceinline__ auto append_step_load(const DecodeArgs& a, int b, int h, int lane, int64_t slot) {
  if constexpr (is_quantised<VT>()) return append_q8_load<KT, VT, QT, D>(a, b, h, lane, slot);
  else return append_rows_load<D, kv_bytes<KT>::value>(a, b, h, lane, slot);
}
template <KV KT, KV VT, KV QT, int D, class P>
__device__ __forceinline__ void append_step_store(const DecodeArgs& a, int h, int lane, int64_t slot, const P& r) {
  if constexpr (is_quantised<VT>()) append_q8_store<KT, VT, QT, D>(a, h, lane, slot, r);
  else append_rows_store(r);
}

// Partition p's result for query head h * G + ha of sequence b, channel d,
// from its (m, l, o), o being the unnormalised sum: the output element, or
// the partition's workspace slot when the call is split.
template <KV OT, int D, int G>
__device__ __forceinline__ void finish_row(const DecodeArgs& a, int b, int h, int p, int ha, int d, float m,
                                           float lsum, float o) {
  const int64_t row = (int64_t)b * a.num_kv_heads * G + h * G + ha;
  const float res = lsum > 0.f ? o / lsum : 0.f;
  if (!a.split) {
    store_out<OT>(a.out, row * D + d, res);
  } else {
    a.o_part[(row * a.part_stride + p) * D + d] = res;
    if (d == 0) {
      a.ml_part[(row * a.part_stride + p) * 2 + 0] = m;
      a.ml_part[(row * a.part_stride + p) * 2 + 1] = lsum;
    }
  }
}

// A partition with nothing of the cache: a zero row (empty partitions of a
// split call are skipped by the merge), and the append if it falls here.
template <KV KT, KV VT, KV QT, KV OT, int D, int G>
__device__ __forceinline__ void finish_empty(const DecodeArgs& a, int b, int h, int p, int tid, bool append,
                                             int64_t slot) {
  if (append) append_step_rows<KT, VT, QT, D>(a, b, h, tid & 63, slot);
  if (!a.split)
    for (int idx = tid; idx < G * D; idx += 256) finish_row<OT, D, G>(a, b, h, p, idx / D, idx % D, -INFINITY, 0.f, 0.f);
}

// A block's table entry, as read (an id outside the pool masks the whole
// block), and its 8-bit scales.
struct BlockRef {
  int phys;
  float ks, vs;
};

// Byte offset of tile (block, KV head h) in a cache; an id outside the
// pool reads block 0 (and is masked).
__device__ __forceinline__ int64_t tile_offset(const DecodeArgs& a, int h, int phys_raw, int tile_bytes) {
  const int phys = ((unsigned)phys_raw < (unsigned)a.num_blocks) ? phys_raw : 0;
  return ((int64_t)phys * a.num_kv_heads + h) * (int64_t)tile_bytes;
}

// The block's K and V scales (8-bit caches with one scale per (block, head);
// 1 otherwise, and with per-token scales, which are read per lane).
// Uniform index, read-only data: scalar loads, which do not wait behind the
// tile copies in flight (those count on vmcnt).
template <bool KQ, bool VQ>
__device__ __forceinline__ void block_scales(const DecodeArgs& a, int h, BlockRef& br) {
  br.ks = 1.f;
  br.vs = 1.f;
  const int phys = ((unsigned)br.phys < (unsigned)a.num_blocks) ? br.phys : 0;
  const int64_t si = (int64_t)phys * a.num_kv_heads + h;
  if constexpr (KQ)
    if (!a.k_tok) br.ks = ((const __attribute__((address_space(4))) float*)a.k_scales)[si];
  if constexpr (VQ)
    if (!a.v_tok) br.vs = ((const __attribute__((address_space(4))) float*)a.v_scales)[si];
}

// End of a partition: every wave's (reference maximum, sum, accumulators)
// is in LDS; each thread combines them for G * D / 256 outputs.
template <KV OT, int D, int G, int NW>
__device__ __forceinline__ void combine_waves(const DecodeArgs& a, int b, int h, int p, int tid,
                                              const float (*red_acc)[G][D], const float (*red_m)[G],
                                              const float (*red_l)[G]) {
  for (int idx = tid; idx < G * D; idx += 256) {
    const int ha = idx / D, d = idx % D;
    float m = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) m = fmaxf(m, red_m[ww][ha]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float f = red_m[ww][ha] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(red_m[ww][ha] - m);
      lsum += red_l[ww][ha] * f;
      o += red_acc[ww][ha][d] * f;
    }
    finish_row<OT, D, G>(a, b, h, p, ha, d, m, lsum, o);
  }
}

// ---------------------------------------------------------------------------
// One workgroup of the cache pass: partition p of (sequence b, KV head h);
// smem is the workgroup's LDS (Cfg::SMEM_B bytes).
template <KV KT, KV VT, KV QT, KV OT, int D, int G>
__device__ __forceinline__ void decode_body(const DecodeArgs& a, int p, int h, int b, char* smem) {
  static_assert(kv_bytes<VT>::value <= kv_bytes<KT>::value, "V is no wider than K");
  static_assert(is_quantised<VT>() || !is_quantised<KT>(), "an 8-bit K goes with an 8-bit V");
  constexpr bool KQ = is_quantised<KT>(), VQ = is_quantised<VT>();
  using C = Cfg<KT, D, G>;
  constexpr int E = C::E, VPT = C::VPT, LPT = C::LPT, R = C::R, TPL = C::TPL, NWT = C::NWT, LW = C::LW;
  // V tiles use K's lane layout (same tokens and channels per lane); a
  // narrower V (16-bit K with 8-bit V) is loaded in proportionally smaller
  // pieces: VEB bytes per element, NWTV words per token per lane.
  constexpr int VEB = kv_bytes<VT>::value, VLW = LW * VEB / C::EB, NWTV = NWT * VEB / C::EB;
  static_assert(VLW == 16 || VLW == 8, "V loads of 16 or 8 bytes");
  constexpr int NS = C::NS, NRS = C::NRS, NF = C::NF, EL = C::EL, NW = C::NW;
  constexpr int LEVELS = C::LEVELS;
  // P.V as f16 dot2 over pairs of tokens (probabilities rounded to f16)
  constexpr bool PV_DOT2 = (VT == KV::F16 || is_quantised<VT>()) && TPL >= 2;

  // LDS: while streaming, per-wave rings of staged K and V tiles; at the end
  // of the partition the same bytes hold the per-wave partial results.
  float (*red_acc)[G][D] = reinterpret_cast<float (*)[G][D]>(smem);
  float (*red_m)[G] = reinterpret_cast<float (*)[G]>(smem + NW * G * D * 4);
  float (*red_l)[G] = reinterpret_cast<float (*)[G]>(smem + NW * G * D * 4 + NW * G * 4);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int Hq = a.num_kv_heads * G;

  // the new token's slot, when the step's append is carried: read next to
  // the sequence's length, so that the append does not wait for it later
  const int64_t new_slot = a.new_slots ? a.new_slots[b] : -1;
  // positions covered elsewhere (sink tiles, or a shared prefix read by the
  // group pass) are skipped here
  const int pre = a.sink_tiles ? 0 : prefix_blocks_of_seq(a, b);
  const SeqSpan span(a.context_lens[b], a.max_blocks, a.window, a.sinks,
                     a.sink_tiles ? a.sinks : 16 * pre);
  // this partition: entries [j0, j1) of the sequence's attended-block list
  const SeqParts parts(span.natt, a.part_blocks, a.num_parts, p);
  const int j0 = parts.j0, j1 = parts.j1;

  // the step's append (append_new_rows): by the partition holding the new
  // token's block, and in it by the wave that reads that block
  const bool appends = a.new_slots != nullptr && p == (parts.n > 0 ? parts.n - 1 : 0);
  constexpr int BPS = C::BPS;
  const int append_wave = j1 > j0 ? ((j1 - 1 - j0) / BPS) % NW : 0;
  auto append_rows = [&]() __attribute__((always_inline)) {
    append_step_rows<KT, VT, QT, D>(a, b, h, lane, new_slot);
  };
  if (j0 >= j1) {
    finish_empty<KT, VT, QT, OT, D, G>(a, b, h, p, tid, appends && w == 0, new_slot);
    return;
  }

  // Register slot k = hs * TPL + i holds (query head hs ^ hmask, tile token
  // row ((i ^ tmask) * R + r)); the masks mirror partners' orders (see above).
  const int r = lane / LPT, c = lane % LPT;
  int M = 0;
  static_for<NRS>([&](auto l) {
    constexpr int kind = 4 - LEVELS + decltype(l)::value;
    M |= level_bit<kind, LEVELS>(c) * (NS >> (decltype(l)::value + 1));
  });
  const int hmask = M / TPL;
  const int tmask = M % TPL;

  auto qrow_of = [&](int hs) {
    const int64_t qoff = ((int64_t)b * Hq + h * G + (hs ^ hmask)) * D;
    return (QT == KV::F32) ? (const void*)((const float*)a.q + qoff)
                           : (const void*)((const uint16_t*)a.q + qoff);
  };
  // 8-bit K: the query times K's channel factors (1 without them), with one
  // power-of-two rescale for the whole KV group, from the largest |q * c|
  // over all g heads (every lane of a row sees all of them, so every lane
  // derives the same exponent), so the partial sums the rows combine agree.
  // The query is loaded after the first tile loads are issued (below), so
  // its latency overlaps theirs.
  QSlice<KT, EL> qs[G];
  int qexp = 0;
  float qfac = 1.f;   // undoes the rescale on the scores
  auto load_query = [&]() __attribute__((always_inline)) {
  if constexpr (KQ) {
    float cf[EL];
    if (a.k_chan) {
      q_slice_f32<KV::F32, EL, LPT, E, VPT>(a.k_chan + (int64_t)h * D, c, cf);
    } else {
#pragma unroll
      for (int e = 0; e < EL; ++e) cf[e] = 1.0f;
    }
    float m = 0.f;
#pragma unroll
    for (int hs = 0; hs < G; ++hs) {
      float f[EL];
      q_slice_f32<QT, EL, LPT, E, VPT>(qrow_of(hs), c, f);
#pragma unroll
      for (int e = 0; e < EL; ++e) m = fmaxf(m, fabsf(f[e] * cf[e]));
    }
    static_for<LEVELS>([&](auto l) { m = fmaxf(m, xlevel<4 - LEVELS + decltype(l)::value>(m)); });
    int ex;
    (void)__builtin_frexpf(m, &ex);             // m = f * 2^ex, f in [0.5, 1)
    qexp = m > 0.f ? 15 - ex : 0;               // largest element lands in [2^14, 2^15)
    qexp = qexp > 100 ? 100 : (qexp < -100 ? -100 : qexp);
#pragma unroll
    for (int hs = 0; hs < G; ++hs) {
      float f[EL];
      q_slice_f32<QT, EL, LPT, E, VPT>(qrow_of(hs), c, f);
      q8_pack<KT, EL>(qs[hs], f, cf, qexp);
    }
  } else {
#pragma unroll
    for (int hs = 0; hs < G; ++hs) load_q<KT, QT, EL, LPT, E, VPT>(qs[hs], qrow_of(hs), c);
  }
  qfac = __builtin_ldexpf(1.0f, -qexp);
  };

  float acc[G][EL];
  float mref[G];
#pragma unroll
  for (int hs = 0; hs < G; ++hs) {
    mref[hs] = -INFINITY;
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[hs][e] = 0.f;
  }
  float lpart[NF];
#pragma unroll
  for (int k = 0; k < NF; ++k) lpart[k] = 0.f;

  const char* kbase = (const char*)a.k_cache;
  const char* vbase = (const char*)a.v_cache;
  // The table is read-only for the whole kernel: reading it through the
  // constant address space makes every entry a scalar load (lgkmcnt), which
  // never waits behind the in-flight tile copies (vmcnt).
  const __attribute__((address_space(4))) int32_t* table =
      (const __attribute__((address_space(4))) int32_t*)(a.block_tables + (int64_t)b * a.max_blocks);

  constexpr int KR = C::KR, TILE_B = C::TILE_B, NDMA = C::NDMA;
  // 16-byte lanes: copy n of a tile moves token rows n / VPT * R .. + R - 1,
  // 16-byte column (n % VPT) * LPT + c, in lane order, so each lane later
  // reads back exactly the bytes it copied.  8-byte lanes: the tile lands in
  // LDS as it is in HBM (row-major) and lanes read their 8 bytes from there.
  // Either way every copy reads 1 KiB contiguously.
  uint32_t dma_off[NDMA];
  if constexpr (LW == 16) {
    static_assert(NDMA == C::LPB, "one copy per 16-byte load");
#pragma unroll
    for (int i = 0; i < TPL; ++i)
#pragma unroll
      for (int v = 0; v < VPT; ++v)
        dma_off[i * VPT + v] = (uint32_t)(((i * R + r) * D + (v * LPT + c) * E) * C::EB);
  } else {
#pragma unroll
    for (int n = 0; n < NDMA; ++n) dma_off[n] = (uint32_t)(n * 1024 + lane * 16);
  }
  // A block's table entry is read two steps before the step that computes
  // the block and its scales one step before, so neither scalar load's
  // latency sits between a step's wait and its next tile loads.
  auto entry_of = [&](int j) __attribute__((always_inline)) { return table[span.logical(j)]; };
  auto tile_of = [&](int phys_raw) __attribute__((always_inline)) { return tile_offset(a, h, phys_raw, TILE_B); };
  auto vtile_of = [&](int phys_raw) __attribute__((always_inline)) {
    return tile_offset(a, h, phys_raw, 16 * D * VEB);
  };
  auto scales_of = [&](BlockRef& br) __attribute__((always_inline)) { block_scales<KQ, VQ>(a, h, br); };
  // Per-token scales ("KV Cache from first principles" 5.2): the 16 K and
  // 16 V scales of a block's slots are copied by LDS DMA (four lanes of 16
  // bytes each) into the ring tile's scale area, waited for with its K
  // tile; a lane reads those of its own token rows.
  const char* toks_area = smem + C::KRING_B + w * KR * BPS * C::TOKS_B;
  auto issue_tok = [&](int phys_raw, int sk) __attribute__((always_inline)) {
    if constexpr (KQ || VQ) {
      const int64_t si = tile_offset(a, h, phys_raw, 16);   // (block, head) * 16 scales
      const uint32_t dst = lds_offset(toks_area) + (uint32_t)(sk * C::TOKS_B);
      if (KQ && a.k_tok && lane < 4) lds_dma16(a.k_scales + si, (uint32_t)(lane * 16), dst);
      if (VQ && a.v_tok && lane < 4) lds_dma16(a.v_scales + si, (uint32_t)(lane * 16), dst + 64);
    }
  };
  // vr is consumed: tokens outside the sequence (or window) are zeroed in it.
  auto compute_block = [&](int j, int sk, const BlockRef& br, const TokWords<NWT> (&kr)[TPL],
                           TokWords<NWTV> (&vr)[TPL]) __attribute__((always_inline)) {
    const int jl = span.logical(j);
    const bool blk_ok = (unsigned)br.phys < (unsigned)a.num_blocks;
    const uint32_t vbits = blk_ok ? span.valid_bits(jl) : 0u;
    float cs = a.scale;  // scale * log2(e), folded on the host
    float vsc = 1.f;
    if constexpr (KQ) cs *= br.ks;   // br.ks, br.vs: 1 with per-token scales
    if constexpr (VQ) vsc = br.vs;
    // per-token scales of the lane's token rows (i ^ tmask) * R + r (1
    // otherwise, and for a row that holds no attended token: its slot's
    // scale may never have been written, and a NaN there would survive the
    // zero probability it is multiplied with)
    float kt[TPL], vt[TPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      kt[i] = 1.f;
      vt[i] = 1.f;
      if constexpr (KQ || VQ) {
        const int row = (i ^ tmask) * R + r;
        const float* ts = (const float*)(toks_area + sk * C::TOKS_B) + row;
        const bool live = (vbits >> row) & 1u;
        if (KQ && a.k_tok && live) kt[i] = ts[0];
        if (VQ && a.v_tok && live) vt[i] = ts[16];
      }
    }

    // 1. partial scores: slot k = hs * TPL + i
    float s[NS];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      float kf[EL];
      uint32_t kh[EL / 2];
      if constexpr (KT == KV::F32) to_f32<KT, EL, NWT>(kr[i], kf);
      if constexpr (KT == KV::FP8) fp8_to_f16_pairs<EL, NWT>(kr[i], kh);
      if constexpr (KT == KV::INT8) int8_to_f16_pairs<EL, NWT>(kr[i], kh);
#pragma unroll
      for (int hs = 0; hs < G; ++hs) s[hs * TPL + i] = qk_partial<KT, EL, NWT>(qs[hs], kr[i], kf, kh);
    }
    // 2. reduce-scatter over the row, then all-reduce for any levels left
    static_for<NRS>([&](auto l) {
      constexpr int lv = decltype(l)::value;
      constexpr int half = NS >> (lv + 1);
#pragma unroll
      for (int k = 0; k < half; ++k) s[k] += xlevel<4 - LEVELS + lv>(s[k + half]);
    });
    static_for<LEVELS - NRS>([&](auto l) {
      constexpr int lv = NRS + decltype(l)::value;
      s[0] += xlevel<4 - LEVELS + lv>(s[0]);
    });
    if constexpr (KQ) cs *= qfac;
#pragma unroll
    for (int k = 0; k < NF; ++k) s[k] *= cs * kt[k % TPL];

    // 3. mask the tail (and a block id outside the pool)
    TokWords<NWTV> (&vv)[TPL] = vr;
    if (vbits != 0xFFFFu) {
#pragma unroll
      for (int k = 0; k < NF; ++k) {
        const int tok = (((k % TPL) ^ tmask) * R + r);
        if (!((vbits >> tok) & 1u)) s[k] = -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        if (!((vbits >> ((i ^ tmask) * R + r)) & 1u)) {
#pragma unroll
          for (int k = 0; k < NWTV; ++k) vv[i].w[k] = 0u;
        }
      }
    }

    // 4. move the reference maxima if some score passed them by > slack
    bool need = false;
#pragma unroll
    for (int k = 0; k < NF; ++k) need |= s[k] > mref[k / TPL] + kLazyMaxSlack;
    if (__any(need)) {
      float sa[NS];
#pragma unroll
      for (int k = 0; k < NF; ++k) sa[k] = s[k];
      static_for<NRS>([&](auto l) {
        constexpr int lv = NRS - 1 - decltype(l)::value;
        constexpr int half = NS >> (lv + 1);
#pragma unroll
        for (int k = 0; k < half; ++k) sa[k + half] = xlevel<4 - LEVELS + lv>(sa[k]);
      });
#pragma unroll
      for (int hs = 0; hs < G; ++hs) {
        float bm = sa[hs * TPL];
#pragma unroll
        for (int i = 1; i < TPL; ++i) bm = fmaxf(bm, sa[hs * TPL + i]);
        const float mnew = fmaxf(mref[hs], bm);
        const float f = exp2_safe_factor(mref[hs], mnew);
#pragma unroll
        for (int e = 0; e < EL; ++e) acc[hs][e] *= f;
#pragma unroll
        for (int k = 0; k < NF; ++k)
          if (k / TPL == hs) lpart[k] *= f;
        mref[hs] = mnew;
      }
    }

    // 5. probabilities of the row's own scores, then all-gather them
    float pf[NS];
#pragma unroll
    for (int k = 0; k < NF; ++k) {
      const float m = mref[k / TPL];
      const float pk = __builtin_amdgcn_exp2f(s[k] - (m == -INFINITY ? 0.f : m));
      lpart[k] += pk;
      pf[k] = pk * vsc * vt[k % TPL];
    }
    static_for<NRS>([&](auto l) {
      constexpr int lv = NRS - 1 - decltype(l)::value;
      constexpr int half = NS >> (lv + 1);
#pragma unroll
      for (int k = 0; k < half; ++k) pf[k + half] = xlevel<4 - LEVELS + lv>(pf[k]);
    });

    // 6. accumulate p * V
    if constexpr (PV_DOT2) {
#pragma unroll
      for (int m2 = 0; m2 < TPL / 2; ++m2) {
        uint32_t vp[EL];
        v_token_pairs<VT, EL, NWTV>(vv[2 * m2], vv[2 * m2 + 1], vp);
#pragma unroll
        for (int hs = 0; hs < G; ++hs) {
          const half2_t pp = __builtin_bit_cast(
              half2_t, pack_f16x2(pf[hs * TPL + 2 * m2], pf[hs * TPL + 2 * m2 + 1]));
#pragma unroll
          for (int e = 0; e < EL; ++e)
            acc[hs][e] = __builtin_amdgcn_fdot2(pp, __builtin_bit_cast(half2_t, vp[e]), acc[hs][e], false);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        float vf[EL];
        to_f32<VT, EL, NWTV>(vv[i], vf);
#pragma unroll
        for (int hs = 0; hs < G; ++hs) {
          const float pw = pf[hs * TPL + i];
#pragma unroll
          for (int e = 0; e < EL; ++e) acc[hs][e] = __builtin_fmaf(pw, vf[e], acc[hs][e]);
        }
      }
    }
  };

  // Staging.  K tiles go through a two-slot per-wave LDS ring by LDS DMA; V
  // tiles go straight to registers.  Scattered 4 KiB tiles stream at ~6.0
  // TB/s on this chip under the default cache policy whichever path they
  // take (LDS DMA or registers, one to three blocks in flight, two or four
  // waves per SIMD all measured alike); non-temporal K copies lift a launch
  // to ~6.2-6.3 TB/s.  Block t + 1's K copy and V loads are in flight while
  // block t is computed.  The V loads
  // are ordinary loads, so the compiler knows when their registers are
  // valid; the one wait per block is a waitcnt it can see (vmcnt(0), which
  // also covers the K copies it cannot see), so it places no waits of its
  // own on V(t) behind the newer loads.  V's register slot (i, v) is token
  // row ((i ^ tmask) * R + r), the order the reduce-scatter's mirrored masks
  // ask for.
  uint32_t roff[TPL][VPT];
#pragma unroll
  for (int i = 0; i < TPL; ++i)
#pragma unroll
    for (int v = 0; v < VPT; ++v)
      roff[i][v] = (uint32_t)((((i ^ tmask) * R + r) * D + (v * LPT + c) * E) * VEB);
  // Ordinary loads: non-temporal V loads measured no faster on a uniform
  // batch and about 40% slower on a batch of uneven lengths.
  // nv: token rows of the block to fetch (rows_of); lanes of rows past it
  // load nothing.
  auto issue_vregs = [&](int phys_raw, TokWords<NWTV> (&vr)[TPL], int nv) __attribute__((always_inline)) {
    const char* src = vbase + vtile_of(phys_raw);
    auto load = [&](int i, int v) __attribute__((always_inline)) {
      if constexpr (VLW == 16) {
        const uint4 x = *(const uint4*)(src + roff[i][v]);
        vr[i].w[4 * v + 0] = x.x; vr[i].w[4 * v + 1] = x.y; vr[i].w[4 * v + 2] = x.z; vr[i].w[4 * v + 3] = x.w;
      } else {
        const uint2 x = *(const uint2*)(src + roff[i][v]);
        vr[i].w[2 * v + 0] = x.x; vr[i].w[2 * v + 1] = x.y;
      }
    };
    if (nv >= 16) {
#pragma unroll
      for (int i = 0; i < TPL; ++i)
#pragma unroll
        for (int v = 0; v < VPT; ++v) load(i, v);
    } else {
#pragma unroll
      for (int i = 0; i < TPL; ++i)
#pragma unroll
        for (int v = 0; v < VPT; ++v)
          if (((i ^ tmask) * R + r) < nv) load(i, v);
    }
  };
  // K(t) from its ring slot: the 16 bytes each lane's DMA copy wrote, read
  // back with ds_read_b128 (consecutive lanes, consecutive 16-byte columns:
  // no bank conflicts) and waited for in the same statement.
  // a wave's ring: KR slots of BPS tiles; tile sk of the ring at sk * TILE_B
  const uint32_t kread0 = lds_offset(smem) + (uint32_t)(w * KR * BPS * TILE_B + lane * 16);
  const uint32_t kread8 = lds_offset(smem) + (uint32_t)(w * KR * BPS * TILE_B + r * D * C::EB + c * 8);
  auto read_k = [&](int sk, TokWords<NWT> (&kr)[TPL]) __attribute__((always_inline)) {
    if constexpr (LW == 16) {
      uint32_t addr[TPL * VPT];
#pragma unroll
      for (int i = 0; i < TPL; ++i)
#pragma unroll
        for (int v = 0; v < VPT; ++v)
          addr[i * VPT + v] = kread0 + (uint32_t)(sk * TILE_B + ((i ^ tmask) * VPT + v) * 1024);
      u32x4_t got[TPL * VPT];
      lds_read16_wait<TPL * VPT>(got, addr);
#pragma unroll
      for (int i = 0; i < TPL; ++i)
#pragma unroll
        for (int v = 0; v < VPT; ++v)
#pragma unroll
          for (int k = 0; k < 4; ++k) kr[i].w[4 * v + k] = got[i * VPT + v][k];
    } else {
      // token row (i ^ tmask) * R + r, bytes [8c, 8c + 8) of the row-major tile
      uint32_t addr[TPL];
#pragma unroll
      for (int i = 0; i < TPL; ++i)
        addr[i] = kread8 + (uint32_t)(sk * TILE_B + (i ^ tmask) * R * D * C::EB);
      u32x2_t got[TPL];
      lds_read8_wait<TPL>(got, addr);
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        kr[i].w[0] = got[i][0];
        kr[i].w[1] = got[i][1];
      }
    }
  };
  {
    const uint32_t kslot0 = lds_offset(smem) + (uint32_t)(w * KR * BPS * TILE_B);
    // nv as for issue_vregs: a copy's lanes of rows past it copy nothing
    // (the slot keeps older bytes there, which compute_block never uses).
    auto issue_k2 = [&](int phys_raw, int sk, int nv) __attribute__((always_inline)) {
      const char* src = kbase + tile_of(phys_raw);
      const uint32_t dst = kslot0 + (uint32_t)(sk * TILE_B);
      if (nv >= 16) {
#pragma unroll
        for (int n = 0; n < NDMA; ++n) lds_dma16(src, dma_off[n], dst + n * 1024);
      } else {
#pragma unroll
        for (int n = 0; n < NDMA; ++n) {
          // token row of this lane's 16 bytes in copy n
          const int row = LW == 16 ? (n / VPT) * R + r : (n * 1024 + lane * 16) / (D * C::EB);
          if (row < nv) lds_dma16(src, dma_off[n], dst + n * 1024);
        }
      }
    };
    // Step t of wave w covers unit w + t * NW: the BPS attended blocks from
    // j0 + (w + t * NW) * BPS.  A block past j1 (the partition's last unit
    // may be short) has entry -1: its loads read block 0 of the pool and it
    // is masked like a block outside the pool.
    const int nunits = (j1 - j0 + BPS - 1) / BPS;
    const int n_my = w < nunits ? (nunits - w + NW - 1) / NW : 0;
    auto blk = [&](int t, int b2) __attribute__((always_inline)) { return j0 + (w + t * NW) * BPS + b2; };
    auto entry_at = [&](int t, int b2) __attribute__((always_inline)) {
      const int j = blk(t, b2);
      if constexpr (BPS == 1) return entry_of(j);   // every step's block is in range
      else return j < j1 ? entry_of(j) : -1;
    };
    auto rows_at = [&](int t, int b2) __attribute__((always_inline)) {
      const int j = blk(t, b2);
      if constexpr (BPS == 1) return span.rows(span.logical(j));
      else return j < j1 ? span.rows(span.logical(j)) : 0;
    };
    TokWords<NWTV> va[BPS][TPL], vb[BPS][TPL];
    constexpr unsigned kWaitVm0 = 0x0F70;     // vmcnt(0), expcnt(7), lgkmcnt(15)
    static_assert(KR == 2, "one step in flight: K(t+1) and V(t+1) while t is computed");
    // A plain copy of the new rows is loaded here, so that its round trip
    // overlaps the first tiles' instead of delaying them, and stored in step
    // 0 once step 1's loads are issued: step 1's wait completes the store
    // before the wave issues any later block's loads, the new token's block
    // (its last step, n_my - 1 >= 2) among them.  (A later step would keep
    // the rows' registers live through the loop, which costs the head_dim-64
    // instantiations a wave per SIMD.)  With fewer than three steps the rows
    // are written before the first loads.
    const bool defer = !is_quantised<VT>() && appends && w == append_wave && n_my >= 3;
    PendingRow pend;
    pend.dst = nullptr;
    if (appends && w == append_wave) {
      if constexpr (!is_quantised<VT>()) {
        if (defer) pend = append_rows_load<D, kv_bytes<KT>::value>(a, b, h, lane, new_slot);
      }
      if (!defer) {
        append_rows();
        if (n_my == 1) wait_vmcnt<0>();    // the new token's block is in this wave's first step
      }
    }
    // bcur: the blocks being computed; bnext: the next step's, entries read
    BlockRef bcur[BPS], bnext[BPS];
#pragma unroll
    for (int b2 = 0; b2 < BPS; ++b2) {
      bcur[b2] = BlockRef{-1, 1.f, 1.f};
      bnext[b2] = BlockRef{-1, 1.f, 1.f};
    }
    if (n_my > 0) {
#pragma unroll
      for (int b2 = 0; b2 < BPS; ++b2) {
        bcur[b2].phys = entry_at(0, b2);
        issue_vregs(bcur[b2].phys, va[b2], rows_at(0, b2));
        issue_k2(bcur[b2].phys, b2, rows_at(0, b2));
        issue_tok(bcur[b2].phys, b2);
        scales_of(bcur[b2]);
      }
      if (n_my > 1)
#pragma unroll
        for (int b2 = 0; b2 < BPS; ++b2) bnext[b2].phys = entry_at(1, b2);
    }
    load_query();
    // A wait the compiler sees: the query loads are complete, so it places
    // none of its own inside the loop, where they would also wait for the
    // prefetches in flight.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    // Step t: K(t) and V(t) are the newest loads in flight, so wait for all,
    // then issue step t + 1 at once: its K slot and V registers held step
    // t - 1, already consumed, so nothing of step t has to be read first.
    auto step = [&](int t, TokWords<NWTV> (&vcur)[BPS][TPL], TokWords<NWTV> (&vnext)[BPS][TPL])
                    __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      wait_vmcnt<0>();                      // (asm, memory clobber) the LDS reads stay below
      BlockRef b0[BPS];
#pragma unroll
      for (int b2 = 0; b2 < BPS; ++b2) b0[b2] = bcur[b2];
      const bool more = t + 1 < n_my;
      if (more) {
#pragma unroll
        for (int b2 = 0; b2 < BPS; ++b2) {
          issue_vregs(bnext[b2].phys, vnext[b2], rows_at(t + 1, b2));
          issue_k2(bnext[b2].phys, ((t + 1) & 1) * BPS + b2, rows_at(t + 1, b2));
          issue_tok(bnext[b2].phys, ((t + 1) & 1) * BPS + b2);
        }
      }
      if (defer && t == 0) append_rows_store(pend);
      TokWords<NWT> kr[TPL];
      read_k((t & 1) * BPS, kr);            // waits for its reads (lgkmcnt(0))
      // scalar loads after that wait, which would otherwise cover them too
      if (more) {
#pragma unroll
        for (int b2 = 0; b2 < BPS; ++b2) {
          scales_of(bnext[b2]);
          bcur[b2] = bnext[b2];
          if (t + 2 < n_my) bnext[b2].phys = entry_at(t + 2, b2);
        }
      }
      __builtin_amdgcn_sched_barrier(0);    // the loads stay ahead of the compute
      compute_block(blk(t, 0), (t & 1) * BPS, b0[0], kr, vcur[0]);
      // further blocks of the step: K read from the ring just before use,
      // so one block's K is held at a time
#pragma unroll
      for (int b2 = 1; b2 < BPS; ++b2) {
        read_k((t & 1) * BPS + b2, kr);
        compute_block(blk(t, b2), (t & 1) * BPS + b2, b0[b2], kr, vcur[b2]);
      }
    };
    int t = 0;
    for (; t + 1 < n_my; t += 2) {
      step(t, va, vb);
      step(t + 1, vb, va);
    }
    if (t < n_my) step(t, va, vb);
  }
  __syncthreads();  // every wave is done with its ring: the LDS is reused below

  // ---- combine: lanes of a row -> rows of a wave -> waves of the group ----
  // per-head sum of probabilities over the row
  float la[NS];
#pragma unroll
  for (int k = 0; k < NF; ++k) la[k] = lpart[k];
  static_for<NRS>([&](auto l) {
    constexpr int lv = NRS - 1 - decltype(l)::value;
    constexpr int half = NS >> (lv + 1);
#pragma unroll
    for (int k = 0; k < half; ++k) la[k + half] = xlevel<4 - LEVELS + lv>(la[k]);
  });
  float lrow[G];
#pragma unroll
  for (int hs = 0; hs < G; ++hs) {
    lrow[hs] = 0.f;
#pragma unroll
    for (int i = 0; i < TPL; ++i) lrow[hs] += la[hs * TPL + i];
  }
  // Rows of the wave: lanes with equal c hold the same heads and columns.
  // Every row's partial is first moved to the wave's reference maximum.
  constexpr int NA = G * EL;               // accumulators per lane, flat: hs * EL + el
  float fa[NA];
#pragma unroll
  for (int hs = 0; hs < G; ++hs) {
    const float mw = across_rows<LPT, true>(mref[hs]);
    const float f = mref[hs] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref[hs] - mw);
    lrow[hs] = across_rows<LPT, false>(lrow[hs] * f);
#pragma unroll
    for (int e = 0; e < EL; ++e) fa[hs * EL + e] = acc[hs][e] * f;
    mref[hs] = mw;
  }
  // Rows inside a 16-lane DPP row (LPT < 16): summed in place.
#pragma unroll
  for (int k = 0; k < NA; ++k) {
    if constexpr (LPT == 4) fa[k] += dpp<DPP_ROW_ROR4>(fa[k]);
    if constexpr (LPT <= 8) fa[k] += dpp<DPP_ROW_ROR8>(fa[k]);
  }
  // Rows 16 and 32 lanes apart: a reduce-scatter with gfx950's lane swaps.
  // v_permlane16_swap(X, Y) with X, Y the two halves of the accumulators
  // leaves, in X' + Y', the pair's sum of X in even 16-lane rows and the
  // pair's sum of Y in odd ones; v_permlane32_swap splits the result again
  // between the lower and upper 32 lanes.  A lane ends with NA / 4 sums:
  // flat indices base + k, base = (bit 5) * NA/4 + (bit 4) * NA/2.
  constexpr int N2 = NA / 2, N4 = NA / 4;
  float h1[N2], h2[N4];
#pragma unroll
  for (int k = 0; k < N2; ++k) {
    const auto sw = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, fa[k]),
                                                     __builtin_bit_cast(uint32_t, fa[k + N2]), false, false);
    h1[k] = __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
  }
#pragma unroll
  for (int k = 0; k < N4; ++k) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, h1[k]),
                                                     __builtin_bit_cast(uint32_t, h1[k + N4]), false, false);
    h2[k] = __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
  }
  // one lane of each in-row group (the rest hold copies) writes its sums
  if (((lane & 15) / LPT) == 0) {
    const int base = ((lane >> 5) & 1) * N4 + ((lane >> 4) & 1) * N2;
#pragma unroll
    for (int k = 0; k < N4; ++k) {
      const int fi = base + k, hs = fi / EL, el = fi % EL;
      red_acc[w][hs ^ hmask][((el / E) * LPT + c) * E + el % E] = h2[k];
    }
  }
  if (r == 0 && c == 0) {
#pragma unroll
    for (int hs = 0; hs < G; ++hs) {
      red_m[w][hs ^ hmask] = mref[hs];
      red_l[w][hs ^ hmask] = lrow[hs];
    }
  }
  __syncthreads();
  combine_waves<OT, D, G, NW>(a, b, h, p, tid, red_acc, red_m, red_l);
}

}  // namespace pkv

#include "decode_mfma.h"

namespace pkv {

// The per-sequence pass an instantiation runs, and its LDS.
template <KV KT, KV VT, KV QT, KV OT, int D, int G>
__device__ __forceinline__ void cache_pass(const DecodeArgs& a, int p, int h, int b, char* smem) {
  if constexpr (UseMfma<KT, VT, D, G>::value) decode_body_mfma<KT, VT, QT, OT, G>(a, p, h, b, smem);
  else decode_body<KT, VT, QT, OT, D, G>(a, p, h, b, smem);
}
template <KV KT, KV VT, int D, int G>
struct PassLds {
  static constexpr int bytes() {
    if constexpr (UseMfma<KT, VT, D, G>::value) return MCfg<KT>::template smem_bytes<G>();
    else return Cfg<KT, D, G>::SMEM_B;
  }
  static constexpr int value = bytes();
};

// Waves per SIMD the register allocation must allow.  The matrix-core
// instantiations are held to three: the compiler then keeps their
// accumulators in ordinary VGPRs (138 registers with 16-bit caches, 123
// with 8-bit ones) instead of accumulator registers that the
// per-tile rescale would copy out and back, 68 moves per tile.  Vector
// instantiations for 8-bit caches with 8 query heads (two blocks per step)
// are held to two.  The fp8 vector instantiations with one query head per
// KV head are held to five (96 registers, no spills, against a natural
// 100 and four): their workgroups are short chains of dependent round
// trips, which more resident waves overlap (13B-shaped fp8 layer without
// groups: 92.4 -> 87.6 us per layer, balanced A/B).  Those with two are
// held to four, which they fit without spills (a natural 129 registers
// would allow three).  The others keep their natural allocation.
template <KV KT, KV VT, int D, int G>
struct MinWaves {
  static constexpr bool eight_bit = kv_bytes<KT>::value == 1;
  static constexpr bool fp8 = KT == KV::FP8 && VT == KV::FP8;
  static constexpr int value =
      UseMfma<KT, VT, D, G>::value ? 3
                                   : ((G == 8 && eight_bit) ? 2 : ((G == 1 && fp8) ? 5 : ((G == 2 && fp8) ? 4 : 1)));
};

template <KV KT, KV VT, KV QT, KV OT, int D, int G>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MinWaves<KT, VT, D, G>::value)))
decode_partition_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[PassLds<KT, VT, D, G>::value];
  const Unit u = unit_of(a, blockIdx.x);
  cache_pass<KT, VT, QT, OT, D, G>(a, u.p, u.h, u.b, smem);
}

// Cache pass and shared-prefix group pass in one launch: the first
// group_wgs workgroups run the group pass (matrix cores, latency-bound at
// this size) while the rest stream the sequences' own blocks, so neither
// waits for the other.  Both parts use the same LDS buffer.  T: the caches'
// element type (K and V alike); QT: the query's and the output's.
template <KV T, KV QT, int D, int G>
struct GroupKernelLds {
  static constexpr int value =
      PassLds<T, T, D, G>::value > GroupLds<D>::BYTES ? PassLds<T, T, D, G>::value : GroupLds<D>::BYTES;
};
// Waves per SIMD the group launch's registers must allow.  With 8-bit
// caches its per-sequence workgroups are short chains of dependent round
// trips moving half the bytes of 16-bit ones, so more of them resident pay:
// held to four waves per SIMD (no spills; 13B MHA layer with an fp8 cache
// 58.7 -> 53.2 us per layer cold, balanced A/B), and with fp8 and one query
// head per KV head to five (96 registers, no spills; 48.3 -> 46.3 us).
// With 16-bit caches four waves measured slower (63.0 -> 64.0 us), so they
// keep their natural allocation (three).
template <KV T, int G>
struct GroupMinWaves {
  static constexpr int value = is_quantised<T>() ? ((T == KV::FP8 && G == 1) ? 5 : 4) : 1;
};
template <KV T, KV QT, int D, int G>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(GroupMinWaves<T, G>::value)))
decode_group_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[GroupKernelLds<T, QT, D, G>::value];
  const int id = blockIdx.x;
  if (id < a.group_wgs) {
    const int pp = id % a.group_num_parts, rest = id / a.group_num_parts;
    group_body<T, QT, D>(a, pp, rest % a.num_kv_heads, rest / a.num_kv_heads, smem);
  } else {
    const Unit u = unit_of(a, id - a.group_wgs);
    cache_pass<T, T, QT, QT, D, G>(a, u.p, u.h, u.b, smem);
  }
}

// Log-sum-exp merge of the partitions of one (sequence, query head) row.
// Partition p carries o_p (its normalised output), m_p (log2 reference) and
// l_p (sum of exp2(s - m_p)); out = sum_p l_p 2^(m_p - M) o_p / sum_p l_p 2^(m_p - M).
// Only the slots written for this row are read: the sequence's own
// partitions, then the pieces of the shared-prefix group pass, if any.
//
// Full-precision sink tokens ("The KV Cache memory ledger" 7: attention-sink
// tokens keep their original precision when the rest is quantised) join
// here as one more term: the first min(S, L) positions of the sequence,
// read as stored (q's dtype) from its side tile, attended with an online
// softmax over at most 16 tokens (lane l holds elements l + 64k).
template <KV QT, KV OT, int D>
__global__ void __launch_bounds__(64) lse_merge_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;
  const int row = blockIdx.x;
  const int b = row / a.num_q_heads;
  const int lane = threadIdx.x;
  const float* ml = a.ml_part + (int64_t)row * a.part_stride * 2;
  const float* op = a.o_part + (int64_t)row * a.part_stride * D;
  // The row's first U workspace slots are loaded before its length is known
  // (which of them were written depends on it), so their round trip
  // overlaps the lookups below; slots past the row's stride re-read the
  // last one and are ignored.
  constexpr int U = 4;
  float mi0[U], li0[U], oi0[U][PER];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int sl = min(u, a.part_stride - 1);
    mi0[u] = ml[2 * sl];
    li0[u] = ml[2 * sl + 1];
#pragma unroll
    for (int k = 0; k < PER; ++k) oi0[u][k] = op[(int64_t)sl * D + k * 64 + lane];
  }
  const int pre = a.sink_tiles ? 0 : prefix_blocks_of_seq(a, b);
  const SeqSpan span(a.context_lens[b], a.max_blocks, a.window, a.sinks,
                     a.sink_tiles ? a.sinks : 16 * pre);
  // slots [0, np) hold the per-sequence pieces, [num_parts, num_parts + ng)
  // those of the shared-prefix pass
  const int np = SeqParts(span.natt, a.part_blocks, a.num_parts, 0).n;
  const int ng = pre > 0 ? SeqParts(pre, a.group_part_blocks, a.group_num_parts, 0).n : 0;
  auto written = [&](int sl) __attribute__((always_inline)) {
    return sl < np || (sl >= a.num_parts && sl < a.num_parts + ng);
  };

  float ms = -INFINITY, ls = 0.f, os[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) os[k] = 0.f;
  if (a.sink_tiles) {
    const int tile = a.sink_of_seq[b];
    const int n = ((unsigned)tile < (unsigned)a.num_sink_tiles) ? min(a.sinks, span.L) : 0;
    const int h = (row % a.num_q_heads) / (a.num_q_heads / a.num_kv_heads);
    const int64_t tbase = ((int64_t)(n > 0 ? tile : 0) * a.num_kv_heads + h) * 16 * D;
    float qv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) qv[k] = load_elem_f32<QT>(a.q, (int64_t)row * D + k * 64 + lane);
    for (int t = 0; t < n; ++t) {
      float part = 0.f;
#pragma unroll
      for (int k = 0; k < PER; ++k)
        part = __builtin_fmaf(qv[k], load_elem_f32<QT>(a.sink_k, tbase + t * D + k * 64 + lane), part);
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) part += __shfl_xor(part, d);
      const float s = part * a.scale;                   // log2 units, same on every lane
      const float mnew = fmaxf(ms, s);
      const float f = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - mnew);
      const float w = __builtin_amdgcn_exp2f(s - mnew);
      ls = __builtin_fmaf(ls, f, w);
#pragma unroll
      for (int k = 0; k < PER; ++k)
        os[k] = __builtin_fmaf(os[k], f, w * load_elem_f32<QT>(a.sink_v, tbase + t * D + k * 64 + lane));
      ms = mnew;
    }
  }

  // One pass with a running reference (the sink term first): every
  // partition joins as l_p 2^(m_p - M) o_p, the sum rescaled when M moves.
  float m = ls > 0.f ? ms : -INFINITY;
  float wsum = ls > 0.f ? ls : 0.f;
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = ls > 0.f ? os[k] : 0.f;
  auto join = [&](float mp, float lp, const float (&opp)[PER]) __attribute__((always_inline)) {
    if (!(lp > 0.f)) return;
    const float mn = fmaxf(m, mp);
    const float f = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    const float g = lp * __builtin_amdgcn_exp2f(mp - mn);
    wsum = __builtin_fmaf(wsum, f, g);
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] = __builtin_fmaf(o[k], f, g * opp[k]);
    m = mn;
  };
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (u < a.part_stride && written(u)) join(mi0[u], li0[u], oi0[u]);
  // The written slots from U on: the rest of the per-sequence pieces, then
  // the group pieces, read U at a time with unconditional loads (an index
  // past the end re-reads the last slot and is then ignored), so their
  // latencies overlap.
  const int n = np + ng;
  int i0 = 0;
  while (i0 < n && (i0 < np ? i0 : a.num_parts + (i0 - np)) < U) ++i0;
  for (; i0 < n; i0 += U) {
    float mi[U], li[U], oi[U][PER];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(i0 + u, n - 1);
      const int p = i < np ? i : a.num_parts + (i - np);
      mi[u] = ml[2 * p];
      li[u] = ml[2 * p + 1];
#pragma unroll
      for (int k = 0; k < PER; ++k) oi[u][k] = op[(int64_t)p * D + k * 64 + lane];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u;
      if (i >= n || (i < np ? i : a.num_parts + (i - np)) < U) continue;
      join(mi[u], li[u], oi[u]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) store_out<OT>(a.out, (int64_t)row * D + k * 64 + lane, o[k] * inv);
}

// ---------------------------------------------------------------------------
void plan_partitions(const pkv_decode_dims& d, int* part_blocks, int* num_parts) {
  // longest attended-block list any sequence can have
  int maxb = d.max_blocks_per_seq;
  if (d.window > 0) {
    const int64_t att = (int64_t)(d.window + 15) / 16 + 1 + (d.sinks + 15) / 16;
    if (att < maxb) maxb = (int)att;
  }
  int pb;
  if (d.partition_blocks > 0) {
    pb = d.partition_blocks;
  } else {
    // Aim for about 512 workgroups: two per CU on 256 CUs, which is what the
    // LDS ring allows resident at once.  Each extra split costs a workspace
    // round trip and shortens the streaming loop, so split no further than
    // that, and never below 16 blocks (256 tokens) per partition.
    const int64_t units = (int64_t)d.num_seqs * d.num_kv_heads;
    int64_t want = (512 + units - 1) / units;
    if (want < 1) want = 1;
    pb = (int)((maxb + want - 1) / want);
    if (pb < 16) pb = 16;
    // The table width only bounds the lengths.  When the batch's real size
    // is known and the plan above would keep fewer than 256 workgroups busy
    // (one per CU), size the pieces from the real size instead (sequences
    // are cut evenly into ceil(len / pb) pieces).  Finer splits of a batch
    // that already fills the chip measured slower, so they are not made.
    if (d.total_blocks > 0) {
      const int64_t total = d.total_blocks < units / d.num_kv_heads * (int64_t)maxb
                                ? d.total_blocks
                                : units / d.num_kv_heads * (int64_t)maxb;
      if (total * d.num_kv_heads < 256 * (int64_t)pb) {
        const int64_t t = (total * d.num_kv_heads + 511) / 512;
        pb = (int)(t < 16 ? 16 : (t > maxb ? maxb : t));
      }
    }
  }
  if (pb > maxb) pb = maxb;
  if (pb < 1) pb = 1;
  *part_blocks = pb;
  *num_parts = (maxb + pb - 1) / pb;
}

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
  // About PKV_GROUP_WGS workgroups for the whole pass, never fewer than
  // PKV_GROUP_MIN_PB blocks per piece: each piece adds a partial result per
  // query row.
  const int64_t units = (int64_t)d.prefix_groups * d.num_kv_heads * *qchunks;
  const int64_t want = units >= PKV_GROUP_WGS ? 1 : (PKV_GROUP_WGS + units - 1) / units;
  int pb = (int)((maxb + want - 1) / want);
  if (pb < PKV_GROUP_MIN_PB) pb = PKV_GROUP_MIN_PB;
  if (pb > maxb) pb = maxb;
  *part_blocks = pb;
  *num_parts = (maxb + pb - 1) / pb;
}

size_t workspace_bytes_for(const pkv_decode_dims& d) {
  int pb, np, gpb, gnp = 0, qc;
  plan_partitions(d, &pb, &np);
  if (d.prefix_groups > 0) plan_groups(d, &gpb, &gnp, &qc);
  // sink tiles and shared-prefix groups are merged in: always split
  if (np <= 1 && !d.sink_tiles && d.prefix_groups <= 0) return 0;
  return (size_t)d.num_seqs * d.num_q_heads * (np + gnp) * (d.head_dim + 2) * sizeof(float);
}

template <KV KT, KV VT, KV QT, KV OT, int D, int G>
static int launch_typed(const DecodeArgs& a, hipStream_t stream) {
  constexpr bool plain16 = (KT == KV::F16 || KT == KV::BF16) && VT == KT && QT == KT && OT == KT;
  // 8-bit caches with groups: K and V of one format, a 16-bit query and
  // output of one type, head_dim 128
  constexpr bool q8group = is_quantised<KT>() && VT == KT && QT == OT && (QT == KV::F16 || QT == KV::BF16) &&
                           D == 128;
  if constexpr (plain16 || q8group) {
    if (a.group_wgs > 0) {
      const int64_t n = (int64_t)a.group_wgs + (int64_t)a.num_parts * a.num_kv_heads * a.num_seqs;
      hipLaunchKernelGGL((decode_group_kernel<KT, QT, D, G>), dim3((unsigned)n), dim3(256), 0, stream, a);
      if (hipGetLastError() != hipSuccess) return PKV_ERR_LAUNCH;
      hipLaunchKernelGGL((lse_merge_kernel<QT, OT, D>), dim3(a.num_seqs * a.num_q_heads), dim3(64), 0,
                         stream, a);
      return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
    }
  }
  if (a.group_wgs > 0) return PKV_ERR_DTYPE;   // no group pass for this type combination
  const int64_t n = (int64_t)a.num_parts * a.num_kv_heads * a.num_seqs;
  if (n > 0x7FFFFFFF) return PKV_ERR_SHAPE;
  hipLaunchKernelGGL((decode_partition_kernel<KT, VT, QT, OT, D, G>), dim3((unsigned)n), dim3(256), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return PKV_ERR_LAUNCH;
  if (a.split) {
    hipLaunchKernelGGL((lse_merge_kernel<QT, OT, D>), dim3(a.num_seqs * a.num_q_heads), dim3(64), 0,
                       stream, a);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_LAUNCH;
  }
  return PKV_OK;
}

template <KV KT, KV VT, KV QT, KV OT, int D>
static int dispatch_g(const DecodeArgs& a, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_typed<KT, VT, QT, OT, D, 1>(a, s);
    case 2: return launch_typed<KT, VT, QT, OT, D, 2>(a, s);
    case 4: return launch_typed<KT, VT, QT, OT, D, 4>(a, s);
    case 8: return launch_typed<KT, VT, QT, OT, D, 8>(a, s);
    default: return PKV_ERR_SHAPE;
  }
}

template <KV KT, KV VT, KV QT, KV OT>
static int dispatch_d(const DecodeArgs& a, hipStream_t s) {
  switch (a.head_dim) {
    case 64: return dispatch_g<KT, VT, QT, OT, 64>(a, s);
    case 128: return dispatch_g<KT, VT, QT, OT, 128>(a, s);
    default: return PKV_ERR_SHAPE;
  }
}

int launch_decode(const DecodeArgs& a, hipStream_t s) {
  const KV kt = (KV)a.kv_dtype, vt = (KV)a.v_dtype, qt = (KV)a.q_dtype, ot = (KV)a.out_dtype;
  if ((kt == KV::F16 || kt == KV::BF16) && (vt == KV::FP8 || vt == KV::INT8)) {
    // 16-bit K with an 8-bit V: q and out of K's type
    if (qt != kt || ot != kt) return PKV_ERR_DTYPE;
    if (kt == KV::F16)
      return vt == KV::FP8 ? dispatch_d<KV::F16, KV::FP8, KV::F16, KV::F16>(a, s)
                           : dispatch_d<KV::F16, KV::INT8, KV::F16, KV::F16>(a, s);
    return vt == KV::FP8 ? dispatch_d<KV::BF16, KV::FP8, KV::BF16, KV::BF16>(a, s)
                         : dispatch_d<KV::BF16, KV::INT8, KV::BF16, KV::BF16>(a, s);
  }
  if (kt == KV::F32 || kt == KV::F16 || kt == KV::BF16) {
    if (vt != kt || qt != kt || ot != kt) return PKV_ERR_DTYPE;
    switch (kt) {
      case KV::F32: return dispatch_d<KV::F32, KV::F32, KV::F32, KV::F32>(a, s);
      case KV::F16: return dispatch_d<KV::F16, KV::F16, KV::F16, KV::F16>(a, s);
      default: return dispatch_d<KV::BF16, KV::BF16, KV::BF16, KV::BF16>(a, s);
    }
  }
#define PKV_Q8_CASE(K, V, Q, O)                                                  \
  if (kt == KV::K && vt == KV::V && qt == KV::Q && ot == KV::O)                  \
    return dispatch_d<KV::K, KV::V, KV::Q, KV::O>(a, s);
  // fp8 K and V: every query / output pairing
  PKV_Q8_CASE(FP8, FP8, BF16, BF16)
  PKV_Q8_CASE(FP8, FP8, F16, F16)
  PKV_Q8_CASE(FP8, FP8, F32, F32)
  PKV_Q8_CASE(FP8, FP8, BF16, F32)
  PKV_Q8_CASE(FP8, FP8, F16, F32)
  // mixed and int8 caches: 16-bit query and output of one type
  PKV_Q8_CASE(FP8, INT8, BF16, BF16)
  PKV_Q8_CASE(FP8, INT8, F16, F16)
  PKV_Q8_CASE(INT8, INT8, BF16, BF16)
  PKV_Q8_CASE(INT8, INT8, F16, F16)
#undef PKV_Q8_CASE
  return PKV_ERR_DTYPE;
}

}  // namespace pkv
