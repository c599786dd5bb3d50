// Per-sequence pass of paged decode attention on the matrix cores, for
// head_dim 128 and 4 or 8 query heads per KV head (gfx950).
//
// Same result as the vector pass in decode_attn.hip ("KV Cache from first
// principles" 2.1-2.2 and 4.3): for sequence b, KV head h and its g query
// heads, softmax(scale * q K^T) V over the attended positions, K and V
// gathered through the block table.  One (block, KV head) tile is still read
// once from HBM for all g heads; what changes is where the arithmetic runs.
// With 8 heads, and 8-bit tiles that must be widened first, the vector pass
// spends as many VALU cycles per tile as the tile takes to stream, so here
// the two products of a tile are matrix-core operations:
//
//   S^T (16 tokens x 16 columns) = K (16 x 128) . Q^T (128 x 16)
//       four v_mfma_f32_16x16x32 over the head dimension; columns >= g are
//       padding (a zero query), so a column is a query head;
//   O^T (128 x 16) += V^T (128 x 16 tokens) . P^T (16 tokens x 16)
//       eight v_mfma_f32_16x16x32, one per 16-channel slice of V.
//
// The matrix cores idle most of the time (12 operations per 4 KiB tile); the
// point is that the VALU work per tile drops to the softmax of four scores
// per lane, the widening of 8-bit codes and a byte shuffle of V.
//
// Lane layout (l = lane, lq = l % 16, lg = l / 16):
//   * S^T leaves lane l with head lq and tokens 4 lg + i (i < 4) of the tile;
//   * the K operand of lane l is token lq, channels 32 lg .. 32 lg + 31 (one
//     8-channel slice per product), staged through LDS;
//   * the P^T operand of lane l is exactly its four probabilities, twice:
//     contraction slots 8 lg + j hold token 4 lg + (j % 4), rounded to the
//     operand type for j < 4 (hi) and the rounding remainder for j >= 4 (lo),
//     so each weight enters the sum to about 22 bits (f16) / 16 bits (bf16);
//   * the V^T operand of lane l is channel 8 lq + c (slice c) of the same
//     four tokens, twice: the lane loads 16 (8) bytes of each of its token
//     rows straight into registers and pairs tokens with one byte permute;
//   * O^T leaves lane l with head lq and channels 32 lg .. 32 lg + 31.
// So the softmax state of a head lives in the four lanes lq + 16 k, which
// keep identical reference maxima; a rescale stays in-lane.
//
// K staging.  Each K tile is copied into a per-wave two-slot LDS ring by
// non-temporal LDS DMA, every copy reading 1 KiB of HBM contiguously.  The
// copy places the 16-byte column x of token row r at column x ^ f(r) of the
// LDS row (f(r) = r for 256-byte rows, r / 2 for 128-byte rows), so that
// the 16 lanes of a lane group, which read the same column of 16 different
// rows, hit 16 different bank groups.
//
// Masking, append, partitions and the end-of-partition combine behave as in
// the vector pass: positions outside the sequence or window get score -inf
// and a zeroed V operand; the step's append is written by the wave that
// reads the new token's block; partial results go to the workspace when
// the call is split.
//
// This file is part of decode_attn.hip's translation unit: it is included
// there after the per-dtype helpers, SeqSpan and the vector pass, whose
// pieces it uses.
#pragma once

namespace pkv {

// Instantiations that run this pass (the others keep the vector pass).
template <KV KT, KV VT, int D, int G>
struct UseMfma {
  static constexpr bool value = D == 128 && (G == 4 || G == 8) && KT != KV::F32;
};

// Tile geometry of one cache (K's or V's: a 16-bit K may go with an 8-bit V).
template <KV T>
struct MCfg {
  static constexpr int D = 128;
  static constexpr int EB = kv_bytes<T>::value;
  static constexpr int ROW_B = D * EB;            // one token row of a tile
  static constexpr int TILE_B = 16 * ROW_B;       // one (block, KV head) tile
  static constexpr int NDMA = TILE_B / 1024;      // 1 KiB LDS DMA copies per tile
  static constexpr int KREADS = 32 * EB / 16;     // 16-byte LDS reads: a lane's 32 channels
  static constexpr int VW = 2 * EB;               // V dwords per token per lane (8 channels)
  static constexpr int NW = 4;                    // waves per workgroup
  static constexpr int KR = 2;                    // K ring slots per wave
  static constexpr int KRING_B = NW * KR * TILE_B;
  // per-token scales of a ring slot's block: 16 K scales, then 16 V scales
  static constexpr int TOKS_B = 128;
  static constexpr int TOKRING_B = NW * KR * TOKS_B;
  // the per-wave partial results of the end-of-partition combine, after
  // the rings: a wave that is done writes its partial while the others
  // still stream (over the rings, every wave would first wait for all;
  // 0.4-0.6 us longer per 70B-shaped launch)
  static constexpr int RED_OFF = KRING_B + TOKRING_B;
  template <int G>
  static constexpr int smem_bytes() {
    constexpr int red = NW * G * (D + 2) * 4;
    return RED_OFF + red > KRING_B + TOKRING_B ? RED_OFF + red : KRING_B + TOKRING_B;
  }
};

// V rows of one tile held by a lane: token 4 lg + i, channels 8 lq .. + 7.
template <int VW> struct VRows { uint32_t w[4][VW]; };

// Probabilities of four tokens -> P^T operand: hi parts of tokens 0..3, then
// the remainders p - hi, each rounded to the operand type (RNE).
template <KV MV>
__device__ __forceinline__ u32x4_t p_operand(const float (&pv)[4]) {
  uint32_t hi[2], lo[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float p0 = pv[2 * k], p1 = pv[2 * k + 1];
    if constexpr (MV == KV::F16) {
      hi[k] = pack_f16x2(p0, p1);
      lo[k] = pack_f16x2(p0 - f16lo(hi[k]), p1 - f16hi(hi[k]));
    } else {
      // one v_cvt_pk_bf16_f32 (round to nearest even) per pair
      hi[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{p0, p1}, bf162_t));
      lo[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                               float2_t{p0 - bf16lo(hi[k]), p1 - bf16hi(hi[k])}, bf162_t));
    }
  }
  return u32x4_t{hi[0], hi[1], lo[0], lo[1]};
}

// V^T operand of slice c (channel 8 lq + c of the lane's four tokens, as
// f16/bf16 pairs (token 0, token 1), (token 2, token 3), then again).
template <KV VT, int VW>
__device__ __forceinline__ void v_operands(const VRows<VW>& v, u32x4_t (&op)[8]) {
  static_for<8>([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    uint32_t p01, p23;
    if constexpr (VT == KV::F16 || VT == KV::BF16) {
      // dword c / 2 holds channels c & ~1 (low half) and c | 1 (high half)
      constexpr uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      p01 = __builtin_amdgcn_perm(v.w[1][c / 2], v.w[0][c / 2], sel);
      p23 = __builtin_amdgcn_perm(v.w[3][c / 2], v.w[2][c / 2], sel);
    } else if constexpr (VT == KV::INT8) {
      // dword c / 4 holds int8 channels 4 (c / 4) .. + 3
      p01 = i8_pair_to_f16<c % 4, c % 4>(v.w[0][c / 4], v.w[1][c / 4]);
      p23 = i8_pair_to_f16<c % 4, c % 4>(v.w[2][c / 4], v.w[3][c / 4]);
    } else {
      // fp8: interleave the bytes of channels (c, c + 1) of two tokens, widen
      // each half; odd c takes the high half of its even neighbour's word
      constexpr uint32_t sel = ((c & 2) ? 0x07030602u : 0x05010400u);
      const uint32_t x01 = __builtin_amdgcn_perm(v.w[1][c / 4], v.w[0][c / 4], sel);
      const uint32_t x23 = __builtin_amdgcn_perm(v.w[3][c / 4], v.w[2][c / 4], sel);
      p01 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x01, 1.0f, (c & 1) != 0));
      p23 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x23, 1.0f, (c & 1) != 0));
    }
    op[c] = u32x4_t{p01, p23, p01, p23};
  });
}

// K operand of slice c from the lane's 32 staged channels (kr: 16-byte LDS
// reads in channel order).  16-bit K is used as stored; 8-bit K is widened
// to f16 exactly.
template <KV KT, int KREADS>
__device__ __forceinline__ void k_operands(const u32x4_t (&kr)[KREADS], u32x4_t (&op)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if constexpr (KT == KV::F16 || KT == KV::BF16) {
      op[c] = kr[c];
    } else {
      // channels 8c .. 8c + 7: dwords 2c, 2c + 1 of the 32 bytes
      const uint32_t d0 = kr[c / 2][(c % 2) * 2], d1 = kr[c / 2][(c % 2) * 2 + 1];
      if constexpr (KT == KV::FP8) {
        op[c] = u32x4_t{
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true))};
      } else {
        op[c] = u32x4_t{i8_pair_to_f16<0, 1>(d0, d0), i8_pair_to_f16<2, 3>(d0, d0),
                        i8_pair_to_f16<0, 1>(d1, d1), i8_pair_to_f16<2, 3>(d1, d1)};
      }
    }
  }
}

// One workgroup: partition p of (sequence b, KV head h).  smem holds
// MCfg<KT>::smem_bytes<G>() bytes.
template <KV KT, KV VT, KV QT, KV OT, int G>
__device__ __forceinline__ void decode_body_mfma(const DecodeArgs& a, int p, int h, int b, char* smem) {
  static_assert(kv_bytes<VT>::value <= kv_bytes<KT>::value, "V is no wider than K");
  static_assert(is_quantised<VT>() || !is_quantised<KT>(), "an 8-bit K goes with an 8-bit V");
  static_assert(G == 4 || G == 8, "4 or 8 query heads per KV head");
  constexpr int D = 128;
  using C = MCfg<KT>;     // K tiles
  using CV = MCfg<VT>;    // V tiles
  constexpr bool KQ = is_quantised<KT>(), VQ = is_quantised<VT>();
  constexpr int EB = C::EB, TILE_B = C::TILE_B, NDMA = C::NDMA, KREADS = C::KREADS, VW = CV::VW;
  constexpr int NW = C::NW, KR = C::KR;
  constexpr KV MK = KQ ? KV::F16 : KT;                    // S^T operands
  constexpr KV MV = VT == KV::BF16 ? KV::BF16 : KV::F16;  // O^T operands

  float (*red_acc)[G][D] = reinterpret_cast<float (*)[G][D]>(smem + C::RED_OFF);
  float (*red_m)[G] = reinterpret_cast<float (*)[G]>(smem + C::RED_OFF + NW * G * D * 4);
  float (*red_l)[G] = reinterpret_cast<float (*)[G]>(smem + C::RED_OFF + NW * G * D * 4 + NW * G * 4);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 15, lg = lane >> 4;
  const bool hv = lq < G;                                 // the lane's column is a query head
  const int Hq = a.num_kv_heads * G;

  const int64_t new_slot = a.new_slots ? a.new_slots[b] : -1;   // read next to the length
  const int pre = a.sink_tiles ? 0 : prefix_blocks_of_seq(a, b);
  const SeqSpan span(a.context_lens[b], a.max_blocks, a.window, a.sinks,
                     a.sink_tiles ? a.sinks : 16 * pre);
  const SeqParts parts(span.natt, a.part_blocks, a.num_parts, p);
  const int j0 = parts.j0, j1 = parts.j1;

  // the step's append (append_new_rows): by the partition holding the new
  // token's block, and in it by the wave that reads that block
  const bool appends = a.new_slots != nullptr && p == (parts.n > 0 ? parts.n - 1 : 0);
  const int append_wave = j1 > j0 ? (j1 - 1 - j0) % NW : 0;
  auto append_rows = [&]() __attribute__((always_inline)) {
    append_step_rows<KT, VT, QT, D>(a, b, h, lane, new_slot);
  };
  if (j0 >= j1) {
    finish_empty<KT, VT, QT, OT, D, G>(a, b, h, p, tid, appends && w == 0, new_slot);
    return;
  }

  // Q^T operand: lane holds q[head lq][32 lg + 8c .. + 7] for slice c (zero
  // for padding columns).  8-bit K: the query times K's channel factors,
  // scaled by a power of two per head (from the head's largest |q c|, over
  // its four lane groups) into f16; the scores undo it.
  u32x4_t qop[4];
  float qfac = 1.f;
  const int64_t qoff = ((int64_t)b * Hq + h * G + (hv ? lq : 0)) * D + lg * 32;
  auto load_query = [&]() __attribute__((always_inline)) {
    if constexpr (!KQ) {
      static_assert(QT == KT, "16-bit caches take a query of the same type");
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>((const uint16_t*)a.q + qoff);
#pragma unroll
      for (int c = 0; c < 4; ++c) qop[c] = hv ? src[c] : u32x4_t{0u, 0u, 0u, 0u};
    } else {
      float f[32], cf[32];
      const void* qrow = (QT == KV::F32) ? (const void*)((const float*)a.q + qoff)
                                         : (const void*)((const uint16_t*)a.q + qoff);
      q_slice_f32<QT, 32, 1, 32, 1>(qrow, 0, f);
      if (a.k_chan) {
        q_slice_f32<KV::F32, 32, 1, 32, 1>(a.k_chan + (int64_t)h * D + lg * 32, 0, cf);
      } else {
#pragma unroll
        for (int e = 0; e < 32; ++e) cf[e] = 1.0f;
      }
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        f[e] = hv ? f[e] * cf[e] : 0.f;
        m = fmaxf(m, fabsf(f[e]));
      }
      m = across_rows<16, true>(m);
      int ex;
      (void)__builtin_frexpf(m, &ex);
      int qexp = m > 0.f ? 15 - ex : 0;              // largest element in [2^14, 2^15)
      qexp = qexp > 100 ? 100 : (qexp < -100 ? -100 : qexp);
      qfac = __builtin_ldexpf(1.0f, -qexp);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          qop[c][k] = pack_f16x2(__builtin_ldexpf(f[8 * c + 2 * k], qexp),
                                 __builtin_ldexpf(f[8 * c + 2 * k + 1], qexp));
    }
  };

  f32x4_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mref = -INFINITY, lsum = 0.f;

  const char* kbase = (const char*)a.k_cache;
  const char* vbase = (const char*)a.v_cache;
  // The block table is read-only for the whole kernel: reading it through
  // the constant address space makes every entry a scalar load, which never
  // waits behind the tile copies in flight.
  const __attribute__((address_space(4))) int32_t* table =
      (const __attribute__((address_space(4))) int32_t*)(a.block_tables + (int64_t)b * a.max_blocks);

  // LDS DMA: copy n, lane l brings 16 bytes of token row r into LDS row r,
  // column (l % per-row) -- i.e. HBM column (l % per-row) ^ f(r).
  uint32_t dma_off[NDMA];
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
  // LDS reads: token row lq, HBM columns holding channels 32 lg .. + 31
  const uint32_t ring0 = lds_offset(smem) + (uint32_t)(w * KR * TILE_B);
  uint32_t kaddr[KREADS];
#pragma unroll
  for (int k = 0; k < KREADS; ++k) {
    if constexpr (EB == 2) kaddr[k] = ring0 + (uint32_t)(lq * 256 + (((lg * 4 + k) ^ lq) & 15) * 16);
    else kaddr[k] = ring0 + (uint32_t)(lq * 128 + (((lg * 2 + k) ^ (lq >> 1)) & 7) * 16);
  }
  // V loads: token rows 4 lg + i, bytes [8 lq EB, + 8 EB); non-temporal,
  // like the K copies (streamed data, read once per step).  A wave
  // instruction reads four whole rows 1 KiB apart.
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = (uint32_t)((lg * 4 + i) * CV::ROW_B + lq * 8 * CV::EB);

  auto entry_of = [&](int j) __attribute__((always_inline)) { return table[span.logical(j)]; };
  auto tile_of = [&](int phys_raw) __attribute__((always_inline)) { return tile_offset(a, h, phys_raw, TILE_B); };
  auto vtile_of = [&](int phys_raw) __attribute__((always_inline)) {
    return tile_offset(a, h, phys_raw, CV::TILE_B);
  };
  auto scales_of = [&](BlockRef& br) __attribute__((always_inline)) { block_scales<KQ, VQ>(a, h, br); };
  // Per-token scales ("KV Cache from first principles" 5.2): the 16 K and
  // 16 V scales of a block's slots are copied by LDS DMA (four lanes of 16
  // bytes each) into the ring slot's scale area next to its K tile, and
  // waited for with it; a lane then reads the four of its tokens.
  const uint32_t toks0 = lds_offset(smem) + (uint32_t)(C::KRING_B + w * KR * C::TOKS_B);
  auto issue_tok = [&](int phys_raw, int sk) __attribute__((always_inline)) {
    if constexpr (KQ || VQ) {
      const int64_t si = tile_offset(a, h, phys_raw, 16);   // (block, head) * 16 scales
      const uint32_t dst = toks0 + (uint32_t)(sk * C::TOKS_B);
      if (KQ && a.k_tok && lane < 4) lds_dma16(a.k_scales + si, (uint32_t)(lane * 16), dst);
      if (VQ && a.v_tok && lane < 4) lds_dma16(a.v_scales + si, (uint32_t)(lane * 16), dst + 64);
    }
  };
  // nv: token rows of the block to fetch (SeqSpan::rows); lanes of rows
  // past it load nothing.
  auto issue_v = [&](int phys_raw, VRows<VW>& vr, int nv) __attribute__((always_inline)) {
    const char* src = vbase + vtile_of(phys_raw);
    auto load = [&](int i) __attribute__((always_inline)) {
      if constexpr (VW == 4) {
        const u32x4_t x = __builtin_nontemporal_load((const u32x4_t*)(src + voff[i]));
        vr.w[i][0] = x[0]; vr.w[i][1] = x[1]; vr.w[i][2] = x[2]; vr.w[i][3] = x[3];
      } else {
        const u32x2_t x = __builtin_nontemporal_load((const u32x2_t*)(src + voff[i]));
        vr.w[i][0] = x[0]; vr.w[i][1] = x[1];
      }
    };
    if (nv >= 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) load(i);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lg * 4 + i < nv) load(i);
    }
  };
  const uint32_t kslot0 = lds_offset(smem) + (uint32_t)(w * KR * TILE_B);
  // nv as for issue_v: a copy's lanes of rows past it copy nothing (the
  // slot keeps older bytes there, which compute_block never uses).
  auto issue_k = [&](int phys_raw, int sk, int nv) __attribute__((always_inline)) {
    const char* src = kbase + tile_of(phys_raw);
    const uint32_t dst = kslot0 + (uint32_t)(sk * TILE_B);
    if (nv >= 16) {
#pragma unroll
      for (int n = 0; n < NDMA; ++n) lds_dma16(src, dma_off[n], dst + n * 1024);
    } else {
#pragma unroll
      for (int n = 0; n < NDMA; ++n) {
        const int row = EB == 2 ? n * 4 + lg : n * 8 + (lane >> 3);   // as in dma_off
        if (row < nv) lds_dma16(src, dma_off[n], dst + n * 1024);
      }
    }
  };
  auto read_k = [&](int sk, u32x4_t (&kr)[KREADS]) __attribute__((always_inline)) {
    uint32_t addr[KREADS];
#pragma unroll
    for (int k = 0; k < KREADS; ++k) addr[k] = kaddr[k] + (uint32_t)(sk * TILE_B);
    lds_read16_wait<KREADS>(kr, addr);
  };

  // One tile: scores, online softmax, P.V.  vr is consumed (masked rows zeroed).
  auto compute_block = [&](int j, int sk, const BlockRef& br, const u32x4_t (&kr)[KREADS], VRows<VW>& vr)
                           __attribute__((always_inline)) {
    const int jl = span.logical(j);
    const bool blk_ok = (unsigned)br.phys < (unsigned)a.num_blocks;
    const uint32_t vbits = blk_ok ? span.valid_bits(jl) : 0u;
    float cs = a.scale;  // scale * log2(e), folded on the host
    float vsc = 1.f;
    if constexpr (KQ) cs *= br.ks * qfac;   // br.ks, br.vs: 1 with per-token scales
    if constexpr (VQ) vsc = br.vs;
    // per-token scales of the lane's tokens 4 lg .. + 3 (1 otherwise).  A
    // token outside the attended ones may have a scale slot never written:
    // its score is selected to -inf below, its weight to 0, so a NaN there
    // reaches neither.
    f32x4_t kt = {1.f, 1.f, 1.f, 1.f}, vt = {1.f, 1.f, 1.f, 1.f};
    if constexpr (KQ || VQ) {
      const char* ts = smem + C::KRING_B + (w * KR + sk) * C::TOKS_B + lg * 16;
      if (KQ && a.k_tok) kt = *(const f32x4_t*)ts;
      if (VQ && a.v_tok) vt = *(const f32x4_t*)(ts + 64);
    }
    u32x4_t kop[4];
    k_operands<KT, KREADS>(kr, kop);
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) s = Mma<MK>::run(kop[c], qop[c], s);

    // this lane's tokens 4 lg + i, for a real head
    const uint32_t mine = hv ? (vbits >> (lg * 4)) & 0xFu : 0u;
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = ((mine >> i) & 1u) ? s[i] * cs * kt[i] : -INFINITY;
    if (vbits != 0xFFFFu) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!((vbits >> (lg * 4 + i)) & 1u)) {
#pragma unroll
          for (int k = 0; k < VW; ++k) vr.w[i][k] = 0u;
        }
    }

    // move the head's reference maximum if a score passed it by > slack;
    // the head's four lane groups agree on the new value
    bool need = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) need |= sc[i] > mref + kLazyMaxSlack;
    if (__any(need)) {
      float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      bm = across_rows<16, true>(bm);
      const float mnew = fmaxf(mref, bm);
      const float f = exp2_safe_factor(mref, mnew);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] *= f;
      lsum *= f;
      mref = mnew;
    }
    const float mo = mref == -INFINITY ? 0.f : mref;
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pe = __builtin_amdgcn_exp2f(sc[i] - mo);
      lsum += pe;
      pv[i] = pe * vsc * vt[i];
      if constexpr (VQ) pv[i] = ((mine >> i) & 1u) ? pv[i] : 0.f;
    }
    const u32x4_t pop = p_operand<MV>(pv);
    u32x4_t vop[8];
    v_operands<VT, VW>(vr, vop);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = Mma<MV>::run(vop[c], pop, acc[c]);
  };

  {
    // wave w takes blocks j0 + w, j0 + w + NW, ...
    const int nunits = j1 - j0;
    const int n_my = w < nunits ? (nunits - w + NW - 1) / NW : 0;
    auto blk = [&](int t) __attribute__((always_inline)) { return j0 + w + t * NW; };
    VRows<VW> va, vb;
    constexpr unsigned kWaitVm0 = 0x0F70;     // vmcnt(0), expcnt(7), lgkmcnt(15)
    static_assert(KR == 2, "one step in flight: K(t+1) and V(t+1) while t is computed");
    // the new rows (copied, or quantised for an fp8 cache): loaded here and
    // stored once the next step's loads are issued -- a copy in step
    // n_my - 3 (in step 0, as the vector pass does, the 70B-shaped step was
    // 1.3 us slower per layer), quantised rows in step 0 (in step n_my - 3
    // the 131072-token fp8 layer was 2.4 us slower) -- and complete at the
    // following step's wait, before the wave loads its last block, the new
    // token's.  The int8 and mixed-format instantiations would need more
    // registers than their waves per SIMD allow, so they write before their
    // first loads.
    constexpr bool kDefer = !is_quantised<VT>() || (KT == KV::FP8 && VT == KV::FP8);
    const bool defer = kDefer && appends && w == append_wave && n_my >= 3;
    const int store_step = is_quantised<VT>() ? 0 : n_my - 3;
    decltype(append_step_load<KT, VT, QT, D>(a, b, h, lane, new_slot)) pend{};
    if (appends && w == append_wave) {
      if (defer) {
        pend = append_step_load<KT, VT, QT, D>(a, b, h, lane, new_slot);
      } else {
        append_rows();
        if (n_my == 1) wait_vmcnt<0>();
      }
    }
    BlockRef bcur{-1, 1.f, 1.f}, bnext{-1, 1.f, 1.f};
    if (n_my > 0) {
      bcur.phys = entry_of(blk(0));
      const int nv = span.rows(span.logical(blk(0)));
      issue_v(bcur.phys, va, nv);
      issue_k(bcur.phys, 0, nv);
      issue_tok(bcur.phys, 0);
      scales_of(bcur);
      if (n_my > 1) bnext.phys = entry_of(blk(1));
    }
    load_query();
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    auto step = [&](int t, VRows<VW>& vcur, VRows<VW>& vnext) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      wait_vmcnt<0>();
      const BlockRef b0 = bcur;
      const bool more = t + 1 < n_my;
      if (more) {
        const int nv = span.rows(span.logical(blk(t + 1)));
        issue_v(bnext.phys, vnext, nv);
        issue_k(bnext.phys, (t + 1) & 1, nv);
        issue_tok(bnext.phys, (t + 1) & 1);
      }
      if (defer && t == store_step) append_step_store<KT, VT, QT, D>(a, h, lane, new_slot, pend);
      u32x4_t kr[KREADS];
      read_k(t & 1, kr);
      if (more) {
        scales_of(bnext);
        bcur = bnext;
        if (t + 2 < n_my) bnext.phys = entry_of(blk(t + 2));
      }
      __builtin_amdgcn_sched_barrier(0);
      compute_block(blk(t), t & 1, b0, kr, vcur);
    };
    int t = 0;
    for (; t + 1 < n_my; t += 2) {
      step(t, va, vb);
      step(t + 1, vb, va);
    }
    if (t < n_my) step(t, va, vb);
  }
  // A head's sum over the wave's four lane groups; its accumulators are
  // already complete per lane (lane lq + 16 lg owns channels 32 lg .. + 31).
  const float lw = across_rows<16, false>(lsum);
  if (hv) {
    float* dst = &red_acc[w][lq][lg * 32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(float4*)(dst + i * 8) = float4{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
      *(float4*)(dst + i * 8 + 4) = float4{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
    }
    if (lg == 0) {
      red_m[w][lq] = mref;
      red_l[w][lq] = lw;
    }
  }
  __syncthreads();
  combine_waves<OT, D, G, NW>(a, b, h, p, tid, red_acc, red_m, red_l);
}

}  // namespace pkv
