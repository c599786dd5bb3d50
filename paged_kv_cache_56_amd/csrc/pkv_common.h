// Shared device helpers for the pagedkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum class KV : int { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3, INT8 = 4 };

// 8-bit codes with a per-(block, head) scale
template <KV T> constexpr bool is_quantised() { return T == KV::FP8 || T == KV::INT8; }

template <KV T> struct kv_bytes;
template <> struct kv_bytes<KV::F32> { static constexpr int value = 4; };
template <> struct kv_bytes<KV::F16> { static constexpr int value = 2; };
template <> struct kv_bytes<KV::BF16> { static constexpr int value = 2; };
template <> struct kv_bytes<KV::FP8> { static constexpr int value = 1; };
template <> struct kv_bytes<KV::INT8> { static constexpr int value = 1; };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }
constexpr int cmin(int a, int b) { return a < b ? a : b; }

// ---- lane exchange inside a 16-lane DPP row ------------------------------
// DPP control codes (GCN/CDNA encoding).
constexpr int DPP_QUAD_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROW_ROR8 = 0x128;      // row_ror:8  (lane c <-> c ^ 8)
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane c <-> 7 - c inside each 8

// Every control used here reads a valid lane for every lane, so the "old"
// operand is never selected (bound_ctrl set: no register needs priming).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// ---- combining the token rows of a wave ----------------------------------
// Lanes l and l' hold the same quantity for different token rows when
// l % LPT == l' % LPT (LPT lanes per row, 4, 8 or 16).  across_rows combines
// the 64 / LPT copies and leaves the result in every lane.  Inside a 16-lane
// DPP row the copies are LPT apart, and rotating the row by 4 and then by 8
// visits all of them.  Across rows, gfx950's lane swaps do it without the
// LDS round trip of a shuffle: with both operands equal to x, the two
// results of v_permlane16_swap hold, in every lane, x and x from the lane 16
// away (rows 0<->1, 2<->3), and v_permlane32_swap likewise for lanes 32
// away, so combining the two results combines the pair.
constexpr int DPP_ROW_ROR4 = 0x124;      // row_ror:4

template <bool MAX>
__device__ __forceinline__ float combine2(float a, float b) { return MAX ? fmaxf(a, b) : a + b; }

template <int LPT, bool MAX>
__device__ __forceinline__ float across_rows(float x) {
  static_assert(LPT == 4 || LPT == 8 || LPT == 16, "lanes per token row");
  if constexpr (LPT == 4) x = combine2<MAX>(x, dpp<DPP_ROW_ROR4>(x));
  if constexpr (LPT <= 8) x = combine2<MAX>(x, dpp<DPP_ROW_ROR8>(x));
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = combine2<MAX>(__builtin_bit_cast(float, (uint32_t)s16[0]), __builtin_bit_cast(float, (uint32_t)s16[1]));
  const uint32_t v = __builtin_bit_cast(uint32_t, x);
  const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return combine2<MAX>(__builtin_bit_cast(float, (uint32_t)s32[0]), __builtin_bit_cast(float, (uint32_t)s32[1]));
}

// ---- asynchronous global -> LDS copies (gfx950 LDS DMA) --------------------
// One instruction moves 16 bytes per lane from `gbase + voff` (per lane) into
// LDS at `lds + 16 * lane`.  The copy is tracked by vmcnt only, so the waits
// below are explicit; the compiler is told nothing about the LDS write except
// a memory clobber, which keeps LDS reads from moving across these points.
// The read is non-temporal (streamed data, read once): on this chip a
// stream of scattered 4 KiB tiles read that way runs about 11% faster than
// under the default cache policy, at the rate of a sequential read.
__device__ __forceinline__ void lds_dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1 nt"
      :
      : "v"(voff), "s"(gbase), "s"(lds)
      : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// N 16-byte LDS reads (ds_read_b128) and the wait for them, in one asm
// statement: the outputs are defined only when the statement ends, after
// the wait, so the compiler cannot use them while they are in flight.  The
// compiler would otherwise split each read into two ds_read2_b32, which
// puts four lanes on every bank when the 64 lanes read consecutive 16-byte
// columns.  addr: LDS byte addresses, 16-byte aligned.
template <int N>
__device__ __forceinline__ void lds_read16_wait(u32x4_t (&out)[N], const uint32_t (&addr)[N]) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "1, 2, 4 or 8 reads");
  if constexpr (N == 1) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(out[0]) : "v"(addr[0]) : "memory");
  } else if constexpr (N == 2) {
    asm volatile(
        "ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(out[0]), "=&v"(out[1])
        : "v"(addr[0]), "v"(addr[1])
        : "memory");
  } else if constexpr (N == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]), "=&v"(out[5]),
          "=&v"(out[6]), "=&v"(out[7])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
          "v"(addr[7])
        : "memory");
  }
}

// The same with 8-byte reads (ds_read_b64), 2 or 4 of them.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <int N>
__device__ __forceinline__ void lds_read8_wait(u32x2_t (&out)[N], const uint32_t (&addr)[N]) {
  static_assert(N == 2 || N == 4, "2 or 4 reads");
  if constexpr (N == 2) {
    asm volatile(
        "ds_read_b64 %0, %2\n\tds_read_b64 %1, %3\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(out[0]), "=&v"(out[1])
        : "v"(addr[0]), "v"(addr[1])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64 %0, %4\n\tds_read_b64 %1, %5\n\tds_read_b64 %2, %6\n\tds_read_b64 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3])
        : "memory");
  }
}

// LDS byte offset of a __shared__ object (the low half of its flat address).
__device__ __forceinline__ uint32_t lds_offset(const void* p) { return (uint32_t)(uintptr_t)p; }

// ---- conversions ----------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(half2_t, w).x;
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(half2_t, w).y;
}

// Two fp32 values -> an f16 pair in one word (one v_cvt_pk_f16_f32, round to
// nearest even), lo in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const half2_t h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- 8-bit codes (quantise on write) ---------------------------------------
// Largest code magnitude: 448 for OCP e4m3fn, 127 for symmetric int8.
template <KV CT> constexpr float qmax() { return CT == KV::FP8 ? 448.0f : 127.0f; }

// N (2 or 4) clamped quotients -> N codes in one word, element 0 in the low
// byte: fp8 by the hardware's round-to-nearest-even e4m3 convert, int8 by
// rint (ties to even; NaN gives 0).
template <KV CT, int N>
__device__ __forceinline__ uint32_t encode_codes(const float (&v)[N]) {
  static_assert(N == 2 || N == 4, "two or four codes");
  if constexpr (CT == KV::FP8) {
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    if constexpr (N == 4) word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
    return (uint32_t)word & (N == 4 ? 0xFFFFFFFFu : 0xFFFFu);
  } else {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const float r = v[e] == v[e] ? __builtin_rintf(v[e]) : 0.f;
      word |= ((uint32_t)(int)r & 0xFFu) << (8 * e);
    }
    return word;
  }
}

}  // namespace pkv
