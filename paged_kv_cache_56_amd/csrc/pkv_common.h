// Shared device helpers for the pagedkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum class KV : int { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };

template <KV T> struct kv_bytes;
template <> struct kv_bytes<KV::F32> { static constexpr int value = 4; };
template <> struct kv_bytes<KV::F16> { static constexpr int value = 2; };
template <> struct kv_bytes<KV::BF16> { static constexpr int value = 2; };
template <> struct kv_bytes<KV::FP8> { static constexpr int value = 1; };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }
constexpr int cmin(int a, int b) { return a < b ? a : b; }

// ---- lane exchange inside a 16-lane DPP row ------------------------------
// DPP control codes (GCN/CDNA encoding).
constexpr int DPP_QUAD_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROW_ROR8 = 0x128;      // row_ror:8  (lane c <-> c ^ 8)
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane c <-> 7 - c inside each 8

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// ---- conversions ----------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(half2_t, w).x;
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(half2_t, w).y;
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <KV T> struct out_store;

}  // namespace pkv
