// Device helpers for gfx950 (CDNA4): vector types, conversions, DPP
// reductions and matrix-core wrappers.  Wave size is 64 everywhere.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Running-max floor (log2 units).  Finite, so that states that have seen no
// valid token rescale by exp2(0) = 1 and weigh exp2(floor - real) = 0.
constexpr float kMaxFloor = -1.0e30f;

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32
}

// ---- DPP within a row of 16 lanes ------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF,
                                      0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // lane i <-> 7-i inside each 8 lanes
constexpr int kRowMirror = 0x140;   // lane i <-> 15-i inside each 16 lanes

// Sum over groups of N consecutive lanes (N = 1, 2, 4, 8, 16, 32, 64); every
// lane of a group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_mov<kQuadSwap1>(x);
  if constexpr (N >= 4) x += dpp_mov<kQuadSwap2>(x);
  if constexpr (N >= 8) x += dpp_mov<kHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_mov<kRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// ---- conversions -------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __builtin_bit_cast(float, w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[0];
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[1];
}

// two fp32 -> packed 16-bit (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// four E4M3FN bytes of a word -> four 16-bit values in two words
__device__ __forceinline__ i32x2 fp8x4_to_bf16x4(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return i32x2{__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
}
__device__ __forceinline__ i32x2 fp8x4_to_f16x4(uint32_t w) {
  f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return i32x2{__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
}
// four E4M3FN bytes -> four fp32
__device__ __forceinline__ f32x4 fp8x4_to_f32x4(uint32_t w) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  return f32x4{lo[0], lo[1], hi[0], hi[1]};
}

// byte-select of two words (v_perm_b32): low halves / high halves
__device__ __forceinline__ uint32_t pack_lo_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);  // a.lo | b.lo << 16
}
__device__ __forceinline__ uint32_t pack_hi_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);  // a.hi | b.hi << 16
}

// ---- matrix cores -------------------------------------------------------------
// 16x16 output tiles; lane l holds D[4*(l/16) + i][l % 16], i = 0..3.
// A operand lane l: A[l % 16][k-slice of lane group l / 16]; B operand lane l:
// B[k-slice of lane group l / 16][l % 16].
template <bool BF16>
__device__ __forceinline__ f32x4 mfma_k32(i32x4 a, i32x4 b, f32x4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <bool BF16>
__device__ __forceinline__ f32x4 mfma_k16(i32x2 a, i32x2 b, f32x4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(
        __builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// ---- caller-visible error flags ------------------------------------------------
// Flag k of the caller's array (null: none) is set to 1 when a kernel takes
// device-resident contents outside their contract; a plain store, so any
// number of lanes may set it at once.
__device__ __forceinline__ void raise_flag(int32_t* flags, int k) {
  if (flags) flags[k] = 1;
}

// ---- loads ----------------------------------------------------------------------
template <int BYTES>
struct Bytes;
template <>
struct Bytes<16> {
  i32x4 v;
  __device__ __forceinline__ uint32_t w(int i) const { return (uint32_t)v[i]; }
  __device__ __forceinline__ void zero() { v = i32x4{0, 0, 0, 0}; }
};
template <>
struct Bytes<8> {
  i32x2 v;
  __device__ __forceinline__ uint32_t w(int i) const { return (uint32_t)v[i]; }
  __device__ __forceinline__ void zero() { v = i32x2{0, 0}; }
};
template <>
struct Bytes<4> {
  int v;
  __device__ __forceinline__ uint32_t w(int) const { return (uint32_t)v; }
  __device__ __forceinline__ void zero() { v = 0; }
};

// cache-policy operand of the load-to-LDS builtin that marks a load
// non-temporal
constexpr int kNonTemporalAux = 2;

// K/V rows are read exactly once per decode call: non-temporal loads keep
// them from displacing reusable lines in the caches (on MI355X this lifts a
// paged gather from ~5.9 to ~6.4 TB/s).
template <int BYTES>
__device__ __forceinline__ Bytes<BYTES> load_bytes(const char* base, uint32_t off) {
  Bytes<BYTES> r;
  if constexpr (BYTES == 16)
    r.v = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(base + off));
  else if constexpr (BYTES == 8)
    r.v = __builtin_nontemporal_load(reinterpret_cast<const i32x2*>(base + off));
  else
    r.v = __builtin_nontemporal_load(reinterpret_cast<const int*>(base + off));
  return r;
}

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane l's bytes land at lds_base + 16 * l; the
// LDS base must be the same for the whole wave.  Non-temporal like the
// register loads above.
__device__ __forceinline__ void load_lds16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0,
                                   kNonTemporalAux);
}

}  // namespace pa
