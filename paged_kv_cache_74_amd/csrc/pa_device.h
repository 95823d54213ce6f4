// Device helpers shared by the paged-KV kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "../../include/pa.h"

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// bf16 <-> f32.  A bfloat16 is the top half of a binary32, so widening is a shift.
__device__ __forceinline__ float bf16lo_f32(uint32_t pair) { return bits_f32(pair << 16); }
__device__ __forceinline__ float bf16hi_f32(uint32_t pair) { return bits_f32(pair & 0xffff0000u); }

// Two f32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  float2_t f = {lo, hi};
  bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

// acc + a.lo*b.lo + a.hi*b.hi with bf16 pairs and f32 accumulation (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Two e4m3 codes (the low or high 16 bits of `src`) -> a bf16 pair.  Every
// e4m3 value is exactly representable in bf16, so with a unit scale the
// conversion is exact.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t src) {
  bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, b);
}

// Two int8 codes (bytes 0, 1 of `src`, or 2, 3 when HI) -> a bf16 pair.  Every
// integer in [-128, 127] is exact in bf16, so the conversion is exact.
template <bool HI>
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t src) {
  const int32_t x = (int32_t)src;
  const float a = (float)((x << (HI ? 8 : 24)) >> 24);
  const float b = (float)((x << (HI ? 0 : 16)) >> 24);
  return pack_bf16(a, b);
}

// Two 8-bit cache codes (fp8 e4m3 or int8) -> a bf16 pair, exactly.
template <int CDT, bool HI>
__device__ __forceinline__ uint32_t code8x2_to_bf16x2(uint32_t src) {
  if constexpr (CDT == PA_INT8) return i8x2_to_bf16x2<HI>(src);
  else return fp8x2_to_bf16x2<HI>(src);
}

// INT4 codes as e4m3 bytes.  Eight sign-magnitude nibbles of `x` (element 2i
// in the low nibble of byte i) become four e4m3 bytes each: an e4m3 subnormal
// is m * 2^-9 for its mantissa m, so the magnitude goes into the mantissa bits
// and the sign into bit 7.  lo: elements 0, 2, 4, 6; hi: elements 1, 3, 5, 7.
__device__ __forceinline__ uint32_t int4_lo_as_e4m3(uint32_t x) {
  return (x & 0x07070707u) | ((x << 4) & 0x80808080u);
}
__device__ __forceinline__ uint32_t int4_hi_as_e4m3(uint32_t x) {
  return ((x >> 4) & 0x07070707u) | (x & 0x80808080u);
}
// Two such bytes -> the bf16 pair of the integer codes, exactly (the scale 2^9
// undoes the subnormal quantum).
template <bool HI>
__device__ __forceinline__ uint32_t int4e4m3_to_bf16x2(uint32_t src) {
  bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 512.0f, HI);
  return __builtin_bit_cast(uint32_t, b);
}

// ---------------------------------------------------------------------------
// Cache encoders of the append (also used by the decode that appends).
// e4m3 (OCP e4m3fn) encoder: saturate to +-448, round half to even, NaN -> 0x7F.
// Integer-only, so the result never depends on the device's float modes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = f32_bits(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                 // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;         // |x| >= 448 (and inf): saturate
  const int e = (int)(a >> 23) - 127;                // unbiased binary32 exponent
  const uint32_t m = (a & 0x7fffffu) | 0x800000u;    // 24-bit significand (normal input)
  // value = m * 2^(e-23).  Normal e4m3 (e >= -6) keeps 3 fraction bits:
  // q = m >> 20 in [8, 16); subnormal e4m3 counts units of 2^-9: q = m >> (14 - e).
  const int shift = e >= -6 ? 20 : 14 - e;
  if (shift >= 26) return sign;                      // below a quarter unit: +-0
  const uint32_t q = m >> shift;
  const uint32_t rem = m & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  const uint32_t r = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
  // Normal: code = (e + 7) * 8 + (r - 8); r == 16 carries into the exponent.
  // Subnormal: code = r (r == 8 is the smallest normal, code 0x08).
  const uint32_t code = e >= -6 ? (uint32_t)((e + 7) * 8) + r - 8u : r;
  return sign | code;
}

// int8 encoder: round half to even, clamp to [-127, 127], NaN -> 0.  (The
// clamp before the rounding changes no result: every value beyond +-127 ends
// at +-127 either way.)
__device__ __forceinline__ uint32_t f32_to_int8(float x) {
  if (!(x == x)) return 0u;
  const float r = __builtin_rintf(fminf(fmaxf(x, -127.0f), 127.0f));
  return (uint32_t)(int32_t)r & 0xffu;
}

template <int DST>
__device__ __forceinline__ uint32_t encode8(float x) {
  if constexpr (DST == PA_FP8_E4M3) return f32_to_e4m3(x);
  else return f32_to_int8(x);
}

// v_perm_b32: byte i of the result is byte sel[i] of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// {a.lo16, b.lo16} and {a.hi16, b.hi16}
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

// DPP lane exchanges inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xf, 0xf, false));
}
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <-> 7-i inside each group of 8
constexpr int DPP_ROR8 = 0x128;         // row rotate by 8: lane i <-> i^8 inside a row

// Sum over the 8 lanes {8k .. 8k+7}; every lane of the group gets the total.
__device__ __forceinline__ float sum8(float v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  v += dpp<DPP_HALF_MIRROR>(v);
  return v;
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Reductions over the 8 lane groups that differ in lane bits 3..5.
__device__ __forceinline__ float max_over_groups(float v) {
  v = fmaxf(v, dpp<DPP_ROR8>(v));
  v = fmaxf(v, shfl_xor(v, 16));
  v = fmaxf(v, shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float sum_over_groups(float v) {
  v += dpp<DPP_ROR8>(v);
  v += shfl_xor(v, 16);
  v += shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-uniform read of a table that no kernel of the call writes: through the
// constant address space, so it becomes a scalar load (counted apart from the
// vector loads in flight) even where the kernel has stores in between.
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ __forceinline__ int32_t uniform_load(const int32_t* p, int i) {
  return ((const_i32*)p)[i];
}

// ---------------------------------------------------------------------------
// host: launch a kernel and report the status of that launch alone.
// hipLaunchKernel returns the launch's own error code; an error left behind by
// an unrelated earlier call (which hipGetLastError would hand back) is not
// reported as this call's failure.
// ---------------------------------------------------------------------------
template <typename... P, size_t... I>
inline pa_status launch_held(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem,
                             hipStream_t stream, std::tuple<P...>& held,
                             std::index_sequence<I...>) {
  void* argv[] = {(void*)&std::get<I>(held)..., nullptr};
  return hipLaunchKernel((const void*)kernel, grid, block, argv, shmem, stream) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

template <typename... P, typename... A>
inline pa_status launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem,
                        hipStream_t stream, A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> held(std::forward<A>(args)...);
  return launch_held(kernel, grid, block, shmem, stream, held, std::index_sequence_for<P...>{});
}

// Device id of the calling thread (0 if it cannot be read), for per-device caches.
constexpr int MAX_DEVICES = 64;
inline int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) dev = 0;
  return dev;
}

}  // namespace pa
