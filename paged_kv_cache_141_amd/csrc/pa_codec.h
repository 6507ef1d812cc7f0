// pa_codec.h -- device-side number formats of the KV cache (gfx950).
//
// The cache write stores K/V as fp32, fp16, bf16 or an 8-bit float with a
// per-tensor scale (techknowgenie "vLLM V1 core refactoring", section on the
// FP8 KV cache: the 8-bit cache halves the bytes of FP16; itwiki "vLLM",
// engine features: --kv-cache-dtype).  The 8-bit format is OCP E4M3FN: bias
// 7, three mantissa bits, subnormals at exponent field 0, largest finite 448,
// NaN at S.1111.111, no infinities.
//
// All encoders round to nearest, ties to even, on the integer image of the
// fp32 input: adding (half quantum - 1) plus the lowest kept bit and then
// truncating rounds ties to the even neighbour.  They are written as plain
// integer code so their result never depends on a hardware rounding mode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

// ---- decode to fp32 (exact) -----------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return u2f(b << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// ---- fp32 -> bf16 bits ------------------------------------------------------
// NaN -> sign | 0x7FC0; values past the largest finite bf16 round to inf.
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  uint32_t u = f2u(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---- fp32 -> fp16 bits ------------------------------------------------------
// NaN -> sign | 0x7E00; |x| >= 65520 (past 65504 by half an ulp) -> inf.
__device__ __forceinline__ uint32_t f32_to_f16(float x) {
  const uint32_t u = f2u(x);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7E00u;
  if (a >= 0x477FF000u) return sign | 0x7C00u;
  if (a < 0x38800000u) {                     // below 2^-14: fp16 subnormal (or zero)
    // |x| * 2^24 counts fp16 subnormal quanta; scaling by a power of two is exact
    const uint32_t q = static_cast<uint32_t>(__builtin_rintf(u2f(a) * 16777216.0f));
    return sign | q;                         // q == 1024 is the smallest normal
  }
  uint32_t r = a + 0xFFFu + ((a >> 13) & 1u);  // keep 10 mantissa bits
  return sign | ((r >> 13) - (112u << 10));    // rebias 127 -> 15
}

// ---- fp32 -> E4M3FN code, with a per-tensor scale ---------------------------
// code = e4m3(fl32(x / scale)): correctly rounded fp32 quotient, RNE to three
// mantissa bits, finite overflow and inf saturate to +-448, NaN -> sign|0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x, float scale) {
  const float y = x / scale;                 // IEEE division (compiled without fast-math)
  const uint32_t u = f2u(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |y| >= 448
  if (a < 0x3C800000u) {                       // below 2^-6: subnormal quanta of 2^-9
    const uint32_t q = static_cast<uint32_t>(__builtin_rintf(u2f(a) * 512.0f));
    return sign | q;                           // q == 8 is the smallest normal
  }
  uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);  // keep 3 mantissa bits
  return sign | ((r >> 20) - (120u << 3));       // rebias 127 -> 7
}

}  // namespace pa
