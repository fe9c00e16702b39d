// MXFP8 activations for the W4A8-MX variant: E4M3 elements with one UE8M0
// scale per 32 consecutive values (b12x PR #22, Measured table: the dynamic
// path quantises activations to MXFP8; flashinfer #4285 review of the direct
// micro kernel: the activation scale column is K / 32).  Encoding per the OCP
// MX definition: the block's shared exponent is floor(log2(max |v|)) - 8 (8
// = exponent of E4M3's largest power of two), clamped to [-127, 127]; each
// value divided by 2^shared is rounded to nearest-even E4M3 and capped at
// 448.  A block of zeros gets scale byte 0; a block holding a NaN or an
// infinity gets scale byte 255 (NaN) and every code 0x7F.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Scale byte of a block from the largest |v| as fp32 bits (an integer max of
// the magnitudes' bits, so NaN and infinity compare above every finite
// value): shared + 127 = exponent field - 8, at least 0.
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits) {
  if (amax_bits >= 0x7F800000u) return 255u;
  const int ef = (int)(amax_bits >> 23);
  return (uint32_t)(ef > 8 ? ef - 8 : 0);
}

// 2^-shared for a finite scale byte (at most 246): fp32 with exponent field
// 254 - byte, always a normal number.
__device__ __forceinline__ float mx_inv_scale(uint32_t sbyte) { return __uint_as_float((254u - sbyte) << 23); }

// E4M3 code of a finite v with |v| < 512: magnitude capped at 448, then
// rounded to nearest-even.  Normal range (>= 2^-6): the fp32 significand is
// rounded to 3 bits in place (a carry moves into the exponent) and the
// exponent rebiased from 127 to 7.  Below 2^-6: steps of 2^-9, where a
// result of 8 is the encoding of the smallest normal.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  a = a < 0x43E00000u ? a : 0x43E00000u;  // 448
  if (a >= 0x3C800000u) {                 // 2^-6
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    return sign | (r - (120u << 3));
  }
  return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
}

// Value of an E4M3 code (finite codes only): exponent field e and mantissa m
// give (1 + m / 8) * 2^(e - 7), or m * 2^-9 for e = 0.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

}  // namespace moe

// MXFP8 quantisation of bf16 rows: codes [rows][cols] (row stride cols),
// scales [rows][sstride] (bytes cols/32 .. sstride-1 of a scale row are not
// written).  cols must be a multiple of 32.
hipError_t launch_mxfp8_quantize(const uint16_t* x, int64_t rows, int cols, uint8_t* codes,
                                 uint8_t* scales, int sstride, hipStream_t st);
