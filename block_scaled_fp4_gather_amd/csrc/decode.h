// Device-side decode of E2M1 nibbles and block scales for gfx950.
//
// E2M1 (+-{0, 0.5, 1, 1.5, 2, 3, 4, 6}) is widened by the CDNA4 conversion
// instructions v_cvt_scalef32_pk_{bf16,f32}_fp4, which turn the two nibbles
// of one byte (low nibble first) into a packed pair.  They are given a unit
// scale; the block scale multiplies the partial dot product of its block
// instead, which is exact for the power-of-two UE8M0 scales and one extra
// rounding for E4M3.  UE8M0 bytes become fp32 by placing the byte in the
// exponent field (byte 0 is the subnormal 2^-127, byte 255 is NaN); E4M3
// bytes go through v_cvt_pk_f32_fp8 (OCP E4M3FN on gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float ue8m0_to_f32(uint32_t b) {
  b &= 0xFFu;
  const uint32_t bits = b == 0u ? 0x00400000u : (b == 255u ? 0x7FC00000u : b << 23);
  return __uint_as_float(bits);
}

// Two E4M3 bytes (positions 2*hi and 2*hi+1 of `word`) to fp32.
__device__ __forceinline__ f32x2_t e4m3x2_to_f32(uint32_t word, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true)
            : __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
}

// 8 nibbles of one dword -> 4 packed bf16 pairs (unit scale, exact).
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t w, bf16x2_t* o) {
  o[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
  o[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
  o[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
  o[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
}

// 8 nibbles of one dword -> 4 fp32 pairs (unit scale, exact).
__device__ __forceinline__ void fp4x8_to_f32(uint32_t w, f32x2_t* o) {
  o[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  o[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  o[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  o[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

// Round fp32 to bf16, nearest-even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Scale of unit (chunk) c of a lane, from its packed scale dwords.
// MXFP4: byte c%4 of dword c/4.  NVFP4: bytes 2(c%2), 2(c%2)+1 of dword c/2.
__device__ __forceinline__ float mx_scale(uint32_t dword, int c) {
  return ue8m0_to_f32(dword >> (8 * (c & 3)));
}

// Compressed scales (the CSF block of a tile, layout.h).  The CSF word of
// chunk c of a lane's row: base byte and the offsets of c's group of chunks.
template <int FMT>
__device__ __forceinline__ uint32_t csf_load(const uint8_t* csf, int lane, int c) {
  return __builtin_nontemporal_load((const uint32_t*)(csf + 256 * (c / (FMT == kMXFP4 ? 24 : 3)) + 4 * lane));
}

// Chunk c's scale bytes from its CSF word, placed where the plain scale word
// holds them (so mx_scale / e4m3x2_to_f32 read them alike): MXFP4 byte c %
// 4; NVFP4 bytes 2 (c % 2) and 2 (c % 2) + 1.  Not for exception rows.
template <int FMT>
__device__ __forceinline__ uint32_t csf_word(uint32_t w, int c) {
  const uint32_t base = w & 0xFFu;
  if (FMT == kMXFP4) return ((base + ((w >> (8 + c % 24)) & 1u)) & 0xFFu) << (8 * (c & 3));
  const uint32_t ob = (w >> (8 + 8 * (c % 3))) & 0xFFu;
  const uint32_t s = ((base + (ob & 15u)) & 0xFFu) | (((base + (ob >> 4)) & 0xFFu) << 8);
  return (c & 1) ? s << 16 : s;
}

// Whether a CSF word belongs to an exception row (base byte 255).
__device__ __forceinline__ bool csf_exception(uint32_t w) { return (w & 0xFFu) == 255u; }

// The scale word of chunk c of a lane's row from the CSF block, or the
// plain word for an exception row.
template <int FMT>
__device__ __forceinline__ uint32_t csf_scale_word(const uint8_t* csf, int lane, int c, uint32_t plain) {
  const uint32_t w = csf_load<FMT>(csf, lane, c);
  return csf_exception(w) ? plain : csf_word<FMT>(w, c);
}

}  // namespace moe
