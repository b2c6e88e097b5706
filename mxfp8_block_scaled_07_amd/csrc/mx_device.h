// Device helpers shared by the MXFP8 kernels (gfx950 only).
//
// MXFP8 = OCP MX: 32-element blocks, E4M3 codes and one E8M0 scale per block
// (digest "Key Questions Answered": one scale per fine-grained sub-block;
// pytorch/ao PR #3203 stacked list: quantize, dequantize and the e8m0 -> fp32
// scale decode).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxmoe.h"

namespace mx {

typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 32;

// Scale byte of a block from the bf16 magnitude bits of its amax:
// floor(log2 amax) - 8 clamped at -127, biased by 127.  For a normal amax the
// floor of log2 is its exponent field minus 127, so the byte is the exponent
// field minus 8; zero and subnormal amax (field 0) clamp to byte 0.
__device__ __forceinline__ uint32_t scale_byte_from_amax(uint32_t amax_bits) {
  const uint32_t e = amax_bits >> 7;
  return e > 8u ? e - 8u : 0u;
}

// fp32 holding 2^(byte-127) for byte in [0, 254]; byte 0 is the fp32
// subnormal 2^-127 (never 0).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return __uint_as_float(b ? (b << 23) : 0x00400000u);
}

// Largest bf16 magnitude (bits, sign cleared) of the two halves of w.
__device__ __forceinline__ uint32_t absmax2(uint32_t w) {
  const v2u16 m = __builtin_bit_cast(v2u16, w & 0x7FFF7FFFu);
  return m[0] > m[1] ? m[0] : m[1];
}

__device__ __forceinline__ v2u16 absbits(uint32_t w) { return __builtin_bit_cast(v2u16, w & 0x7FFF7FFFu); }

__device__ __forceinline__ v2u16 vmax(v2u16 a, v2u16 b) { return __builtin_elementwise_max(a, b); }

__device__ __forceinline__ uint32_t hmax(v2u16 a) { return a[0] > a[1] ? a[0] : a[1]; }

// The E4M3 conversion rounds to nearest even but turns magnitudes that round
// past 448 into the NaN code (0x7F / 0xFF).  Saturation maps exactly those
// bytes to 0x7E / 0xFE: a byte whose low 7 bits are all ones gains a carry
// into bit 7 when 1 is added to its low 7 bits; subtract 1 from such bytes.
__device__ __forceinline__ uint32_t saturate_e4m3x4(uint32_t w) {
  const uint32_t t = (w & 0x7F7F7F7Fu) + 0x01010101u;
  return w - ((t & 0x80808080u) >> 7);
}

// Four bf16 (two packed words) -> four E4M3 codes of x / scale, RNE, saturating.
__device__ __forceinline__ uint32_t cvt4_e4m3(uint32_t x01, uint32_t x23, float scale) {
  v2s r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf, x01), scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf, x23), scale, true);
  return saturate_e4m3x4(__builtin_bit_cast(uint32_t, r));
}

// Four E4M3 codes -> four bf16 (two packed words) of code * scale, RNE.
__device__ __forceinline__ uint2 cvt4_bf16(uint32_t codes, float scale) {
  const v2bf lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, false);
  const v2bf hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// Max over the 4 lanes of a quad (lanes 4q..4q+3) via DPP quad permutes.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // lane ^ 1
  v = v > o ? v : o;
  o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);           // lane ^ 2
  return v > o ? v : o;
}

typedef float v2f __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (low half = a), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
}

// fp32 -> bf16 bits, round to nearest even (finite and infinite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Scale layout of an MX tensor viewed as a matrix of R rows (batch entries
// stacked) and C columns: 128-column panels, stored panel-major; inside
// panel p, row r keeps the scale bytes of its blocks 4p..4p+3 in one dword.
// A GEMM k step then reads the scales of consecutive rows as consecutive
// dwords.  Byte of (row r, block b): ((b >> 2) * R + r) * 4 + (b & 3);
// bytes of blocks past the last one (C % 128 != 0) are zero.
__device__ __forceinline__ int64_t scale_index(int64_t R, int64_t r, int64_t b) {
  return ((b >> 2) * R + r) * 4 + (b & 3);
}

// Store the scale byte of block b (of nb) of row r; the row's last block also
// zeroes the pad bytes of its panel.
__device__ __forceinline__ void put_scale(uint8_t* s, int64_t R, int64_t r, int64_t b, int64_t nb, uint32_t v) {
  s[scale_index(R, r, b)] = (uint8_t)v;
  if (b == nb - 1)
    for (int64_t j = b + 1; j < ((nb + 3) & ~(int64_t)3); ++j) s[scale_index(R, r, j)] = 0;
}

inline int launch_status() { return hipGetLastError() == hipSuccess ? MX_OK : MX_EHIP; }

}  // namespace mx
