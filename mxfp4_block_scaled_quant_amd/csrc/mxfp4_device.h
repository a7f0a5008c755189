// Device-side helpers shared by the gfx950 kernels of libmxfp4.
//
// Operand layout of the block-scaled FP4 MFMA used throughout
// (v_mfma_scale_f32_16x16x128_f8f6f4 with both formats E2M1), as measured on
// MI355X: lane l of a wave supplies 16 bytes = 32 FP4 values of row l%16,
// K block l/16 (one whole 1x32 MX block), for each of A (16 x 128) and
// B (128 x 16); the lane's 32-bit scale register supplies that block's E8M0
// byte, the op_sel operand picking which of its 4 bytes; result lane l,
// register i holds D[4*(l/16) + i][l%16].  Products are exact and the sum
// is rounded like fp32 (error ~2^-25 of sum |a*b| per instruction).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v2s __attribute__((ext_vector_type(2)));

// E8M0 1.0: fill for every padded scale (0xFF would be NaN).
constexpr uint32_t kE8M0One = 0x7F;
constexpr uint32_t kE8M0OneX4 = 0x7F7F7F7Fu;

// Buffer resource for raw buffer loads: base, byte size (num_records),
// default stride 0, gfx9 data format word.  Loads at offsets >= size return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// An offset guaranteed to be out of range for any resource: masked lanes use it.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ int4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// One block-scaled FP4 MFMA step: acc += (A * 2^(sa-127)) x (B * 2^(sb-127)).
// The scale bytes are taken from byte SEL of each scale register.
template <int SEL_A, int SEL_B>
__device__ __forceinline__ v4f mfma_fp4(const int4& a, const int4& b, uint32_t sa, uint32_t sb, v4f acc) {
  v8i A = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  v8i B = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 4, SEL_A, (int)sa, SEL_B, (int)sb);
}

// fp32 -> bf16 bits, round to nearest even, by gfx950's conversion
// instruction: identical to integer RNE rounding (add 0x7FFF plus the kept
// LSB, truncate) for every non-NaN fp32 pattern, and NaN stays NaN (checked
// exhaustively over all 2^32 inputs on MI355X).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two fp32 values -> packed bf16 pair (lo in bits 0-15), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  const v2bf h = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// ---- Encoding one MX block (OCP MX v1.0, conversion of a vector of 32
// values into one block with E2M1 elements and an E8M0 scale).
//
// Scale byte from the largest |bf16| bit pattern of the block: the biased
// exponent E of amax, less emax(E2M1) = 2, clamped at 0 (zero and subnormal
// amax give 0).  |bf16| bit patterns order like their values.
__device__ __forceinline__ uint32_t e8m0_of_amax_bits(uint32_t amax_bits) {
  const uint32_t e = amax_bits >> 7;
  return e > 2 ? e - 2 : 0;
}

// Packed per-half max of |bf16| over dwords holding two bf16 each.
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t absmax_pairs(uint32_t m, uint32_t w) {
  const v2u16 a = __builtin_bit_cast(v2u16, m), b = __builtin_bit_cast(v2u16, w & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

// The fp32 value 2^(b-127) of a scale byte (b = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t b) { return __uint_as_float(b ? (b << 23) : 0x00400000u); }

// Eight bf16 values (four dwords, element 2j in the low half of dword j) ->
// eight E2M1 codes in one dword (element i in bits 4i..4i+3), each |v| /
// 2^(b-127) rounded to the nearest E2M1 magnitude, ties to the even code,
// saturating at 6, sign copied.  gfx950's scaled FP4 conversion divides by
// its scale operand and rounds exactly this way for every finite bf16 input
// and every scale byte (checked over all 65536 patterns on MI355X; the
// quantisation kernels' parity tests pin it against the oracle bytewise).
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e2m1_pack8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, float scale) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf16, w0), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf16, w1), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf16, w2), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf16, w3), scale, 3);
  return r;
}

// The largest |bf16| bit pattern of a block held as 8 values by each of
// the 4 lanes of a quad (lanes 4q..4q+3), in every lane of the quad: a
// packed max over the lane's dwords, then two quad permutes (DPP, no LDS).
__device__ __forceinline__ uint32_t quad_amax_bits(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  uint32_t m = absmax_pairs(absmax_pairs(absmax_pairs(absmax_pairs(0u, w0), w1), w2), w3);
  uint32_t a = max(m & 0xFFFFu, m >> 16);
  a = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0xB1, 0xF, 0xF, true));  // lane ^ 1
  a = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0x4E, 0xF, 0xF, true));  // lane ^ 2
  return a;
}

// A whole 1x32 block held by one lane (four 16-byte pieces in element order)
// -> its 16 code bytes (the lane's operand of the block-scaled FP4 MFMA) and
// its scale byte.
__device__ __forceinline__ int4 quant_block32(const int4 (&v)[4], uint32_t& b) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = absmax_pairs(m, (uint32_t)v[i].x);
    m = absmax_pairs(m, (uint32_t)v[i].y);
    m = absmax_pairs(m, (uint32_t)v[i].z);
    m = absmax_pairs(m, (uint32_t)v[i].w);
  }
  b = e8m0_of_amax_bits(max(m & 0xFFFFu, m >> 16));
  const float sc = e8m0_value(b);
  int4 c;
  c.x = (int)e2m1_pack8((uint32_t)v[0].x, (uint32_t)v[0].y, (uint32_t)v[0].z, (uint32_t)v[0].w, sc);
  c.y = (int)e2m1_pack8((uint32_t)v[1].x, (uint32_t)v[1].y, (uint32_t)v[1].z, (uint32_t)v[1].w, sc);
  c.z = (int)e2m1_pack8((uint32_t)v[2].x, (uint32_t)v[2].y, (uint32_t)v[2].z, (uint32_t)v[2].w, sc);
  c.w = (int)e2m1_pack8((uint32_t)v[3].x, (uint32_t)v[3].y, (uint32_t)v[3].z, (uint32_t)v[3].w, sc);
  return c;
}

// Byte offset of scale (row r, block c) in the GEMM scale layout with G groups.
__device__ __forceinline__ uint32_t gemm_scale_offset(uint32_t r, uint32_t c, uint32_t G) {
  uint32_t t = c >> 2, kb = c & 3, g = t >> 2, j = t & 3;
  return ((r >> 4) * G + g) * 256u + ((kb << 4) + (r & 15)) * 4u + j;
}

}  // namespace mxfp4
