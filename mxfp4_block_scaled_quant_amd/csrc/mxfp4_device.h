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

// Byte offset of scale (row r, block c) in the GEMM scale layout with G groups.
__device__ __forceinline__ uint32_t gemm_scale_offset(uint32_t r, uint32_t c, uint32_t G) {
  uint32_t t = c >> 2, kb = c & 3, g = t >> 2, j = t & 3;
  return ((r >> 4) * G + g) * 256u + ((kb << 4) + (r & 15)) * 4u + j;
}

}  // namespace mxfp4
