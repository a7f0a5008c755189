// Per-1x32 MXFP4 quantisation of bf16 rows (gfx950).
//
// What it computes: P1 §Modifications quantises activations per 1x32 block
// before the FP4 GEMM and P2 §2 returns packed FP4 [rows, K/2] plus one E8M0
// byte per block; the arithmetic is the OCP-MX conversion of a 32-value
// vector into one MX block (the pages name the formats only):
//   b = max(E(amax) - 2, 0)           E = biased exponent field of amax
//   code = nearest E2M1 magnitude of |v| / 2^(b-127), ties to even, <= 6
//   sign bit copied from v; element 2j -> low nibble of byte j.
// The scaled magnitude is formed exactly by rewriting the exponent field (no
// rounding), and the nearest-even choice is a sum of seven threshold tests
// against the rounding midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5 (strict '>'
// where the midpoint rounds down to the even code, '>=' where it rounds up).
//
// Work split: one wave per 512-element row segment (16 blocks); lane l owns
// 8 consecutive elements (one 16-byte load, one 4-byte store), lanes
// 4j..4j+3 share block j and combine their amax with two xor shuffles.
// In the GEMM scale layout the grid also covers the padding rows (up to a
// multiple of 16) and padding blocks (up to a multiple of 16 per row), where
// it writes 0x7F: P2 §2 pads activation scales with E8M0 1.0 because whole
// tiles are read and 0xFF would be NaN.
#include "mxfp4_device.h"
#include "mxfp4_launch.h"

namespace mxfp4 {

__device__ __forceinline__ uint32_t e2m1_code(uint32_t h, uint32_t b) {
  const uint32_t mag = h & 0x7FFFu;
  const uint32_t ev = mag >> 7, m7 = mag & 0x7Fu;
  float y;
  if (ev == 0) {
    // bf16 subnormal (or zero): |v| = m7 * 2^-133, so y = m7 * 2^(-6-b).
    y = __builtin_ldexpf((float)m7, -6 - (int)b);
  } else {
    // |v| = 2^(ev-127) (1 + m7/128); y = |v| 2^(127-b): exponent ev + 127 - b.
    const int ye = (int)ev + 127 - (int)b;
    y = ye <= 0 ? 0.0f : __uint_as_float(((uint32_t)ye << 23) | (m7 << 16));
  }
  uint32_t c = (y > 0.25f) + (y >= 0.75f) + (y > 1.25f) + (y >= 1.75f) +
               (y > 2.5f) + (y >= 3.5f) + (y > 5.0f);
  return c | ((h >> 12) & 8u);
}

template <int LAYOUT>
__global__ __launch_bounds__(256) void quant_1x32_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int K,
    uint8_t* __restrict__ q, int64_t ldq, uint8_t* __restrict__ scales,
    int rows_cover, int segs, int G) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= (int64_t)rows_cover * segs) return;
  const int r = (int)(wave / segs), seg = (int)(wave % segs);
  const int nblocks = K >> 5;
  const int c = seg * 16 + (lane >> 2);
  const bool valid = (r < M) && (c < nblocks);
  const int k0 = seg * 512 + lane * 8;

  uint32_t h[8];
  uint32_t amax = 0;
  if (valid) {
    const int4 v = *reinterpret_cast<const int4*>(x + (int64_t)r * ldx + k0);
    const uint32_t w[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = w[i] & 0xFFFFu;
      h[2 * i + 1] = w[i] >> 16;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = max(amax, h[i] & 0x7FFFu);
  }
  // Lanes of one block are 4 aligned lanes, all valid or all invalid.
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
  const uint32_t e = amax >> 7;
  const uint32_t b = e > 2 ? e - 2 : 0;

  if (valid) {
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= e2m1_code(h[i], b) << (4 * i);
    *reinterpret_cast<uint32_t*>(q + (int64_t)r * ldq + (k0 >> 1)) = packed;
  }
  if ((lane & 3) == 0) {
    if (LAYOUT == 0) {
      if (valid) scales[(int64_t)r * nblocks + c] = (uint8_t)b;
    } else {
      scales[gemm_scale_offset(r, c, G)] = valid ? (uint8_t)b : (uint8_t)kE8M0One;
    }
  }
}

hipError_t launch_quant_1x32(const void* x, int64_t M, int64_t K, int64_t ldx, void* q,
                             int64_t ldq, void* scales, int layout, hipStream_t stream) {
  const int Kt = (int)((K + 127) / 128);
  const int G = (Kt + 3) / 4;
  const int segs = (int)((K + 511) / 512);
  const int rows_cover = layout == 0 ? (int)M : (int)((M + 15) / 16 * 16);
  const int64_t waves = (int64_t)rows_cover * segs;
  if (waves == 0) return hipSuccess;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (layout == 0)
    quant_1x32_kernel<0><<<grid, 256, 0, stream>>>((const uint16_t*)x, ldx, (int)M, (int)K,
                                                    (uint8_t*)q, ldq, (uint8_t*)scales,
                                                    rows_cover, segs, G);
  else
    quant_1x32_kernel<1><<<grid, 256, 0, stream>>>((const uint16_t*)x, ldx, (int)M, (int)K,
                                                    (uint8_t*)q, ldq, (uint8_t*)scales,
                                                    rows_cover, segs, G);
  return hipGetLastError();
}

}  // namespace mxfp4
