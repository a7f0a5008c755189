// Per-1x32 MXFP4 quantisation of bf16 rows (gfx950).
//
// What it computes: P1 §Modifications quantises activations per 1x32 block
// before the FP4 GEMM and P2 §2 returns packed FP4 [rows, K/2] plus one E8M0
// byte per block; the arithmetic is the OCP-MX conversion of a 32-value
// vector into one MX block (the pages name the formats only):
//   b = max(E(amax) - 2, 0)           E = biased exponent field of amax
//   code = nearest E2M1 magnitude of |v| / 2^(b-127), ties to even, <= 6
//   sign bit copied from v; element 2j -> low nibble of byte j.
// The scale byte comes from integer compares on the |bf16| bit patterns; the
// elements are encoded by gfx950's scaled bf16 -> FP4 conversion, which
// divides by 2^(b-127) and rounds to nearest-even with saturation exactly
// as above.
//
// Two output forms:
//  * ROWMAJOR (weights before a preshuffle, interop): a wave per one or
//    four 512-element row segments (16 blocks each); lane l owns 8
//    consecutive elements of a segment (one 16-byte load, one 4-byte store),
//    lanes 4j..4j+3 share block j and combine their amax with two xor
//    shuffles.
//  * GEMM (what the FP4 GEMM reads): a workgroup per one or four 1 KiB units
//    of the GEMM data layout (16 rows x one 128-wide K-step), same 8
//    elements per lane.  The grid covers the padding rows (to 16) and K-steps (to the
//    4-step scale group) and writes 0x00 data and 0x7F scales there: P2 §2
//    pads scale tiles with E8M0 1.0 because whole tiles are read and 0xFF
//    would be NaN.
#include "mxfp4_device.h"
#include "mxfp4_launch.h"

namespace mxfp4 {

// Row-major: wave w of the grid takes the U consecutive 512-element row
// segments U*w .. U*w+U-1 (segment = row * segs + seg), all U loads issued
// before the first is used (U > 1 keeps more bytes in flight per wave where
// there are many segments).
template <int U>
__global__ __launch_bounds__(256) void quant_1x32_rowmajor_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int K,
    uint8_t* __restrict__ q, int64_t ldq, uint8_t* __restrict__ scales, int segs) {
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * U;
  const int nblocks = K >> 5;
  const int64_t total = (int64_t)M * segs;
  uint32_t w[U][4];
  bool valid[U];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int64_t wave = wave0 + j;
    const int r = (int)(wave / segs), seg = (int)(wave % segs);
    const int c = seg * 16 + (lane >> 2);
    // lanes of one block are 4 aligned lanes, all valid or all invalid
    valid[j] = wave < total && r < M && c < nblocks;
    const int k0 = seg * 512 + lane * 8;
    w[j][0] = w[j][1] = w[j][2] = w[j][3] = 0;
    if (valid[j]) {
      const int4 v = *reinterpret_cast<const int4*>(x + (int64_t)r * ldx + k0);
      w[j][0] = (uint32_t)v.x, w[j][1] = (uint32_t)v.y, w[j][2] = (uint32_t)v.z, w[j][3] = (uint32_t)v.w;
    }
  }
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int64_t wave = wave0 + j;
    if (wave >= total) break;  // uniform across the wave
    const int r = (int)(wave / segs), seg = (int)(wave % segs);
    const int c = seg * 16 + (lane >> 2);
    const int k0 = seg * 512 + lane * 8;
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = absmax_pairs(m, w[j][i]);
    uint32_t amax = max(m & 0xFFFFu, m >> 16);
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
    const uint32_t b = e8m0_of_amax_bits(amax);
    if (valid[j]) {
      const uint32_t packed = e2m1_pack8(w[j][0], w[j][1], w[j][2], w[j][3], e8m0_value(b));
      *reinterpret_cast<uint32_t*>(q + (int64_t)r * ldq + (k0 >> 1)) = packed;
    }
    if ((lane & 3) == 0 && valid[j]) scales[(int64_t)r * nblocks + c] = (uint8_t)b;
  }
}

// GEMM layout: a 256-thread workgroup takes U consecutive 1 KiB units
// (16-row strip s, K-step t; unit = s * 4G + t).  In each, lane L takes row
// r = L/16 and the 8 elements [8q, 8q+8) of block kb of that K-step, (kb, q)
// = ((L%16)/4, L%4): 16 consecutive lanes read one row's 256 contiguous
// bytes; the 4 lanes of a block combine their amax with two xor shuffles
// and store their 4 packed bytes into the block's 16-byte slot kb*16 + r.
// Units past the last K-step only fill scale padding.  All U loads are
// issued before the first is used (U > 1 keeps more bytes in flight per
// wave where there are many units).
template <int U>
__global__ __launch_bounds__(256) void quant_1x32_gemm_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int K, uint8_t* __restrict__ q,
    uint8_t* __restrict__ scales, int Kt, int G, int units) {
  const int L = threadIdx.x;
  const int r = L >> 4, kb = (L >> 2) & 3, sub = L & 3;
  uint32_t w[U][4];
  bool valid[U];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int unit = (int)blockIdx.x * U + j;
    const int tq = unit % (4 * G), s = unit / (4 * G);
    const int row = s * 16 + r, c = tq * 4 + kb;
    // the 4 lanes of a block are aligned and all valid or all invalid
    valid[j] = unit < units && row < M && c < (K >> 5);
    w[j][0] = w[j][1] = w[j][2] = w[j][3] = 0;
    if (valid[j]) {
      const int4 v = *reinterpret_cast<const int4*>(x + (int64_t)row * ldx + (int64_t)c * 32 + sub * 8);
      w[j][0] = (uint32_t)v.x, w[j][1] = (uint32_t)v.y, w[j][2] = (uint32_t)v.z, w[j][3] = (uint32_t)v.w;
    }
  }
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int unit = (int)blockIdx.x * U + j;
    if (unit >= units) break;  // uniform across the workgroup
    const int tq = unit % (4 * G), s = unit / (4 * G);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = absmax_pairs(m, w[j][i]);
    uint32_t amax = max(m & 0xFFFFu, m >> 16);
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
    const uint32_t b = valid[j] ? e8m0_of_amax_bits(amax) : kE8M0One;
    if (tq < Kt) {
      const uint32_t packed = valid[j] ? e2m1_pack8(w[j][0], w[j][1], w[j][2], w[j][3], e8m0_value(b)) : 0u;
      *reinterpret_cast<uint32_t*>(q + (int64_t)(s * Kt + tq) * 1024 + (kb * 16 + r) * 16 + sub * 4) = packed;
    }
    if (sub == 0) scales[(int64_t)(s * G + (tq >> 2)) * 256 + (kb * 16 + r) * 4 + (tq & 3)] = (uint8_t)b;
  }
}

hipError_t launch_quant_1x32(const void* x, int64_t M, int64_t K, int64_t ldx, void* q,
                             int64_t ldq, void* scales, int layout, hipStream_t stream) {
  const int Kt = (int)((K + 127) / 128);
  const int G = (Kt + 3) / 4;
  if (layout == 0) {
    const int segs = (int)((K + 511) / 512);
    const int64_t waves = M * segs;
    if (waves == 0) return hipSuccess;
    // Four segments per wave where there are many: measured on MI355X,
    // M = 8192 x K = 5120 / 14336 21.9 / 53.4 -> 18.5 / 49.0 us; decode sizes
    // keep one per wave (M = 16: 2.0 us against 3.0).
    if (waves >= 8192)
      quant_1x32_rowmajor_kernel<4><<<dim3((unsigned)((waves + 15) / 16)), 256, 0, stream>>>(
          (const uint16_t*)x, ldx, (int)M, (int)K, (uint8_t*)q, ldq, (uint8_t*)scales, segs);
    else
      quant_1x32_rowmajor_kernel<1><<<dim3((unsigned)((waves + 3) / 4)), 256, 0, stream>>>(
          (const uint16_t*)x, ldx, (int)M, (int)K, (uint8_t*)q, ldq, (uint8_t*)scales, segs);
  } else {
    const int64_t units = (M + 15) / 16 * (int64_t)(4 * G);
    if (units == 0) return hipSuccess;
    // Four units per workgroup where there are many: measured on MI355X,
    // M = 8192 x K = 5120 / 14336 21.2 / 55.6 -> 18.9 / 49.8 us, M = 2048 x
    // 5120 7.4 -> 6.8 us; with few units (decode sizes) one per workgroup
    // keeps the launch latency lowest (M = 16: 2.1 us against 2.8).
    if (units >= 4096)
      quant_1x32_gemm_kernel<4><<<dim3((unsigned)((units + 3) / 4)), 256, 0, stream>>>(
          (const uint16_t*)x, ldx, (int)M, (int)K, (uint8_t*)q, (uint8_t*)scales, Kt, G, (int)units);
    else
      quant_1x32_gemm_kernel<1><<<dim3((unsigned)units), 256, 0, stream>>>(
          (const uint16_t*)x, ldx, (int)M, (int)K, (uint8_t*)q, (uint8_t*)scales, Kt, G, (int)units);
  }
  return hipGetLastError();
}

}  // namespace mxfp4
