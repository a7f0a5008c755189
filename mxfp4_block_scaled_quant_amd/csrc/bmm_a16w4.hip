// A16WFP4 batched GEMM on gfx950: bf16 activations x MXFP4 weights.
//
// P3 §Motivation and §Modifications keep the MLA absorbed K/V projection
// weights in packed MXFP4 and run the per-head products on bf16
// activations, writing the V-up result batch-major.  Computed here:
//   out[b, m, n] = round(sum_k x[b, m, k] * dq(W)[b, n, k])
// with the activations used exactly (no activation quantisation), the
// weights dequantised exactly to bf16 in registers (an E2M1 value times a
// power of two always fits bf16), the bf16 16x16x32 MFMA with fp32
// accumulation, and one RNE rounding to bf16 (or fp32 out).  Output
// strides (sob, som) cover both [B, M, N] and batch-major [M, B, N].
//
// Organisation: a 256-thread workgroup owns one head and a 64 (m) x 128 (n)
// output tile; wave w takes 32 columns (2 MFMA tiles) over all 64 rows (4
// MFMA tiles).  The weight acts as the MFMA's A operand (16 output columns
// n per tile) and the activations as its B operand (16 rows m), so each lane
// ends with 4 consecutive n of one m and writes them as two bf16 pairs.
// Per 1x32 block c, lane (q = l/16, r = l%16) takes elements 8q..8q+7 of
// the block from both operands (a consistent pairing of the MFMA's K
// slots): 16 bytes of one activation row, and 4 bytes of weight row r from
// the preshuffled unit (slot (c%4)*16 + r, bytes 4q..4q+3) with its scale.
#include "mxfp4_device.h"
#include "mxfp4_launch.h"

namespace mxfp4 {

struct BmmArgs {
  const uint16_t* x;
  int64_t sxb, sxm;
  const uint8_t* w;
  const uint8_t* ws;
  void* out;
  int64_t sob, som;
  int out_f32;
  int M, N, K, Kt, G, Ns;
};

// Exact E2M1 code x 2^(sc-127) as fp32 (power-of-two product, no rounding;
// sc == 0 gives the fp32 subnormal 2^-127).
__device__ __forceinline__ float dq_fp4(uint32_t code, float scale) {
  const uint32_t mag = code & 7u, e = mag >> 1, mb = mag & 1u;
  const uint32_t bits = e == 0 ? (mb ? 0x3F000000u : 0u) : (((e + 126u) << 23) | (mb << 22));
  return __uint_as_float(bits | ((code & 8u) << 28)) * scale;
}

__device__ __forceinline__ v8bf dequant8(uint32_t word, uint32_t sc) {
  const float scale = __uint_as_float(sc == 0 ? 0x00400000u : (sc << 23));
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = __float_as_uint(dq_fp4((word >> (8 * i)) & 0xFu, scale)) >> 16;
    const uint32_t hi = __float_as_uint(dq_fp4((word >> (8 * i + 4)) & 0xFu, scale)) >> 16;
    h[i] = lo | (hi << 16);
  }
  return __builtin_bit_cast(v8bf, (int4){(int)h[0], (int)h[1], (int)h[2], (int)h[3]});
}

template <int MTW, int NTW>
__global__ __launch_bounds__(256) void bmm_a16w4_kernel(BmmArgs p) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int m0 = blockIdx.x * (MTW * 16);
  const int n0 = (blockIdx.y * 4 + wv) * (NTW * 16);
  if (n0 >= p.N) return;
  const int q = lane >> 4, r = lane & 15;
  const int nblocks = p.K >> 5;

  const int rows = min(MTW * 16, p.M - m0);
  const auto rx = make_rsrc(p.x + b * p.sxb + (int64_t)m0 * p.sxm,
                            (uint32_t)(((int64_t)(rows - 1) * p.sxm + p.K) * 2));
  const auto rw = make_rsrc(p.w + (int64_t)b * p.Ns * p.Kt * 1024, (uint32_t)p.Ns * p.Kt * 1024u);
  const auto rs = make_rsrc(p.ws + (int64_t)b * p.Ns * p.G * 256, (uint32_t)p.Ns * p.G * 256u);

  v4f acc[NTW][MTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int i = 0; i < MTW; ++i) acc[j][i] = (v4f){0.f, 0.f, 0.f, 0.f};

  for (int c = 0; c < nblocks; ++c) {
    const int t = c >> 2, kb = c & 3, g = t >> 2, jsel = t & 3;
    int4 xf[MTW];
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int m = i * 16 + r;
      const uint32_t off = m < rows ? (uint32_t)(((int64_t)m * p.sxm + c * 32 + q * 8) * 2) : kOOB;
      xf[i] = buf_load16(rx, off);
    }
    v8bf wf[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int s = (n0 >> 4) + j;
      const bool ok = s < p.Ns;
      const uint32_t word =
          buf_load4(rw, ok ? (uint32_t)((s * p.Kt + t) * 1024 + (kb * 16 + r) * 16 + q * 4) : kOOB);
      const uint32_t sw =
          buf_load4(rs, ok ? (uint32_t)((s * p.G + g) * 256 + (kb * 16 + r) * 4) : kOOB);
      wf[j] = dequant8(word, (sw >> (8 * jsel)) & 0xFFu);
    }
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int i = 0; i < MTW; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], __builtin_bit_cast(v8bf, xf[i]),
                                                            acc[j][i], 0, 0, 0);
  }

  // Lane l, register e of tile (j, i): n = n0 + 16j + 4(l/16) + e, m = m0 + 16i + l%16.
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int m = m0 + i * 16 + r;
      const int n = n0 + j * 16 + 4 * q;
      if (m >= p.M) continue;
      const int64_t base = (int64_t)b * p.sob + (int64_t)m * p.som + n;
      if (p.out_f32) {
        float* o = reinterpret_cast<float*>(p.out) + base;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < p.N) o[e] = acc[j][i][e];
      } else {
        uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + base;
        if (n + 3 < p.N) {
          const uint32_t lo = f32_to_bf16_rne(acc[j][i][0]) | ((uint32_t)f32_to_bf16_rne(acc[j][i][1]) << 16);
          const uint32_t hi = f32_to_bf16_rne(acc[j][i][2]) | ((uint32_t)f32_to_bf16_rne(acc[j][i][3]) << 16);
          reinterpret_cast<uint32_t*>(o)[0] = lo;
          reinterpret_cast<uint32_t*>(o)[1] = hi;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < p.N) o[e] = f32_to_bf16_rne(acc[j][i][e]);
        }
      }
    }
}

hipError_t launch_bmm_a16w4(const void* x, int64_t sxb, int64_t sxm, const void* w,
                            const void* ws, void* out, int64_t sob, int64_t som, int out_f32,
                            int64_t B, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  BmmArgs p;
  p.x = (const uint16_t*)x;
  p.sxb = sxb;
  p.sxm = sxm;
  p.w = (const uint8_t*)w;
  p.ws = (const uint8_t*)ws;
  p.out = out;
  p.sob = sob;
  p.som = som;
  p.out_f32 = out_f32;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.Kt = (int)((K + 127) / 128);
  p.G = (p.Kt + 3) / 4;
  p.Ns = (int)((N + 15) / 16);
  constexpr int MTW = 4, NTW = 2;
  const dim3 grid((unsigned)((M + MTW * 16 - 1) / (MTW * 16)),
                  (unsigned)((N + 4 * NTW * 16 - 1) / (4 * NTW * 16)), (unsigned)B);
  bmm_a16w4_kernel<MTW, NTW><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace mxfp4
