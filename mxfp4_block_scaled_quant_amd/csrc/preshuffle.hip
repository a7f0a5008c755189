// Load-time weight preshuffle into the library's gfx950 layout (and the same
// permutation for row-major quantised activations handed over by a producer).
//
// P1 §Modifications and P2 §2 (process_weights_after_loading) rearrange the
// FP4 weights and their E8M0 scales once after loading, into the order the
// FP4 GEMM reads.  The permutation here is this library's own: each 1 KiB
// unit is a 16-row x 128-K tile whose 16-byte slot kb*16 + r holds row r's
// whole 1x32 block kb, so one dwordx4 load per lane fills the operand of a
// 16x16x128 block-scaled MFMA; units of a 16-row strip run along K.  Scales
// go to the GEMM scale layout (one 256-byte tile = 16 rows x 4 K-steps x 4
// blocks; dword kb*16 + r, byte = K-step within the group).  Rows are padded
// to 16 with zero data; blocks are padded to the unit/tile with zero data
// and E8M0 1.0 scales (P2 §2: pad scales with 1.0, never the NaN 0xFF).
#include "mxfp4_device.h"
#include "mxfp4_launch.h"

namespace mxfp4 {

// One 16-byte slot of the preshuffled data; source row (b, n) at byte
// (b*N + n)*ldw.
__device__ __forceinline__ void preshuffle_data_slot(const uint8_t* __restrict__ w, int64_t ldw, int N, int K,
                                                     uint8_t* __restrict__ out, int Ns, int Kt, int64_t slot) {
  const int l = (int)(slot & 63);
  const int kb = l >> 4, r = l & 15;
  const int64_t unit = slot >> 6;
  const int t = (int)(unit % Kt);
  const int64_t bs = unit / Kt;
  const int s = (int)(bs % Ns);
  const int64_t b = bs / Ns;
  const int n = s * 16 + r, c = t * 4 + kb;
  int4 v = {0, 0, 0, 0};
  if (n < N && c < (K >> 5))
    v = *reinterpret_cast<const int4*>(w + ((b * N + n) * ldw + (int64_t)c * 16));
  *reinterpret_cast<int4*>(out + slot * 16) = v;
}

// One 4-byte scale dword of the GEMM scale layout (per batch); source row
// (b, n) at byte (b*N + n)*lds.
__device__ __forceinline__ void preshuffle_scale_dword(const uint8_t* __restrict__ ws, int64_t lds, int N, int K,
                                                       uint8_t* __restrict__ out, int Ns, int G, int64_t d) {
  const int l = (int)(d & 63);
  const int kb = l >> 4, r = l & 15;
  const int64_t unit = d >> 6;
  const int g = (int)(unit % G);
  const int64_t bs = unit / G;
  const int s = (int)(bs % Ns);
  const int64_t b = bs / Ns;
  const int n = s * 16 + r;
  const int nblocks = K >> 5;
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = (g * 4 + j) * 4 + kb;
    uint32_t byte = kE8M0One;
    if (n < N && c < nblocks) byte = ws[(b * N + n) * lds + c];
    word |= byte << (8 * j);
  }
  *reinterpret_cast<uint32_t*>(out + d * 4) = word;
}

// One thread per data slot, then one per scale dword: both permutations in
// one launch (a launch costs about 2 us of fixed time at decode sizes).
__global__ __launch_bounds__(256) void preshuffle_kernel(const uint8_t* __restrict__ w, int64_t ldw,
                                                         const uint8_t* __restrict__ ws, int64_t lds, int N, int K,
                                                         uint8_t* __restrict__ out, uint8_t* __restrict__ sout,
                                                         int Ns, int Kt, int G, int64_t slots, int64_t dwords) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < slots)
    preshuffle_data_slot(w, ldw, N, K, out, Ns, Kt, i);
  else if (i - slots < dwords)
    preshuffle_scale_dword(ws, lds, N, K, sout, Ns, G, i - slots);
}

// The scales alone.
__global__ __launch_bounds__(256) void preshuffle_scale_kernel(const uint8_t* __restrict__ ws, int64_t lds, int N,
                                                               int K, uint8_t* __restrict__ out, int Ns, int G,
                                                               int64_t total_dwords) {
  const int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (d < total_dwords) preshuffle_scale_dword(ws, lds, N, K, out, Ns, G, d);
}

hipError_t launch_preshuffle_strided(const void* w_fp4, int64_t ldw, const void* w_scales,
                                     int64_t lds, int64_t batch, int64_t N, int64_t K,
                                     void* w_out, void* ws_out, hipStream_t stream) {
  const int Ns = (int)((N + 15) / 16);
  const int Kt = (int)((K + 127) / 128);
  const int G = (Kt + 3) / 4;
  const int64_t slots = batch * Ns * (int64_t)Kt * 64;
  const int64_t dwords = batch * Ns * (int64_t)G * 64;
  if (w_fp4) {
    const int64_t total = slots + dwords;
    preshuffle_kernel<<<dim3((unsigned)((total + 255) / 256)), 256, 0, stream>>>(
        (const uint8_t*)w_fp4, ldw, (const uint8_t*)w_scales, lds, (int)N, (int)K, (uint8_t*)w_out,
        (uint8_t*)ws_out, Ns, Kt, G, slots, dwords);
    return hipGetLastError();
  }
  preshuffle_scale_kernel<<<dim3((unsigned)((dwords + 255) / 256)), 256, 0, stream>>>(
      (const uint8_t*)w_scales, lds, (int)N, (int)K, (uint8_t*)ws_out, Ns, G, dwords);
  return hipGetLastError();
}

hipError_t launch_preshuffle(const void* w_fp4, const void* w_scales, int64_t batch, int64_t N,
                             int64_t K, void* w_out, void* ws_out, hipStream_t stream) {
  return launch_preshuffle_strided(w_fp4, K / 2, w_scales, K / 32, batch, N, K, w_out, ws_out,
                                   stream);
}

}  // namespace mxfp4
