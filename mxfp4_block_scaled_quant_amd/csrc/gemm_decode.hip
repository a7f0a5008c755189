// W4A4 block-scaled FP4 GEMM for small M (decode, M <= 64) on gfx950.
//
// Computes out[m, n] = round(sum_k dq(A)[m,k] dq(W)[n,k] + bias[n]) (P2 §2:
// quantised activations times the preshuffled [N, K] weight in the NT form
// of a linear layer, bias added after; P1 §Accuracy Tests: equal to the
// dequantised reference).  At M <= 64 the product is bound by streaming the
// weights from HBM, so the kernel is organised around that stream:
//
//  * a workgroup owns NS 16-row weight strips over the whole K; its KW waves
//    split K into contiguous runs of 128-wide K-steps (intra-workgroup
//    split-K), so no partial sums leave the chip;
//  * per K-step a wave issues one 16-byte load per lane for each strip (a
//    whole 1 KiB preshuffled unit, fully coalesced) and one per 16-row
//    activation tile (row-major packed FP4, masked to zero past M and past
//    K), plus the matching scale dwords, for UNROLL steps before it issues
//    the MFMAs, to keep several KiB in flight per wave;
//  * block scales are applied by the MFMA itself (v_mfma_scale 16x16x128,
//    both operands E2M1), accumulation in fp32;
//  * the KW partial tiles are summed through LDS in a fixed order (run to
//    run identical results), the bias is added in fp32 and the result is
//    rounded once to bf16 (or stored as fp32).
#include "mxfp4_device.h"
#include "mxfp4_launch.h"

namespace mxfp4 {

template <int MT, int NS, int KW, int UNROLL>
__global__ __launch_bounds__(64 * KW) void gemm_decode_kernel(GemmArgs p) {
  __shared__ v4f red[KW][MT * NS][64];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int s0 = blockIdx.x * NS;
  const int nblocks = p.K >> 5;

  // Contiguous run of K-steps for this wave.
  const int per = p.Kt / KW, rem = p.Kt % KW;
  const int t0 = wv * per + min(wv, rem);
  const int t1 = t0 + per + (wv < rem ? 1 : 0);

  const uint32_t a_bytes = (uint32_t)min<int64_t>((int64_t)p.M * p.lda, 0x7FFFFFFF);
  const auto ra = make_rsrc(p.a, a_bytes);
  const auto rw = make_rsrc(p.w, (uint32_t)p.Ns * p.Kt * 1024u);
  const auto ras = make_rsrc(p.as, (uint32_t)((p.M + 15) / 16) * p.G * 256u);
  const auto rws = make_rsrc(p.ws, (uint32_t)p.Ns * p.G * 256u);

  const int kb = lane >> 4, rl = lane & 15;
  v4f acc[MT][NS];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  for (int tb = t0; tb < t1; tb += UNROLL) {
    int4 af[UNROLL][MT], bf[UNROLL][NS];
    uint32_t sa[UNROLL][MT], sb[UNROLL][NS];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int t = tb + u;
      const bool tv = t < t1;
      const int c = t * 4 + kb;
      const int g = t >> 2;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int row = i * 16 + rl;
        const uint32_t off = (tv && row < p.M && c < nblocks)
                                 ? (uint32_t)(row * p.lda + t * 64 + kb * 16)
                                 : kOOB;
        af[u][i] = buf_load16(ra, off);
        sa[u][i] = buf_load4(ras, tv ? (uint32_t)((i * p.G + g) * 256 + lane * 4) : kOOB);
      }
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int s = s0 + j;
        const bool ok = tv && s < p.Ns;
        bf[u][j] = buf_load16(rw, ok ? (uint32_t)((s * p.Kt + t) * 1024 + lane * 16) : kOOB);
        sb[u][j] = buf_load4(rws, ok ? (uint32_t)((s * p.G + g) * 256 + lane * 4) : kOOB);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int sh = ((tb + u) & 3) * 8;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j)
          acc[i][j] = mfma_fp4<0, 0>(af[u][i], bf[u][j], sa[u][i] >> sh, sb[u][j] >> sh, acc[i][j]);
    }
  }

#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) red[wv][i * NS + j][lane] = acc[i][j];
  __syncthreads();

  // Ordered sum over the KW waves; thread -> (tile, lane, register) with the
  // lane fastest so 16 consecutive threads write 16 consecutive columns.
  constexpr int TOTAL = MT * NS * 64 * 4;
  for (int idx = threadIdx.x; idx < TOTAL; idx += 64 * KW) {
    const int l = idx & 63;
    const int reg = (idx >> 6) & 3;
    const int tile = idx >> 8;
    const int i = tile / NS, j = tile % NS;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < KW; ++w) v += red[w][tile][l][reg];
    const int m = i * 16 + 4 * (l >> 4) + reg;
    const int n = (s0 + j) * 16 + (l & 15);
    if (m < p.M && n < p.N) {
      if (p.bias) v += bf16_to_f32(p.bias[n]);
      if (p.out_f32)
        reinterpret_cast<float*>(p.out)[(int64_t)m * p.ldo + n] = v;
      else
        reinterpret_cast<uint16_t*>(p.out)[(int64_t)m * p.ldo + n] = f32_to_bf16_rne(v);
    }
  }
}

template <int MT, int NS, int KW>
static hipError_t launch_decode_t(const GemmArgs& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.Ns + NS - 1) / NS));
  gemm_decode_kernel<MT, NS, KW, 4><<<grid, 64 * KW, 0, stream>>>(p);
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_decode_mt(const GemmArgs& p, hipStream_t stream) {
  // Enough waves per strip that each runs ~5 K-steps; two strips per
  // workgroup once there are plenty of strips.
  const int kw_want = (p.Kt + 4) / 5;
  const bool two = p.Ns >= 2048;
  if (kw_want >= 12) return two ? launch_decode_t<MT, 2, 16>(p, stream) : launch_decode_t<MT, 1, 16>(p, stream);
  if (kw_want >= 6) return two ? launch_decode_t<MT, 2, 8>(p, stream) : launch_decode_t<MT, 1, 8>(p, stream);
  if (kw_want >= 3) return two ? launch_decode_t<MT, 2, 4>(p, stream) : launch_decode_t<MT, 1, 4>(p, stream);
  return two ? launch_decode_t<MT, 2, 1>(p, stream) : launch_decode_t<MT, 1, 1>(p, stream);
}

hipError_t launch_gemm_decode(const GemmArgs& p, hipStream_t stream) {
  const int mt = (p.M + 15) / 16;
  switch (mt) {
    case 1: return launch_decode_mt<1>(p, stream);
    case 2: return launch_decode_mt<2>(p, stream);
    case 3: return launch_decode_mt<3>(p, stream);
    default: return launch_decode_mt<4>(p, stream);
  }
}

}  // namespace mxfp4
