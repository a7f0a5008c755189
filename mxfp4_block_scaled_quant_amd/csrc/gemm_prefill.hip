// W4A4 block-scaled FP4 GEMM for large M (prefill) on gfx950.
//
// Same operation as the decode kernel (P2 §2: quantised activations times
// the preshuffled [N, K] weight, NT form, bias after; P1 §Accuracy Tests:
// equal to the dequantised reference), organised for the MFMA roofline:
//
//  * a 512-thread workgroup computes a 256 x 256 output tile; its 8 waves
//    form a 2 (M) x 4 (N) grid of 128 x 64 wave tiles, each 8 x 4 MFMA
//    tiles of 16 x 16 held in 32 fp32 accumulators per lane;
//  * operands stream through LDS in stages of two 128-wide K-steps (64 KiB
//    per stage, two stages in flight): each 1 KiB MFMA operand fragment is
//    fetched by one buffer_load_dwordx4 ... lds per wave (global -> LDS with
//    no register staging), so LDS holds fragments in exactly the lane order
//    the MFMA consumes and every ds_read_b128 is conflict free;
//  * activation and weight fragments are whole 1 KiB units of the GEMM
//    layouts (padding already zero); tiles past the last 16-row strip read
//    zeros through out-of-range buffer offsets;
//  * block scales: one dword per lane per 16-row tile per 4 K-steps, read
//    straight into registers; the op_sel byte selector of the scaled MFMA
//    walks the 4 K-steps, so the K loop is unrolled by 4 (two stages);
//  * epilogue: bias in fp32, one RNE rounding to bf16 (or fp32 out).
#include "mxfp4_device.h"
#include "mxfp4_launch.h"

namespace mxfp4 {

namespace {

constexpr int kBM = 256, kBN = 256;
constexpr int kFragsA = 2 * (kBM / 16);     // 2 K-steps x 16 row tiles
constexpr int kFragsB = 2 * (kBN / 16);     // 2 K-steps x 16 strips
constexpr int kFrags = kFragsA + kFragsB;   // 64 fragments of 1 KiB per stage

typedef __attribute__((address_space(3))) void* lds_ptr_t;

struct TileCtx {
  __amdgpu_buffer_rsrc_t ra, rw, ras, rws;
  int Kt, G, mstrips, strips;  // 16-row activation tiles / weight strips inside this tile
};

// Issue the global->LDS loads of one stage (K-steps 2*st, 2*st+1).
__device__ __forceinline__ void issue_stage(const TileCtx& c, int4 (*buf)[64], int st, int wv, int lane) {
#pragma unroll
  for (int q = 0; q < kFrags / 8; ++q) {
    const int f = wv * (kFrags / 8) + q;
    uint32_t off;
    __amdgpu_buffer_rsrc_t r;
    if (f < kFragsA) {
      const int u = f >> 4, i = f & 15;
      const int t = st * 2 + u;
      off = (t < c.Kt && i < c.mstrips) ? (uint32_t)((i * c.Kt + t) * 1024 + lane * 16) : kOOB;
      r = c.ra;
    } else {
      const int u = (f - kFragsA) >> 4, j = (f - kFragsA) & 15;
      const int t = st * 2 + u;
      off = (t < c.Kt && j < c.strips) ? (uint32_t)((j * c.Kt + t) * 1024 + lane * 16) : kOOB;
      r = c.rw;
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)&buf[f][0], 16, (int)off, 0, 0, 0);
  }
}

// Two K-steps from one LDS stage; op_sel bytes SEL and SEL+1.
template <int SEL>
__device__ __forceinline__ void compute_stage(int4 (*buf)[64], v4f (&acc)[8][4], const uint32_t (&sa)[8],
                                              const uint32_t (&sb)[4], int wm, int wn, int lane) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    int4 af[8], bf[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) af[i] = buf[u * 16 + wm * 8 + i][lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = buf[kFragsA + u * 16 + wn * 4 + j][lane];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (u == 0)
          acc[i][j] = mfma_fp4<SEL, SEL>(af[i], bf[j], sa[i], sb[j], acc[i][j]);
        else
          acc[i][j] = mfma_fp4<SEL + 1, SEL + 1>(af[i], bf[j], sa[i], sb[j], acc[i][j]);
      }
  }
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace

__global__ __launch_bounds__(512, 1) void gemm_prefill_kernel(GemmArgs p, int tiles_m) {
  __shared__ int4 smem[2][kFrags][64];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int wm = wv >> 2, wn = wv & 3;

  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * kBM;
  const int s0 = tn * (kBN / 16);

  TileCtx c;
  c.Kt = p.Kt;
  c.G = p.G;
  const int strips = min(kBN / 16, p.Ns - s0);
  c.strips = strips;
  const int mstrips = min(kBM / 16, ((p.M + 15) >> 4) - m0 / 16);
  c.mstrips = mstrips;
  c.ra = make_rsrc(p.a + (int64_t)(m0 / 16) * p.Kt * 1024, (uint32_t)mstrips * p.Kt * 1024u);
  c.rw = make_rsrc(p.w + (int64_t)s0 * p.Kt * 1024, (uint32_t)strips * p.Kt * 1024u);
  c.ras = make_rsrc(p.as + (int64_t)(m0 / 16) * p.G * 256, (uint32_t)mstrips * p.G * 256u);
  c.rws = make_rsrc(p.ws + (int64_t)s0 * p.G * 256, (uint32_t)strips * p.G * 256u);

  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  issue_stage(c, smem[0], 0, wv, lane);
  for (int g = 0; g < p.G; ++g) {
    uint32_t sa[8], sb[4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      sa[i] = buf_load4(c.ras, (uint32_t)(((wm * 8 + i) * c.G + g) * 256 + lane * 4));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sb[j] = buf_load4(c.rws, (uint32_t)(((wn * 4 + j) * c.G + g) * 256 + lane * 4));
    wait_vm_all();
    __syncthreads();
    issue_stage(c, smem[1], 2 * g + 1, wv, lane);
    compute_stage<0>(smem[0], acc, sa, sb, wm, wn, lane);
    wait_vm_all();
    __syncthreads();
    if (g + 1 < p.G) issue_stage(c, smem[0], 2 * g + 2, wv, lane);
    compute_stage<2>(smem[1], acc, sa, sb, wm, wn, lane);
  }

  // Epilogue: lane l, register r of tile (i, j) is row 4*(l/16)+r, column l%16.
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = (s0 + wn * 4 + j) * 16 + (lane & 15);
      const float bv = (p.bias && n < p.N) ? bf16_to_f32(p.bias[n]) : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 128 + i * 16 + 4 * (lane >> 4) + r;
        if (m < p.M && n < p.N) {
          const float v = acc[i][j][r] + bv;
          if (p.out_f32)
            reinterpret_cast<float*>(p.out)[(int64_t)m * p.ldo + n] = v;
          else
            reinterpret_cast<uint16_t*>(p.out)[(int64_t)m * p.ldo + n] = f32_to_bf16_rne(v);
        }
      }
    }
}

hipError_t launch_gemm_prefill(const GemmArgs& p, hipStream_t stream) {
  const int tiles_m = (p.M + kBM - 1) / kBM;
  const int tiles_n = (p.Ns * 16 + kBN - 1) / kBN;
  gemm_prefill_kernel<<<dim3((unsigned)(tiles_m * tiles_n)), 512, 0, stream>>>(p, tiles_m);
  return hipGetLastError();
}

}  // namespace mxfp4
