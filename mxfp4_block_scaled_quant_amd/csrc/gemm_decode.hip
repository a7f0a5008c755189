// W4A4 block-scaled FP4 GEMM for small M (decode, M <= 64) on gfx950.
//
// Computes out[m, n] = round(sum_k dq(A)[m,k] dq(W)[n,k] + bias[n]) (P2 §2:
// quantised activations times the preshuffled [N, K] weight in the NT form
// of a linear layer, bias added after; P1 §Accuracy Tests: equal to the
// dequantised reference).  At M <= 64 the product is bound by streaming the
// weights from HBM, so the kernel is organised around that stream:
//
//  * a workgroup owns NS 16-row weight strips over the whole K; its KW waves
//    split the K-step groups (4 K-steps of 128 = one scale dword) evenly
//    (intra-workgroup split-K), so no partial sums leave the chip;
//  * a wave issues every load of a round of GPR groups at once -- per K-step
//    one 16-byte load per lane for each strip (a whole preshuffled 1 KiB
//    unit, non-temporal: it is read exactly once) and for each 16-row
//    activation tile (a 1 KiB unit of the GEMM activation layout, shared by
//    all workgroups through L2), plus one scale dword per tile and group --
//    and only then waits, so typically the whole K-run of a wave costs one
//    memory round trip;
//  * block scales are applied by the MFMA itself (v_mfma_scale 16x16x128,
//    both operands E2M1, op_sel picking the K-step's byte), fp32 accumulate;
//  * the KW partial tiles are summed through LDS in a fixed order (results
//    identical run to run; every thread's reads of the KW partials in flight
//    at once), the bias is added in fp32 and the result is rounded once to
//    bf16 (or stored as fp32).
#include "mxfp4_device.h"
#include "mxfp4_launch.h"

namespace mxfp4 {

namespace {

constexpr int kAuxNT = 2;  // cache policy bits of a buffer load: non-temporal

template <int SEL>
__device__ __forceinline__ v4f mfma_sel(const int4& a, const int4& b, uint32_t sa, uint32_t sb, v4f acc) {
  return mfma_fp4<SEL, SEL>(a, b, sa, sb, acc);
}

}  // namespace

// Sums the KW waves' partial tiles through LDS in a fixed order (wave 0
// first, so results are identical run to run), adds the bias in fp32 and
// stores the tile rows below M: bf16 rounded once to nearest even, or fp32.
// The partials sit at [tile][register][wave][lane] as fp32 in an area sized
// for MAXW waves, so a thread reads its value of every wave as one 4-byte
// load per wave, all in flight at once (one LDS round trip; slots past KW
// are read and ignored), and consecutive lanes read consecutive words.
// Measured on MI355X against per-output loops over the waves (one LDS round
// trip per wave, 4-way bank conflicts): M = 64 decode shapes 8-12% faster,
// M <= 16 within 1%.
// The bias of a thread's output columns in reduce_store / reduce_store_fp4
// (column (s0 + j) * 16 + lane % 16 of strip j) as raw bf16 bits, 0 past N
// or without a bias: loaded with the weights, so the reduction does not
// wait a memory round trip for them (measured on MI355X: +0.65 us per
// launch at N = 34816 with the load in the reduction, against the same
// launch without bias).  A buffer load, so that no branch guards it (a
// guarded load gets its wait at the end of the branch, before the weight
// loads are even issued).
template <int NS>
__device__ __forceinline__ void load_bias(const GemmArgs& p, int s0, uint32_t (&bb)[NS]) {
  const int lane = threadIdx.x & 63;
  const auto rb = make_rsrc(p.bias, p.bias ? (uint32_t)p.N * 2u : 0u);
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const uint32_t n = (uint32_t)((s0 + j) * 16 + (lane & 15));
    bb[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, n < (uint32_t)p.N ? n * 2u : kOOB, 0, 0);
  }
}

template <int MT, int NS, int MAXW>
__device__ __forceinline__ void reduce_store(float* red, const v4f (&acc)[MT][NS], const GemmArgs& p, int s0,
                                             const uint32_t (&bb)[NS]) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int KW = blockDim.x >> 6;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(((i * NS + j) * 4 + r) * MAXW + wv) * 64 + lane] = acc[i][j][r];
  __syncthreads();
  for (int sl = wv; sl < MT * NS * 4; sl += KW) {
    const int tile = sl >> 2, r = sl & 3;
    const int i = tile / NS, j = tile % NS;
    const int m = i * 16 + 4 * (lane >> 4) + r;
    const int n = (s0 + j) * 16 + (lane & 15);
    const float* src = red + sl * MAXW * 64 + lane;
    float part[MAXW];
#pragma unroll
    for (int w = 0; w < MAXW; ++w) part[w] = src[w * 64];
    float v = part[0];
#pragma unroll
    for (int w = 1; w < MAXW; ++w)
      if (w < KW) v += part[w];
    if (m < p.M && n < p.N) {
      if (p.bias) v += bf16_to_f32((uint16_t)bb[j]);
      if (p.out_f32)
        reinterpret_cast<float*>(p.out)[(int64_t)m * p.ldo + n] = v;
      else
        reinterpret_cast<uint16_t*>(p.out)[(int64_t)m * p.ldo + n] = f32_to_bf16_rne(v);
    }
  }
}

// LDS bytes of reduce_store's partials.
template <int MT, int NS, int MAXW>
constexpr size_t reduce_lds_bytes() {
  return (size_t)MT * NS * 4 * MAXW * 64 * sizeof(float);
}

// Where the activations come from.  Row-major: as a producer hands them over
// (packed FP4 [M, K/2], row stride lda bytes; scales [M, K/32], row stride
// lds bytes), gathered into the same MFMA operands: lane l's 16 bytes of row
// r, block kb are one contiguous piece of the row, and its scale dword is
// assembled from the 4 K-steps' bytes (one 16-byte load of the group's
// scales when the rows allow it, else four byte loads).  Same values, same
// MFMAs.  The scale-load form is a template choice, not a branch: a load
// inside a branch gets its wait at the branch's end, which held every load
// issued before it (the weights) up before the activations were even
// requested (measured: 2-3 us per launch at N = 34816).
constexpr int kASrcGemm = 0;   // quantised, GEMM layouts
constexpr int kASrcRow16 = 1;  // quantised, row-major; 16-byte scale loads
constexpr int kASrcRow8 = 2;   // quantised, row-major; byte scale loads
constexpr int kASrcBf16 = 3;   // bf16 rows, quantised in the kernel (persistent form, one row tile)
// MXFP4 output (two strips = 32 columns per workgroup, one 1x32 block per
// row): the summed rows are rounded to bf16 into an LDS staging area, then
// 4 threads per row each take 8 of the block's values, combine the block's
// amax, and encode it like the quantisation kernels (scale byte from the
// amax's exponent, scaled conversion): 4 code bytes per thread, the scale
// byte from the first.  Bitwise the bf16 output quantised afterwards.
template <int MT>
__device__ __forceinline__ void reduce_store_fp4(v4f* red, const v4f (&acc)[MT][2], const GemmArgs& p, int s0,
                                                 const uint32_t (&bb)[2]) {
  constexpr int NS = 2;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int KW = blockDim.x >> 6;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) red[(wv * MT * NS + i * NS + j) * 64 + lane] = acc[i][j];
  __syncthreads();
  uint16_t* stg = reinterpret_cast<uint16_t*>(red + KW * MT * NS * 64);  // [MT*16][32] bf16
  constexpr int TOTAL = MT * NS * 64 * 4;
  for (int idx = threadIdx.x; idx < TOTAL; idx += blockDim.x) {
    const int l = idx & 63;
    const int reg = (idx >> 6) & 3;
    const int tile = idx >> 8;
    const int i = tile / NS, j = tile % NS;
    float v = 0.f;
    for (int w = 0; w < KW; ++w) v += red[(w * MT * NS + tile) * 64 + l][reg];
    const int m = i * 16 + 4 * (l >> 4) + reg;
    const int n = (s0 + j) * 16 + (l & 15);
    if (p.bias && n < p.N) v += bf16_to_f32((uint16_t)bb[j]);
    stg[m * 32 + j * 16 + (l & 15)] = f32_to_bf16_rne(v);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < MT * 64; idx += blockDim.x) {
    const int m = idx >> 2, piece = idx & 3;
    const int4 v = *reinterpret_cast<const int4*>(stg + m * 32 + piece * 8);
    const uint32_t b = e8m0_of_amax_bits(quad_amax_bits((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w));
    const uint32_t code = e2m1_pack8((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w, e8m0_value(b));
    if (m < p.M && s0 * 16 < p.N) {
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(p.out) + (int64_t)m * p.ldo + s0 * 8 + piece * 4) = code;
      if (piece == 0) p.out_scales[(int64_t)m * p.ldos + (s0 >> 1)] = (uint8_t)b;
    }
  }
}

template <int MT, int NS, int GPR, int MAXW, int ASRC, bool HOLDA>
__global__ __launch_bounds__(64 * MAXW) void gemm_decode_kernel(GemmArgs p, int gpw) {
  constexpr bool AROW = ASRC == kASrcRow16 || ASRC == kASrcRow8;
  static_assert(ASRC != kASrcBf16, "bf16 activations: the persistent form only");
  extern __shared__ v4f red[];  // reduce_store's partials (or reduce_store_fp4's)
  constexpr int STEPS = 4 * GPR;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int s0 = blockIdx.x * NS;
  const int nblk = p.K >> 5;

  const auto ra = make_rsrc(p.a, AROW ? (uint32_t)(p.M - 1) * p.lda + (uint32_t)(p.K >> 1)
                                      : (uint32_t)MT * p.Kt * 1024u);
  const auto rw = make_rsrc(p.w, (uint32_t)p.Ns * p.Kt * 1024u);
  const auto ras = make_rsrc(p.as, AROW ? (uint32_t)(p.M - 1) * p.lds + (uint32_t)nblk
                                        : (uint32_t)MT * p.G * 256u);
  const auto rws = make_rsrc(p.ws, (uint32_t)p.Ns * p.G * 256u);

  v4f acc[MT][NS];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  uint32_t bb[NS];

  const int g_begin = wv * gpw;
  const int g_end = min(g_begin + gpw, p.G);
  for (int gr = g_begin; gr < g_end; gr += GPR) {
    int4 bf[STEPS][NS], af[STEPS][MT];
    uint32_t sa[GPR][MT], sb[GPR][NS];
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      const int t = gr * 4 + u;
      const bool tv = (gr + u / 4) < g_end && t < p.Kt;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int s = s0 + j;
        const uint32_t off = (tv && s < p.Ns) ? (uint32_t)((s * p.Kt + t) * 1024 + lane * 16) : kOOB;
        bf[u][j] = __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, kAuxNT));
      }
    }
#pragma unroll
    for (int q = 0; q < GPR; ++q) {
      const int g = gr + q;
      const bool gv = g < g_end;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int s = s0 + j;
        sb[q][j] = buf_load4(rws, (gv && s < p.Ns) ? (uint32_t)((s * p.G + g) * 256 + lane * 4) : kOOB);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if constexpr (AROW) {
          const int row = i * 16 + (lane & 15);
          const bool ok = gv && row < p.M;
          uint32_t word = 0;
          if constexpr (ASRC == kASrcRow16) {
            // the group's 16 scale bytes of the row in one load (whole
            // groups: K % 512 == 0); this lane's block kb is byte kb of
            // each dword
            const int4 v = buf_load16(ras, ok ? (uint32_t)row * p.lds + (uint32_t)(g * 16) : kOOB);
            const uint32_t sh = (uint32_t)(lane >> 4) * 8u;
            word = ((uint32_t)v.x >> sh & 0xFFu) | ((uint32_t)v.y >> sh & 0xFFu) << 8 |
                   ((uint32_t)v.z >> sh & 0xFFu) << 16 | ((uint32_t)v.w >> sh & 0xFFu) << 24;
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int c = (g * 4 + j) * 4 + (lane >> 4);
              const uint32_t off = (ok && c < nblk) ? (uint32_t)row * p.lds + (uint32_t)c : kOOB;
              word |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(ras, off, 0, 0) << (8 * j);
            }
          }
          sa[q][i] = word;
        } else {
          sa[q][i] = buf_load4(ras, gv ? (uint32_t)((i * p.G + g) * 256 + lane * 4) : kOOB);
        }
      }
    }
    if constexpr (AROW && GPR == 1 && HOLDA) {
      // Row-major rows are a few KiB that every workgroup reads piece by
      // piece; requested alongside the weights they slowed the stream
      // (N = 14336, K = 5120, M = 1 / 4 / 16: 9.13 / 9.33 / 10.72 us),
      // requested once the weights and scales are in they do not (8.47 /
      // 8.67 / 9.93).  Where one row tile's waves have several groups the
      // launch holds nothing (K = 14336, N = 5120, M = 1 / 4 / 16: 9.31 /
      // 9.70 / 11.45 us with the wait, 9.03 / 9.30 / 11.09 without).
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      const int t = gr * 4 + u;
      const bool tv = (gr + u / 4) < g_end && t < p.Kt;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        // rows past M are zero padding: skip their bytes
        const int row = i * 16 + (lane & 15);
        const bool rv = row < p.M;
        if constexpr (AROW) {
          const bool cv = t * 4 + (lane >> 4) < nblk;
          af[u][i] = buf_load16(ra, (tv && rv && cv) ? (uint32_t)row * p.lda + (uint32_t)(t * 64 + (lane >> 4) * 16)
                                                       : kOOB);
        } else {
          af[u][i] = buf_load16(ra, (tv && rv) ? (uint32_t)((i * p.Kt + t) * 1024 + lane * 16) : kOOB);
        }
      }
    }
    // the bias after the operands (every round: no branch), so that the
    // MFMAs' waits do not include it; row-major operands leave no registers
    // for it (two strips and two groups per round spill), so there it is
    // loaded after the loop
    if constexpr (!AROW) load_bias<NS>(p, s0, bb);
    // Keep every load of the round ahead of the first wait: without this the
    // scheduler interleaves loads and MFMAs to save registers, which turns one
    // memory round trip into several.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < STEPS; ++u)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const uint32_t a_s = sa[u / 4][i], b_s = sb[u / 4][j];
          switch (u & 3) {
            case 0: acc[i][j] = mfma_sel<0>(af[u][i], bf[u][j], a_s, b_s, acc[i][j]); break;
            case 1: acc[i][j] = mfma_sel<1>(af[u][i], bf[u][j], a_s, b_s, acc[i][j]); break;
            case 2: acc[i][j] = mfma_sel<2>(af[u][i], bf[u][j], a_s, b_s, acc[i][j]); break;
            default: acc[i][j] = mfma_sel<3>(af[u][i], bf[u][j], a_s, b_s, acc[i][j]); break;
          }
        }
  }

  if constexpr (AROW) load_bias<NS>(p, s0, bb);
  if constexpr (NS == 2) {
    if (p.out_fp4) {
      reduce_store_fp4<MT>(red, acc, p, s0, bb);
      return;
    }
  }
  reduce_store<MT, NS, MAXW>(reinterpret_cast<float*>(red), acc, p, s0, bb);
}

// Persistent form, for more rows (each workgroup of the form above re-reads
// all M activation rows of its K-run, bytes that grow with M while the
// weights do not): one workgroup per compute unit walks the strips
// s = blockIdx.x + k * gridDim.x, one scale group (4 K-steps) per wave; a
// wave loads its group's activation operands and scales once (from any of
// the sources above; bf16 rows are encoded here), and they stay in
// registers; the weights of the next D strips (with their scales and the
// bias of their columns) are in flight in a ring of registers while the
// current strip's MFMAs and reduction run.  Per strip a
// wave's partial tile is the one gemm_decode_kernel forms with one group per
// wave, and reduce_store sums them in the same order: bitwise the same
// output.  The reduction areas alternate between strips, so the one barrier
// inside reduce_store also orders a strip's LDS reads before the writes two
// strips later.  With MXFP4 output (NS = 2) a step is a pair of adjacent
// strips (one 1x32 block per row), walked the same way, and
// reduce_store_fp4 reduces it in one area: its second barrier already
// orders every read of a step before the next step's writes.
template <int MT, int MAXW, int D, int ASRC, int NS = 1, int GPW = 1>
__global__ __launch_bounds__(64 * MAXW) void gemm_decode_persist_kernel(GemmArgs p) {
  constexpr bool AROW = ASRC == kASrcRow16 || ASRC == kASrcRow8;
  static_assert(GPW == 1 || (GPW == 2 && ASRC == kASrcGemm && NS == 1), "two groups per wave: GEMM layout, one strip");
  extern __shared__ v4f red[];
  constexpr size_t kRedFloats = reduce_lds_bytes<MT, 1, MAXW>() / sizeof(float);
  const int lane = threadIdx.x & 63;
  const int g = (threadIdx.x >> 6) * GPW;  // this wave's (first) scale group
  const bool gv = g < p.G;
  const int nblk = p.K >> 5;
  const auto ra = make_rsrc(p.a, AROW ? (uint32_t)(p.M - 1) * p.lda + (uint32_t)(p.K >> 1)
                                      : (uint32_t)MT * p.Kt * 1024u);
  const auto rw = make_rsrc(p.w, (uint32_t)p.Ns * p.Kt * 1024u);
  const auto ras = make_rsrc(p.as, AROW ? (uint32_t)(p.M - 1) * p.lds + (uint32_t)nblk
                                        : (uint32_t)MT * p.G * 256u);
  const auto rws = make_rsrc(p.ws, (uint32_t)p.Ns * p.G * 256u);

  // This wave's activation operands and scales, as gemm_decode_kernel reads
  // them (from the GEMM layout, or gathered from the row-major form); from
  // bf16 rows, each lane loads the whole 1x32 block its operand of K-step u
  // in row tile i holds (row 16i + lane % 16, block (4g + u) * 4 + lane / 16:
  // 64 bytes) and encodes it below: the first tile once the weight ring is
  // in flight, the others after it, two blocks at a time (registers).
  int4 af[GPW][4][MT];
  uint32_t sa[GPW][MT];
  int4 xv[ASRC == kASrcBf16 ? 4 : 1][4];
  [[maybe_unused]] const auto rx = make_rsrc(p.x, ASRC == kASrcBf16 ? p.x_bytes : 0u);
  [[maybe_unused]] auto load_x = [&](int i, int u, int4 (&v)[4]) {
    const int row = i * 16 + (lane & 15);
    const int kb = (g * 4 + u) * 4 + (lane >> 4);
    const bool ok = gv && row < p.M && kb < nblk;
    const uint32_t off = (uint32_t)row * (uint32_t)p.ldx * 2u + (uint32_t)kb * 64u;
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = buf_load16(rx, ok ? off + (uint32_t)c * 16u : kOOB);
  };
  if constexpr (ASRC == kASrcBf16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) load_x(0, u, xv[u]);
  }
#pragma unroll
  for (int q = 0; q < GPW; ++q)
#pragma unroll
  for (int u = 0; u < 4 && ASRC != kASrcBf16; ++u) {
    const int t = (g + q) * 4 + u;
    const bool tv = g + q < p.G && t < p.Kt;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      // rows past M are zero padding: skip their bytes
      const int row = i * 16 + (lane & 15);
      const bool rv = row < p.M;
      if constexpr (AROW) {
        const bool cv = t * 4 + (lane >> 4) < nblk;
        af[q][u][i] = buf_load16(ra, (tv && rv && cv) ? (uint32_t)row * p.lda + (uint32_t)(t * 64 + (lane >> 4) * 16)
                                                        : kOOB);
      } else {
        af[q][u][i] = buf_load16(ra, (tv && rv) ? (uint32_t)((i * p.Kt + t) * 1024 + lane * 16) : kOOB);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < GPW; ++q)
#pragma unroll
  for (int i = 0; i < MT && ASRC != kASrcBf16; ++i) {
    if constexpr (AROW) {
      const int row = i * 16 + (lane & 15);
      const bool ok = gv && row < p.M;
      uint32_t word = 0;
      if constexpr (ASRC == kASrcRow16) {
        const int4 v = buf_load16(ras, ok ? (uint32_t)row * p.lds + (uint32_t)(g * 16) : kOOB);
        const uint32_t sh = (uint32_t)(lane >> 4) * 8u;
        word = ((uint32_t)v.x >> sh & 0xFFu) | ((uint32_t)v.y >> sh & 0xFFu) << 8 |
               ((uint32_t)v.z >> sh & 0xFFu) << 16 | ((uint32_t)v.w >> sh & 0xFFu) << 24;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = (g * 4 + j) * 4 + (lane >> 4);
          const uint32_t off = (ok && c < nblk) ? (uint32_t)row * p.lds + (uint32_t)c : kOOB;
          word |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(ras, off, 0, 0) << (8 * j);
        }
      }
      sa[q][i] = word;
    } else {
      sa[q][i] = buf_load4(ras, g + q < p.G ? (uint32_t)((i * p.G + g + q) * 256 + lane * 4) : kOOB);
    }
  }

  static_assert(NS == 1 || (NS == 2 && ASRC == kASrcGemm), "pairs of strips: MXFP4 output from the GEMM layout");
  const int Nu = (p.Ns + NS - 1) / NS;  // steps of NS strips
  const int nk = (int)blockIdx.x < Nu ? (Nu - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  int4 bf[D][NS][GPW][4];
  uint32_t sb[D][NS][GPW], bb[D][NS];
  // Weights and scale of this wave's group of the k-th step's strips, and
  // the bias of their columns that the reduction gives this thread, into
  // ring slot `slot` (strips past the end load zeros).
  auto issue = [&](int k, int4 (&b)[NS][GPW][4], uint32_t (&sc)[NS][GPW], uint32_t (&bias)[NS]) {
    const int s0 = ((int)blockIdx.x + k * (int)gridDim.x) * NS;
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int q = 0; q < GPW; ++q) {
        const int s = s0 + j;
        const bool sv = k < nk && g + q < p.G && s < p.Ns;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t = (g + q) * 4 + u;
          const uint32_t off = (sv && t < p.Kt) ? (uint32_t)((s * p.Kt + t) * 1024 + lane * 16) : kOOB;
          b[j][q][u] = __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, kAuxNT));
        }
        sc[j][q] = buf_load4(rws, sv ? (uint32_t)((s * p.G + g + q) * 256 + lane * 4) : kOOB);
      }
    load_bias<NS>(p, k < nk ? s0 : p.Ns, bias);
  };
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, bf[d], sb[d], bb[d]);
  if constexpr (ASRC == kASrcBf16) {
    // the first tile's encoding waits for x only: the ring's loads stay in
    // flight (the later tiles' loads queue behind them)
    __builtin_amdgcn_sched_barrier(0);
    sa[0][0] = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t b;
      af[0][u][0] = quant_block32(xv[u], b);
      sa[0][0] |= b << (8 * u);
    }
#pragma unroll
    for (int i = 1; i < MT; ++i) {
      sa[0][i] = 0;
#pragma unroll
      for (int h = 0; h < 4; h += 2) {
        // one pair of blocks in registers at a time (no load hoisted above)
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        load_x(i, h, xv[0]);
        load_x(i, h + 1, xv[1]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          uint32_t b;
          af[0][h + u][i] = quant_block32(xv[u], b);
          sa[0][i] |= b << (8 * (h + u));
        }
      }
    }
  }

  for (int k0 = 0; k0 < nk; k0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int k = k0 + d;
      if (k >= nk) break;  // the same for every wave of the workgroup
      v4f acc[MT][NS];
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < GPW; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NS; ++j) {
              const int4& av = af[q][u][i];
              const int4& wv4 = bf[d][j][q][u];
              switch (u) {
                case 0: acc[i][j] = mfma_sel<0>(av, wv4, sa[q][i], sb[d][j][q], acc[i][j]); break;
                case 1: acc[i][j] = mfma_sel<1>(av, wv4, sa[q][i], sb[d][j][q], acc[i][j]); break;
                case 2: acc[i][j] = mfma_sel<2>(av, wv4, sa[q][i], sb[d][j][q], acc[i][j]); break;
                default: acc[i][j] = mfma_sel<3>(av, wv4, sa[q][i], sb[d][j][q], acc[i][j]); break;
              }
            }
      uint32_t bias[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) bias[j] = bb[d][j];
      issue(k + D, bf[d], sb[d], bb[d]);
      const int s0 = ((int)blockIdx.x + k * (int)gridDim.x) * NS;
      if constexpr (NS == 2)
        reduce_store_fp4<MT>(red, acc, p, s0, bias);
      else
        reduce_store<MT, 1, MAXW>(reinterpret_cast<float*>(red) + (size_t)(k & 1) * kRedFloats, acc, p, s0, bias);
    }
  }
  // the ring's last loads (past the end: zeros) land before the waves end
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The same product with the activation quantisation fused in, for M <= 4:
// the A operand is encoded from bf16 x in registers instead of being read
// from a quantised copy.  Per scale group (4 K-steps x 4 blocks = 16 blocks
// per row) a wave encodes all M x 16 blocks in one pass, one whole 1x32
// block per lane (lane l: row l/16, block l%16 of the group; 64 bytes
// loaded, amax, scale byte and 16 code bytes on its own, no cross-lane
// step), then moves each block to its MFMA lane (row r, K-step u, block kb
// -> lane kb*16 + r of step u) with one LDS-crossbar permute per dword;
// rows r >= M take zero codes.  The x loads are issued ahead of the weight
// stream and encoded while the weights are in flight.  Every workgroup
// encodes the x rows it needs; the K split, the per-wave MFMA order and the
// reduction are those of gemm_decode_kernel for one row tile, so the two
// paths give identical bits.
constexpr int kFusedRows = 4;

__device__ __forceinline__ uint32_t lane_permute(uint32_t src_lane, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(src_lane * 4u), (int)v);
}

template <int NS, int GPR, int MAXW>
__global__ __launch_bounds__(64 * MAXW) void linear_decode_kernel(GemmArgs p, int gpw) {
  extern __shared__ v4f red[];  // reduce_store's partials
  constexpr int STEPS = 4 * GPR;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int s0 = blockIdx.x * NS;

  const auto rx = make_rsrc(p.x, p.x_bytes);
  const auto rw = make_rsrc(p.w, (uint32_t)p.Ns * p.Kt * 1024u);
  const auto rws = make_rsrc(p.ws, (uint32_t)p.Ns * p.G * 256u);

  // Encoding pass: lane -> (row er, block ec of the group).  Rows past M and
  // blocks past K load nothing (zero data: scale byte 0, codes 0).
  const int er = lane >> 4, ec = lane & 15;
  const bool erv = er < p.M;
  const uint32_t xlane = (uint32_t)er * (uint32_t)p.ldx * 2u + (uint32_t)ec * 64u;
  const int nblk = p.K >> 5;
  // MFMA lane -> its row (lane % 16) and block kb (lane / 16); the encoding
  // lane of step u is row*16 + u*4 + kb.
  const int mr = lane & 15;
  const bool mrv = mr < p.M;
  const uint32_t src0 = (uint32_t)((mr & 3) * 16 + (lane >> 4));

  v4f acc[1][NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) acc[0][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  uint32_t bb[NS];
  load_bias<NS>(p, s0, bb);

  const int g_begin = wv * gpw;
  const int g_end = min(g_begin + gpw, p.G);
  for (int gr = g_begin; gr < g_end; gr += GPR) {
    int4 xv[GPR][4];
#pragma unroll
    for (int q = 0; q < GPR; ++q) {
      const int g = gr + q;
      const bool ok = erv && g < g_end && g * 16 + ec < nblk;
      const uint32_t off = xlane + (uint32_t)g * 1024u;
#pragma unroll
      for (int c = 0; c < 4; ++c) xv[q][c] = buf_load16(rx, ok ? off + c * 16 : kOOB);
    }
    int4 bf[STEPS][NS];
    uint32_t sb[GPR][NS];
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      const int t = gr * 4 + u;
      const bool tv = (gr + u / 4) < g_end && t < p.Kt;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int s = s0 + j;
        const uint32_t off = (tv && s < p.Ns) ? (uint32_t)((s * p.Kt + t) * 1024 + lane * 16) : kOOB;
        bf[u][j] = __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, kAuxNT));
      }
    }
#pragma unroll
    for (int q = 0; q < GPR; ++q) {
      const int g = gr + q;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int s = s0 + j;
        sb[q][j] = buf_load4(rws, (g < g_end && s < p.Ns) ? (uint32_t)((s * p.G + g) * 256 + lane * 4) : kOOB);
      }
    }
    // Loads stay ahead of the encoding, and the encoding ahead of the MFMAs
    // (which wait for the weights).
    __builtin_amdgcn_sched_barrier(0);
    int4 af[STEPS];
    uint32_t sa[STEPS];
#pragma unroll
    for (int q = 0; q < GPR; ++q) {
      uint32_t b;
      const int4 c = quant_block32(xv[q], b);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t src = src0 + (uint32_t)u * 4u;
        int4 a;
        a.x = (int)lane_permute(src, (uint32_t)c.x);
        a.y = (int)lane_permute(src, (uint32_t)c.y);
        a.z = (int)lane_permute(src, (uint32_t)c.z);
        a.w = (int)lane_permute(src, (uint32_t)c.w);
        const uint32_t sc = lane_permute(src, b);
        af[q * 4 + u] = mrv ? a : (int4){0, 0, 0, 0};
        sa[q * 4 + u] = sc;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < STEPS; ++u)
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        switch (u & 3) {
          case 0: acc[0][j] = mfma_fp4<0, 0>(af[u], bf[u][j], sa[u], sb[u / 4][j], acc[0][j]); break;
          case 1: acc[0][j] = mfma_fp4<0, 1>(af[u], bf[u][j], sa[u], sb[u / 4][j], acc[0][j]); break;
          case 2: acc[0][j] = mfma_fp4<0, 2>(af[u], bf[u][j], sa[u], sb[u / 4][j], acc[0][j]); break;
          default: acc[0][j] = mfma_fp4<0, 3>(af[u], bf[u][j], sa[u], sb[u / 4][j], acc[0][j]); break;
        }
      }
  }

  reduce_store<1, NS, MAXW>(reinterpret_cast<float*>(red), acc, p, s0, bb);
}

// HOLDA: row-major activation loads wait for the round's weights (one group
// per round only).
template <int MT, int NS, int GPR, int MAXW, bool HOLDA = true>
static hipError_t launch_decode_t(const GemmArgs& p, int kw, int gpw, hipStream_t stream) {
  const dim3 grid((unsigned)((p.Ns + NS - 1) / NS));
  // partial tiles (MXFP4 output: KW of them, plus the bf16 staging rows)
  const size_t lds = p.out_fp4 ? (size_t)kw * MT * NS * 64 * sizeof(v4f) + (size_t)MT * 16 * 32 * 2
                               : reduce_lds_bytes<MT, NS, MAXW>();
  // Row-major activations at one row tile are never loaded two groups per
  // round (launch_decode_mt gives them one: two strips of two groups spill
  // with the 16-byte scale loads), so those forms are not built.
  constexpr bool kRowForms = !(MT == 1 && GPR == 2);
  if constexpr (kRowForms) {
    if (p.a_rowmajor && p.scales_vec)
      gemm_decode_kernel<MT, NS, GPR, MAXW, kASrcRow16, HOLDA><<<grid, 64 * kw, lds, stream>>>(p, gpw);
    else if (p.a_rowmajor)
      gemm_decode_kernel<MT, NS, GPR, MAXW, kASrcRow8, HOLDA><<<grid, 64 * kw, lds, stream>>>(p, gpw);
    else
      gemm_decode_kernel<MT, NS, GPR, MAXW, kASrcGemm, false><<<grid, 64 * kw, lds, stream>>>(p, gpw);
  } else {
    if (p.a_rowmajor) return hipErrorInvalidValue;
    gemm_decode_kernel<MT, NS, GPR, MAXW, kASrcGemm, false><<<grid, 64 * kw, lds, stream>>>(p, gpw);
  }
  return hipGetLastError();
}

// Launch shape, from a sweep on MI355X: every wave owns whole scale groups
// (4 K-steps), the groups split evenly and loaded in rounds of two groups
// (one group beyond a single row tile, for registers); two strips per
// workgroup reuse each activation tile unless the strips are plentiful and
// M tiny.  At most 16 waves per workgroup at one row tile; 8 with two or
// three (at their register counts a compute unit holds several workgroups
// of a few waves, which beat fewer workgroups of more waves with fewer
// load rounds each); 12 with four (a compute unit holds 12 of those waves
// either way, and fewer load rounds per wave win).  Where every strip fits
// in one round of compute units (N/16 <= CUs) one strip per workgroup, so
// that all of them stream: two strips per workgroup left half of them idle
// (us, bias, two strips -> one; K = 5120, M = 1 / 16 / 64: N = 1024 4.41 /
// 4.70 / 6.60 -> 3.57 / 3.90 / 5.14, N = 4096 4.88 / 5.17 / 7.09 -> 4.16 /
// 4.52 / 5.93; K = 14336: N = 2048 8.10 / 8.83 / 13.82 -> 5.77 / 6.16 /
// 10.79, N = 4096 8.82 / 9.57 / 14.57 -> 7.58 / 7.91 / 11.76), and at one
// row tile with more than 16 groups at most 8 waves of four groups in one
// round (14 waves of two groups put one workgroup on a compute unit at a
// time); with more row tiles and 16-32 groups likewise at most 8 waves,
// loading four groups per round at two row tiles and two at three or four
// (K = 14336, N = 2048, M = 17 / 32 / 64: 7.46 / 8.22 / 10.79 -> 6.91 /
// 7.17 / 9.79 us; K = 8192: 5.35 / 5.79 / 7.09 -> 5.04 / 5.07 / 6.65; at
// K = 6144 no faster).  Just past one round (N = 5120, 320 strips) the
// two-strip workgroups stay: one strip in 7 waves took 10.96 us against
// 9.19 (M = 1, K = 14336; 64 compute units stream twice).
// Where the persistent form pays: many strips per compute unit, the more
// the fewer activation rows, and at least ten waves (groups) per workgroup.
// Measured on MI355X with a bf16 bias, rotated weight copies (us,
// streaming / persistent), K = 5120: N = 34816 (8.5 strips per CU): M = 8
// 17.0 / 18.1, M = 9 18.8 / 18.1, M = 12 18.9 / 18.1, M = 16 19.0 / 18.2,
// M = 32 22.5 / 19.9, M = 64 31.7 / 23.9; N = 28672 (7 per CU): M = 8 14.6 /
// 15.2, M = 9 16.8 / 15.2; N = 24576 (6 per CU): M = 16 13.1 / 13.6, M = 17
// 16.3 / 14.5, M = 64 21.0 / 17.8; N = 14336 (3.5 per CU): M = 48 11.5 /
// 12.3, M = 64 14.1 / 13.1; N = 8192: 10-19% slower at every M; with M <= 8
// 3-19% slower everywhere (the streaming form keeps more loads in flight per
// compute unit); with fewer waves too (K = 4096, N = 16384: 12-19% slower
// up to M = 48, 2% faster at 64).
static bool decode_persist_pays(int M, int Ns, int cus, int kw) {
  // (at four row tiles eight waves suffice on six strips per unit: K = 4096,
  // M = 64, N = 24576 / 32768 / 57344: 17.8 / 22.9 / 38.0 -> 16.2 / 19.7 /
  // 30.9 us)
  if (kw >= 8 && kw < 10 && M > 48) return Ns >= 6 * cus || (Ns > 2 * cus && Ns < 3 * cus);
  if (kw < 10 || M <= 8) return false;
  // (and from two row tiles between two and three strips per unit, where
  // two-strip workgroups leave some units four: N = 10240, K = 5120, M =
  // 20 / 32 / 40 / 64: 9.3 / 9.7 / 10.5 / 13.3 -> 9.0 / 9.1 / 10.1 / 10.8
  // us; N = 11264, K = 6144, M = 20 / 64: 10.8 / 14.6 -> 10.1 / 12.2; with
  // 8 waves (K = 4096) only at M = 64: 11.3 -> 9.8)
  if (M > 16 && Ns > 2 * cus && Ns < 3 * cus) return true;
  if (M > 48) return Ns >= 3 * cus;
  // (between four and five strips per unit, too: K = 5120, N = 18432, M =
  // 20 / 32 / 48: 13.6 / 14.2 / 15.7 -> 12.9 / 13.2 / 14.8 us)
  if (M > 16) return Ns > 4 * cus;
  return Ns >= 7 * cus;
}

// Row-major (prequantised) activations: every workgroup of the streaming form
// gathers its rows' 16-byte pieces afresh, so loading them once per wave pays
// sooner than from the GEMM layout.  Measured as above (us, streaming /
// persistent), K = 5120: N = 24576 (6 strips per CU): M = 1 14.4 / 13.4,
// M = 16 14.6 / 14.0, M = 17 17.7 / 14.9, M = 64 30.7 / 21.2; N = 34816:
// M = 1 19.3 / 17.8, M = 64 48.1 / 27.0; N = 14336 (3.5 per CU): M = 16
// 9.96 / 10.1, M = 17 10.5 / 10.9, M = 32 13.0 / 12.3, M = 64 20.4 / 16.6;
// N = 8192 (two per CU): 8-16% slower at every M; K = 4096 (eight waves),
// N = 16384 (four per CU): M = 17 9.8 / 10.3, M = 32 11.3 / 11.2, M = 33
// 14.2 / 12.0, M = 64 18.8 / 14.6.
static bool decode_persist_pays_rowmajor(int M, int Ns, int cus, int kw) {
  if (kw < 8) return false;
  if (M >= 32) return Ns >= 3 * cus;
  return kw >= 10 && Ns >= 6 * cus;
}

// MXFP4 output: the persistent form in steps of two strips pays with more
// than one row tile (measured, us, one-workgroup-per-two-strips form ->
// persistent, K = 5120: N = 34816, M = 64 37.28 -> 32.74; N = 24576, M = 32 /
// 64 19.03 / 24.48 -> 16.59 / 22.56; N = 14336, M = 64 16.40 -> 15.57), not
// with one (N = 34816, M = 16: 19.89 -> 21.62; its ring holds one step,
// as registers allow).
// (Steps of two strips are what the streaming form's workgroups hold, so
// the persistent walk evens nothing out there: the rule measured before
// the balance cases above.)
static bool decode_persist_fp4_pays(int M, int Ns, int cus, int kw) {
  if (M <= 16 || kw < 10) return false;
  return M > 48 ? Ns >= 3 * cus : Ns >= 6 * cus;
}

template <int MT, int MAXW>
static hipError_t launch_decode_persist(const GemmArgs& p, int kw, hipStream_t stream) {
  // strips in flight per wave, as registers allow at 12 waves (six at one
  // row tile measured no faster than four)
  constexpr int D = MT == 4 ? 3 : 4;
  const int grid = p.Ns < p.cus ? p.Ns : p.cus;
  const size_t lds = 2 * reduce_lds_bytes<MT, 1, MAXW>();
  if (p.a_rowmajor && p.scales_vec)
    gemm_decode_persist_kernel<MT, MAXW, D, kASrcRow16><<<grid, 64 * kw, lds, stream>>>(p);
  else if (p.a_rowmajor)
    gemm_decode_persist_kernel<MT, MAXW, D, kASrcRow8><<<grid, 64 * kw, lds, stream>>>(p);
  else
    gemm_decode_persist_kernel<MT, MAXW, D, kASrcGemm><<<grid, 64 * kw, lds, stream>>>(p);
  return hipGetLastError();
}

// The persistent form with two scale groups per wave (13-24 groups, one or
// two row tiles, GEMM-layout activations, bf16 / fp32 output), on at least
// five strips per compute unit.  Measured on MI355X (us, streaming ->
// persistent, N = 28672): K = 6656 / 7680 / 8704 / 10240 / 11264, M = 16:
// 21.5 / 23.4 / 26.7 / 30.2 / 29.6 -> 21.0 / 22.4 / 25.1 / 27.0 / 29.1;
// M = 32: 22.3 / 24.5 / 32.0 / 31.7 / 34.4 -> 20.6 / 22.6 / 27.0 / 29.6 /
// 31.6; K = 12288, M = 32: 36.5 -> 33.5.  Not at M <= 8 (K = 8192, N =
// 28672, M = 1 / 8: 20.1 / 20.6 -> 23.1 / 24.1), nor at M <= 16 with many
// strips per unit (N = 57344, K = 7168: 39.9 -> 41.6), nor at 16 groups
// below 25 rows, where the streaming form's 16 waves of one group do well
// (N = 28672, K = 8192, M = 16 / 24: 23.6 / 23.6 -> 24.5 / 24.0).
static bool decode_persist2_pays(int M, int Ns, int cus, int G) {
  // Two row tiles between two and three strips per unit, where two-strip
  // workgroups leave some units four strips and the persistent walk at most
  // three: K = 11008, M = 24, N = 10240 / 11264: 17.3 / 17.6 -> 14.8 / 15.2
  // us; K = 8192, N = 10240, M = 32: 13.3 -> 12.3; at exactly three (N =
  // 12288) only with 18 or more groups (K = 11008, M = 24: 18.0 -> 15.8;
  // K = 8192, M = 20: 13.07 -> 13.20); not at two (N = 8192, K = 8192: 8.9
  // -> 10.4) nor at 3.25-4 (N = 13312, K = 9216: 15.0 -> 15.9).
  if (M > 16)
    return (Ns > 2 * cus && (Ns < 3 * cus || (Ns == 3 * cus && G >= 18))) ||
           (Ns >= 5 * cus && (G != 16 || M > 24));
  if (M > 8) return Ns >= 5 * cus && Ns <= 8 * cus && G != 16;
  return false;
}

template <int MT>
static hipError_t launch_decode_persist2(const GemmArgs& p, hipStream_t stream) {
  const int kw = (p.G + 1) / 2;
  const int grid = p.Ns < p.cus ? p.Ns : p.cus;
  if (kw <= 8) {
    gemm_decode_persist_kernel<MT, 8, 2, kASrcGemm, 1, 2><<<grid, 64 * kw, 2 * reduce_lds_bytes<MT, 1, 8>(), stream>>>(p);
  } else {
    gemm_decode_persist_kernel<MT, 12, 1, kASrcGemm, 1, 2><<<grid, 64 * kw, 2 * reduce_lds_bytes<MT, 1, 12>(), stream>>>(p);
  }
  return hipGetLastError();
}

// MXFP4 output in the persistent form: steps of two strips (one 1x32
// block per row), one reduction area (two barriers per step).
template <int MT>
static hipError_t launch_decode_persist_fp4(const GemmArgs& p, int kw, hipStream_t stream) {
  constexpr int D = 1;  // steps in flight per wave (two strips each)
  const int Nu = (p.Ns + 1) / 2;
  const int grid = Nu < p.cus ? Nu : p.cus;
  const size_t lds = (size_t)kw * MT * 2 * 64 * sizeof(v4f) + (size_t)MT * 16 * 32 * 2;
  gemm_decode_persist_kernel<MT, 12, D, kASrcGemm, 2><<<grid, 64 * kw, lds, stream>>>(p);
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_decode_mt(const GemmArgs& p, hipStream_t stream) {
  constexpr int MAXW = MT == 1 ? 16 : MT == 4 ? 12 : 8;
  // (29-32 groups at 9-16 rows on many strips: three groups per wave in at
  // most 11 waves, as 16 waves of two leave a compute unit one workgroup at
  // a time — K = 16384, M = 16, N = 16384 / 24576 / 32768: 27.3 / 38.8 /
  // 50.2 -> 24.1 / 34.4 / 45.1 us; K = 15360, N = 16384: 23.3 -> 22.8)
  const bool three = MT == 1 && p.M > 8 && p.G > 28 && p.G <= 32 && p.Ns >= 4 * p.cus;
  const int gpw = three ? (p.G + 11) / 12 : (p.G + MAXW - 1) / MAXW;
  const int kw = (p.G + gpw - 1) / gpw;
  // persistent form: one group per wave, bf16 / fp32 output, activations in
  // the GEMM layout or row-major (path 7 of the test hook forces it where it
  // applies, 8 keeps the streaming form); the same K split as the streaming
  // form wherever that has one group per wave too, so the same bits (two or
  // three row tiles above 4096 of K give each streaming wave two groups, so
  // their sums differ in order)
  const bool persist_ok = p.G <= 12 && !p.out_fp4;
  const int ov = get_gemm_path_override();
  const bool persist =
      persist_ok && (ov == 7 || (ov != 8 && (p.a_rowmajor ? decode_persist_pays_rowmajor(p.M, p.Ns, p.cus, p.G)
                                                          : decode_persist_pays(p.M, p.Ns, p.cus, p.G))));
  if (persist) return launch_decode_persist<MT, 12>(p, p.G, stream);
  if constexpr (MT <= 2) {
    if (p.G > 12 && p.G <= 24 && !p.out_fp4 && !p.a_rowmajor &&
        (ov == 7 || (ov != 8 && decode_persist2_pays(p.M, p.Ns, p.cus, p.G))))
      return launch_decode_persist2<MT>(p, stream);
  }
  // MXFP4 output (GEMM-layout activations): the same form in steps of two
  // strips
  if (p.out_fp4 && !p.a_rowmajor && p.G <= 12 && (ov == 7 || (ov != 8 && decode_persist_fp4_pays(p.M, p.Ns, p.cus, p.G))))
    return launch_decode_persist_fp4<MT>(p, p.G, stream);
  // one strip per workgroup never with MXFP4 output (a workgroup encodes
  // whole 32-column blocks)
  const bool one_round = p.Ns <= p.cus && !p.out_fp4;
  // (and at K <= 2048 with one or four row tiles: N = 14336, K = 2048, M = 1
  // / 16 / 64: 5.24 / 5.53 / 10.36 -> 5.01 / 5.37 / 8.50 us; K = 1024, M = 64:
  // 11.56 -> 8.52; two and three row tiles, or K >= 3072, were slower)
  const bool small_k = p.G <= 4 && (MT == 1 || MT == 4);
  // (and at one row tile between two and three strips per compute unit:
  // two-strip workgroups leave some units four strips, one-strip ones at
  // most three — K = 8192, N = 10240 / 12288, M = 1: 11.33 / 11.89 -> 9.44 /
  // 10.27 us, M = 16: 11.81 / 12.38 -> 10.59 / 11.15; K = 5120, N = 10240,
  // M = 1 / 16: 7.93 / 8.66 -> 6.92 / 7.83.  Where both forms give each unit
  // the same number of strips two per workgroup share the activations:
  // N = 6144 and 14336 stay, 0.3-0.8 us faster at M = 16)
  // The same between four and four and a half strips per unit at 9-16 rows
  // (K = 5120 / 8192 / 14336, N = 18432, M = 16: 11.9 / 17.4 / 28.0 ->
  // 11.3 / 16.1 / 27.4 us; neutral at 4.75, slower at exactly five), and
  // between six and six and a half with at most 16 groups (K = 8192,
  // N = 25088, M = 9 / 16: 22.2 / 22.3 -> 20.8 / 21.3; at K = 14336 slower).
  const bool balance = MT == 1 && ((p.Ns > 2 * p.cus && p.Ns <= 3 * p.cus) ||
                                   (p.Ns > 4 * p.cus && 2 * p.Ns <= 9 * p.cus) ||
                                   (p.G <= 16 && p.Ns > 6 * p.cus && 2 * p.Ns <= 13 * p.cus));
  // (and at M <= 4 up to 16 groups from two strips per unit: K = 8192,
  // N = 8192 / 14336, M = 1: 7.95 / 12.64 -> 7.66 / 12.03 us; K = 5120,
  // N = 8192: 6.01 -> 5.83; neutral at N = 13312-14336, K = 5120)
  const bool few_rows = MT == 1 && p.M <= 4 && p.G <= 16 && p.Ns >= 2 * p.cus;
  const bool one_strip = ((p.Ns >= 1024 && p.M <= 8) || one_round || small_k || balance || few_rows) && !p.out_fp4;
  if constexpr (MT == 1) {
    if (one_round && p.G > 16 && p.G <= 32) return launch_decode_t<1, 1, 4, 8>(p, (p.G + 3) / 4, 4, stream);
    // (row-major activations: one group per round, so the 16-byte scale
    // loads fit the registers, and no hold on them — K = 14336, N = 5120 /
    // 14336, M = 16: 12.97 / 26.59 -> 11.09 / 22.97 us; the GEMM layout
    // likewise once the two-strip workgroups fill a round of compute units —
    // N = 14336, K = 14336, M = 1 / 16: 19.94 / 21.02 -> 19.14 / 20.35;
    // N = 12288, K = 10240: 14.86 / 15.56 -> 13.68 / 14.80; but N = 5120,
    // 160 workgroups: 9.18 -> 9.43.  One group or two per round, the same K
    // split and order, so the same bits)
    if (gpw >= 2 && (p.a_rowmajor || p.Ns >= 2 * p.cus))
      return one_strip ? launch_decode_t<MT, 1, 1, MAXW, false>(p, kw, gpw, stream)
                       : launch_decode_t<MT, 2, 1, MAXW, false>(p, kw, gpw, stream);
    if (gpw >= 2)
      return one_strip ? launch_decode_t<MT, 1, 2, MAXW>(p, kw, gpw, stream)
                       : launch_decode_t<MT, 2, 2, MAXW>(p, kw, gpw, stream);
  }
  if constexpr (MT > 1) {
    // one round of compute units and 16-32 groups: at most 8 waves, each
    // loading four groups (two row tiles) or two (three and four) per round
    if (one_round && p.G >= 16 && p.G <= 32) {
      const int g8 = (p.G + 7) / 8;
      const int gp = MT == 2 ? (g8 < 4 ? 4 : g8) : (g8 + 1) / 2 * 2;
      return launch_decode_t<MT, 1, MT == 2 ? 4 : 2, 8>(p, (p.G + gp - 1) / gp, gp, stream);
    }
  }
  return one_strip ? launch_decode_t<MT, 1, 1, MAXW>(p, kw, gpw, stream)
                   : launch_decode_t<MT, 2, 1, MAXW>(p, kw, gpw, stream);
}

hipError_t launch_gemm_decode(const GemmArgs& p, hipStream_t stream) {
  switch ((p.M + 15) / 16) {
    case 1: return launch_decode_mt<1>(p, stream);
    case 2: return launch_decode_mt<2>(p, stream);
    case 3: return launch_decode_mt<3>(p, stream);
    default: return launch_decode_mt<4>(p, stream);
  }
}

hipError_t launch_gemm_decode_rows(const GemmArgs& p0, hipStream_t stream) {
  for (int r0 = 0; r0 < p0.M; r0 += 64) {
    GemmArgs p = p0;
    p.M = p0.M - r0 < 64 ? p0.M - r0 : 64;
    if (p0.a_rowmajor) {
      p.a = p0.a + (size_t)r0 * p0.lda;
      p.as = p0.as + (size_t)r0 * p0.lds;
    } else {
      // 64 rows are four whole 16-row tiles of both GEMM layouts
      p.a = p0.a + (size_t)(r0 / 16) * p0.Kt * 1024;
      p.as = p0.as + (size_t)(r0 / 16) * p0.G * 256;
    }
    if (p0.out_fp4) {
      p.out = (uint8_t*)p0.out + (size_t)r0 * p0.ldo;
      p.out_scales = p0.out_scales + (size_t)r0 * p0.ldos;
    } else {
      p.out = (uint8_t*)p0.out + (size_t)r0 * p0.ldo * (p0.out_f32 ? 4 : 2);
    }
    const hipError_t e = launch_gemm_decode(p, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Fused form (M <= 4): the K split of the one-row-tile decode kernel.
template <int NS, int GPR>
static hipError_t launch_linear_t(const GemmArgs& p, int kw, int gpw, hipStream_t stream) {
  const dim3 grid((unsigned)((p.Ns + NS - 1) / NS));
  const size_t lds = reduce_lds_bytes<1, NS, 16>();
  linear_decode_kernel<NS, GPR, 16><<<grid, 64 * kw, lds, stream>>>(p, gpw);
  return hipGetLastError();
}

bool linear_fused_pays(int M, int N, int K) {
  // Every workgroup re-reads and re-encodes the bf16 rows, so the fused
  // call beats quantisation + GEMM (about 2 us for the extra launch) only
  // while that traffic is small: measured on MI355X, at M = 1 for every
  // decode shape, and up to M = 4 when there are few workgroups (N < 16384)
  // and one round of groups per wave (K <= 8192).  With two rounds
  // (K <= 16384) it still pays at M = 2, and up to M = 4 while the strips
  // fit in about one round of compute units (N <= 4096): K = 14336,
  // N = 4096, M = 2 / 4: 9.76 / 9.85 -> 7.56 / 8.86 us; N = 14336, M = 2:
  // 22.36 -> 20.68 us; but N = 5120, M = 4: 11.63 -> 13.03 us.  On many
  // strips (N >= 16384) only at M = 2 (K = 4096, N = 24576 / 28672:
  // 12.45 / 13.62 -> 10.87 / 12.11 us; K = 8192, N = 20480: 17.44 ->
  // 15.84), and not at M >= 3 between two and three strips per compute
  // unit (N = 8192-12288), where the GEMM runs one strip per workgroup and
  // the fused kernel two (K = 8192, N = 10240, M = 3 / 4: 12.57 / 13.00 ->
  // 11.64 / 11.66 us through quantisation + GEMM).
  if (M < 1 || M > kFusedRows) return false;
  if (M == 1) return true;
  if (N >= 16384) return M == 2 && K <= 16384;
  if (M >= 3 && N > 8192 && N <= 12288) return false;
  if (K <= 8192) return true;
  return K <= 16384 && (M == 2 || N <= 4096);
}

hipError_t launch_linear_decode(const GemmArgs& p, hipStream_t stream) {
  if (p.M > kFusedRows) return hipErrorInvalidValue;
  // Up to 8192-wide K: at most 16 waves of one group each, one strip per
  // workgroup when strips are plentiful or all fit in one round of compute
  // units (N = 4096, K = 5120, M = 1 / 4: 5.01 / 5.56 -> 4.41 / 4.88 us;
  // K = 8192: 6.41 / 7.26 -> 5.45 / 6.09).  Wider K: at most 8 waves of two
  // groups per round and one strip (fewer waves re-encoding the rows, and
  // two strips would not fit the registers; four groups per round in 7
  // waves measured slower: K = 14336, N = 5120, M = 1: 12.14 against 10.66).
  // As the GEMM, one strip between two and three strips per compute unit,
  // where each workgroup's re-encoding of x is cheap (M <= 2: K = 5120,
  // N = 10240 / 12288, M = 1: 8.83 / 9.08 -> 7.27 / 7.78 us; K = 8192,
  // N = 10240, M = 1 / 2: 11.81 / 12.15 -> 9.63 / 10.20; at M = 4 mixed,
  // N = 12288: 9.85 -> 10.59).  At M = 1 one strip everywhere (one row to
  // encode): K = 5120, N = 13312 / 14336: 9.20 / 9.44 -> 8.52 / 8.74 us;
  // K = 8192, N = 14336: 13.07 -> 12.13.  At M = 2 past three strips per
  // unit also one strip with 12 or 16 groups (waves even over the four
  // SIMDs): K = 6144, N = 12800 / 16128: 10.45 / 11.31 -> 10.31 / 10.90 us;
  // K = 8192, N = 12800 / 14336 / 16128: 12.78 / 13.30 / 14.15 -> 12.11 /
  // 12.68 / 13.26; not with 10, 11 or 14 groups (K = 7168, N = 14336 /
  // 16128: 12.27 / 12.99 -> 13.32 / 14.19; K = 5120, N = 16128: 10.15 ->
  // 10.89).
  if (p.G <= 16) {
    const int kw = p.G;
    const bool balance = (p.Ns > 2 * p.cus && p.Ns <= 3 * p.cus && p.M <= 2) || p.M == 1 ||
                         (p.M == 2 && p.Ns > 3 * p.cus && p.G >= 12 && p.G % 4 == 0);
    return (p.Ns >= 1024 || p.Ns <= p.cus || balance) ? launch_linear_t<1, 1>(p, kw, 1, stream)
                                                      : launch_linear_t<2, 1>(p, kw, 1, stream);
  }
  // From 20 groups on, at most 12 waves (two or three groups each, the
  // latter one per round) beat 8 waves of three or four: K = 14336, M = 1,
  // N = 5120 / 8192 / 14336: 10.71 / 12.52 / 19.82 -> 10.45 / 11.74 /
  // 19.06 us; K = 10240, N = 2048: 5.82 -> 5.21 (at 17 groups, K = 8704,
  // N = 20480, 8 waves stay: 19.52 against 20.22).
  const int gpw = p.G >= 20 ? (p.G + 11) / 12 : (p.G + 7) / 8;
  const int kw = (p.G + gpw - 1) / gpw;
  return (p.G >= 20 && gpw == 3) ? launch_linear_t<1, 1>(p, kw, gpw, stream)
                                 : launch_linear_t<1, 2>(p, kw, gpw, stream);
}
// Fused quantisation in the persistent form (M <= 32: one or two row
// tiles, at most 12 scale groups): each wave encodes its group's blocks of
// the rows once.  The same operands, K split and order as quantisation +
// the persistent GEMM, so the same bits.  (Three or four tiles of encoded
// operands beside the weight ring spill at the 12-wave register budget, so
// those forms are not built.)
bool linear_persist_applies(int M, int K, int64_t x_bytes) {
  const int G = (K / 32 + 15) / 16;
  return M >= 1 && M <= 32 && G <= 12 && x_bytes <= (int64_t)0x7FFFFFFF;  // 31-bit buffer offsets
}

// Every workgroup encodes the bf16 rows itself (4x the bytes of their FP4
// form through each compute unit's L2 path before the first MFMA), so the
// fusion beats quantisation + GEMM only while the rows are few and the
// weight strips many.  Measured on MI355X (us, default two launches /
// fused persistent; rotated weight copies, bf16 out), K = 5120: N = 24576
// (6 strips per CU): M = 2 15.0 / 14.0, M = 4 15.0 / 14.3, M = 8 15.1 /
// 15.2, M = 16 15.3 / 17.0; N = 34816: M = 2 18.6 / 18.3, M = 4 18.9 /
// 18.7, M = 16 20.2 / 21.3; N = 14336 and 16384 (K = 6144): 5-22% slower
// at every M; M = 1 stays with the streaming fused kernel (N = 34816: 16.4
// against 18.2).
bool linear_persist_pays(int M, int N, int K, int cus) {
  const int ov = get_gemm_path_override();
  if (ov == 7) return true;
  if (ov == 8) return false;
  const int Ns = (N + 15) / 16;
  const int G = (K / 32 + 15) / 16;
  return M >= 2 && M <= 4 && G >= 10 && Ns >= 6 * cus;
}

template <int MT, int D>
static void launch_linear_persist_mt(const GemmArgs& p, hipStream_t stream) {
  const int grid = p.Ns < p.cus ? p.Ns : p.cus;
  gemm_decode_persist_kernel<MT, 12, D, kASrcBf16><<<grid, 64 * p.G, 2 * reduce_lds_bytes<MT, 1, 12>(), stream>>>(p);
}

hipError_t launch_linear_persist(const GemmArgs& p, hipStream_t stream) {
  if (p.M < 1 || p.M > 32 || p.G > 12) return hipErrorInvalidValue;
  // ring depth: as the GEMM-layout form at one row tile; at two, the
  // encoding's registers are live beside the ring, which holds one step
  if (p.M <= 16)
    launch_linear_persist_mt<1, 4>(p, stream);
  else
    launch_linear_persist_mt<2, 1>(p, stream);
  return hipGetLastError();
}

}  // namespace mxfp4
