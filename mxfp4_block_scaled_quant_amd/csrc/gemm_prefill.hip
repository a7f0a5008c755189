// W4A4 block-scaled FP4 GEMM for large M (prefill) on gfx950.
//
// Same operation as the decode kernel (P2 §2: quantised activations times
// the preshuffled [N, K] weight, NT form, bias after; P1 §Accuracy Tests:
// equal to the dequantised reference), organised for the MFMA roofline:
//
//  * a 512-thread workgroup computes a 256 x 256 output tile; its 8 waves
//    (two per SIMD, so one can issue while the other waits) form a 2 x 4
//    grid of 128 x 64 wave tiles, 8 x 4 MFMA tiles of 16 x 16 each (128
//    fp32 accumulators per lane).  One K-step (128) is 32 MFMAs per wave
//    against 12 KiB of operand reads from LDS;
//  * operands stream through four single-K-step LDS buffers (32 KiB each):
//    every 1 KiB operand unit of the GEMM layouts (activations and weights
//    alike) is fetched by one buffer_load_dwordx4 ... lds per wave, so LDS
//    holds fragments in the lane order the MFMA consumes (conflict-free
//    ds_read_b128).  Loads run three K-steps ahead; each step needs one
//    wait (hand-counted vmcnt) and one barrier;
//  * the next step's fragments are read while this step's MFMAs run: each
//    activation fragment is re-read right after its row of 8 MFMAs, weight
//    fragments alternate between two register sets;
//  * block scales: one dword per lane per 16-row tile per 4 K-steps, loaded
//    a group ahead; op_sel walks the 4 K-steps of a dword;
//  * the MFMA takes the weight as its A operand and the activations as B, so
//    a lane ends with 4 consecutive output columns of one row; the epilogue
//    adds the bias in fp32, rounds once to bf16 and transposes through LDS to
//    write whole 16-byte chunks of output rows (fp32 output, used for the
//    pre-cast checks, is stored directly);
//  * tiles are ordered in groups of 8 row-tiles and dealt to the 8 XCDs in
//    contiguous runs, so the workgroups sharing an XCD's L2 share operands.
#include "mxfp4_device.h"
#include "mxfp4_launch.h"

namespace mxfp4 {

namespace {

constexpr int kBM = 256, kBN = 256;
constexpr int kTilesA = kBM / 16;            // 16 activation units per K-step
constexpr int kTilesB = kBN / 16;            // 16 weight units per K-step
constexpr int kUnits = kTilesA + kTilesB;    // 32 units of 1 KiB per K-step
constexpr int kBufs = 4;                     // LDS buffers (K-steps in flight)
constexpr int kWaves = 8;
constexpr int kLoadsPerWave = kUnits / kWaves;  // 4 buffer->LDS loads per wave per step
constexpr int kWM = 8, kWN = 4;                 // wave tile: 8 x 4 MFMA tiles (128 x 64)
constexpr int kScaleLoads = kWM + kWN;          // scale dwords per wave per group
constexpr int kGroupM = 8;                   // row-tiles per ordering group
constexpr int kRowB = 144;                   // epilogue staging row stride (bytes)
constexpr int kStageBytes = kBufs * kUnits * 64 * 16;
constexpr int kEpiBytes = kWaves * 128 * kRowB;
constexpr int kLdsBytes = kStageBytes > kEpiBytes ? kStageBytes : kEpiBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS per workgroup");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Base pointers and byte sizes of this tile's operand windows.  Buffer
// descriptors are built after any selection between them: a select between
// descriptors becomes a vector select, which then costs a waterfall loop per
// buffer instruction.
struct Ctx {
  const uint8_t *pa, *pw, *pas, *pws;
  uint32_t na, nw, nas, nws;
  int Kt, G;
};

typedef int4 StageBuf[kUnits][64];
// Fragment registers: a native 4 x 32-bit vector, so inline assembly can take
// it as a register operand.
typedef int v4i __attribute__((ext_vector_type(4)));

template <int SEL>
__device__ __forceinline__ v4f mfma_fp4v(v4i a, v4i b, uint32_t sa, uint32_t sb, v4f acc) {
  const v8i A = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  const v8i B = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 4, SEL, (int)sa, SEL, (int)sb);
}

// Issue this wave's 4 buffer->LDS loads of K-step t into stage buffer `buf`.
// Waves 0-3 fetch the 16 activation units, waves 4-7 the 16 weight units.
// The unit's position goes in the vector offset, so units past the tile's
// last strip fall outside the window (zeros); steps past K use an empty
// window; the step's position goes in the scalar offset.
__device__ __forceinline__ void issue_step(const Ctx& c, StageBuf& buf, int t, int wv, const uint32_t (&voff)[4]) {
  const bool is_a = wv < 4;
  const uint8_t* base = is_a ? c.pa : c.pw;
  const uint32_t size = t < c.Kt ? (is_a ? c.na : c.nw) : 0u;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, size);
  const int u0 = (is_a ? 0 : kTilesA) + (wv & 3) * kLoadsPerWave;
#pragma unroll
  for (int q = 0; q < kLoadsPerWave; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)&buf[u0 + q][0], 16, voff[q], t << 10, 0, 0);
}

// Scale dwords of group g for this wave's 8 row tiles and 4 column strips.
__device__ __forceinline__ void issue_scales(const Ctx& c, uint32_t (&sa)[kWM], uint32_t (&sb)[kWN], int g,
                                             const uint32_t (&soff_a)[kWM], const uint32_t (&soff_b)[kWN]) {
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(c.pas, g < c.G ? c.nas : 0u);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(c.pws, g < c.G ? c.nws : 0u);
#pragma unroll
  for (int i = 0; i < kWM; ++i) sa[i] = __builtin_amdgcn_raw_buffer_load_b32(ras, soff_a[i], g << 8, 0);
#pragma unroll
  for (int j = 0; j < kWN; ++j) sb[j] = __builtin_amdgcn_raw_buffer_load_b32(rws, soff_b[j], g << 8, 0);
}

// Fragment reads from LDS are written as inline assembly with hand-counted
// lgkmcnt waits.  The compiler cannot tell the LDS written by buffer->LDS
// loads from the LDS these reads use, so for its own LDS reads it would
// wait for every buffer->LDS load in flight (draining the prefetch) and sink
// each read to just before its first use.
template <int OFF>
__device__ __forceinline__ void ds_read16(v4i& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}

// lgkmcnt(N) wait that the given fragments depend on, so no MFMA reading
// them is scheduled above it.
template <int N>
__device__ __forceinline__ void wait_lgkm(v4i& a, v4i& b, v4i& c, v4i& d) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "i"(N));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (the fence
// waits for every buffer->LDS load in flight, draining the prefetch).  The
// waits before it are explicit; the empty statements keep the compiler from
// moving memory operations across it.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS addresses of this lane's fragments: stage buffers 0-1 are reached
// from the first base, 2-3 from the second (the read offset field is 16 bits).
struct FragAddr {
  uint32_t a01, a23, b01, b23;
};

template <int BUF, int I>
__device__ __forceinline__ void read_a(v4i& v, const FragAddr& fa) {
  ds_read16<(BUF & 1) * (int)sizeof(StageBuf) + I * 1024>(v, BUF < 2 ? fa.a01 : fa.a23);
}
template <int BUF, int J>
__device__ __forceinline__ void read_b(v4i& v, const FragAddr& fa) {
  ds_read16<(BUF & 1) * (int)sizeof(StageBuf) + J * 1024>(v, BUF < 2 ? fa.b01 : fa.b23);
}

// First half of the next step's fragments (weights 0-3, activations 0-3),
// then the second half (activations 4-7): 8 + 4 LDS reads in this order.
template <int BUF>
__device__ __forceinline__ void read_first_half(v4i (&af)[kWM], v4i (&bf)[kWN], const FragAddr& fa) {
  read_b<BUF, 0>(bf[0], fa);
  read_b<BUF, 1>(bf[1], fa);
  read_b<BUF, 2>(bf[2], fa);
  read_b<BUF, 3>(bf[3], fa);
  read_a<BUF, 0>(af[0], fa);
  read_a<BUF, 1>(af[1], fa);
  read_a<BUF, 2>(af[2], fa);
  read_a<BUF, 3>(af[3], fa);
}
template <int BUF>
__device__ __forceinline__ void read_second_half(v4i (&af)[kWM], const FragAddr& fa) {
  read_a<BUF, 4>(af[4], fa);
  read_a<BUF, 5>(af[5], fa);
  read_a<BUF, 6>(af[6], fa);
  read_a<BUF, 7>(af[7], fa);
}

// MFMAs of activation rows I0..I0+3 of one K-step: acc[i][j] (+)= W-strip j
// (A operand) x activation tile i (B operand).
template <int SEL, int I0>
__device__ __forceinline__ void mfma_rows(v4f (&acc)[kWM][kWN], const v4i (&af)[kWM], const v4i (&bf)[kWN],
                                          const uint32_t (&sa)[kWM], const uint32_t (&sb)[kWN]) {
#pragma unroll
  for (int i = I0; i < I0 + 4; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j) acc[i][j] = mfma_fp4v<SEL>(bf[j], af[i], sb[j], sa[i], acc[i][j]);
}

// One K-step t = 4*g + J, its operands in stage buffer J:
//  * rows 0-3 (their fragments, and the weight fragments, were read in the
//    second half of the previous step: wait for all but the last 4 reads);
//  * then the step's one barrier.  Before it this wave's reads of buffer J
//    are done and its buffer->LDS loads of step t+1 have landed; after it
//    buffer J is refilled with step t+4 (at J == 0 after the scale loads of
//    group g+1), and the first half of step t+1's fragments is read from
//    buffer J+1 (weights into the other weight set);
//  * rows 4-7, then the second half of step t+1's fragments.
// Loads in flight after the ones step t+1 needs: steps t+2 and t+3 plus,
// for J = 1 and 2, the 12 scale loads issued at J = 0.
template <int J>
__device__ __forceinline__ void main_step(const Ctx& c, StageBuf& cur, v4f (&acc)[kWM][kWN], v4i (&af)[kWM],
                                          v4i (&bf_cur)[kWN], v4i (&bf_nxt)[kWN], const uint32_t (&sa)[kWM],
                                          const uint32_t (&sb)[kWN], uint32_t (&sa_nxt)[kWM],
                                          uint32_t (&sb_nxt)[kWN], int g, int wv, const FragAddr& fa,
                                          const uint32_t (&voff)[4], const uint32_t (&soff_a)[kWM],
                                          const uint32_t (&soff_b)[kWN]) {
  const int t = 4 * g + J;
  constexpr int kNext = (J + 1) & 3;
  wait_lgkm<4>(af[0], af[1], af[2], af[3]);
  wait_lgkm<4>(bf_cur[0], bf_cur[1], bf_cur[2], bf_cur[3]);
  mfma_rows<J, 0>(acc, af, bf_cur, sa, sb);
  __builtin_amdgcn_sched_barrier(0);
  wait_lgkm<0>(af[4], af[5], af[6], af[7]);
  if (J == 1 || J == 2)
    wait_vm<2 * kLoadsPerWave + kScaleLoads>();
  else
    wait_vm<2 * kLoadsPerWave>();
  barrier_nofence();
  if (J == 0) issue_scales(c, sa_nxt, sb_nxt, g + 1, soff_a, soff_b);
  issue_step(c, cur, t + 4, wv, voff);
  read_first_half<kNext>(af, bf_nxt, fa);
  __builtin_amdgcn_sched_barrier(0);
  mfma_rows<J, 4>(acc, af, bf_cur, sa, sb);
  __builtin_amdgcn_sched_barrier(0);
  read_second_half<kNext>(af, fa);
}

}  // namespace

__global__ __launch_bounds__(512, 1) void gemm_prefill_kernel(GemmArgs p, int tiles_m, int tiles_n) {
  // The four stage buffers (128 KiB); the bf16 epilogue reuses the space
  // (144 KiB) for its transpose.
  __shared__ int4 lds_raw[kLdsBytes / 16];
  StageBuf* smem = reinterpret_cast<StageBuf*>(lds_raw);
  const int lane = threadIdx.x & 63;
  // The wave index is uniform across the wave; saying so keeps the buffer
  // resource and LDS address of every buffer->LDS load in scalar registers.
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wv >> 2, wn = wv & 3;

  // Tile order: consecutive ids run down a group of kGroupM row-tiles, then
  // across columns; ids are dealt to the XCDs (round-robin by workgroup id)
  // in contiguous runs.
  const int ntiles = tiles_m * tiles_n;
  int id = blockIdx.x;
  {
    const int per_xcd = (ntiles + 7) / 8;
    const int xcd = id % 8, k = id / 8;
    const int full = ntiles - (per_xcd - 1) * 8;  // XCDs that get per_xcd ids
    id = xcd < full ? xcd * per_xcd + k : full * per_xcd + (xcd - full) * (per_xcd - 1) + k;
  }
  const int group = id / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (id % (kGroupM * tiles_n)) % gm;
  const int tn = (id % (kGroupM * tiles_n)) / gm;

  const int m0 = tm * kBM;
  const int s0 = tn * kTilesB;
  Ctx c;
  c.Kt = p.Kt;
  c.G = p.G;
  const int strips = min(kTilesB, p.Ns - s0);
  const int mstrips = min(kTilesA, ((p.M + 15) >> 4) - m0 / 16);
  c.pa = p.a + (int64_t)(m0 / 16) * p.Kt * 1024;
  c.na = (uint32_t)mstrips * p.Kt * 1024u;
  c.pw = p.w + (int64_t)s0 * p.Kt * 1024;
  c.nw = (uint32_t)strips * p.Kt * 1024u;
  c.pas = p.as + (int64_t)(m0 / 16) * p.G * 256;
  c.nas = (uint32_t)mstrips * p.G * 256u;
  c.pws = p.ws + (int64_t)s0 * p.G * 256;
  c.nws = (uint32_t)strips * p.G * 256u;

  uint32_t voff[kLoadsPerWave];
#pragma unroll
  for (int q = 0; q < kLoadsPerWave; ++q)
    voff[q] = (uint32_t)((((wv & 3) * kLoadsPerWave + q) * p.Kt) << 10) + lane * 16;
  uint32_t soff_a[kWM], soff_b[kWN];
#pragma unroll
  for (int i = 0; i < kWM; ++i) soff_a[i] = (uint32_t)(((wm * kWM + i) * p.G) << 8) + lane * 4;
#pragma unroll
  for (int j = 0; j < kWN; ++j) soff_b[j] = (uint32_t)(((wn * kWN + j) * p.G) << 8) + lane * 4;
  FragAddr fa;
  {
    const uint32_t base = (uint32_t)(uintptr_t)(lds_ptr_t)&smem[0][0][0] + lane * 16;
    fa.a01 = base + wm * kWM * 1024;
    fa.b01 = base + (kTilesA + wn * kWN) * 1024;
    fa.a23 = fa.a01 + 2 * (uint32_t)sizeof(StageBuf);
    fa.b23 = fa.b01 + 2 * (uint32_t)sizeof(StageBuf);
  }

  // Zero accumulators the compiler cannot see through, so it does not peel
  // the first K-group to specialise it (which costs accumulator copies).
  float zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  v4f acc[kWM][kWN];
#pragma unroll
  for (int i = 0; i < kWM; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j) acc[i][j] = (v4f){zero, zero, zero, zero};

  uint32_t sa[kWM], sb[kWN], sa_n[kWM], sb_n[kWN];
  v4i af[kWM], b0[kWN], b1[kWN];

  // Prologue: scales of group 0 and steps 0..3 in flight; once step 0 has
  // landed everywhere, read its fragments in the order the loop expects.
  issue_scales(c, sa, sb, 0, soff_a, soff_b);
  issue_step(c, smem[0], 0, wv, voff);
  issue_step(c, smem[1], 1, wv, voff);
  issue_step(c, smem[2], 2, wv, voff);
  issue_step(c, smem[3], 3, wv, voff);
  wait_vm<3 * kLoadsPerWave>();
  barrier_nofence();
  read_first_half<0>(af, b0, fa);
  read_second_half<0>(af, fa);

  for (int g = 0; g < p.G; ++g) {
    main_step<0>(c, smem[0], acc, af, b0, b1, sa, sb, sa_n, sb_n, g, wv, fa, voff, soff_a, soff_b);
    main_step<1>(c, smem[1], acc, af, b1, b0, sa, sb, sa_n, sb_n, g, wv, fa, voff, soff_a, soff_b);
    main_step<2>(c, smem[2], acc, af, b0, b1, sa, sb, sa_n, sb_n, g, wv, fa, voff, soff_a, soff_b);
    main_step<3>(c, smem[3], acc, af, b1, b0, sa, sb, sa_n, sb_n, g, wv, fa, voff, soff_a, soff_b);
#pragma unroll
    for (int i = 0; i < kWM; ++i) sa[i] = sa_n[i];
#pragma unroll
    for (int j = 0; j < kWN; ++j) sb[j] = sb_n[j];
  }
  // Drain the reads and loads of steps past the end before the stage
  // buffers are reused for the output.
  wait_lgkm<0>(af[4], af[5], af[6], af[7]);
  wait_vm<0>();
  __syncthreads();

  // Epilogue.  Lane l, register r of tile (i, j): output row
  // m0 + wm*128 + 16i + l%16, column (s0 + wn*4 + j)*16 + 4*(l/16) + r.
  const int ncol0 = (s0 + wn * kWN) * 16;
  const int mrow0 = m0 + wm * 128;
  if (p.out_f32) {
#pragma unroll
    for (int i = 0; i < kWM; ++i)
#pragma unroll
      for (int j = 0; j < kWN; ++j) {
        const int m = mrow0 + i * 16 + (lane & 15);
        const int n = ncol0 + j * 16 + 4 * (lane >> 4);
        if (m >= p.M) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < p.N)
            reinterpret_cast<float*>(p.out)[(int64_t)m * p.ldo + n + r] =
                acc[i][j][r] + (p.bias ? bf16_to_f32(p.bias[n + r]) : 0.f);
      }
    return;
  }
  // bf16: stage this wave's 128 x 64 tile in LDS (row stride 144 bytes to
  // spread banks), then write 16-byte chunks of whole rows.
  uint8_t* stage = reinterpret_cast<uint8_t*>(lds_raw) + wv * 128 * kRowB;
  float bias4[kWN][4];
#pragma unroll
  for (int j = 0; j < kWN; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = ncol0 + j * 16 + 4 * (lane >> 4) + r;
      bias4[j][r] = (p.bias && n < p.N) ? bf16_to_f32(p.bias[n]) : 0.f;
    }
#pragma unroll
  for (int i = 0; i < kWM; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j) {
      const uint32_t lo = f32_to_bf16_rne(acc[i][j][0] + bias4[j][0]) |
                          ((uint32_t)f32_to_bf16_rne(acc[i][j][1] + bias4[j][1]) << 16);
      const uint32_t hi = f32_to_bf16_rne(acc[i][j][2] + bias4[j][2]) |
                          ((uint32_t)f32_to_bf16_rne(acc[i][j][3] + bias4[j][3]) << 16);
      const int row = i * 16 + (lane & 15);
      const int col = j * 16 + 4 * (lane >> 4);
      *reinterpret_cast<uint2*>(stage + row * kRowB + col * 2) = make_uint2(lo, hi);
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes done
  __builtin_amdgcn_wave_barrier();
  // 8 lanes cover a 128-byte row; 8 rows per pass, 16 passes.
#pragma unroll 4
  for (int pass = 0; pass < 16; ++pass) {
    const int row = pass * 8 + (lane >> 3);
    const int col = (lane & 7) * 8;
    const int m = mrow0 + row;
    const int n = ncol0 + col;
    if (m >= p.M) continue;
    const int4 v = *reinterpret_cast<const int4*>(stage + row * kRowB + col * 2);
    uint16_t* dst = reinterpret_cast<uint16_t*>(p.out) + (int64_t)m * p.ldo + n;
    if (n + 8 <= p.N && (((uintptr_t)dst & 15) == 0)) {
      *reinterpret_cast<int4*>(dst) = v;
    } else {
      const uint32_t w[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < p.N) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  }
}

hipError_t launch_gemm_prefill(const GemmArgs& p, hipStream_t stream) {
  const int tiles_m = (p.M + kBM - 1) / kBM;
  const int tiles_n = (p.Ns * 16 + kBN - 1) / kBN;
  gemm_prefill_kernel<<<dim3((unsigned)(tiles_m * tiles_n)), 64 * kWaves, 0, stream>>>(p, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace mxfp4
