// A16WFP4 batched GEMM on gfx950: bf16 activations x MXFP4 weights.
//
// P3 §Motivation and §Modifications keep the MLA absorbed K/V projection
// weights in packed MXFP4 and run the per-head products on bf16
// activations, writing the V-up result batch-major.  Computed here:
//   out[b, m, n] = round(sum_k x[b, m, k] * dq(W)[b, n, k])
// with the activations used exactly (no activation quantisation), the
// weights dequantised exactly to bf16 in registers (an E2M1 value times a
// power of two fits bf16 for every scale byte quantisation produces), the bf16 16x16x32 MFMA with fp32
// accumulation, and one RNE rounding to bf16 (or fp32 out).  The weight
// dequantisation uses gfx950's scaled FP4 -> bf16 conversion instruction.  Output
// strides (sob, som) cover both [B, M, N] and batch-major [M, B, N].
//
// Two kernels.  The streaming kernel (shapes whose weight slice fits in
// registers, which covers the MLA K-up 512 x 192 and V-up 256 x 512 heads):
// a 512-thread workgroup owns one head (with few m-tiles per head, one
// column block of it: 128 columns for M <= 64, half the head a little
// above) and a run of 16-row m-tiles; each of its 8 waves dequantises its
// 1/8 of the workgroup's output columns once into registers (bf16 MFMA
// fragments), and the activation m-tiles stream through a ring of two or
// three LDS stages by buffer->LDS loads (in the MFMA's lane order), one
// barrier per m-tile, so activations are read from HBM once, weights once
// per workgroup, and output written once.  Waves 0-3 issue all activation
// loads and waves 4-7 all output stores (through a double-buffered LDS
// staging area, as whole rows of the workgroup's columns, non-temporal): a
// wave's memory counter retires loads and stores in issue order, so a wave
// that both stores and waits for its loads would wait for its stores too.
// The general kernel (any K):
// a 256-thread workgroup owns one head and a 64 (m) x 128 (n) output tile;
// wave w takes 32 columns (2 MFMA tiles) over all 64 rows (4 MFMA tiles).  The weight acts as the MFMA's A operand (16 output columns
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

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) times
// 2^(sc-127) as bf16 pairs: gfx950's scaled FP4 -> bf16 conversion, one
// instruction per byte.  Exact whenever the product fits bf16, which holds
// for every scale byte up to 252 (all that quantising bf16 data produces;
// bytes 253-254 with the largest codes overflow to +-inf); measured
// bit-identical to the exact product for every byte and every scale byte
// 0..254 (sc = 0 passes the fp32 subnormal 2^-127).
__device__ __forceinline__ v8bf dequant8(uint32_t word, uint32_t sc) {
  const float scale = __uint_as_float(sc == 0 ? 0x00400000u : (sc << 23));
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3);
  return (v8bf){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
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
          const uint32_t lo = pack_bf16x2(acc[j][i][0], acc[j][i][1]);
          const uint32_t hi = pack_bf16x2(acc[j][i][2], acc[j][i][3]);
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

// ---------------------------------------------------------------------------
// Streaming kernel.

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int kWavesS = 8;

// LDS of one instance (KF K-fragments, NT column tiles, output element
// size ESZ, NS stages): NS stages of KF KiB (fragment c of a stage at c
// KiB), a 1 KiB target for padding loads, then two output staging buffers,
// each holding the m-tile's 16 output rows over the workgroup's 8*NT*16
// columns (wave w's columns at w*NT*16; rows padded by 16 bytes to spread
// banks), so that stores go out as whole rows.  A shallow ring: measured on MI355X with activations read
// from HBM, a three-stage ring beats deeper ones (K-up / V-up, M = 4096:
// 23.2 / 24.1 us with three stages, 23.3 / 24.9 with four, 24.5 / 28.1 with
// eight: the larger start-up burst of every workgroup delays its first
// m-tile), and with up to four m-tiles per workgroup two stages do (M =
// 1024: 9.1 / 9.8 us against 9.4 / 10.5; M = 256: 5.1 / 5.7 against 5.3 /
// 6.0).
template <int KF, int NT, int ESZ, int NS>
struct BmmLds {
  static constexpr int kRowB = NT * 16 * ESZ;                 // one wave's part of a row
  static constexpr int kRowStride = kWavesS * kRowB + 16;
  static constexpr int kStgBuf = 16 * kRowStride;             // one staging buffer
  static constexpr int kStage = KF * 1024;
  static constexpr int kStages = NS;
  static constexpr int kTrash = kStages * kStage;
  static constexpr int kStg = kTrash + 1024;
  static constexpr int kBytes = kStg + 2 * kStgBuf;
  static_assert(kBytes <= 160 * 1024, "LDS per workgroup");
};

__device__ __forceinline__ lds_ptr_t lds_at(uint32_t addr) { return (lds_ptr_t)(uintptr_t)addr; }

__device__ __forceinline__ uint32_t lane_here() {
  uint32_t l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 4 x 4 transpose between a lane's four registers and the wave's four
// 16-lane rows: afterwards register j of row q holds what register q of row j
// held.  gfx950's lane-swap instructions: the 32-lane swap exchanges the upper
// half of its first operand with the lower half of its second; the 16-lane
// swap exchanges the odd rows of its first operand with the even rows of its
// second.  Together they transpose the 2 x 2 blocks, then each block.
__device__ __forceinline__ void transpose_rows4(uint32_t (&d)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto e = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  d[0] = c[0];
  d[1] = c[1];
  d[2] = e[0];
  d[3] = e[1];
}

template <int OFF>
__device__ __forceinline__ void ds_read16(v4i& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
__device__ __forceinline__ void read_frag(v4i& v, uint32_t addr) { ds_read16<0>(v, addr); }

// lgkmcnt(n) wait (n a compile-time value after unrolling) that `v` depends on.
__device__ __forceinline__ void wait_lgkm_n(v4i& v, int n) {
  switch (n) {
#define MXFP4_W(N_) \
  case N_: asm volatile("s_waitcnt lgkmcnt(" #N_ ")" : "+v"(v)); break;
    MXFP4_W(0) MXFP4_W(1) MXFP4_W(2) MXFP4_W(3) MXFP4_W(4) MXFP4_W(5) MXFP4_W(6) MXFP4_W(7)
    MXFP4_W(8) MXFP4_W(9) MXFP4_W(10) MXFP4_W(11) MXFP4_W(12) MXFP4_W(13) MXFP4_W(14)
    default: asm volatile("s_waitcnt lgkmcnt(15)" : "+v"(v)); break;
#undef MXFP4_W
  }
}

template <int OFF>
__device__ __forceinline__ void ds_write8(uint32_t addr, v2i v) {
  asm volatile("ds_write_b64 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_write16(uint32_t addr, v4i v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF));
}

// A loading wave's (0-3) share of m-tile `mt` of head b into stage `st`:
// K-fragment c (16 rows x 32 K, lane l = row l%16, elements 8(l/16)..+7)
// goes to LDS stage + c KiB in the MFMA's lane order, loaded by wave c % 4.
// A loading wave always issues KD loads per m-tile (padding ones load zeros,
// past KF into a trash slot), so its count of memory operations is fixed.
// Rows past M and m-tiles past the end fall outside the descriptor (zeros).
template <int KD, int KF, int STAGE, int TRASH>
__device__ __forceinline__ void issue_xtile(const BmmArgs& p, int b, int mt, int nmt, int st, int kf, int wv,
                                            uint32_t lane) {
  const int m0 = mt * 16;
  const int rows = mt < nmt ? min(16, p.M - m0) : 0;
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc(p.x + b * p.sxb + (int64_t)m0 * p.sxm,
                rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * p.sxm + p.K) * 2) : 0u);
  const uint32_t row = lane & 15u;
  const uint32_t voff = (int)row < rows ? (uint32_t)(row * p.sxm + (lane >> 4) * 8) * 2 : kOOB;
#pragma unroll
  for (int d = 0; d < KD; ++d) {
    const int c = d * 4 + wv;
    // Fragments from K to KF are zero-filled (out-of-range offset), so the
    // MFMAs over them add nothing; loads past KF go to the trash slot.
    const uint32_t lds = c < KF ? (uint32_t)(st * STAGE + c * 1024) : (uint32_t)TRASH;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_at(lds), 16, c < kf ? voff : kOOB, c * 64, 0, 0);
  }
}

// A wave's 16 x (NT*16) output block of an m-tile to its LDS staging block
// at `slot`: lane (r = l%16, q = l/16) writes columns 16j + 4q..+3 of row r.
template <int NT, bool F32, int ROWSTRIDE>
__device__ __forceinline__ void stage_write(const v4f (&acc)[NT], uint32_t slot, uint32_t lane) {
  constexpr int esz = F32 ? 4 : 2;
  const uint32_t waddr = slot + (lane & 15u) * ROWSTRIDE + (lane >> 4) * 4 * esz;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (F32) {
      // The MFMA results pass through an exact vector copy (identity DPP
      // move) before the inline-assembly LDS write: the compiler inserts the
      // wait states an MFMA result needs before a vector instruction reads
      // it, but not before an assembly statement does.
      v4i d;
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] = __builtin_amdgcn_mov_dpp((int)__float_as_uint(acc[j][e]), 0xE4, 0xF, 0xF, false);
      switch (j) {
        case 0: ds_write16<0>(waddr, d); break;
        case 1: ds_write16<64>(waddr, d); break;
        case 2: ds_write16<128>(waddr, d); break;
        default: ds_write16<192>(waddr, d); break;
      }
    } else {
      const uint32_t lo = pack_bf16x2(acc[j][0], acc[j][1]);
      const uint32_t hi = pack_bf16x2(acc[j][2], acc[j][3]);
      const v2i d = {(int)lo, (int)hi};
      switch (j) {
        case 0: ds_write8<0>(waddr, d); break;
        case 1: ds_write8<32>(waddr, d); break;
        case 2: ds_write8<64>(waddr, d); break;
        default: ds_write8<96>(waddr, d); break;
      }
    }
  }
}

// Store of rows 4*quarter..+3 of a staged m-tile (m-tile mt, the
// workgroup's columns from 16-column strip c0) from staging buffer `stg`:
// piece k is row 4*quarter + k / CPR, 16-byte piece k % CPR of it, so
// consecutive lanes write consecutive bytes of a row and every store covers
// whole rows of the workgroup's columns.  VEC: whole pieces (N a multiple of
// the piece, aligned rows), written non-temporal (the output is not read
// again here); otherwise each element on its own.  Out-of-range elements get
// an out-of-range offset.  Measured on MI355X against the earlier staging of
// one wave's 16 x NT*16 block per store (V-up rows then 64 bytes: half
// lines), back-to-back launches at M = 4096: V-up 26.4 -> 22.5 us, K-up
// (128-byte rows before) unchanged at 20.2-20.9 us.
template <int NT, bool F32, bool VEC, int ROWSTRIDE>
__device__ __forceinline__ void stage_store(const BmmArgs& p, int b, int mt, int c0, uint32_t stg, int quarter,
                                            uint32_t lane) {
  constexpr int esz = F32 ? 4 : 2;
  constexpr int EPP = 16 / esz;              // elements per piece
  constexpr int CPR = kWavesS * NT * esz;    // pieces per staged row
  constexpr int PER = 4 * CPR / 64;          // pieces per lane
  static_assert(4 * CPR % 64 == 0, "whole pieces per lane");
  const int m0 = mt * 16;
  const int rows = max(0, min(16, p.M - m0));
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(reinterpret_cast<uint8_t*>(p.out) + ((int64_t)b * p.sob + (int64_t)m0 * p.som) * esz,
                rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * p.som + p.N) * esz) : 0u);
  v4i v[PER];
  int n[PER];
  bool ok[PER];
  uint32_t base[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const uint32_t k = lane + 64u * e;
    const uint32_t row = (uint32_t)quarter * 4u + k / CPR, piece = k % CPR;
    n[e] = c0 * 16 + (int)piece * EPP;
    ok[e] = (int)row < rows;
    base[e] = (uint32_t)(row * p.som + n[e]) * esz;
    ds_read16<0>(v[e], stg + row * ROWSTRIDE + piece * 16);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    asm volatile("" : "+v"(v[e]));
    if (VEC) {
      __builtin_amdgcn_raw_buffer_store_b128(v[e], ro, ok[e] && n[e] < p.N ? base[e] : kOOB, 0, 2);
    } else {
#pragma unroll
      for (int x = 0; x < EPP; ++x) {
        const uint32_t off = ok[e] && n[e] + x < p.N ? base[e] + x * esz : kOOB;
        const uint32_t word = (uint32_t)v[e][(x * esz) >> 2];
        if (F32)
          __builtin_amdgcn_raw_buffer_store_b32(word, ro, off, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(word >> (16 * (x & 1))), ro, off, 0, 0);
      }
    }
  }
}

}  // namespace

// KF: maximum K-fragments (K/32) held per column tile; NT: 16-column tiles
// per wave.  Grid: B heads x S workgroups per head x NB column blocks;
// workgroup (b, s, nb) takes m-tiles [s*T, min((s+1)*T, nmt)) and the
// 8*NT column tiles from 8*NT*nb (NB > 1 when there are few m-tiles: more
// workgroups, each with a smaller weight slice to load and dequantise).
template <int KF, int NT, bool F32, bool VEC, int NS>
__global__ __launch_bounds__(512, 1) void bmm_stream_kernel(BmmArgs p, int S, int T, int NB) {
  constexpr int KD = (KF + 3) / 4;  // loads per loading wave per m-tile
  constexpr int esz = F32 ? 4 : 2;
  using L = BmmLds<KF, NT, esz, NS>;
  constexpr int kStages = L::kStages;
  static_assert((kStages - 2) * KD <= 63, "loading waves' wait within the counter's range");
  // The stage, trash and staging addresses are absolute: this is the
  // kernel's only LDS allocation, so it starts at address 0.
  __shared__ int4 lds_raw[L::kBytes / 16];
  const uint32_t lane = lane_here();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool loader = wv < 4;
  const int nb = blockIdx.x % NB;
  const int b = (blockIdx.x / NB) / S;
  const int s = (blockIdx.x / NB) % S;
  const int cb = nb * kWavesS * NT;  // first column tile of this workgroup
  const int kf = p.K >> 5;
  const int nmt = (p.M + 15) >> 4;
  const int mt0 = s * T;
  const int cnt = max(0, min(T, nmt - mt0));  // m-tiles of this workgroup (uniform)
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)&lds_raw[0];

  // Weights of this wave's column tiles, loaded first (their wait then does
  // not cover the activation loads issued after them).
  const int s0 = cb + wv * NT;  // first 16-column strip
  const uint32_t r = lane & 15u;
  const auto rw = make_rsrc(p.w + (int64_t)b * p.Ns * p.Kt * 1024, (uint32_t)p.Ns * p.Kt * 1024u);
  const auto rs = make_rsrc(p.ws + (int64_t)b * p.Ns * p.G * 256, (uint32_t)p.Ns * p.G * 256u);
  // Scale dword (kb*16 + r) of group g holds the scales of K-fragments
  // c = 16g + kb + 4i, i = 0..3 (byte i): 4 dwords per 16 fragments.
  constexpr int KG = (KF + 15) / 16;  // scale groups
  constexpr int KU = (KF + 3) / 4;    // 1 KiB weight units per column tile
  int4 wunit[NT][KU];
  uint32_t wsc[NT][KG * 4];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int st = s0 + j;
    // Each 1 KiB unit (16 rows x 4 blocks) in one load, lane l taking slot
    // l (block l/16 of row l%16: contiguous across the wave); transposed
    // once loaded (below).  Units past K load zeros.
#pragma unroll
    for (int t = 0; t < KU; ++t) {
      const bool ok = st < p.Ns && t * 4 < kf;
      wunit[j][t] = buf_load16(rw, ok ? (uint32_t)((st * p.Kt + t) * 1024) + lane * 16u : kOOB);
    }
#pragma unroll
    for (int g = 0; g < KG; ++g)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bool ok = st < p.Ns && g * 16 + kb < kf;
        wsc[j][g * 4 + kb] = buf_load4(rs, ok ? (uint32_t)((st * p.G + g) * 256 + (kb * 16 + r) * 4) : kOOB);
      }
  }

  // Activation m-tiles 0..kStages-2 in flight.
  if (loader) {
#pragma unroll
    for (int x = 0; x < kStages - 1; ++x)
      issue_xtile<KD, KF, L::kStage, L::kTrash>(p, b, mt0 + x, x < cnt ? nmt : 0, x, kf, wv, lane);
  }

  // Each unit transposed across the four 16-lane rows: lane (q, r) then
  // holds dword q of each of the unit's four blocks of row r, its MFMA
  // operand (blocks past K are zero in the preshuffled data).
  uint32_t wword[NT][KF];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int t = 0; t < KU; ++t) {
      uint32_t d[4] = {(uint32_t)wunit[j][t].x, (uint32_t)wunit[j][t].y, (uint32_t)wunit[j][t].z,
                       (uint32_t)wunit[j][t].w};
      transpose_rows4(d);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        if (t * 4 + kb < KF) wword[j][t * 4 + kb] = d[kb];
    }

  // Dequantise the weights (exact).  An invalid fragment loaded zeros: code
  // 0 gives 0.  (One fragment at a time: the scheduling barriers keep the
  // compiler from interleaving all of them, whose temporaries would not fit
  // in registers.)
  v8bf wf[NT][KF];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int c = 0; c < KF; ++c) {
      wf[j][c] = dequant8(wword[j][c], (wsc[j][(c >> 4) * 4 + (c & 3)] >> (8 * ((c >> 2) & 3))) & 0xFFu);
      __builtin_amdgcn_sched_barrier(0);
    }

  const uint32_t stg = lds0 + L::kStg;                           // staging buffer 0
  const uint32_t slot = stg + (uint32_t)wv * L::kRowB;               // this wave's columns in it
  for (int i = 0; i < cnt; ++i) {
    const int stage = i % kStages;
    // Loading waves: their loads of m-tile i were issued kStages-1
    // iterations ago, each iteration since adding KD loads.
    if (loader) wait_vm<(kStages - 2) * KD>();
    // This wave's staging writes of m-tile i-1 done before the barrier.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_nofence();  // m-tile i landed everywhere; stage (i-1) % kStages and staging buffer (i-1) & 1 are complete
    if (loader) {
      issue_xtile<KD, KF, L::kStage, L::kTrash>(p, b, mt0 + i + kStages - 1, i + kStages - 1 < cnt ? nmt : 0,
                                                (i + kStages - 1) % kStages, kf, wv, lane);
    } else if (i > 0) {
      // Storing waves: rows 4*(wv-4)..+3 of m-tile i-1.
      const uint32_t buf = (uint32_t)((i - 1) & 1) * L::kStgBuf;
      stage_store<NT, F32, VEC, L::kRowStride>(p, b, mt0 + i - 1, cb, stg + buf, wv - 4, lane);
    }
    // PA partial sums per column tile (fragment c adds into part c % PA), so
    // several independent accumulation chains keep the MFMA pipe busy; the
    // parts are added in a fixed order at the end (deterministic).
    constexpr int PA0 = 4 / NT < 1 ? 1 : 4 / NT;
    constexpr int PA = PA0 < KF ? PA0 : KF;
    v4f part[NT][PA];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int a = 0; a < PA; ++a) part[j][a] = (v4f){0.f, 0.f, 0.f, 0.f};
    const uint32_t xa = lds0 + (uint32_t)stage * L::kStage + lane * 16;
    // Fragments in chunks of up to 16: all of a chunk's reads are issued,
    // then each fragment's MFMAs start as soon as that read has returned.
    constexpr int CK = KF < 16 ? KF : 16;
#pragma unroll
    for (int c0 = 0; c0 < KF; c0 += CK) {
      v4i xf[CK];
#pragma unroll
      for (int c = 0; c < CK; ++c)
        if (c0 + c < KF) read_frag(xf[c], xa + (uint32_t)(c0 + c) * 1024u);
#pragma unroll
      for (int c = 0; c < CK; ++c)
        if (c0 + c < KF) {
          const int left = (KF - c0 < CK ? KF - c0 : CK) - 1 - c;  // reads issued after this one
          wait_lgkm_n(xf[c], left);
#pragma unroll
          for (int j = 0; j < NT; ++j)
            part[j][(c0 + c) % PA] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                wf[j][c0 + c], __builtin_bit_cast(v8bf, xf[c]), part[j][(c0 + c) % PA], 0, 0, 0);
        }
    }
    v4f acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int w = PA; w > 1; w = (w + 1) / 2)
#pragma unroll
        for (int a = 0; a + (w + 1) / 2 < w; ++a) part[j][a] += part[j][a + (w + 1) / 2];
      acc[j] = part[j][0];
    }
    stage_write<NT, F32, L::kRowStride>(acc, slot + (uint32_t)(i & 1) * L::kStgBuf, lane);
  }
  // The last m-tile's stores, once every wave has staged it.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier_nofence();
  if (!loader && cnt > 0) {
    const uint32_t buf = (uint32_t)((cnt - 1) & 1) * L::kStgBuf;
    stage_store<NT, F32, VEC, L::kRowStride>(p, b, mt0 + cnt - 1, cb, stg + buf, wv - 4, lane);
  }
  // Loads issued past the last m-tile (empty descriptors) still write LDS:
  // let them finish before the workgroup ends.
  wait_vm<0>();
}

hipError_t launch_bmm_a16w4(const void* x, int64_t sxb, int64_t sxm, const void* w,
                            const void* ws, void* out, int64_t sob, int64_t som, int out_f32,
                            int64_t B, int64_t M, int64_t N, int64_t K, hipStream_t stream, int cus) {
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

  // Streaming kernel when a wave's weight slice fits in registers and 16
  // rows of output and activations stay within 32-bit buffer offsets.
  const int kf = (int)(K / 32);
  const int nt = (p.Ns + kWavesS - 1) / kWavesS;
  const int esz = out_f32 ? 4 : 2;
  const bool offsets_ok = (15 * som + N) * esz <= 0x7FFFFFFF && (15 * sxm + K) * 2 <= 0x7FFFFFFF;
  const int nmt = (int)((M + 15) / 16);
  // Few m-tiles (M <= 64): one column tile per wave and the head's columns
  // split over NB workgroups (the activations, small here, are read once per
  // block).  Measured on MI355X: M = 1 K-up 5.8 -> 3.6 us, V-up 7.4 -> 5.5 us;
  // slower from 16 m-tiles on.
  const bool small = nmt <= 4;
  int cfg = 0, NB = 1;
  if (offsets_ok) {
    if (small && kf <= 32) {
      cfg = kf == 6 ? 5 : kf <= 8 ? 6 : kf <= 16 ? 7 : 3;
      NB = (p.Ns + kWavesS - 1) / kWavesS;
    } else if (nt <= 4 && kf == 6) cfg = 4;  // MLA K-up heads (K = 192)
    else if (nt <= 4 && kf <= 8) cfg = 1;
    else if (nt <= 2 && kf <= 16) cfg = 2;
    else if (nt <= 1 && kf <= 32) cfg = 3;
  }
  // A few m-tiles per workgroup (5 to 32 m-tiles per head at K = 192, 5 to
  // 15 at K = 512, with 16 heads on 256 compute units): the head's columns
  // over two workgroups, each loading and dequantising half the weights and
  // reading the activations itself.  Measured on MI355X, back-to-back
  // launches (us, whole head / two column halves): K-up M = 80 4.60 / 3.65,
  // M = 128 4.67 / 3.76, M = 256 5.06 / 4.53, M = 512 6.28 / 6.18, M = 1024
  // 8.00 / 8.76; V-up M = 128 5.13 / 4.18, M = 192 5.22 / 5.09, M = 256
  // 5.34 / 5.93.
  const int s_full = (int)((cus + B - 1) / B);
  if (cfg == 4 && nt > 2 && nmt <= 2 * s_full) {
    cfg = 8;
    NB = 2;
  } else if (cfg == 2 && kf == 16 && nt == 2 && nmt < s_full) {
    cfg = 9;
    NB = 2;
  }
  if (cfg) {
    // Workgroups per head and column block: enough to fill the device (the
    // small-M blocks keep those of a whole head), each with whole m-tiles.
    int S = small ? s_full : (int)((cus + B * NB - 1) / (B * NB));
    if (S > nmt) S = nmt;
    if (S < 1) S = 1;
    const int T = (nmt + S - 1) / S;
    S = (nmt + T - 1) / T;
    // vector mode: whole 16-byte pieces of output rows
    const int per = 16 / esz;
    const bool vec = N % per == 0 && som % per == 0 && sob % per == 0 && ((uintptr_t)out & 15) == 0;
    const dim3 grid((unsigned)(B * S * NB)), block(64 * kWavesS);
#define MXFP4_BMM_LAUNCH_NS(KF_, NT_, NS_)                                                                      \
  do {                                                                                                          \
    if (out_f32 && vec) bmm_stream_kernel<KF_, NT_, true, true, NS_><<<grid, block, 0, stream>>>(p, S, T, NB);  \
    else if (out_f32) bmm_stream_kernel<KF_, NT_, true, false, NS_><<<grid, block, 0, stream>>>(p, S, T, NB);   \
    else if (vec) bmm_stream_kernel<KF_, NT_, false, true, NS_><<<grid, block, 0, stream>>>(p, S, T, NB);       \
    else bmm_stream_kernel<KF_, NT_, false, false, NS_><<<grid, block, 0, stream>>>(p, S, T, NB);               \
  } while (0)
#define MXFP4_BMM_LAUNCH(KF_, NT_)                   \
  do {                                               \
    if (T <= 4) MXFP4_BMM_LAUNCH_NS(KF_, NT_, 2);    \
    else MXFP4_BMM_LAUNCH_NS(KF_, NT_, 3);           \
  } while (0)
    if (cfg == 4) MXFP4_BMM_LAUNCH(6, 4);
    else if (cfg == 8) MXFP4_BMM_LAUNCH(6, 2);
    else if (cfg == 9) MXFP4_BMM_LAUNCH(16, 1);
    else if (cfg == 1) MXFP4_BMM_LAUNCH(8, 4);
    else if (cfg == 2) MXFP4_BMM_LAUNCH(16, 2);
    else if (cfg == 5) MXFP4_BMM_LAUNCH_NS(6, 1, 2);
    else if (cfg == 6) MXFP4_BMM_LAUNCH_NS(8, 1, 2);
    else if (cfg == 7) MXFP4_BMM_LAUNCH_NS(16, 1, 2);
    else MXFP4_BMM_LAUNCH(32, 1);
#undef MXFP4_BMM_LAUNCH_NS
#undef MXFP4_BMM_LAUNCH
    return hipGetLastError();
  }

  constexpr int MTW = 4, NTW = 2;
  const dim3 grid((unsigned)((M + MTW * 16 - 1) / (MTW * 16)),
                  (unsigned)((N + 4 * NTW * 16 - 1) / (4 * NTW * 16)), (unsigned)B);
  bmm_a16w4_kernel<MTW, NTW><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace mxfp4
