// W4A4 block-scaled FP4 GEMM for large M (prefill) on gfx950.
//
// Same operation as the decode kernel (P2 §2: quantised activations times
// the preshuffled [N, K] weight, NT form, bias after; P1 §Accuracy Tests:
// equal to the dequantised reference), organised for the MFMA roofline:
//
//  * persistent: one 512-thread workgroup per compute unit walks a list of
//    256 x 256 output tiles (or 256 x 128: this source built again with
//    MXFP4_PREFILL_BN = 128, for shapes where 256-wide tiles would leave
//    most compute units idle).  Its 8 waves (two per SIMD, so one can issue
//    while the other waits) form a 2 x 4 grid of 128 x 64 (128 x 32) wave
//    tiles, 8 x 4 (8 x 2) MFMA tiles of 16 x 16 each (128 (64) fp32
//    accumulators per lane);
//  * operands stream through four single-K-step LDS stages (32 (24) KiB each):
//    every 1 KiB operand unit of the GEMM layouts (activations and weights
//    alike) is fetched by one buffer_load_dwordx4 ... lds, so LDS holds
//    fragments in the lane order the MFMA consumes (conflict-free
//    ds_read_b128).  Loads run three K-steps ahead, across tile boundaries:
//    the last steps of a tile already fetch the first steps of the next;
//  * one barrier per K-step, in its middle: before it, hand-counted waits for
//    this wave's loads of the next step; after it, the freed stage is
//    refilled and the next step's fragments are read while the rest of this
//    step's MFMAs run;
//  * block scales: one dword per lane per 16-row tile per 4 K-steps.  The
//    next group's scales go to LDS by the same kind of load and are read into
//    registers at the group boundary; op_sel walks the 4 K-steps of a dword;
//  * the MFMA takes the weight as its A operand and the activations as B, so
//    a lane ends with 4 consecutive output columns of one row; the epilogue
//    adds the bias in fp32, rounds once and stores straight from registers
//    (buffer stores, out-of-range lanes masked by offset) while the next
//    tile's operands are already in flight;
//  * tiles are ordered in groups of 8 row-tiles; each XCD's workgroups take
//    consecutive tiles, so the tiles in flight on an XCD share its L2;
//  * split schedule, where whole tiles would leave the last round of
//    workgroups part-empty: the r tiles short of whole rounds are each cut
//    along K into s slices of whole groups of 4 K-steps (s = workgroups / r,
//    at most the groups a tile has), and each workgroup takes one slice
//    before its whole tiles.  Slices are dealt slice-major (workgroup
//    j r + t takes slice j of tile t), so the workgroups of one slice run
//    at the same K at the same time, like whole tiles, and share operands in
//    L2; and the slices come first, so their parts' memory traffic overlaps
//    other workgroups' whole tiles.  Each slice takes an arrival ticket for
//    its tile; every slice but the last to arrive stores its fp32
//    accumulators to the workspace (device-scope stores) and raises a flag;
//    the last adds the slices in K order (so the sum does not depend on
//    arrival order) and runs the tile's epilogue.  Only that last slice
//    ever waits, and only for slices whose workgroups already hold a
//    ticket, so the wait always ends.
//
// Every register counts: at two waves per SIMD a wave has 256 registers, 128
// of them accumulators and 64 operand fragments (256 wide).
#include "mxfp4_device.h"
#include "mxfp4_launch.h"

#ifndef MXFP4_PREFILL_BN
#define MXFP4_PREFILL_BN 256
#endif
#if MXFP4_PREFILL_BN == 256
#define MXFP4_PREFILL_KERNEL gemm_prefill_kernel
#define MXFP4_PREFILL_TILES launch_prefill_tiles_256
#else
#define MXFP4_PREFILL_KERNEL gemm_prefill_n128_kernel
#define MXFP4_PREFILL_TILES launch_prefill_tiles_128
#endif

namespace mxfp4 {

namespace {

// Output tile width: 256 (this file as it stands) or 128 (the same source
// built again with MXFP4_PREFILL_BN = 128, for M where 256-wide tiles
// leave most compute units idle).  The tile is 256 rows either way.
constexpr int kBM = 256, kBN = MXFP4_PREFILL_BN;
static_assert(kBN == 256 || kBN == 128, "tile width");
constexpr int kTilesA = kBM / 16;            // 16 activation units per K-step
constexpr int kTilesB = kBN / 16;            // 16 (8) weight units per K-step
constexpr int kUnits = kTilesA + kTilesB;    // 32 (24) units of 1 KiB per K-step
constexpr int kBufs = 4;                     // LDS stages (K-steps in flight)
constexpr int kWaves = 8;
constexpr int kLoadsPerWave = kUnits / kWaves;  // 4 (3) buffer->LDS loads per wave per step
constexpr int kWM = 8, kWN = kBN / 64;          // wave tile: 8 x 4 (8 x 2) MFMA tiles, 128 x 64 (128 x 32)
constexpr int kScaleLoads = kUnits / 4;         // scale loads of a group (4 tiles each): one per wave (6 of 8)
constexpr int kGroupM = 8;                   // row-tiles per ordering group
// LDS: unit u of stage b at u * 4 KiB + b * 1 KiB (so a wave reaches its
// fragments in all four stages from one base register), then the scales of
// one group: 16 activation tiles, then the weight strips, 256 bytes each;
// then each wave's bias values of the tile (256 bytes per wave); then each
// wave's 16-row bf16 staging area of the epilogue; then the arrival rank;
// then (128-wide) a dummy 1 KiB for the scale loads of waves that have none.
constexpr int kStageBytes = kUnits * kBufs * 1024;  // 128 (96) KiB
constexpr int kScaleLds = kStageBytes;
constexpr int kBiasLds = kScaleLds + kUnits * 256;  // + 8 (6) KiB
constexpr int kEpiRowB = kWN * 32 + 16;              // epilogue staging row stride (bytes)
constexpr int kEpiLds = kBiasLds + kWaves * 256;     // + 2 KiB
constexpr int kSkLds = kEpiLds + kWaves * 16 * kEpiRowB;     // + 18 (10) KiB
constexpr int kDummyLds = kSkLds + 16;
constexpr int kLdsBytes = kDummyLds + (kScaleLoads < kWaves ? 1024 : 0);  // 156 KiB in all (113)
static_assert(kLdsBytes <= 160 * 1024, "LDS per workgroup");
#ifndef MXFP4_STORE_AUX
#define MXFP4_STORE_AUX 0
#endif
// Cache policy of the staged bf16 epilogue's stores (not read again by this
// kernel): non-temporal where a wave's row piece is a whole 128-byte line
// (256 wide).  Measured on MI355X: 1-2% faster at five of the six M >= 2048
// prefill shapes (e.g. M = 8192, N = 5120, K = 14336 295 -> 289 us), no
// change at the sixth; on half lines non-temporal stores were slower.
constexpr int kStagedStoreAux = kWN == 4 ? 2 : 0;
// Staged epilogues: a wave's 16-row block is read back as 16-byte pieces of
// whole rows, kLpr lanes per row (16 kWN columns of bf16), so each lane
// holds 8 consecutive columns of a row, kWN / 2 pieces per block.
constexpr int kLpr = 2 * kWN;
constexpr int kLprShift = kWN == 4 ? 3 : 2;

// Split schedule of one launch (PrefillSplit): tiles [0, r) of the tile
// order are cut into s slices each (r = 0: whole tiles only).  Workspace:
// a give-up word, an arrival counter per split tile and a ready flag per
// slot, all zeroed before every launch, then one fp32 part slot of a tile per
// slice (slot = the slice's workgroup).
using SkArgs = PrefillSplit;
constexpr uint32_t kPartBytes = kBM * kBN * 4;  // 256 (128) KiB: one tile's fp32 accumulators
// Cache policy of the part stores and loads: device scope (sc1), as the
// memory model's relaxed device-scope atomics: written through, and read
// past, the XCD-local caches, so another XCD's part is seen once its flag
// is.  (Measured: no slower than cached accesses.)
constexpr int kPartAux = 16;
constexpr int kSpinLimit = 1 << 20;  // ready-flag polls before giving up (a guard: about a second)

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// Fragment registers: a native 4 x 32-bit vector, so inline assembly can take
// it as a register operand.
typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ lds_ptr_t lds_at(uint32_t addr) { return (lds_ptr_t)(uintptr_t)addr; }

// Lane id, recomputed where it is used (two instructions): a volatile
// statement the compiler cannot hoist into a register that would stay live
// through the K loop, where every register counts.
__device__ __forceinline__ uint32_t lane_here() {
  uint32_t l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

template <int SEL>
__device__ __forceinline__ v4f mfma_fp4v(v4i a, v4i b, uint32_t sa, uint32_t sb, v4f acc) {
  const v8i A = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  const v8i B = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 4, SEL, (int)sa, SEL, (int)sb);
}

// One output tile: its first 16-row activation strip and strip count, its
// first 16-column weight strip and strip count (counts are 0 for an empty
// tile past the end).  Buffer descriptors are derived from it where a load is
// issued, after any selection between tiles: a select between descriptors
// becomes a vector select, which then costs a waterfall loop per load.
// A work item: the groups [g0, g1) of 4 K-steps of one tile (a slice of a
// split tile unless that is all G of them).
struct Tile {
  int ms, mstrips, s0, strips;
  int g0, g1;
};

// Linear tile L (all its groups): tiles run down groups of kGroupM
// row-tiles, then across columns.
__device__ __forceinline__ Tile tile_at(const GemmArgs& p, int L, int tiles_m, int tiles_n) {
  Tile t = {0, 0, 0, 0, 0, 0};
  if (L >= tiles_m * tiles_n) return t;
  t.g1 = p.G;
  const int group = L / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int r = L % (kGroupM * tiles_n);
  t.ms = (first_m + r % gm) * kTilesA;
  t.mstrips = min(kTilesA, ((p.M + 15) >> 4) - t.ms);
  t.s0 = (r / gm) * kTilesB;
  t.strips = min(kTilesB, p.Ns - t.s0);
  return t;
}

// This workgroup's share of a launch: first, if slot < r s, slice
// slot / r of split tile slot % r (nsk = 1); then the whole tiles
// r + k grid + slot.
struct Share {
  int slot, grid, nsk, n;
};

// Groups [g0, g1) of slice j of s: the G groups cut as evenly as whole
// groups allow.
__device__ __forceinline__ Tile work_at(const GemmArgs& p, const SkArgs& sk, const Share& s, int i, int tiles_m,
                                        int tiles_n) {
  if (i < s.nsk) {
    const int j = s.slot / sk.r;
    Tile tl = tile_at(p, s.slot - j * sk.r, tiles_m, tiles_n);
    tl.g0 = j * p.G / sk.s;
    tl.g1 = (j + 1) * p.G / sk.s;
    return tl;
  }
  return tile_at(p, sk.r + (i - s.nsk) * s.grid + s.slot, tiles_m, tiles_n);
}

// This wave's buffer->LDS load of unit q (of its 4) of K-step t of tile
// `tl` into stage J.  Waves 0-3 fetch the 16 activation units, waves 4-7 the
// 16 weight units.  Each unit has its own descriptor (the unit's row of
// K-steps); units past the tile's last strip and steps past K get an empty
// one and load zeros.  The vector offset is the lane's 16 bytes, the step
// goes in the scalar offset (in range whenever the descriptor is not empty).
__device__ __forceinline__ void issue_unit(const GemmArgs& p, const Tile& tl, int J, int t, int q, int wv,
                                           uint32_t lane16) {
  // unit gu of the step's kUnits (activation units first): wave wv loads
  // units wv * kLoadsPerWave + q (all activation units in waves 0-3 at
  // 256 wide; at 128 wide wave 5 loads one of each kind)
  const int gu = wv * kLoadsPerWave + q;
  const bool is_a = gu < kTilesA;
  const int first = is_a ? tl.ms : tl.s0;
  const int count = t < p.Kt ? (is_a ? tl.mstrips : tl.strips) : 0;
  const uint8_t* base = is_a ? p.a : p.w;
  const int u = is_a ? gu : gu - kTilesA;
  const uint32_t row_bytes = (uint32_t)p.Kt * 1024u;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (int64_t)(first + u) * row_bytes, u < count ? row_bytes : 0u);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_at((gu * kBufs + J) * 1024), 16, lane16, t << 10, 0, 0);
}

__device__ __forceinline__ void issue_step(const GemmArgs& p, const Tile& tl, int J, int t, int wv,
                                           uint32_t lane16) {
#pragma unroll
  for (int q = 0; q < kLoadsPerWave; ++q) issue_unit(p, tl, J, t, q, wv, lane16);
}

// This wave's one buffer->LDS load of the scales of group g of tile `tl`:
// wave w fetches the 4 tiles 4w..4w+3 of the step's units (activation tiles
// first, then weight strips; lane l: tile l/16, bytes (l%16)*16 of its
// 256).  Tiles past the last strip fall outside the descriptor through the
// vector offset (zeros), and an empty descriptor covers groups past K (the
// group goes in the scalar offset) and, at 128 wide, waves 6-7, whose zeros
// land in a dummy area: every wave issues the load, so the waits count the
// same operations in every wave.
__device__ __forceinline__ void issue_scales(const GemmArgs& p, const Tile& tl, int g, int wv) {
  const int gt = wv * 4;
  const bool is_a = gt < kTilesA;
  const bool none = gt >= kUnits;
  const int first = is_a ? tl.ms : tl.s0;
  const int count = none ? 0 : is_a ? tl.mstrips : tl.strips;
  const int rt0 = is_a ? gt : gt - kTilesA;
  const int G = p.G;
  const int left = __builtin_amdgcn_readfirstlane(max(0, count - rt0));
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc((is_a ? p.as : p.ws) + (int64_t)(first + rt0) * G * 256, g < G ? (uint32_t)(left * G * 256) : 0u);
  const uint32_t lds = none ? (uint32_t)kDummyLds : (uint32_t)(kScaleLds + gt * 256);
  const uint32_t l = lane_here();
  const uint32_t svoff = (l >> 4) * (uint32_t)(G * 256) + (l & 15) * 16;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_at(lds), 16, svoff, g << 8, 0, 0);
}

// This wave's buffer->LDS load of the bias of its 16 kWN output columns of
// tile `tl` (lanes 0 .. 8 kWN - 1 one bf16 pair each; N is a multiple of 4
// here, so the window ends on a whole pair; no bias: an empty window,
// zeros).
__device__ __forceinline__ void issue_bias(const GemmArgs& p, const Tile& tl, int wv, int wn) {
  const uint32_t lane = lane_here();
  const int col0 = (tl.s0 + wn * kWN) * 16;
  const int cols = __builtin_amdgcn_readfirstlane(p.bias ? max(0, min(16 * kWN, p.N - col0)) : 0);
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc(p.bias ? (const void*)(p.bias + col0) : (const void*)p.a, (uint32_t)(cols * 2));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_at(kBiasLds + wv * 256), 4, lane < 8 * kWN ? lane * 4 : kOOB, 0,
                                           0, 0);
}

// LDS reads are written as inline assembly with hand-counted lgkmcnt
// waits.  The compiler cannot tell the LDS written by buffer->LDS loads from
// the LDS these reads use, so for its own LDS reads it would wait for every
// buffer->LDS load in flight (draining the prefetch) and sink each read to
// just before its first use.
template <int OFF>
__device__ __forceinline__ void ds_read16(v4i& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_read4(uint32_t& v, uint32_t addr) {
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
typedef int v2i __attribute__((ext_vector_type(2)));
template <int OFF>
__device__ __forceinline__ void ds_read8(v2i& v, uint32_t addr) {
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_write8(uint32_t addr, v2i v) {
  asm volatile("ds_write_b64 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF));
}
__device__ __forceinline__ void ds_write4(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v));
}

// lgkmcnt(N) waits that the given registers depend on, so no MFMA reading
// them is scheduled above it.
template <int N>
__device__ __forceinline__ void wait_lgkm(v4i& a, v4i& b, v4i& c, v4i& d) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "i"(N));
}
template <int N>
__device__ __forceinline__ void wait_lgkm_scales(uint32_t (&sa)[kWM], uint32_t (&sb)[kWN]) {
  if constexpr (kWN == 4) {
    asm volatile("s_waitcnt lgkmcnt(%12)"
                 : "+v"(sa[0]), "+v"(sa[1]), "+v"(sa[2]), "+v"(sa[3]), "+v"(sa[4]), "+v"(sa[5]), "+v"(sa[6]),
                   "+v"(sa[7]), "+v"(sb[0]), "+v"(sb[1]), "+v"(sb[2]), "+v"(sb[3])
                 : "i"(N));
  } else {
    asm volatile("s_waitcnt lgkmcnt(%10)"
                 : "+v"(sa[0]), "+v"(sa[1]), "+v"(sa[2]), "+v"(sa[3]), "+v"(sa[4]), "+v"(sa[5]), "+v"(sa[6]),
                   "+v"(sa[7]), "+v"(sb[0]), "+v"(sb[1])
                 : "i"(N));
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// vmcnt(N_SET) if `flag` (a uniform value) is non-zero, else vmcnt(N).  The
// branch stays inside one assembly statement: as control flow the compiler
// would see, it costs register copies around the whole K loop.
template <int N, int N_SET>
__device__ __forceinline__ void wait_vm_sel(int flag) {
  if (N == N_SET) {
    wait_vm<N>();
  } else {
    asm volatile(
        "s_cmp_eq_u32 %0, 0\n\t"
        "s_cbranch_scc1 1f\n\t"
        "s_waitcnt vmcnt(%2)\n\t"
        "s_branch 2f\n"
        "1:\n\t"
        "s_waitcnt vmcnt(%1)\n"
        "2:" ::"s"(flag),
        "i"(N), "i"(N_SET)
        : "memory", "scc");
  }
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

// LDS base addresses of this lane's fragment reads: activation fragments
// (unit wm*8) and weight fragments (unit 16 + wn*4).
struct ReadAddr {
  uint32_t a, b;
};

// First half of stage BUF's fragments (weights 0-3, activations 0-3), then
// the second half (activations 4-7): 8 + 4 LDS reads in this order.
template <int BUF>
__device__ __forceinline__ void read_first_half(v4i (&af)[kWM], v4i (&bf)[kWN], const ReadAddr& ra) {
  ds_read16<0 * 4096 + BUF * 1024>(bf[0], ra.b);
  ds_read16<1 * 4096 + BUF * 1024>(bf[1], ra.b);
  if constexpr (kWN == 4) {
    ds_read16<2 * 4096 + BUF * 1024>(bf[2], ra.b);
    ds_read16<3 * 4096 + BUF * 1024>(bf[3], ra.b);
  }
  ds_read16<0 * 4096 + BUF * 1024>(af[0], ra.a);
  ds_read16<1 * 4096 + BUF * 1024>(af[1], ra.a);
  ds_read16<2 * 4096 + BUF * 1024>(af[2], ra.a);
  ds_read16<3 * 4096 + BUF * 1024>(af[3], ra.a);
}
template <int BUF>
__device__ __forceinline__ void read_second_half(v4i (&af)[kWM], const ReadAddr& ra) {
  ds_read16<4 * 4096 + BUF * 1024>(af[4], ra.a);
  ds_read16<5 * 4096 + BUF * 1024>(af[5], ra.a);
  ds_read16<6 * 4096 + BUF * 1024>(af[6], ra.a);
  ds_read16<7 * 4096 + BUF * 1024>(af[7], ra.a);
}
// The 12 scale dwords of the group in LDS.
__device__ __forceinline__ void read_scales(uint32_t (&sa)[kWM], uint32_t (&sb)[kWN], int wm, int wn) {
  const uint32_t l4 = lane_here() * 4;
  const uint32_t a = l4 + (uint32_t)(kScaleLds + wm * kWM * 256);
  const uint32_t b = l4 + (uint32_t)(kScaleLds + (kTilesA + wn * kWN) * 256);
  ds_read4<0 * 256>(sa[0], a);
  ds_read4<1 * 256>(sa[1], a);
  ds_read4<2 * 256>(sa[2], a);
  ds_read4<3 * 256>(sa[3], a);
  ds_read4<4 * 256>(sa[4], a);
  ds_read4<5 * 256>(sa[5], a);
  ds_read4<6 * 256>(sa[6], a);
  ds_read4<7 * 256>(sa[7], a);
  ds_read4<0 * 256>(sb[0], b);
  ds_read4<1 * 256>(sb[1], b);
  if constexpr (kWN == 4) {
    ds_read4<2 * 256>(sb[2], b);
    ds_read4<3 * 256>(sb[3], b);
  }
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

template <int SEL, int I>
__device__ __forceinline__ void mfma_row(v4f (&acc)[kWM][kWN], const v4i (&af)[kWM], const v4i (&bf)[kWN],
                                         const uint32_t (&sa)[kWM], const uint32_t (&sb)[kWN]) {
#pragma unroll
  for (int j = 0; j < kWN; ++j) acc[I][j] = mfma_fp4v<SEL>(bf[j], af[I], sb[j], sa[I], acc[I][j]);
}

// Zero accumulators, each from its own opaque statement: from one shared
// zero the compiler would keep a single zero register live through the loop
// (or specialise the first K-step), both of which cost registers.
__device__ __forceinline__ void zero_acc(v4f (&acc)[kWM][kWN]) {
#pragma unroll
  for (int i = 0; i < kWM; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j) {
      float z0, z1, z2, z3;
      asm volatile("v_mov_b32 %0, 0\n\tv_mov_b32 %1, 0\n\tv_mov_b32 %2, 0\n\tv_mov_b32 %3, 0"
                   : "=v"(z0), "=v"(z1), "=v"(z2), "=v"(z3));
      acc[i][j] = (v4f){z0, z1, z2, z3};
    }
}

// Per-wave state of the K loop.
struct Pipe {
  v4f acc[kWM][kWN];
  v4i af[kWM], b0[kWN], b1[kWN];
  uint32_t sa[kWM], sb[kWN];
};

// One K-step (step J of a group of 4), its operands in stage J:
//  * rows 0-3 (their fragments, the weight fragments and at J == 0 the
//    group's scales were read before the previous step's last 4 reads: wait
//    for all but those);
//  * then the step's one barrier.  Before it this wave's reads of stage J
//    are done and its buffer->LDS loads of the next step have landed; after
//    it the first half of the next step's fragments is read from stage J+1
//    (weights into the other weight set), and stage J is refilled with step
//    `td` of tile `dt` (four steps on in the stream of steps, possibly in
//    the next tile; at J == 0 after the scales of group td/4 and the bias of
//    the current tile `ct`), one unit after each of rows 4-7;
//  * at J == 3 the next group's scales are read (they landed with the loads
//    the barrier waited for); then the second half of the next step's
//    fragments.
// Loads in flight issued after the ones the next step needs: two steps of 4
// loads plus, for J = 1 and 2, the scale and bias loads issued at J = 0,
// plus, in a tile's first group (`first`), the kStores output stores of the
// previous tile's epilogue (or the prologue's dropped stores).
template <int J, int kStores, bool kBias>
__device__ __forceinline__ void main_step(const GemmArgs& p, Pipe& P, v4i (&bf_cur)[kWN], v4i (&bf_nxt)[kWN],
                                          const Tile& dt, const Tile& ct, int td, int first, int wv, int wm,
                                          int wn, const ReadAddr& ra, uint32_t lane16) {
  constexpr int kNext = (J + 1) & 3;
  constexpr int kAfter = 2 * kLoadsPerWave + ((J == 1 || J == 2) ? 1 + (kBias ? 1 : 0) : 0);
  wait_lgkm<4>(P.af[0], P.af[1], P.af[2], P.af[3]);
  wait_lgkm<4>(bf_cur[0], bf_cur[1], bf_cur[2], bf_cur[3]);
  if (J == 0) wait_lgkm_scales<4>(P.sa, P.sb);
  mfma_rows<J, 0>(P.acc, P.af, bf_cur, P.sa, P.sb);
  __builtin_amdgcn_sched_barrier(0);
  wait_lgkm<0>(P.af[4], P.af[5], P.af[6], P.af[7]);
  wait_vm_sel<kAfter, kAfter + (J < 3 ? kStores : 0)>(first);
  barrier_nofence();
  read_first_half<kNext>(P.af, bf_nxt, ra);
  // Rows 4-7 with this wave's buffer->LDS loads spread between them: issued
  // back to back by all waves right after the barrier, they would queue up
  // in the address unit and stall instruction issue (and the MFMAs behind).
  if (J == 0) issue_scales(p, dt, td >> 2, wv);
  if (J == 0 && kBias) issue_bias(p, ct, wv, wn);
  __builtin_amdgcn_sched_barrier(0);
  mfma_row<J, 4>(P.acc, P.af, bf_cur, P.sa, P.sb);
  issue_unit(p, dt, J, td, 0, wv, lane16);
  __builtin_amdgcn_sched_barrier(0);
  mfma_row<J, 5>(P.acc, P.af, bf_cur, P.sa, P.sb);
  issue_unit(p, dt, J, td, 1, wv, lane16);
  __builtin_amdgcn_sched_barrier(0);
  mfma_row<J, 6>(P.acc, P.af, bf_cur, P.sa, P.sb);
  issue_unit(p, dt, J, td, 2, wv, lane16);
  __builtin_amdgcn_sched_barrier(0);
  mfma_row<J, 7>(P.acc, P.af, bf_cur, P.sa, P.sb);
  if constexpr (kLoadsPerWave == 4) issue_unit(p, dt, J, td, 3, wv, lane16);
  __builtin_amdgcn_sched_barrier(0);
  if (J == 3) read_scales(P.sa, P.sb, wm, wn);
  read_second_half<kNext>(P.af, ra);
}

// Output store modes:
//  0  bf16, staged: each 16-row block goes through LDS and leaves as whole
//     16-byte pieces of output rows (N and ldo multiples of 8, 16-byte
//     aligned output): 16 stores per wave per tile;
//  1  bf16, single elements: 128 stores;
//  2  fp32, 4-column groups (16-byte stores; N and ldo multiples of 4,
//     16-byte aligned output): 32 stores;
//  3  fp32, single elements: 128 stores.
// The stores of modes 0 and 2 stay in flight into the next tile and are
// counted by its waits (vmcnt retires loads and stores in issue order); the
// 128 of an element mode would exceed the counter's range (63), so that
// epilogue waits for them instead.
template <int MODE>
struct OutMode {
  static constexpr bool kF32 = MODE == 2 || MODE == 3;
  static constexpr bool kFp4 = MODE == 4;
  static constexpr bool kStaged = MODE == 0 || MODE == 4;
  static constexpr bool kVec = MODE == 2;
  // per 16-row block: kWN / 2 row-piece stores (bf16), or as many code and
  // as many scale stores (MXFP4)
  static constexpr int kStores = MODE == 0 ? kWN / 2 * kWM : kFp4 ? kWN * kWM : kVec ? kWM * kWN : 4 * kWM * kWN;
  static constexpr bool kDrain = !kStaged && !kVec;
  static constexpr int kInFlight = kDrain ? 0 : kStores;  // stores the next tile's waits count
  static constexpr bool kBiasLds = !kDrain;  // bias staged in LDS (whole pairs: N % 4 == 0)
};

// This lane's 4 bias columns of each 16-column strip j of the wave (columns
// 16j + 4*(lane/16) ...), from the bias this wave staged in LDS.
__device__ __forceinline__ void read_bias(v2i (&bl)[kWN], int wv, int lane) {
  const uint32_t ba = kBiasLds + (uint32_t)(lane >> 4) * 8 + (uint32_t)wv * 256;
  ds_read8<0>(bl[0], ba);
  ds_read8<32>(bl[1], ba);
  if constexpr (kWN == 4) {
    ds_read8<64>(bl[2], ba);
    ds_read8<96>(bl[3], ba);
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bl[0]), "+v"(bl[1]), "+v"(bl[2]), "+v"(bl[3]));
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bl[0]), "+v"(bl[1]));
  }
}

// Staged bf16 epilogue (mode 0).  Per 16-row block i: each lane writes its
// 4 x kWN results (bias added in fp32, one rounding) to the wave's staging
// rows, then reads back kWN / 2 16-byte pieces of whole rows (kLpr lanes
// per row) and stores them.  The wave's own LDS operations run in order, so
// no barrier is needed.
__device__ __forceinline__ void epilogue_staged(const GemmArgs& p, const Tile& tl, v4f (&acc)[kWM][kWN], int wv,
                                                int wm, int wn) {
  const int lane = (int)lane_here();
  const int row0 = tl.ms * 16 + wm * 128;
  const int n = (tl.s0 + wn * kWN) * 16 + (lane & (kLpr - 1)) * 8;  // this lane's 8 stored columns
  v2i bl[kWN];
  read_bias(bl, wv, lane);
  const uint32_t wst = kEpiLds + (uint32_t)wv * 16 * kEpiRowB;
  const uint32_t waddr = wst + (uint32_t)(lane & 15) * kEpiRowB + (uint32_t)(lane >> 4) * 8;
  const uint32_t raddr = wst + (uint32_t)(lane >> kLprShift) * kEpiRowB + (uint32_t)(lane & (kLpr - 1)) * 16;
  const uint32_t voff0 = n < p.N ? (uint32_t)((lane >> kLprShift) * p.ldo + n) * 2 : kOOB;
  const uint32_t voff1 = n < p.N ? voff0 + (uint32_t)(8 * p.ldo) * 2 : kOOB;
  uint8_t* const out = reinterpret_cast<uint8_t*>(p.out);
#pragma unroll
  for (int i = 0; i < kWM; ++i) {
#pragma unroll
    for (int j = 0; j < kWN; ++j) {
      const float b0 = __uint_as_float((uint32_t)bl[j].x << 16), b1 = __uint_as_float((uint32_t)bl[j].x & 0xFFFF0000u);
      const float b2 = __uint_as_float((uint32_t)bl[j].y << 16), b3 = __uint_as_float((uint32_t)bl[j].y & 0xFFFF0000u);
      const uint32_t lo = pack_bf16x2(acc[i][j][0] + b0, acc[i][j][1] + b1);
      const uint32_t hi = pack_bf16x2(acc[i][j][2] + b2, acc[i][j][3] + b3);
      const v2i d = {(int)lo, (int)hi};
      if (j == 0) ds_write8<0>(waddr, d);
      if (j == 1) ds_write8<32>(waddr, d);
      if (j == 2) ds_write8<64>(waddr, d);
      if (j == 3) ds_write8<96>(waddr, d);
    }
    v4i r0, r1;
    ds_read16<0>(r0, raddr);
    if constexpr (kWN == 4) {
      ds_read16<8 * kEpiRowB>(r1, raddr);
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r0), "+v"(r1));
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r0));
    }
    const int rb = row0 + i * 16;
    // (uniform, but max/min would be computed in a vector register, which
    // would turn every store into a waterfall loop over the descriptor)
    const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(16, p.M - rb)));
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + (int64_t)rb * p.ldo * 2, (uint32_t)(nrows * p.ldo * 2));
    __builtin_amdgcn_raw_buffer_store_b128(r0, ro, voff0, 0, kStagedStoreAux);
    if constexpr (kWN == 4) __builtin_amdgcn_raw_buffer_store_b128(r1, ro, voff1, 0, kStagedStoreAux);
  }
}

// MXFP4 epilogue (mode 4): as mode 0 up to the row pieces read back from the
// staging rows.  A lane then holds 8 consecutive bf16 values of a row, and
// the 4 lanes of a quad hold one 1x32 block along N: the block's amax is
// combined by two quad permutes, the scale byte taken from its exponent and
// the 8 values encoded by the scaled conversion, as in the quantisation
// kernels.  Each lane stores its 4 code bytes, the quad's first lane the
// scale byte (the other lanes' scale stores go to an out-of-range offset, so
// every store is issued and the waits' counts stay exact).
__device__ __forceinline__ void epilogue_fp4(const GemmArgs& p, const Tile& tl, v4f (&acc)[kWM][kWN], int wv,
                                             int wm, int wn) {
  const int lane = (int)lane_here();
  const int row0 = tl.ms * 16 + wm * 128;
  const int n = (tl.s0 + wn * kWN) * 16 + (lane & (kLpr - 1)) * 8;  // this lane's 8 columns
  v2i bl[kWN];
  read_bias(bl, wv, lane);
  const uint32_t wst = kEpiLds + (uint32_t)wv * 16 * kEpiRowB;
  const uint32_t waddr = wst + (uint32_t)(lane & 15) * kEpiRowB + (uint32_t)(lane >> 4) * 8;
  const uint32_t raddr = wst + (uint32_t)(lane >> kLprShift) * kEpiRowB + (uint32_t)(lane & (kLpr - 1)) * 16;
  const uint32_t ldq = (uint32_t)p.ldo, lds = (uint32_t)p.ldos;
  const uint32_t doff0 = n < p.N ? (uint32_t)(lane >> kLprShift) * ldq + (uint32_t)(n >> 1) : kOOB;
  const uint32_t doff1 = n < p.N ? doff0 + 8 * ldq : kOOB;
  const bool first = (lane & 3) == 0;
  const uint32_t soff0 = (n < p.N && first) ? (uint32_t)(lane >> kLprShift) * lds + (uint32_t)(n >> 5) : kOOB;
  const uint32_t soff1 = (n < p.N && first) ? soff0 + 8 * lds : kOOB;
  uint8_t* const out = reinterpret_cast<uint8_t*>(p.out);
#pragma unroll
  for (int i = 0; i < kWM; ++i) {
#pragma unroll
    for (int j = 0; j < kWN; ++j) {
      const float b0 = __uint_as_float((uint32_t)bl[j].x << 16), b1 = __uint_as_float((uint32_t)bl[j].x & 0xFFFF0000u);
      const float b2 = __uint_as_float((uint32_t)bl[j].y << 16), b3 = __uint_as_float((uint32_t)bl[j].y & 0xFFFF0000u);
      const uint32_t lo = pack_bf16x2(acc[i][j][0] + b0, acc[i][j][1] + b1);
      const uint32_t hi = pack_bf16x2(acc[i][j][2] + b2, acc[i][j][3] + b3);
      const v2i d = {(int)lo, (int)hi};
      if (j == 0) ds_write8<0>(waddr, d);
      if (j == 1) ds_write8<32>(waddr, d);
      if (j == 2) ds_write8<64>(waddr, d);
      if (j == 3) ds_write8<96>(waddr, d);
    }
    v4i r0, r1;
    ds_read16<0>(r0, raddr);
    if constexpr (kWN == 4) {
      ds_read16<8 * kEpiRowB>(r1, raddr);
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r0), "+v"(r1));
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r0));
    }
    const int rb = row0 + i * 16;
    // (uniform: see epilogue_staged)
    const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(16, p.M - rb)));
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(out + (int64_t)rb * p.ldo, (uint32_t)nrows * ldq);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.out_scales + (int64_t)rb * p.ldos, (uint32_t)nrows * lds);
    const uint32_t b0 = e8m0_of_amax_bits(quad_amax_bits((uint32_t)r0.x, (uint32_t)r0.y, (uint32_t)r0.z, (uint32_t)r0.w));
    const uint32_t c0 = e2m1_pack8((uint32_t)r0.x, (uint32_t)r0.y, (uint32_t)r0.z, (uint32_t)r0.w, e8m0_value(b0));
    if constexpr (kWN == 4) {
      const uint32_t b1 = e8m0_of_amax_bits(quad_amax_bits((uint32_t)r1.x, (uint32_t)r1.y, (uint32_t)r1.z, (uint32_t)r1.w));
      const uint32_t c1 = e2m1_pack8((uint32_t)r1.x, (uint32_t)r1.y, (uint32_t)r1.z, (uint32_t)r1.w, e8m0_value(b1));
      __builtin_amdgcn_raw_buffer_store_b32(c0, rd, doff0, 0, MXFP4_STORE_AUX);
      __builtin_amdgcn_raw_buffer_store_b32(c1, rd, doff1, 0, MXFP4_STORE_AUX);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)b0, rs, soff0, 0, MXFP4_STORE_AUX);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)b1, rs, soff1, 0, MXFP4_STORE_AUX);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(c0, rd, doff0, 0, MXFP4_STORE_AUX);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)b0, rs, soff0, 0, MXFP4_STORE_AUX);
    }
  }
}

// Tile epilogue of modes 1-3: bias (fp32), one rounding, stores of every
// accumulator.  Rows are addressed through one buffer descriptor per 16-row block whose
// size ends at the last valid row; columns past N get an out-of-range
// offset.  Each store instruction is issued unconditionally, so the count of
// memory operations the K loop's waits rely on is exact.
template <int MODE>
__device__ __forceinline__ void epilogue(const GemmArgs& p, const Tile& tl, v4f (&acc)[kWM][kWN], int wv, int wm,
                                         int wn) {
  using OM = OutMode<MODE>;
  const int lane = (int)lane_here();
  constexpr int esz = OM::kF32 ? 4 : 2;
  const int row0 = tl.ms * 16 + wm * 128;  // wave's first output row
  const int ncol0 = (tl.s0 + wn * kWN) * 16 + 4 * (lane >> 4);
  const uint32_t lrow = (uint32_t)((lane & 15) * p.ldo) * esz;
  uint8_t* const out = reinterpret_cast<uint8_t*>(p.out);
  // Bias staged in LDS by this wave (mode 2): 4 columns per j.
  v2i bl[kWN];
  if (OM::kBiasLds) read_bias(bl, wv, lane);
#pragma unroll
  for (int j = 0; j < kWN; ++j) {
    const int n = ncol0 + j * 16;
    float bias[4];
    if (OM::kBiasLds) {
      bias[0] = __uint_as_float((uint32_t)bl[j].x << 16);
      bias[1] = __uint_as_float((uint32_t)bl[j].x & 0xFFFF0000u);
      bias[2] = __uint_as_float((uint32_t)bl[j].y << 16);
      bias[3] = __uint_as_float((uint32_t)bl[j].y & 0xFFFF0000u);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) bias[r] = (p.bias && n + r < p.N) ? bf16_to_f32(p.bias[n + r]) : 0.f;
    }
    const uint32_t voff = lrow + (uint32_t)n * esz;
#pragma unroll
    for (int i = 0; i < kWM; ++i) {
      const int rb = row0 + i * 16;
      // (uniform, but max/min would be computed in a vector register, which
      // would turn every store into a waterfall loop over the descriptor)
      const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(16, p.M - rb)));
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + (int64_t)rb * p.ldo * esz, (uint32_t)(nrows * p.ldo * esz));
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[i][j][r] + bias[r];
      if (OM::kVec) {
        const uint32_t off = n < p.N ? voff : kOOB;
        if (OM::kF32) {
          __builtin_amdgcn_raw_buffer_store_b128(
              (v4i){(int)__float_as_uint(v[0]), (int)__float_as_uint(v[1]), (int)__float_as_uint(v[2]),
                    (int)__float_as_uint(v[3])},
              ro, off, 0, 0);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t off = n + r < p.N ? voff + r * esz : kOOB;
          if (OM::kF32)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[r]), ro, off, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v[r]), ro, off, 0, 0);
        }
      }
    }
  }
  if (OM::kDrain) wait_vm<0>();
}

// The four K-steps of group g of work item c, loading four steps on (from
// item cn when g is c's last group).
template <int kStores, bool kBias>
__device__ __forceinline__ void group_body(const GemmArgs& p, Pipe& P, const Tile& c, const Tile& cn, int g,
                                           int wv, int wm, int wn, const ReadAddr& ra, uint32_t lane16) {
  const bool last = g + 1 == c.g1;
  Tile dt;
  dt.ms = last ? cn.ms : c.ms;
  dt.mstrips = last ? cn.mstrips : c.mstrips;
  dt.s0 = last ? cn.s0 : c.s0;
  dt.strips = last ? cn.strips : c.strips;
  const int t4 = last ? 4 * cn.g0 : 4 * (g + 1);
  // 1 in the item's first group, from a scalar instruction the compiler
  // cannot see through (it would peel the first group to fold the test,
  // which costs register copies around the loop).
  int first;
  asm volatile("s_cmp_eq_u32 %1, %2\n\ts_cselect_b32 %0, 1, 0" : "=s"(first) : "s"(g), "s"(c.g0) : "scc");
  main_step<0, kStores, kBias>(p, P, P.b0, P.b1, dt, c, t4 + 0, first, wv, wm, wn, ra, lane16);
  main_step<1, kStores, kBias>(p, P, P.b1, P.b0, dt, c, t4 + 1, first, wv, wm, wn, ra, lane16);
  main_step<2, kStores, kBias>(p, P, P.b0, P.b1, dt, c, t4 + 2, first, wv, wm, wn, ra, lane16);
  main_step<3, kStores, kBias>(p, P, P.b1, P.b0, dt, c, t4 + 3, first, wv, wm, wn, ra, lane16);
}

// kStores stores that write nothing (no records in the descriptor), as
// inline assembly so identical stores are not merged: they stand for an
// epilogue's stores in the counts of the next item's waits.
template <int kStores>
__device__ __forceinline__ void drop_stores() {
  const v4i none = {0, 0, 0, 0x00020000};
  const uint32_t zero = 0;
#pragma unroll
  for (int q = 0; q < kStores; ++q)
    asm volatile("buffer_store_dword %0, %1, %2, 0 offen" ::"v"(zero), "v"(kOOB), "s"(none) : "memory");
}

// End of this workgroup's slice (kme of S = sk.s) of split tile t: take the
// tile's arrival ticket.  Not the last to arrive: store the accumulators
// to this workgroup's part slot, raise its flag, and return false (no
// epilogue; the stores the next item's waits count are stood in for).  The
// last: wait for the other slices' flags, sum the slices in K order into acc
// (with two slices, acc plus the other: the same either way) and return
// true.  Slice k of tile t is workgroup (and part slot) k r + t.
// acc[i][j] (+)= the part at byte offset o of the part buffer, 8 loads in
// flight at a time (all 32 at once would not fit beside the accumulators).
template <bool kAdd>
__device__ __forceinline__ void add_part(v4f (&acc)[kWM][kWN], __amdgpu_buffer_rsrc_t rp, uint32_t o) {
#pragma unroll
  for (int h = 0; h < kWM * kWN / 8; ++h) {
    v4i v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = __builtin_amdgcn_raw_buffer_load_b128(rp, o + (uint32_t)(h * 8 + e) * 1024u, 0, kPartAux);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = (h * 8 + e) / kWN, j = (h * 8 + e) % kWN;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[i][j][r] = kAdd ? acc[i][j][r] + __uint_as_float((uint32_t)v[e][r]) : __uint_as_float((uint32_t)v[e][r]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int kStores>
__device__ bool sk_combine(const SkArgs& sk, const Share& s, Pipe& P, int wv) {
  // Let every LDS read and memory operation this wave has in flight land
  // (the next item's fragments and loads), so nothing below races them.
  // (Naming the fragment registers here, as the loop's waits do, would make
  // them new values on this path only, and the merge after it would copy
  // them all.)
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  const int S = sk.s, kme = s.slot / sk.r, t = s.slot - kme * sk.r;
  const uint32_t lane = lane_here();
  if (wv == 0 && lane == 0) {
    const uint32_t r = __hip_atomic_fetch_add(sk.ctrl + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ds_write4(kSkLds, r);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  barrier_nofence();
  uint32_t rank;
  ds_read4<0>(rank, kSkLds);
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(rank));
  // (all waves must read the rank before wave 0 may write the next one: the
  // next write follows at least one more barrier, in the next item's loop)
  const bool last = (int)__builtin_amdgcn_readfirstlane(rank) == S - 1;
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(sk.part, (uint32_t)s.grid * kPartBytes);
  const uint32_t lofs = (uint32_t)wv * (kPartBytes / kWaves) + lane * 16u;
  if (!last || S > 2) {
    const int my = s.slot;
    const uint32_t o = (uint32_t)my * kPartBytes + lofs;
#pragma unroll
    for (int i = 0; i < kWM; ++i)
#pragma unroll
      for (int j = 0; j < kWN; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(
            (v4i){(int)__float_as_uint(P.acc[i][j][0]), (int)__float_as_uint(P.acc[i][j][1]),
                  (int)__float_as_uint(P.acc[i][j][2]), (int)__float_as_uint(P.acc[i][j][3])},
            rp, o + (uint32_t)(i * kWN + j) * 1024u, 0, kPartAux);
    wait_vm<0>();
    barrier_nofence();
    if (wv == 0 && lane == 0) __hip_atomic_store(sk.flags + my, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!last) {
      wait_vm<0>();
      drop_stores<kStores>();
      return false;
    }
  }
  bool waited_out = false;
  for (int k = 0; k < S; ++k) {
    if (k == kme) continue;
    const int id = k * sk.r + t;
    bool seen = false;
    for (int it = 0; it < kSpinLimit && !seen; ++it) {
      const uint32_t f = __hip_atomic_load(sk.flags + id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      seen = __builtin_amdgcn_readfirstlane(f) != 0;
      if (!seen) __builtin_amdgcn_s_sleep(2);
    }
    waited_out = waited_out || !seen;
  }
  // a wait that gave up (never expected: every slice waited for already
  // holds its ticket, so it is running) is made visible in the workspace
  if (waited_out && wv == 0 && lane == 0)
    __hip_atomic_fetch_or(sk.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (S == 2) {
    add_part<true>(P.acc, rp, (uint32_t)((1 - kme) * sk.r + t) * kPartBytes + lofs);
  } else {
    // every part, this one's too, is in the workspace: p_0 + p_1 + ... in order
    add_part<false>(P.acc, rp, (uint32_t)t * kPartBytes + lofs);
    for (int k = 1; k < S; ++k) add_part<true>(P.acc, rp, (uint32_t)(k * sk.r + t) * kPartBytes + lofs);
  }
  return true;
}

__global__ void sk_clear_kernel(uint32_t* words, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) words[i] = 0;
}

}  // namespace

template <int MODE>
__global__ __launch_bounds__(512, 1) void MXFP4_PREFILL_KERNEL(GemmArgs p, int tiles_m, int tiles_n, SkArgs sk) {
  constexpr int kStores = OutMode<MODE>::kInFlight;
  constexpr bool kBiasLds = OutMode<MODE>::kBiasLds;
  // The stage and scale addresses above are absolute LDS addresses: this is
  // the kernel's only LDS allocation, so it starts at address 0.
  __shared__ int4 lds_raw[kLdsBytes / 16];
  const int lane = threadIdx.x & 63;
  // The wave index is uniform across the wave; saying so keeps the buffer
  // resource and LDS address of every buffer->LDS load in scalar registers.
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wv >> 2, wn = wv & 3;
  const int G = p.G;

  // Workgroups are dealt to the 8 XCDs round-robin; with a grid that is a
  // multiple of 8, slot numbers are remapped so each XCD's workgroups hold
  // consecutive slots (and so consecutive tiles, or slices of consecutive
  // tiles).
  const int ntiles = tiles_m * tiles_n;
  Share s;
  s.grid = gridDim.x;
  s.slot = (s.grid & 7) == 0 ? (blockIdx.x & 7) * (s.grid >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  {
    s.nsk = s.slot < sk.r * sk.s ? 1 : 0;
    const int rest = ntiles - sk.r;
    s.n = s.nsk + (rest > s.slot ? (rest - s.slot + s.grid - 1) / s.grid : 0);
  }

  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)&lds_raw[0];
  const uint32_t lane16 = lane * 16;
  ReadAddr ra;
  ra.a = lds0 + wm * kWM * 4096 + lane16;
  ra.b = lds0 + (kTilesA + wn * kWN) * 4096 + lane16;

  Pipe P;
  zero_acc(P.acc);

  Tile c = work_at(p, sk, s, 0, tiles_m, tiles_n);
  Tile cn = work_at(p, sk, s, 1, tiles_m, tiles_n);

  // Prologue: scales of the first item's first group and its first 4 steps
  // in flight; then as many dropped stores as an epilogue leaves in flight,
  // so every item's first group counts the same operations.  Once the
  // scales and the first step have landed everywhere, read them in the
  // order the loop expects.
  issue_scales(p, c, c.g0, wv);
  issue_step(p, c, 0, 4 * c.g0 + 0, wv, lane16);
  issue_step(p, c, 1, 4 * c.g0 + 1, wv, lane16);
  issue_step(p, c, 2, 4 * c.g0 + 2, wv, lane16);
  issue_step(p, c, 3, 4 * c.g0 + 3, wv, lane16);
  drop_stores<kStores>();
  wait_vm<3 * kLoadsPerWave + kStores>();
  barrier_nofence();
  read_scales(P.sa, P.sb, wm, wn);
  read_first_half<0>(P.af, P.b0, ra);
  read_second_half<0>(P.af, ra);

  for (int k = 0;;) {
    for (int g = c.g0; g < c.g1; ++g) group_body<kStores, kBiasLds>(p, P, c, cn, g, wv, wm, wn, ra, lane16);
    const bool out = k >= s.nsk || sk_combine<kStores>(sk, s, P, wv);
    if (out) {
      if (OutMode<MODE>::kFp4)
        epilogue_fp4(p, c, P.acc, wv, wm, wn);
      else if (OutMode<MODE>::kStaged)
        epilogue_staged(p, c, P.acc, wv, wm, wn);
      else
        epilogue<MODE>(p, c, P.acc, wv, wm, wn);
    }
    if (++k == s.n) break;
    // The next item's first fragments and scales, already read in the last
    // group, are read again from LDS (they stay there until the next
    // group's first barrier): so their registers are free across the
    // epilogue and the combine.
    read_scales(P.sa, P.sb, wm, wn);
    read_first_half<0>(P.af, P.b0, ra);
    read_second_half<0>(P.af, ra);
    zero_acc(P.acc);
    c = cn;
    cn = work_at(p, sk, s, k + 1, tiles_m, tiles_n);
  }
  // The loads issued past the last item (empty descriptors) still write
  // zeros to LDS: let them and the LDS reads finish before the workgroup
  // ends.
  wait_lgkm<0>(P.af[4], P.af[5], P.af[6], P.af[7]);
  wait_vm<0>();
}

// This tile width's launch on `grid` workgroups: the split schedule's
// counters cleared first (a kernel, not a memset: the launch may be
// captured into a graph), then the GEMM in the output mode the call needs.
hipError_t MXFP4_PREFILL_TILES(const GemmArgs& p, int grid, const PrefillSplit& sk, hipStream_t stream) {
  const int tiles_m = (p.M + kBM - 1) / kBM;
  const int tiles_n = (p.Ns * 16 + kBN - 1) / kBN;
  if (sk.r) sk_clear_kernel<<<1, 256, 0, stream>>>(sk.err, 1 + sk.r + grid);
  const bool a16 = ((uintptr_t)p.out & 15) == 0;
  const int mode = p.out_fp4 ? 4
                 : p.out_f32 ? ((p.N % 4 == 0 && p.ldo % 4 == 0 && a16) ? 2 : 3)
                             : ((p.N % 8 == 0 && p.ldo % 8 == 0 && a16) ? 0 : 1);
  const dim3 g((unsigned)grid), b(64 * kWaves);
  switch (mode) {
    case 0: MXFP4_PREFILL_KERNEL<0><<<g, b, 0, stream>>>(p, tiles_m, tiles_n, sk); break;
    case 1: MXFP4_PREFILL_KERNEL<1><<<g, b, 0, stream>>>(p, tiles_m, tiles_n, sk); break;
    case 2: MXFP4_PREFILL_KERNEL<2><<<g, b, 0, stream>>>(p, tiles_m, tiles_n, sk); break;
    case 4: MXFP4_PREFILL_KERNEL<4><<<g, b, 0, stream>>>(p, tiles_m, tiles_n, sk); break;
    default: MXFP4_PREFILL_KERNEL<3><<<g, b, 0, stream>>>(p, tiles_m, tiles_n, sk); break;
  }
  return hipGetLastError();
}

#if MXFP4_PREFILL_BN == 256
namespace {

constexpr int kMaxSkGrid = 256;  // the split schedule's workgroups (and workspace) at most

// Bytes of the split schedule's words (give-up word, counters, flags),
// rounded up to 256 so the parts after them stay aligned.
size_t sk_words_bytes(int r, int grid) { return ((size_t)(1 + r + grid) * 4 + 255) / 256 * 256; }

struct PrefillPlan {
  int bn, grid, r, s;
  size_t bytes;  // workspace
};

// The plan at tile width bn.  split: 0 = by the measured rule below, 1 =
// whole tiles, 2 = split wherever the tiles leave a round part-empty and a
// tile has more than one group.
// The rule, from both schedules timed on MI355X (256 CUs) at M = 512 ...
// 8192 for (N, K) = (14336, 5120), (5120, 14336), (34816, 5120): moving a
// slice's 256 KiB part costs about as much as 7 groups of MFMAs, so split
// where the r leftover tiles fill at most half a round and each slice keeps
// at least 7 groups (3584 of K), or at least 4 where the leftover tiles fill
// at most a quarter of a round (whole tiles then leave most compute units
// idle).  Measured: K = 14336 gains 6-20% (M = 512: 79.9 -> 64.3 us; M =
// 8192: 289 -> 267 us); K = 5120 (slices of at most 5 groups) loses 3-39%
// and stays on whole tiles.
PrefillPlan plan_width(int bn, int M, int N, int K, int cus, int split) {
  const int tiles_m = (M + kBM - 1) / kBM;
  const int tiles_n = ((N + 15) / 16 * 16 + bn - 1) / bn;
  const int T = tiles_m * tiles_n;
  const int G = ((K + 127) / 128 + 3) / 4;
  const int C = cus < kMaxSkGrid ? cus : kMaxSkGrid;
  PrefillPlan whole = {bn, T < cus ? T : cus, 0, 0, 0};
  if (split == 1 || C < 2) return whole;
  const int r = T % C;
  int s = r ? C / r : 0;
  if (s > G) s = G;
  if (s < 2) return whole;
  if (split == 0 && (2 * r > C || (G / s < 7 && (4 * r > C || G / s < 4)))) return whole;
  PrefillPlan pl;
  pl.bn = bn;
  pl.r = r;
  pl.s = s;
  pl.grid = T >= C ? C : r * s;
  pl.bytes = sk_words_bytes(r, pl.grid) + (size_t)pl.grid * kBM * bn * 4;
  return pl;
}

// The plan for the kernel-selection override (0: automatic; 3 / 4: 256 wide,
// whole tiles / split forced; 5 / 6: 128 wide, the same).  Automatic: 128
// wide where 256-wide tiles fill at most half a round of the compute units
// and 128-wide ones fit in one, else 256 wide; then that width's split
// rule.  Measured on MI355X (both widths, both schedules, M = 512 ... 8192,
// the three sweep shapes): a 128-wide tile does its work 1.27x slower per
// flop when every compute unit is busy (M = 8192: 263 -> 335 us), so it pays
// only where 256-wide tiles leave most units idle — M = 512, N = 14336,
// K = 5120: 33.0 -> 25.7 us; M = 512, N = 5120, K = 14336: 66.3 (256 wide,
// split) -> 41.5 us (128 wide, split); M = 1024 there: 74.4 -> 55.3 us;
// with more tiles it lost up to 28% (and won at most 4%, at two shapes this
// rule leaves at 256).
PrefillPlan plan_prefill(int M, int N, int K, int cus) {
  switch (get_gemm_path_override()) {
    case 3: return plan_width(256, M, N, K, cus, 1);
    case 4: return plan_width(256, M, N, K, cus, 2);
    case 5: return plan_width(128, M, N, K, cus, 1);
    case 6: return plan_width(128, M, N, K, cus, 2);
    default: break;
  }
  const int C = cus < kMaxSkGrid ? cus : kMaxSkGrid;
  const int tiles_m = (M + kBM - 1) / kBM;
  const int n16 = (N + 15) / 16 * 16;
  const int t256 = tiles_m * ((n16 + 255) / 256), t128 = tiles_m * ((n16 + 127) / 128);
  return plan_width(2 * t256 <= C && t128 <= C ? 128 : 256, M, N, K, cus, 0);
}

}  // namespace

size_t gemm_prefill_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return plan_prefill((int)M, (int)N, (int)K, kMaxSkGrid).bytes;
}

hipError_t launch_gemm_prefill(const GemmArgs& p, hipStream_t stream) {
  PrefillPlan pl = plan_prefill(p.M, p.N, p.K, p.cus);
  if (pl.r && (!p.work || p.work_bytes < pl.bytes)) pl = plan_width(pl.bn, p.M, p.N, p.K, p.cus, 1);
  PrefillSplit sk = {0, 1, nullptr, nullptr, nullptr, nullptr};
  if (pl.r) {
    sk.r = pl.r;
    sk.s = pl.s;
    sk.err = reinterpret_cast<uint32_t*>(p.work);
    sk.ctrl = sk.err + 1;
    sk.flags = sk.ctrl + pl.r;
    sk.part = p.work + sk_words_bytes(pl.r, pl.grid);
  }
  return pl.bn == 128 ? launch_prefill_tiles_128(p, pl.grid, sk, stream)
                      : launch_prefill_tiles_256(p, pl.grid, sk, stream);
}
#endif

}  // namespace mxfp4
