// Internal launchers behind the C ABI (include/mxfp4.h).  Arguments are
// already validated by the caller; each returns the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mxfp4 {

// Validated, device-side view of one W4A4 GEMM call.
struct GemmArgs {
  const uint8_t* a;    // packed FP4 activations, GEMM data layout
  const uint8_t* as;   // activation scales, GEMM scale layout
  const uint8_t* w;    // preshuffled weights
  const uint8_t* ws;   // weight scales, GEMM scale layout
  const uint16_t* bias;  // bf16 [N] or nullptr
  void* out;           // [M, N], row stride ldo elements
  int64_t ldo;
  int out_f32;
  int M, N, K, Kt, G, Ns;  // Kt = ceil(K/128), G = ceil(Kt/4), Ns = ceil(N/16)
  int cus;                 // compute units of the device (persistent grids)
  // bf16 activations [M, K] of the fused-quantisation path (else unused):
  // row stride ldx elements, x_bytes = ((M-1)*ldx + K)*2 readable bytes.
  const uint16_t* x;
  int ldx;
  uint32_t x_bytes;
  // Row-major quantised activations (small-M kernel only): a is [M, K/2]
  // with row stride lda bytes, as [M, K/32] with row stride lds bytes.
  int a_rowmajor;
  uint32_t lda, lds;
  int scales_vec;  // row-major scales: lds % 16 == 0, 16-byte aligned, K % 512 == 0
  // MXFP4 output (out_fp4 != 0): out is packed FP4 [M, N/2] with row stride
  // ldo BYTES, out_scales E8M0 [M, N/32] with row stride ldos bytes.
  int out_fp4;
  uint8_t* out_scales;
  int64_t ldos;
  // Workspace of the large-M kernel's split schedule (it falls back to whole
  // tiles when this is smaller than gemm_prefill_workspace_bytes asks).
  uint8_t* work;
  size_t work_bytes;
};

hipError_t launch_gemm_decode(const GemmArgs& p, hipStream_t stream);
// The small-M kernel over any M: one launch per 64 rows (rows 64c .. 64c+63
// of the activations and the output), each as launch_gemm_decode of those
// rows alone.
hipError_t launch_gemm_decode_rows(const GemmArgs& p, hipStream_t stream);
hipError_t launch_gemm_prefill(const GemmArgs& p, hipStream_t stream);
// The large-M kernel's split (split-K) schedule of one launch: tiles [0, r)
// cut into s K slices (r = 0: whole tiles); in the workspace, in this order:
// the give-up word (raised when a slice's bounded wait for another slice's
// flag expired -- the tile's sum is then not to be trusted), the tiles'
// arrival counters, the slices' ready flags, then (256-byte aligned) the
// parts.
struct PrefillSplit {
  int r, s;
  uint8_t* part;
  uint32_t* err;
  uint32_t* ctrl;
  uint32_t* flags;
};
// The large-M kernel at output-tile width 256 / 128 on `grid` workgroups.
hipError_t launch_prefill_tiles_256(const GemmArgs& p, int grid, const PrefillSplit& sk, hipStream_t stream);
hipError_t launch_prefill_tiles_128(const GemmArgs& p, int grid, const PrefillSplit& sk, hipStream_t stream);
// Workspace the large-M kernel's split schedule takes for this shape on up
// to 256 compute units (0: whole tiles only).
size_t gemm_prefill_workspace_bytes(int64_t M, int64_t N, int64_t K);
// Activation quantisation fused into the small-M GEMM (M <= 4), and whether
// that beats quantisation + GEMM for a shape.
hipError_t launch_linear_decode(const GemmArgs& p, hipStream_t stream);
bool linear_fused_pays(int M, int N, int K);
// The fused quantisation in the small-M kernel's persistent form: whether the
// shape fits it (x_bytes = ((M-1)*ldx + K)*2), whether it is chosen, and
// its launch (p.x / ldx / x_bytes set).
bool linear_persist_applies(int M, int K, int64_t x_bytes);
bool linear_persist_pays(int M, int N, int K, int cus);
hipError_t launch_linear_persist(const GemmArgs& p, hipStream_t stream);

hipError_t launch_quant_1x32(const void* x, int64_t M, int64_t K, int64_t ldx, void* q,
                             int64_t ldq, void* scales, int layout, hipStream_t stream);

hipError_t launch_preshuffle(const void* w_fp4, const void* w_scales, int64_t batch, int64_t N,
                             int64_t K, void* w_out, void* ws_out, hipStream_t stream);
// Same permutation from row-strided sources (ldw / lds bytes per row); a
// NULL w_fp4 permutes the scales only.
hipError_t launch_preshuffle_strided(const void* w_fp4, int64_t ldw, const void* w_scales,
                                     int64_t lds, int64_t batch, int64_t N, int64_t K,
                                     void* w_out, void* ws_out, hipStream_t stream);

// mxfp4_linear's steps behind its C entry points (csrc/api.hip): the host
// argument checks (everything but the workspace), the activation workspace
// bytes without the large-M GEMM's split part (0 where the quantisation is
// fused), and the launches on a given workspace -- the split schedule only
// when `split` and the workspace holds it, else whole tiles.
int linear_check(const void* x, int64_t ldx, const void* w_pre, const void* ws_pre, const void* bias,
                 const void* out, int64_t ldo, int out_dtype, int64_t M, int64_t N, int64_t K);
size_t linear_act_bytes(int64_t M, int64_t N, int64_t K);
int linear_run(const void* x, int64_t ldx, const void* w_pre, const void* ws_pre, const void* bias,
               void* out, int64_t ldo, int out_dtype, int64_t M, int64_t N, int64_t K, void* workspace,
               size_t workspace_bytes, bool split, int cus, hipStream_t s);
// The current device's compute units if it is a gfx950 (MXFP4_OK), else MXFP4_ERR_DEVICE.
int device_cus(int* cus);

hipError_t launch_bmm_a16w4(const void* x, int64_t sxb, int64_t sxm, const void* w,
                            const void* ws, void* out, int64_t sob, int64_t som, int out_f32,
                            int64_t B, int64_t M, int64_t N, int64_t K, hipStream_t stream, int cus);

// Kernel-selection override of the calling thread, set only through the
// test hook (include/mxfp4_testing.h) to exercise each GEMM path on every
// shape: 0 = automatic by M, 1 = decode
// kernel, 2 = prefill kernel (schedule by estimate), 3 = prefill kernel with
// whole tiles only, 4 = prefill kernel with the split schedule wherever a
// tile has more than one group of 4 K-steps; 5 and 6: the same as 3 and 4
// with 128-wide output tiles.
void set_gemm_path_override(int path);
int get_gemm_path_override();

}  // namespace mxfp4
