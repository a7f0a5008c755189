// C ABI of libmxfp4 (declared in include/mxfp4.h): argument validation, size
// queries, device check and dispatch to the gfx950 kernels.  Validation runs
// entirely on the host before any HIP call, so a rejected call enqueues
// nothing and works on a machine without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/mxfp4.h"
#include "../../include/mxfp4_testing.h"
#include "mxfp4_launch.h"

namespace mxfp4 {

// The test hook's forced kernel choice: per thread, so a call on one thread
// never sees another thread's setting between its size query and its GEMM.
static thread_local int t_gemm_path = 0;
void set_gemm_path_override(int path) { t_gemm_path = path; }
int get_gemm_path_override() { return t_gemm_path; }

namespace {

constexpr int64_t kMaxBuf = 0x7FFFFFFFll;  // buffer-resource offsets stay below 2^31
constexpr int64_t kMaxK = 1 << 20;         // keeps per-tile 32-bit offsets far from wrapping
constexpr int64_t kFusedMaxM = 4;          // mxfp4_linear quantises inside the GEMM up to 4 rows

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Which GEMM kernel a call of M rows and N columns takes: 1 = small-M,
// 2 = large-M, 3 = small-M once per 64 rows.  Up to 256 rows the large-M
// kernel runs a single row of 256-row tiles, one per 128 (or 256) columns
// on few compute units, its K-steps latency-bound; the small-M kernel
// streams the weights on all of them, once per 64 rows, so it wins while
// those c = ceil(M/64) passes move few weight bytes: c * N <= 16384.
// Measured on MI355X (us, one tile row -> c launches): N = 4096, K = 4096,
// M = 65 / 128 / 192 18.7 / 18.7 / 18.7 -> 8.7 / 10.3 / 15.0; N = 8192,
// K = 14336, M = 65 / 128 34.4 / 35.0 -> 27.8 / 32.8; N = 4096, K = 14336,
// M = 192 / 256 51.9 / 52.3 -> 31.8 / 42.4; N = 1024, K = 4096, M = 256
// 18.6 -> 17.9.  Past that bound the tile row wins (N = 8192, M = 192:
// 19.0 -> 20.5 at K = 4096; N = 14336, K = 8192, M = 128: 28.1 -> 36.0).
int gemm_path(int64_t M, int64_t N) {
  const int path = get_gemm_path_override();
  if ((path == 1 || path == 7 || path == 8) && M <= 64) return 1;
  if (path >= 2 && path <= 6) return 2;
  if (M <= 64) return 1;
  const int64_t c = (M + 63) / 64;
  return c <= 4 && c * N <= 16384 ? 3 : 2;
}

// Row-major operands for the small-M kernel (per launch of up to 64 rows):
// every workgroup gathers all its rows in 64-byte pieces, which on long K
// with many rows, or on many strips, costs more than permuting them once
// into the GEMM layouts (one more launch, data and scales together).
// Measured on MI355X (us, gathered -> permuted first): K = 5120, N = 10240 /
// 14336, M = 48 16.5 / 14.7 -> 13.3 / 14.0; K = 8192, N = 28672, M = 16 /
// 32 / 64 27.5 / 32.0 / 55.8 -> 26.0 / 27.7 / 37.6; N = 10240, M = 16
// 13.4 -> 13.0; K = 14336, N = 5120, M = 48 / 64 20.0 / 25.1 -> 16.1 /
// 17.9.  Not with K <= 4096 (N = 28672, M = 64: 20.0 -> 25.2), nor with
// fewer rows on fewer strips (K = 8192, N = 8192, M = 16 / 32: 9.1 / 11.0
// -> 10.6 / 11.8); the rule's worst miss is 0.36 us (K = 5120, N = 6144,
// M = 48).
bool prequant_permute(int64_t M, int64_t N, int64_t K) {
  const int64_t rows = M < 64 ? M : 64;
  const int64_t G = cdiv(cdiv(K, 128), 4);
  return G >= 10 && (rows > 32 || (rows > 8 && G > 12 && N >= 10240));
}

hipError_t launch_gemm_path(int path, const GemmArgs& p, hipStream_t s) {
  return path == 1 ? launch_gemm_decode(p, s) : path == 3 ? launch_gemm_decode_rows(p, s) : launch_gemm_prefill(p, s);
}

int64_t gemm_scale_bytes(int64_t rows, int64_t K) {
  const int64_t kt = cdiv(K, 128), g = cdiv(kt, 4);
  return cdiv(rows, 16) * g * 256;
}
int64_t gemm_data_bytes(int64_t rows, int64_t K) { return cdiv(rows, 16) * cdiv(K, 128) * 1024; }
int64_t weight_bytes_one(int64_t N, int64_t K) { return gemm_data_bytes(N, K); }

// Per device ordinal: 0 = unknown, 1 = gfx950, 2 = other; and its compute
// unit count (written before the kind is published).
std::atomic<int> g_dev_kind[64];
std::atomic<int> g_dev_cus[64];

// Checks that the current device is a gfx950; on success *cus (if given)
// receives its compute-unit count.
int check_device(int* cus = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MXFP4_ERR_DEVICE;
  if (dev < 0 || dev >= 64) return MXFP4_ERR_DEVICE;
  if (g_dev_kind[dev].load(std::memory_order_acquire) == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MXFP4_ERR_DEVICE;
    g_dev_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1, std::memory_order_relaxed);
    g_dev_kind[dev].store(strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2, std::memory_order_release);
  }
  if (g_dev_kind[dev].load(std::memory_order_acquire) != 1) return MXFP4_ERR_DEVICE;
  if (cus) *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  return MXFP4_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_LAUNCH; }

// Whether mxfp4_linear quantises inside the GEMM kernel for this shape.
bool linear_fused(int64_t M, int64_t N, int64_t K) {
  return M <= kFusedMaxM && N <= kMaxBuf && K <= kMaxK && linear_fused_pays((int)M, (int)N, (int)K);
}

}  // namespace

int device_cus(int* cus) { return check_device(cus); }

// Quantised activations in the GEMM layouts, then the GEMM's workspace, in
// one workspace: byte offsets of the scales and of the GEMM's part.
size_t act_scales_offset(int64_t M, int64_t K) { return (size_t)cdiv(gemm_data_bytes(M, K), 256) * 256; }
size_t act_gemm_offset(int64_t M, int64_t K) {
  return (act_scales_offset(M, K) + (size_t)gemm_scale_bytes(M, K) + 255) / 256 * 256;
}

size_t linear_act_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 32 || linear_fused(M, N, K)) return 0;
  return act_scales_offset(M, K) + (size_t)gemm_scale_bytes(M, K);
}

int linear_check(const void* x, int64_t ldx, const void* w_pre, const void* ws_pre, const void* bias,
                 const void* out, int64_t ldo, int out_dtype, int64_t M, int64_t N, int64_t K) {
  if (out_dtype != MXFP4_OUT_BF16 && out_dtype != MXFP4_OUT_F32) return MXFP4_ERR_ARG;
  if (M < 0 || N <= 0 || K <= 0 || K % 32 || K > kMaxK || N > kMaxBuf || M > kMaxBuf)
    return MXFP4_ERR_SHAPE;
  if (ldo < N || ldx < K) return MXFP4_ERR_SHAPE;
  if (ldo > kMaxBuf / 256 / (out_dtype == MXFP4_OUT_F32 ? 4 : 2)) return MXFP4_ERR_SHAPE;
  if (weight_bytes_one(N, K) > kMaxBuf || gemm_scale_bytes(N, K) > kMaxBuf ||
      gemm_data_bytes(M, K) > kMaxBuf || gemm_scale_bytes(M, K) > kMaxBuf)
    return MXFP4_ERR_SHAPE;
  // the fused kernel addresses x through one 32-bit buffer range
  if (M > 0 && linear_fused(M, N, K) && ((M - 1) * ldx + K) * 2 > kMaxBuf) return MXFP4_ERR_SHAPE;
  if (M == 0) return MXFP4_OK;
  if (!x || !w_pre || !ws_pre || !out) return MXFP4_ERR_NULL;
  if (!aligned(x, 16) || ldx % 8 || !aligned(w_pre, 16) || !aligned(ws_pre, 4) || !aligned(out, 4) ||
      (bias && !aligned(bias, 2)))
    return MXFP4_ERR_ALIGN;
  return MXFP4_OK;
}

int linear_run(const void* x, int64_t ldx, const void* w_pre, const void* ws_pre, const void* bias,
               void* out, int64_t ldo, int out_dtype, int64_t M, int64_t N, int64_t K, void* workspace,
               size_t workspace_bytes, bool split, int cus, hipStream_t s) {
  GemmArgs p{};
  p.cus = cus;
  p.w = (const uint8_t*)w_pre;
  p.ws = (const uint8_t*)ws_pre;
  p.bias = (const uint16_t*)bias;
  p.out = out;
  p.ldo = ldo;
  p.out_f32 = out_dtype == MXFP4_OUT_F32;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.Kt = (int)cdiv(K, 128);
  p.G = (int)cdiv(p.Kt, 4);
  p.Ns = (int)cdiv(N, 16);
  const int64_t x_bytes = ((M - 1) * ldx + K) * 2;
  if (linear_persist_applies((int)M, (int)K, x_bytes) && linear_persist_pays((int)M, (int)N, (int)K, cus)) {
    // quantised inside the persistent form: the workspace stays untouched
    p.x = (const uint16_t*)x;
    p.ldx = (int)ldx;
    p.x_bytes = (uint32_t)x_bytes;
    return launched(launch_linear_persist(p, s));
  }
  if (linear_fused(M, N, K)) {
    p.x = (const uint16_t*)x;
    p.ldx = (int)ldx;
    p.x_bytes = (uint32_t)(((M - 1) * ldx + K) * 2);
    return launched(launch_linear_decode(p, s));
  }
  // Larger M: quantise into the workspace, then the GEMM kernel for that M
  // (the large-M kernel's split schedule in the rest of the workspace, when
  // allowed and the workspace holds it; else whole tiles).
  uint8_t* q = (uint8_t*)workspace;
  uint8_t* sc = q + act_scales_offset(M, K);
  const int st = launched(launch_quant_1x32(x, M, K, ldx, q, 0, sc, MXFP4_LAYOUT_GEMM, s));
  if (st) return st;
  p.a = q;
  p.as = sc;
  if (split && workspace_bytes > act_gemm_offset(M, K)) {
    p.work = q + act_gemm_offset(M, K);
    p.work_bytes = workspace_bytes - act_gemm_offset(M, K);
  }
  return launched(launch_gemm_path(M <= 64 ? 1 : gemm_path(M, N), p, s));
}

}  // namespace mxfp4

using namespace mxfp4;

extern "C" {

const char* mxfp4_status_str(int status) {
  switch (status) {
    case MXFP4_OK: return "ok";
    case MXFP4_ERR_NULL: return "a required pointer is NULL";
    case MXFP4_ERR_SHAPE: return "invalid shape (sizes must be positive and K a multiple of 32)";
    case MXFP4_ERR_ALIGN: return "pointer or stride misaligned";
    case MXFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case MXFP4_ERR_DEVICE: return "current HIP device is not gfx950 (MI355X)";
    case MXFP4_ERR_LAUNCH: return "HIP kernel launch failed";
    case MXFP4_ERR_ARG: return "enum argument out of range";
    default: return "unknown status";
  }
}

int mxfp4_abi_version(void) { return 103; }

size_t mxfp4_data_bytes(int64_t rows, int64_t K, int layout) {
  if (rows < 0 || K <= 0 || K % 32) return 0;
  if (layout == MXFP4_LAYOUT_ROWMAJOR) return (size_t)(rows * (K / 2));
  if (layout == MXFP4_LAYOUT_GEMM) return (size_t)gemm_data_bytes(rows, K);
  return 0;
}

size_t mxfp4_scale_bytes(int64_t rows, int64_t K, int layout) {
  if (rows < 0 || K <= 0 || K % 32) return 0;
  if (layout == MXFP4_LAYOUT_ROWMAJOR) return (size_t)(rows * (K / 32));
  if (layout == MXFP4_LAYOUT_GEMM) return (size_t)gemm_scale_bytes(rows, K);
  return 0;
}

size_t mxfp4_weight_bytes(int64_t batch, int64_t N, int64_t K) {
  if (batch <= 0 || N <= 0 || K <= 0 || K % 32) return 0;
  return (size_t)(batch * weight_bytes_one(N, K));
}

size_t mxfp4_weight_scale_bytes(int64_t batch, int64_t N, int64_t K) {
  if (batch <= 0 || N <= 0 || K <= 0 || K % 32) return 0;
  return (size_t)(batch * gemm_scale_bytes(N, K));
}

size_t mxfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 32 || K > kMaxK || N > kMaxBuf || M > kMaxBuf) return 0;
  return gemm_path(M, N) == 2 ? gemm_prefill_workspace_bytes(M, N, K) : 0;
}


int mxfp4_quant_1x32(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, int64_t ldq,
                     void* scales, int layout, void* stream) {
  if (layout != MXFP4_LAYOUT_ROWMAJOR && layout != MXFP4_LAYOUT_GEMM) return MXFP4_ERR_ARG;
  if (M < 0 || K <= 0 || K % 32 || M > kMaxBuf || K > kMaxK) return MXFP4_ERR_SHAPE;
  if (ldx < K) return MXFP4_ERR_SHAPE;
  if (layout == MXFP4_LAYOUT_ROWMAJOR && ldq < K / 2) return MXFP4_ERR_SHAPE;
  if (mxfp4_scale_bytes(M, K, layout) > (size_t)kMaxBuf ||
      (layout == MXFP4_LAYOUT_GEMM && mxfp4_data_bytes(M, K, layout) > (size_t)kMaxBuf))
    return MXFP4_ERR_SHAPE;
  if (M == 0) return MXFP4_OK;  // nothing to read or write in either layout
  if (!x || !q || !scales) return MXFP4_ERR_NULL;
  if (!aligned(x, 16) || ldx % 8) return MXFP4_ERR_ALIGN;
  if (layout == MXFP4_LAYOUT_ROWMAJOR && (!aligned(q, 4) || ldq % 4)) return MXFP4_ERR_ALIGN;
  if (layout == MXFP4_LAYOUT_GEMM && (!aligned(q, 16) || !aligned(scales, 4))) return MXFP4_ERR_ALIGN;
  int st = check_device();
  if (st) return st;
  return launched(launch_quant_1x32(x, M, K, ldx, q, ldq, scales, layout, (hipStream_t)stream));
}

int mxfp4_preshuffle_weight(const void* w_fp4, const void* w_scales, int64_t batch, int64_t N,
                            int64_t K, void* w_out, void* ws_out, void* stream) {
  if (batch <= 0 || N <= 0 || K <= 0 || K % 32) return MXFP4_ERR_SHAPE;
  if (weight_bytes_one(N, K) > kMaxBuf || gemm_scale_bytes(N, K) > kMaxBuf || N > kMaxBuf ||
      K > kMaxK)
    return MXFP4_ERR_SHAPE;
  if (!w_fp4 || !w_scales || !w_out || !ws_out) return MXFP4_ERR_NULL;
  if (!aligned(w_fp4, 16) || !aligned(w_out, 16) || !aligned(ws_out, 4)) return MXFP4_ERR_ALIGN;
  int st = check_device();
  if (st) return st;
  return launched(launch_preshuffle(w_fp4, w_scales, batch, N, K, w_out, ws_out, (hipStream_t)stream));
}

int mxfp4_gemm_a4w4(const void* a_fp4, const void* a_scales, const void* w_pre,
                    const void* ws_pre, const void* bias, void* out, int64_t ldo, int out_dtype,
                    int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (out_dtype != MXFP4_OUT_BF16 && out_dtype != MXFP4_OUT_F32) return MXFP4_ERR_ARG;
  if (M < 0 || N <= 0 || K <= 0 || K % 32 || K > kMaxK || N > kMaxBuf || M > kMaxBuf)
    return MXFP4_ERR_SHAPE;
  if (ldo < N) return MXFP4_ERR_SHAPE;
  // 256 output rows (one prefill tile) must stay addressable by 32-bit offsets
  if (ldo > kMaxBuf / 256 / (out_dtype == MXFP4_OUT_F32 ? 4 : 2)) return MXFP4_ERR_SHAPE;
  if (weight_bytes_one(N, K) > kMaxBuf || gemm_scale_bytes(N, K) > kMaxBuf ||
      gemm_data_bytes(M, K) > kMaxBuf || gemm_scale_bytes(M, K) > kMaxBuf)
    return MXFP4_ERR_SHAPE;
  const size_t need = mxfp4_gemm_workspace_bytes(M, N, K);
  if (workspace_bytes < need) return MXFP4_ERR_WORKSPACE;
  if (M == 0) return MXFP4_OK;
  if (!a_fp4 || !a_scales || !w_pre || !ws_pre || !out || (need && !workspace)) return MXFP4_ERR_NULL;
  if (!aligned(a_fp4, 16) || !aligned(a_scales, 4) || !aligned(w_pre, 16) ||
      !aligned(ws_pre, 4) || !aligned(out, 4) || (bias && !aligned(bias, 2)) ||
      (workspace && !aligned(workspace, 16)))
    return MXFP4_ERR_ALIGN;
  int cus = 0;
  int st = check_device(&cus);
  if (st) return st;
  GemmArgs p{};
  p.cus = cus;
  p.a = (const uint8_t*)a_fp4;
  p.as = (const uint8_t*)a_scales;
  p.w = (const uint8_t*)w_pre;
  p.ws = (const uint8_t*)ws_pre;
  p.bias = (const uint16_t*)bias;
  p.out = out;
  p.ldo = ldo;
  p.out_f32 = out_dtype == MXFP4_OUT_F32;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.Kt = (int)cdiv(K, 128);
  p.G = (int)cdiv(p.Kt, 4);
  p.Ns = (int)cdiv(N, 16);
  p.x = nullptr;
  p.ldx = 0;
  p.x_bytes = 0;
  p.a_rowmajor = 0;
  p.lda = p.lds = 0;
  p.scales_vec = 0;
  p.out_fp4 = 0;
  p.out_scales = nullptr;
  p.ldos = 0;
  p.work = (uint8_t*)workspace;
  p.work_bytes = workspace ? workspace_bytes : 0;
  hipStream_t s = (hipStream_t)stream;
  return launched(launch_gemm_path(gemm_path(M, N), p, s));
}

size_t mxfp4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N <= 0 || K <= 0 || K % 32) return 0;
  if (M == 0 || linear_fused(M, N, K)) return 0;
  const size_t g = M <= 64 ? 0 : mxfp4_gemm_workspace_bytes(M, N, K);
  return g ? act_gemm_offset(M, K) + g : act_scales_offset(M, K) + (size_t)gemm_scale_bytes(M, K);
}

int mxfp4_linear(const void* x, int64_t ldx, const void* w_pre, const void* ws_pre,
                 const void* bias, void* out, int64_t ldo, int out_dtype, int64_t M, int64_t N,
                 int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  int st = linear_check(x, ldx, w_pre, ws_pre, bias, out, ldo, out_dtype, M, N, K);
  if (st) return st;
  const size_t need = mxfp4_linear_workspace_bytes(M, N, K);
  if (workspace_bytes < need) return MXFP4_ERR_WORKSPACE;
  if (M == 0) return MXFP4_OK;
  if (need && !workspace) return MXFP4_ERR_NULL;
  if (need && !aligned(workspace, 16)) return MXFP4_ERR_ALIGN;
  int cus = 0;
  st = check_device(&cus);
  if (st) return st;
  return linear_run(x, ldx, w_pre, ws_pre, bias, out, ldo, out_dtype, M, N, K, workspace, workspace_bytes,
                    true, cus, (hipStream_t)stream);
}

int mxfp4_gemm_a4w4_mxfp4_out(const void* a_fp4, const void* a_scales, const void* w_pre,
                              const void* ws_pre, const void* bias, void* out_fp4, int64_t ldq,
                              void* out_scales, int64_t lds, int64_t M, int64_t N, int64_t K,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || N <= 0 || N % 32 || K <= 0 || K % 32 || K > kMaxK || N > kMaxBuf || M > kMaxBuf)
    return MXFP4_ERR_SHAPE;
  if (ldq < N / 2 || lds < N / 32) return MXFP4_ERR_SHAPE;
  // 256 output rows (one prefill tile) stay addressable by 32-bit offsets
  if (ldq > kMaxBuf / 256 || lds > kMaxBuf / 256) return MXFP4_ERR_SHAPE;
  if (weight_bytes_one(N, K) > kMaxBuf || gemm_scale_bytes(N, K) > kMaxBuf ||
      gemm_data_bytes(M, K) > kMaxBuf || gemm_scale_bytes(M, K) > kMaxBuf)
    return MXFP4_ERR_SHAPE;
  const size_t need = mxfp4_gemm_workspace_bytes(M, N, K);
  if (workspace_bytes < need) return MXFP4_ERR_WORKSPACE;
  if (M == 0) return MXFP4_OK;
  if (!a_fp4 || !a_scales || !w_pre || !ws_pre || !out_fp4 || !out_scales || (need && !workspace))
    return MXFP4_ERR_NULL;
  if (!aligned(a_fp4, 16) || !aligned(a_scales, 4) || !aligned(w_pre, 16) || !aligned(ws_pre, 4) ||
      !aligned(out_fp4, 4) || ldq % 4 || (bias && !aligned(bias, 2)) || (workspace && !aligned(workspace, 16)))
    return MXFP4_ERR_ALIGN;
  int cus = 0;
  int st = check_device(&cus);
  if (st) return st;
  GemmArgs p{};
  p.cus = cus;
  p.a = (const uint8_t*)a_fp4;
  p.as = (const uint8_t*)a_scales;
  p.w = (const uint8_t*)w_pre;
  p.ws = (const uint8_t*)ws_pre;
  p.bias = (const uint16_t*)bias;
  p.out = out_fp4;
  p.ldo = ldq;
  p.out_f32 = 0;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.Kt = (int)cdiv(K, 128);
  p.G = (int)cdiv(p.Kt, 4);
  p.Ns = (int)cdiv(N, 16);
  p.x = nullptr;
  p.ldx = 0;
  p.x_bytes = 0;
  p.a_rowmajor = 0;
  p.lda = p.lds = 0;
  p.scales_vec = 0;
  p.out_fp4 = 1;
  p.out_scales = (uint8_t*)out_scales;
  p.ldos = lds;
  p.work = (uint8_t*)workspace;
  p.work_bytes = workspace ? workspace_bytes : 0;
  hipStream_t s = (hipStream_t)stream;
  return launched(launch_gemm_path(gemm_path(M, N), p, s));
}

int mxfp4_shuffle_scales(const void* scales, int64_t lds, int64_t rows, int64_t K, void* out,
                         void* stream) {
  if (rows < 0 || K <= 0 || K % 32 || K > kMaxK || rows > kMaxBuf) return MXFP4_ERR_SHAPE;
  if (lds < K / 32 || gemm_scale_bytes(rows, K) > kMaxBuf) return MXFP4_ERR_SHAPE;
  if (rows == 0) return MXFP4_OK;
  if (!scales || !out) return MXFP4_ERR_NULL;
  if (!aligned(out, 4)) return MXFP4_ERR_ALIGN;
  int st = check_device();
  if (st) return st;
  return launched(launch_preshuffle_strided(nullptr, 0, scales, lds, 1, rows, K, nullptr, out,
                                            (hipStream_t)stream));
}

size_t mxfp4_linear_prequantized_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N <= 0 || K <= 0 || K % 32) return 0;
  const int path = M <= 64 ? 1 : gemm_path(M, N);
  if (path != 2) return prequant_permute(M, N, K) ? act_scales_offset(M, K) + (size_t)gemm_scale_bytes(M, K) : 0;
  const size_t g = gemm_prefill_workspace_bytes(M, N, K);
  return g ? act_gemm_offset(M, K) + g : act_scales_offset(M, K) + (size_t)gemm_scale_bytes(M, K);
}

int mxfp4_linear_prequantized(const void* x_fp4, int64_t ldq, const void* x_scales, int64_t lds,
                              const void* w_pre, const void* ws_pre, const void* bias, void* out,
                              int64_t ldo, int out_dtype, int64_t M, int64_t N, int64_t K,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (out_dtype != MXFP4_OUT_BF16 && out_dtype != MXFP4_OUT_F32) return MXFP4_ERR_ARG;
  if (M < 0 || N <= 0 || K <= 0 || K % 32 || K > kMaxK || N > kMaxBuf || M > kMaxBuf)
    return MXFP4_ERR_SHAPE;
  if (ldo < N || ldq < K / 2 || lds < K / 32) return MXFP4_ERR_SHAPE;
  if (ldo > kMaxBuf / 256 / (out_dtype == MXFP4_OUT_F32 ? 4 : 2)) return MXFP4_ERR_SHAPE;
  if (weight_bytes_one(N, K) > kMaxBuf || gemm_scale_bytes(N, K) > kMaxBuf ||
      gemm_data_bytes(M, K) > kMaxBuf || gemm_scale_bytes(M, K) > kMaxBuf)
    return MXFP4_ERR_SHAPE;
  // the small-M kernel reads the row-major operands itself (M <= 64, or 64
  // rows per launch), through 32-bit ranges
  const int path = M <= 64 ? 1 : gemm_path(M, N);
  const bool rows_direct = path != 2 && !prequant_permute(M, N, K);
  const int64_t mr = M < 64 ? M : 64;
  if (M > 0 && rows_direct && ((mr - 1) * ldq + K / 2 > kMaxBuf || (mr - 1) * lds + K / 32 > kMaxBuf))
    return MXFP4_ERR_SHAPE;
  const size_t need = mxfp4_linear_prequantized_workspace_bytes(M, N, K);
  if (workspace_bytes < need) return MXFP4_ERR_WORKSPACE;
  if (M == 0) return MXFP4_OK;
  if (!x_fp4 || !x_scales || !w_pre || !ws_pre || !out || (need && !workspace)) return MXFP4_ERR_NULL;
  if (!aligned(x_fp4, 16) || ldq % 16 || !aligned(w_pre, 16) || !aligned(ws_pre, 4) ||
      !aligned(out, 4) || (bias && !aligned(bias, 2)) || (need && !aligned(workspace, 16)))
    return MXFP4_ERR_ALIGN;
  int cus = 0;
  int st = check_device(&cus);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  GemmArgs p{};
  p.cus = cus;
  p.w = (const uint8_t*)w_pre;
  p.ws = (const uint8_t*)ws_pre;
  p.bias = (const uint16_t*)bias;
  p.out = out;
  p.ldo = ldo;
  p.out_f32 = out_dtype == MXFP4_OUT_F32;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.Kt = (int)cdiv(K, 128);
  p.G = (int)cdiv(p.Kt, 4);
  p.Ns = (int)cdiv(N, 16);
  p.x = nullptr;
  p.ldx = 0;
  p.x_bytes = 0;
  p.out_fp4 = 0;
  p.out_scales = nullptr;
  p.ldos = 0;
  if (rows_direct) {
    // the small-M kernel gathers the row-major operands itself: one launch
    // per 64 rows
    p.a = (const uint8_t*)x_fp4;
    p.as = (const uint8_t*)x_scales;
    p.a_rowmajor = 1;
    p.lda = (uint32_t)ldq;
    p.lds = (uint32_t)lds;
    p.scales_vec = lds % 16 == 0 && aligned(x_scales, 16) && (K / 32) % 16 == 0;
    return launched(launch_gemm_decode_rows(p, s));
  }
  // else: permute into the GEMM layouts in the workspace, then the GEMM
  uint8_t* q = (uint8_t*)workspace;
  uint8_t* sc = q + act_scales_offset(M, K);
  st = launched(launch_preshuffle_strided(x_fp4, ldq, x_scales, lds, 1, M, K, q, sc, s));
  if (st) return st;
  p.a = q;
  p.as = sc;
  p.a_rowmajor = 0;
  p.lda = p.lds = 0;
  p.scales_vec = 0;
  p.work = q + act_gemm_offset(M, K);
  p.work_bytes = workspace_bytes > act_gemm_offset(M, K) ? workspace_bytes - act_gemm_offset(M, K) : 0;
  return launched(launch_gemm_path(path, p, s));
}

int a16wfp4_bmm(const void* x, int64_t sxb, int64_t sxm, const void* w_pre, const void* ws_pre,
                void* out, int64_t sob, int64_t som, int out_dtype, int64_t B, int64_t M,
                int64_t N, int64_t K, void* stream) {
  if (out_dtype != MXFP4_OUT_BF16 && out_dtype != MXFP4_OUT_F32) return MXFP4_ERR_ARG;
  if (B <= 0 || M < 0 || N <= 0 || K <= 0 || K % 32 || K > kMaxK || B > 65535 ||
      M > kMaxBuf || N > kMaxBuf)
    return MXFP4_ERR_SHAPE;
  if (sxm < K || sxb < 0 || sob < 0 || som < 0) return MXFP4_ERR_SHAPE;
  // output rows must not overlap: heads outside rows ([B, M, N]-like) or
  // rows outside heads (batch-major [M, B, N]-like)
  {
    const bool heads_outer = (M <= 1 || som >= N) && (B <= 1 || sob >= (M - 1) * som + N);
    const bool rows_outer = (B <= 1 || sob >= N) && (M <= 1 || som >= (B - 1) * sob + N);
    if (M > 0 && !heads_outer && !rows_outer) return MXFP4_ERR_SHAPE;
  }
  if (weight_bytes_one(N, K) > kMaxBuf || gemm_scale_bytes(N, K) > kMaxBuf ||
      (64 * sxm + K) * 2 > kMaxBuf)
    return MXFP4_ERR_SHAPE;
  if (M == 0) return MXFP4_OK;
  if (!x || !w_pre || !ws_pre || !out) return MXFP4_ERR_NULL;
  if (!aligned(x, 16) || sxb % 8 || sxm % 8 || !aligned(w_pre, 16) || !aligned(ws_pre, 4) ||
      !aligned(out, 4) || sob % 2 || som % 2)
    return MXFP4_ERR_ALIGN;
  int cus = 0;
  int st = check_device(&cus);
  if (st) return st;
  return launched(launch_bmm_a16w4(x, sxb, sxm, w_pre, ws_pre, out, sob, som,
                                   out_dtype == MXFP4_OUT_F32, B, M, N, K, (hipStream_t)stream, cus));
}

// Test hook (include/mxfp4_testing.h): force a GEMM kernel on this thread.
int mxfp4_testing_set_gemm_path(int path) {
  if (path < 0 || path > 8) return MXFP4_ERR_ARG;
  set_gemm_path_override(path);
  return MXFP4_OK;
}

}  // extern "C"
