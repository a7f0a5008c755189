/*
 * mxfp4.h -- C ABI of the MI355X (gfx950) W4A4 MXFP4 linear and A16WFP4 BMM.
 *
 * Sources cited below:
 *   P1  web page "[AMD] Add opt-in AITER ASM FP4 GEMM for Quark dense linear"
 *       (sgl-project/sglang pull request 39598): Modifications, Accuracy Tests.
 *   P2  web page "[sglang] SGLang, AMD GPU에서 Quark 모델의 FP4 GEMM 성능 최적화:
 *       AITER ASM 활용" (analysis of that pull request with its diff), section
 *       "2. AITER ASM FP4 GEMM 통합" (scale swizzle, activation-scale padding,
 *       registered quantisation and GEMM ops, apply_weights).
 *   P3  web page "[AMD] [GLM5] use tuned MXFP4 kernels for MLA absorbed BMM"
 *       (sgl-project/sglang pull request 34317): Motivation, Modifications.
 *   OCP-MX  OCP Microscaling Formats (MX) Specification v1.0: E2M1 elements,
 *       E8M0 scales, conversion of a 32-value vector into one MX block.
 *
 * Conventions shared by every entry point
 *   - Every data pointer is DEVICE memory owned by the caller.  The library
 *     never allocates, frees or synchronises; each call validates its
 *     arguments on the host, enqueues its kernels on `stream` (a hipStream_t;
 *     NULL is the default stream) and returns.
 *   - Returns MXFP4_OK (0) or an mxfp4_status code; on error nothing is
 *     enqueued.  Argument checks run before any HIP call, so they also work
 *     on a host without a GPU.
 *   - bf16 is IEEE binary32 truncated to its top 16 bits.  Packed FP4 holds
 *     two E2M1 codes per byte, element 2j in the low nibble of byte j (the
 *     float4_e2m1fn_x2 packing named in P2 §2).  Scales are E8M0 bytes,
 *     value 2^(b-127); 0xFF (NaN) is never written, padding is 0x7F (1.0).
 *   - K must be a positive multiple of 32 (one scale per 1x32 block).
 *
 * Layouts (all byte offsets; the library's own design for gfx950's
 * 16x16x128 block-scaled FP4 MFMA):
 *   GEMM data layout (quantised activations and preshuffled weights alike),
 *   R rows, Kt = ceil(K/128), per batch entry b of Rp = 16*ceil(R/16) rows:
 *     pair (r, k), k even: s = r/16, t = k/128, kb = (k%128)/32,
 *     offset = ((b*Rp/16 + s)*Kt + t)*1024 + (kb*16 + r%16)*16 + (k%32)/2,
 *     element k in the low nibble; padding bytes (rows >= R, k >= K) 0x00.
 *     A 1 KiB unit (s, t) is a 16-row x 128-K tile whose 16-byte slot
 *     kb*16 + r%16 is that row's whole 1x32 block kb: the operand of MFMA
 *     lane kb*16 + r%16.  Size B*Rp*Kt*64.
 *   GEMM scale layout, G = ceil(Kt/4):
 *     scale (r, c): t = c/4, kb = c%4, g = t/4, j = t%4,
 *     offset = ((r/16)*G + g)*256 + (kb*16 + r%16)*4 + j;  size Rp*G*16,
 *     batch entries concatenated; padding bytes 0x7F.
 *   ROWMAJOR: packed FP4 [R, K/2] (row stride given) and scales [R, K/32].
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbols by default; the entry points
 * declared here are its only exports. */
#pragma GCC visibility push(default)

typedef enum {
  MXFP4_OK = 0,
  MXFP4_ERR_NULL = 1,      /* a required pointer is NULL                        */
  MXFP4_ERR_SHAPE = 2,     /* a size <= 0 (or < 0 where 0 is allowed), K % 32   */
  MXFP4_ERR_ALIGN = 3,     /* pointer or stride not aligned as documented       */
  MXFP4_ERR_WORKSPACE = 4, /* workspace missing or smaller than required        */
  MXFP4_ERR_DEVICE = 5,    /* the current HIP device is not gfx950              */
  MXFP4_ERR_LAUNCH = 6,    /* a HIP launch failed                               */
  MXFP4_ERR_ARG = 7        /* an enum argument is out of range                  */
} mxfp4_status;

enum { MXFP4_LAYOUT_ROWMAJOR = 0, MXFP4_LAYOUT_GEMM = 1 };
enum { MXFP4_OUT_BF16 = 0, MXFP4_OUT_F32 = 1 };

/* Static string naming a status code (never NULL). */
const char* mxfp4_status_str(int status);

/* ABI version: major * 100 + minor.  1.02: the GEMM entry points may ask
 * for a workspace (mxfp4_gemm_workspace_bytes) for large M.  1.03: the
 * workspace's first word reports a give-up of the split schedule's bounded
 * wait; overlapping BMM output strides are rejected; the kernel-selection
 * test hook moved to mxfp4_testing.h and acts per thread. */
int mxfp4_abi_version(void);

/* Bytes of the packed FP4 data / the scales for `rows` x K in `layout`:
 * rows*K/2 and rows*K/32 for ROWMAJOR, the padded GEMM-layout sizes
 * otherwise.  0 on invalid arguments. */
size_t mxfp4_data_bytes(int64_t rows, int64_t K, int layout);
size_t mxfp4_scale_bytes(int64_t rows, int64_t K, int layout);

/* Bytes of the preshuffled weight data / its scales for `batch` matrices of
 * N x K.  0 on invalid arguments. */
size_t mxfp4_weight_bytes(int64_t batch, int64_t N, int64_t K);
size_t mxfp4_weight_scale_bytes(int64_t batch, int64_t N, int64_t K);

/* Workspace bytes mxfp4_gemm_a4w4 and mxfp4_gemm_a4w4_mxfp4_out need for
 * this shape: 0 where the GEMM needs none (every M <= 64 call, calls of up
 * to 256 rows on few columns, and most larger ones on whole output tiles),
 * else the split schedule's (see
 * mxfp4_gemm_a4w4), sized for up to 256 compute units: a give-up word, 4
 * bytes per split tile and per workgroup (these rounded up to 256 bytes),
 * then one fp32 output tile per workgroup (256 KiB, or 128 KiB with
 * 128-wide tiles; up to 64 MiB).
 * (A test build may force another plan for the calling thread:
 * mxfp4_testing.h.)  0 on invalid shapes. */
size_t mxfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * Per-1x32 MXFP4 quantisation (P1 §Modifications: activations are quantised
 * per 1x32 before the FP4 GEMM; P2 §2: the quantisation op returns packed
 * FP4 and one E8M0 scale per block; the scheme quantises weights the same
 * way).  Arithmetic per OCP-MX, reading as follows: per block amax, scale
 * byte b = max(E(amax) - 2, 0) with E the biased exponent field of amax,
 * element |v| / 2^(b-127) rounded to the nearest E2M1 magnitude with ties to
 * the even code and saturation at 6, sign bit copied from v.
 *
 *   x       bf16 [M, K], row stride ldx ELEMENTS (ldx >= K, ldx % 8 == 0,
 *           x 16-byte aligned)
 *   layout  ROWMAJOR: q is [M, K/2] with row stride ldq BYTES (ldq >= K/2,
 *             ldq % 4 == 0, q 4-byte aligned); scales [M, K/32].
 *           GEMM: q and scales in the GEMM layouts above
 *             (mxfp4_data_bytes / mxfp4_scale_bytes bytes; ldq ignored;
 *             q 16-byte aligned, scales 4-byte aligned); every padding byte
 *             is written (0x00 data, 0x7F scales: P2 §2 pads scale tiles with
 *             1.0 because whole tiles are read and 0xFF is NaN).  This is the
 *             form mxfp4_gemm_a4w4 reads, and for a weight it is bytewise the
 *             output of mxfp4_preshuffle_weight.
 *   M >= 0 (M == 0 enqueues nothing), K > 0, K % 32 == 0.
 */
int mxfp4_quant_1x32(const void* x, int64_t M, int64_t K, int64_t ldx,
                     void* q, int64_t ldq, void* scales, int scale_layout,
                     void* stream);

/*
 * Load-time weight preshuffle (P1 §Modifications and P2 §2: weights and
 * their E8M0 scales are rearranged once after loading into the layout the
 * FP4 GEMM reads).  Permutation only, from already quantised ROWMAJOR bytes
 * (e.g. a checkpoint's) into the GEMM layouts, batch entries each padded to
 * a multiple of 16 rows.  A bf16 weight can instead be quantised straight
 * into the GEMM layout with mxfp4_quant_1x32.
 *
 *   w_fp4     packed FP4 [batch, N, K/2], contiguous, 16-byte aligned
 *   w_scales  ROWMAJOR scales [batch, N, K/32], contiguous
 *   w_out     mxfp4_weight_bytes(batch, N, K) bytes, 16-byte aligned
 *   ws_out    mxfp4_weight_scale_bytes(batch, N, K) bytes, 4-byte aligned
 *   batch >= 1, N >= 1, K > 0, K % 32 == 0.
 */
int mxfp4_preshuffle_weight(const void* w_fp4, const void* w_scales,
                            int64_t batch, int64_t N, int64_t K,
                            void* w_out, void* ws_out, void* stream);

/*
 * W4A4 block-scaled FP4 GEMM with optional bias (P2 §2, apply_weights and
 * the registered GEMM op: Y[M, N] = dq(A) dq(W)^T in the NT form of a linear
 * layer, output (M, N), bias added after; P1 §Accuracy Tests: equal to a
 * separately dequantised reference).  Computed as
 *   out[m, n] = round(sum_k dq(A)[m,k] dq(W)[n,k] + bias[n])
 * with fp32 accumulation and one round-to-nearest-even cast for bf16.
 *
 *   a_fp4, a_scales  activations in the GEMM layouts (from mxfp4_quant_1x32
 *             with MXFP4_LAYOUT_GEMM), 16- and 4-byte aligned
 *   w_pre, ws_pre    weights in the same layouts (one batch entry)
 *   bias      bf16 [N] or NULL
 *   out       [M, N], row stride ldo ELEMENTS, bf16 or fp32 per out_dtype
 *             (N <= ldo < 2^22 for bf16, < 2^21 for fp32; 4-byte aligned)
 *   workspace mxfp4_gemm_workspace_bytes(M, N, K) bytes, 16-byte aligned
 *             (NULL when that is 0); scratch owned by the call until it
 *             completes on `stream`: its contents need no initialisation
 *             and are not kept, except that after a call that used it (a
 *             nonzero size) its first 32-bit word is nonzero if a bounded
 *             wait of the split schedule gave up (never expected; the sum of
 *             that tile is then not to be trusted).  Calls that overlap in
 *             time (other streams) need workspaces of their own.
 *   M >= 0 (M == 0 enqueues nothing), N >= 1, K > 0, K % 32 == 0.
 * For 64 < M <= 256 with ceil(M/64) * N <= 16384 the small-M kernel runs
 * once per 64 rows (each launch as a call on those rows alone would be).
 * Otherwise, for M > 64 the output is cut into 256 x 256 tiles, or 256 x 128 where the
 * wider ones would leave most compute units idle (measured rule).  Where
 * whole tiles would leave the last round of compute units at most half full
 * and K is long enough to pay for it,
 * the tiles short of whole rounds are each cut along K into equal slices
 * for the otherwise idle workgroups (split-K): a split tile's fp32 partial
 * sums meet in the workspace and are added in K order by the last
 * workgroup to finish a slice (found by an atomic ticket), so results are
 * still identical run to run, whatever order the slices finish in.  The
 * call then launches a small kernel that clears the workspace's counters
 * before the GEMM (no memset: the pair can be captured into a graph).
 */
int mxfp4_gemm_a4w4(const void* a_fp4, const void* a_scales,
                    const void* w_pre, const void* ws_pre, const void* bias,
                    void* out, int64_t ldo, int out_dtype,
                    int64_t M, int64_t N, int64_t K,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The whole W4A4 linear from bf16 activations (P2 §2, apply_weights: the
 * activations are quantised per 1x32 and fed with the preshuffled weight to
 * the FP4 GEMM, bias added after).  Same result as mxfp4_quant_1x32 (GEMM
 * layout) followed by mxfp4_gemm_a4w4:
 *   out[m, n] = round(sum_k dq(Q(x))[m,k] dq(W)[n,k] + bias[n]).
 * Where it is faster (M = 1; M = 2 for K <= 16384; M <= 4 for N < 16384
 * and K <= 8192, except M >= 3 for 8192 < N <= 12288; M <= 4 for N <= 4096
 * and K <= 16384; 2 <= M <= 4 with 4608 < K <= 6144 and at least six
 * 16-column weight strips per compute unit) the quantisation runs inside
 * the GEMM kernel: one launch, no
 * quantised copy of x, bitwise the same output as the two-call form.
 * Otherwise x is quantised into `workspace` and the GEMM kernel for that M
 * then reads it.
 *
 *   x       bf16 [M, K], row stride ldx ELEMENTS (ldx >= K, ldx % 8 == 0,
 *           16-byte aligned); for M <= 4, ((M-1)*ldx + K)*2 < 2^31
 *   w_pre, ws_pre, bias, out, ldo, out_dtype: as for mxfp4_gemm_a4w4
 *   workspace  mxfp4_linear_workspace_bytes(M, N, K) bytes (0 when the
 *           quantisation is fused: then it may be NULL; the last fused case
 *           above, which depends on the device, still asks for it and leaves
 *           it untouched), 16-byte aligned; overwritten, caller-owned
 *   M >= 0 (M == 0 enqueues nothing), N >= 1, K > 0, K % 32 == 0.
 */
size_t mxfp4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);
int mxfp4_linear(const void* x, int64_t ldx, const void* w_pre, const void* ws_pre,
                 const void* bias, void* out, int64_t ldo, int out_dtype,
                 int64_t M, int64_t N, int64_t K,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * mxfp4_linear for callers that cannot allocate device memory or pass a
 * workspace (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments without the workspace, the same
 * result as mxfp4_linear (bitwise, wherever mxfp4_linear does not take the
 * large-M kernel's split schedule; this entry point always runs whole tiles).
 * The quantised activations go to the library's own scratch array, a fixed
 * 32 MiB of device memory per GPU that the library runs on, held until the
 * process ends: this call allocates nothing.  Shapes whose quantised
 * activations exceed it (ceil(M/16) * (ceil(K/128) * 1024 + ceil(K/512) * 256)
 * bytes: M above 4400 at K = 14336, above 12336 at K = 5120) return
 * MXFP4_ERR_WORKSPACE, before anything is enqueued.  Every call on a
 * GPU shares that GPU's scratch: calls that overlap in time on one GPU
 * (other streams) race, and must not be made.
 */
int mxfp4_linear_noalloc(const void* x, int64_t ldx, const void* w_pre, const void* ws_pre,
                         const void* bias, void* out, int64_t ldo, int out_dtype,
                         int64_t M, int64_t N, int64_t K, void* stream);

/*
 * W4A4 GEMM with MXFP4 output for the next layer (the producer side of the
 * prequantised input of P2 §2: the next layer's activations leave this
 * GEMM already quantised, instead of as bf16 that a separate quantisation
 * reads back).  The output row y = round_bf16(sum_k dq(A) dq(W) + bias) is
 * quantised per 1x32 block along N exactly as mxfp4_quant_1x32 would
 * quantise the bf16 output of mxfp4_gemm_a4w4 (bitwise the same bytes),
 * inside the GEMM's epilogue.
 *
 *   a_fp4, a_scales, w_pre, ws_pre, bias: as for mxfp4_gemm_a4w4
 *   out_fp4     packed FP4 [M, N/2], row stride ldq BYTES (N/2 <= ldq,
 *               ldq % 4 == 0, 4-byte aligned)
 *   out_scales  E8M0 [M, N/32], row stride lds BYTES (N/32 <= lds)
 *   (ldq, lds < 2^23); the ROWMAJOR form mxfp4_linear_prequantized reads.
 *   M >= 0 (M == 0 enqueues nothing), N >= 32, N % 32 == 0, K > 0,
 *   K % 32 == 0; workspace as for mxfp4_gemm_a4w4.
 */
int mxfp4_gemm_a4w4_mxfp4_out(const void* a_fp4, const void* a_scales, const void* w_pre,
                              const void* ws_pre, const void* bias, void* out_fp4, int64_t ldq,
                              void* out_scales, int64_t lds, int64_t M, int64_t N, int64_t K,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Scale re-layout for activations quantised elsewhere (P2 §2: a fused
 * producer hands over (packed FP4, row-major E8M0 scales); the scales are
 * swizzled into the GEMM's order and padded with E8M0 1.0 before the GEMM).
 *
 *   scales  ROWMAJOR [rows, K/32], row stride lds BYTES (lds >= K/32)
 *   out     mxfp4_scale_bytes(rows, K, MXFP4_LAYOUT_GEMM) bytes, 4-byte
 *           aligned: the GEMM scale layout, every padding byte 0x7F
 *   rows >= 0 (0 enqueues nothing), K > 0, K % 32 == 0.
 */
int mxfp4_shuffle_scales(const void* scales, int64_t lds, int64_t rows, int64_t K,
                         void* out, void* stream);

/*
 * The W4A4 linear from activations quantised elsewhere (P2 §2, the
 * prequantised-input form of apply_weights): packed FP4 and E8M0 scales in
 * the ROWMAJOR form mxfp4_quant_1x32 also writes, as a fused producer
 * (normalisation + quantisation) would hand them over.
 *   out[m, n] = round(sum_k dq(x)[m,k] dq(W)[n,k] + bias[n])
 * For M <= 64 the GEMM kernel reads the row-major operands directly (one
 * launch; bitwise the result of mxfp4_gemm_a4w4 on the same values in the
 * GEMM layouts), and so it does once per 64 rows where mxfp4_gemm_a4w4 runs
 * the small-M kernel per 64 rows (M <= 256, ceil(M/64) * N <= 16384) --
 * except with K > 4608 and more than 32 rows per launch, or more than 8
 * with K > 6144 and N >= 10240, where they are first permuted into the
 * GEMM layouts in `workspace` (one more launch, faster there); for larger
 * M they are permuted into `workspace` first, then the tiled kernel runs.
 *
 *   x_fp4     packed FP4 [M, K/2], row stride ldq BYTES (ldq >= K/2,
 *             ldq % 16 == 0, 16-byte aligned)
 *   x_scales  E8M0 [M, K/32], row stride lds BYTES (lds >= K/32)
 *   w_pre, ws_pre, bias, out, ldo, out_dtype: as for mxfp4_gemm_a4w4
 *   workspace mxfp4_linear_prequantized_workspace_bytes(M, N, K) bytes (0
 *             where the small-M kernel reads the operands: may be NULL),
 *             16-byte aligned, caller-owned
 *   M >= 0 (M == 0 enqueues nothing), N >= 1, K > 0, K % 32 == 0.
 */
size_t mxfp4_linear_prequantized_workspace_bytes(int64_t M, int64_t N, int64_t K);
int mxfp4_linear_prequantized(const void* x_fp4, int64_t ldq, const void* x_scales,
                              int64_t lds, const void* w_pre, const void* ws_pre,
                              const void* bias, void* out, int64_t ldo, int out_dtype,
                              int64_t M, int64_t N, int64_t K,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * A16WFP4 batched GEMM (P3 §Motivation and §Modifications: the MLA absorbed
 * K/V projection weights stay in packed MXFP4, the batched products take
 * bf16 activations, and the V-up result is written batch-major).  For each
 * b < B:
 *   out[b, m, n] = round(sum_k x[b, m, k] * dq(W)[b, n, k])
 * with exact bf16 activations, fp32 accumulation and one RNE cast for bf16.
 *
 *   x      bf16, element (b, m, k) at x[b*sxb + m*sxm + k] (ELEMENTS;
 *          sxb, sxm % 8 == 0, pointer 16-byte aligned)
 *   w_pre  preshuffled weights of `B` matrices N x K, ws_pre their scales
 *   out    element (b, m, n) at out[b*sob + m*som + n] (ELEMENTS; sob, som
 *          even, pointer 4-byte aligned).  [B, M, N]: sob = M*N, som = N;
 *          batch-major [M, B, N]: sob = N, som = B*N.  Rows must not
 *          overlap: either som >= N and sob >= (M-1)*som + N, or sob >= N
 *          and som >= (B-1)*sob + N (a stride of a size-1 dimension is
 *          free); otherwise MXFP4_ERR_SHAPE.
 *   B >= 1, M >= 0 (M == 0 enqueues nothing), N >= 1, K > 0, K % 32 == 0.
 */
int a16wfp4_bmm(const void* x, int64_t sxb, int64_t sxm,
                const void* w_pre, const void* ws_pre,
                void* out, int64_t sob, int64_t som, int out_dtype,
                int64_t B, int64_t M, int64_t N, int64_t K, void* stream);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
