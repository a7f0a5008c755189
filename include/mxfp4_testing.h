/*
 * mxfp4_testing.h -- test-only entry point of libmxfp4 (not part of the
 * method; the product path never calls it).
 *
 * The parity tests run every GEMM kernel and schedule on every shape, which
 * the automatic choice would not: this forces the choice for the CALLING
 * THREAD only (a thread-local setting; other threads keep the automatic
 * choice).  Size queries made on that thread follow the forced plan, so query
 * workspace sizes after setting it, on the same thread.
 */
#ifndef MXFP4_TESTING_H
#define MXFP4_TESTING_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Forces the GEMM kernel of mxfp4_gemm_a4w4 (and of the large-M share of
 * mxfp4_gemm_a4w4_mxfp4_out, mxfp4_linear and mxfp4_linear_prequantized) on
 * this thread: 0 = choose by M (the default); 1 = the small-M streaming
 * kernel (M <= 64 only; larger M still uses the tiled kernel); 2 = the
 * LDS-tiled kernel on its own plan; 3 = the tiled kernel on whole 256-wide
 * tiles only; 4 = the tiled kernel with the split schedule wherever the
 * tiles leave a round of compute units part-empty and a tile has more than
 * 512 of K; 5 and 6 = as 3 and 4 with 128-wide tiles; 7 and 8 = the
 * small-M kernel (M <= 64) in its persistent form wherever that form
 * applies (one scale group per wave, bf16 or fp32 output, activations in
 * the GEMM layout or row-major), and in its one-workgroup-per-strip form
 * only.
 * Returns MXFP4_OK, or MXFP4_ERR_ARG for other values.
 */
#pragma GCC visibility push(default)
int mxfp4_testing_set_gemm_path(int path);
#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_TESTING_H */
