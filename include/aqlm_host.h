/*
 * aqlm_host.h - C ABI of the host (CPU) matrix-vector product for additive
 * multi-codebook quantized layers, built as its own library (libaqlm_host.so)
 * beside the MI355X one. It serves callers whose activations live in host
 * memory; it is never called by the GPU entry points and the GPU library
 * never falls back to it.
 *
 * The operation and the packed format are those of aqlm.h: every weight
 * vector is the sum of one codeword from each of M codebooks, scaled by its
 * row's scale ("Additive quantization that actually survives one-bit
 * weights", section "What it does"). The pages mention CPU kernels next to the
 * GPU ones ("AQLM (additive / multi-codebook quantization)", field "Kernels":
 * token generation by lookup, with no per-element dequantization; "Additive
 * quantization that actually survives one-bit weights", "Key highlights").
 *
 * Method. For 8-bit codebooks (B == 8) each call first builds, per
 * activation row b and group j, the table T[b][j][m][c] = <x_b[j], C_m[c]>
 * (float32), after which a group costs M table reads and adds:
 *   y[b][o] = fp16( scale[o] * sum_j sum_m T[b][j][m][codes[o][j][m]] ).
 * For B > 8 (tables of 2^B entries per group would not fit in cache) each
 * group's codewords are summed in float32 in ascending m and dotted with the
 * activations in float32. Either way the result equals x . W^T within the
 * product tolerance of aqlm.h's GEMV (float32 accumulation in a fixed order,
 * one round to float16); it is not bit-identical to the GPU library.
 */
#ifndef AQLM_HOST_H
#define AQLM_HOST_H

#include <stdint.h>

#include "aqlm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * aqlm_host_gemv: y[b][o] = sum_i x[b][i] * W[o][i] for b < batch,
 * 1 <= batch <= 8 (batch == 0 is a no-op returning AQLM_OK).
 *   layer    the packed layer as in aqlm.h (element or bit-packed codes),
 *            except that codes, codebooks and scales are HOST pointers (no
 *            alignment requirement)
 *   x        host, [batch][in] float16 bits
 *   y        host, [batch][out] float16 bits, written in full
 *   threads  worker threads (OpenMP); <= 0 uses the runtime's default
 * Supported schemes, shape rules and status codes are those of aqlm.h
 * (AQLM_ERR_ALIGN and AQLM_ERR_HIP are never returned). The call allocates
 * its float32 tables and activations on the host heap and frees them before
 * returning, blocks until y is written, keeps no state and is reentrant.
 * Each output is summed by one thread in a fixed order, so results do not
 * depend on the thread count.
 */
AQLM_API int aqlm_host_gemv(const aqlm_layer *layer, const uint16_t *x, int64_t batch, uint16_t *y,
                            int32_t threads);

/* Instruction set the host library selected at run time: "avx2" (AVX2, FMA
 * and F16C present) or "scalar". Static string, never NULL. */
AQLM_API const char *aqlm_host_isa(void);

#ifdef __cplusplus
}
#endif

#endif /* AQLM_HOST_H */
