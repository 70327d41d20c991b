/*
 * aqlm_encode.h - C ABI of the toy encoder kernels in libaqlm_mi355x.so:
 * the steps that turn a dense float16 weight matrix into the packed format of
 * aqlm.h (codes, codebooks, scales) by residual k-means codebooks and greedy
 * nearest-codeword codes under the plain squared error.
 *
 * The pages describe AQLM as classic additive quantization adapted to LLM
 * weights: codes are chosen by nearest-neighbour style search over sums of
 * codewords, codebooks and codes are learned by beam search and Adam, and a
 * residual K-means initialisation of the codebooks beats a random one
 * ("Extreme Compression of Large Language Models via Additive Quantization"
 * summary, "Approach"; table "Measured effects reported in the paper";
 * "Limitations"). These kernels cover the part that needs neither calibration
 * data nor training: residual k-means and greedy (beam width one) codes.
 * A caller runs them in this order per layer (the Python driver does):
 *   aqlm_encode_normalize                       scales and group vectors
 *   for each codebook m:
 *     aqlm_encode_init                          K starting centroids
 *     repeat: aqlm_encode_assign, aqlm_encode_update     (Lloyd k-means)
 *     aqlm_encode_round                         codebook m as float16
 *     aqlm_encode_assign with residual          codes of m, residual for m + 1
 *
 * Common rules. Every array pointer is a DEVICE pointer on the current HIP
 * device, 16-byte aligned; the caller owns every buffer and the library keeps
 * none. Work is enqueued on `stream` (a hipStream_t, NULL = default stream)
 * and the call returns without synchronising; arguments are validated on the
 * host first and nothing is enqueued on error. g is 8 or 16; K = 2^B with
 * 8 <= B <= 16. A group vector is g consecutive float32 values; vector i of a
 * layer [out][in] is group i % (in/g) of row i / (in/g). Codes are written
 * and read in the packed layout [n][M] (code of codebook m at element
 * i * M + m), uint8 when B == 8 and uint16 otherwise. Results are
 * deterministic and bit-identical to the CPU oracle of the toy encoder: the
 * squared error is float32 with terms added in ascending k and every
 * operation rounded (no fused multiply-add), ties go to the lowest code, and
 * means are exact sums in 24-bit fixed point. Status codes are aqlm.h's.
 */
#ifndef AQLM_ENCODE_H
#define AQLM_ENCODE_H

#include <stdint.h>

#include "aqlm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Row scales and normalised group vectors of a dense layer W [out][in]
 * (float16 bits, finite values): scales[o] = max_k |W[o][k]| as float16 (1.0
 * for a row of zeros); vecs[o * in + k] = float(W[o][k]) / float(scales[o]),
 * correctly rounded, so every value lies in [-1, 1]. in % g is not required
 * here; out >= 1, in >= 1.
 */
AQLM_API int aqlm_encode_normalize(const uint16_t *W, int64_t out, int64_t in, uint16_t *scales,
                                   float *vecs, void *stream);

/*
 * Starting centroids: centroids[c] = vecs[indices[c]] for c < K (g floats
 * each). indices is a device array of K int64 values in [0, n); a value
 * outside gives a zero centroid instead of a read out of bounds.
 */
AQLM_API int aqlm_encode_init(const float *vecs, int64_t n, int32_t g, const int64_t *indices,
                              int32_t K, float *centroids, void *stream);

/*
 * Nearest centroid: for each of the n vectors, the code c < K with the
 * smallest float32 squared error against centroids[c] (lowest c on a tie) is
 * written to codes[i * M + m] (uint8 when K == 256, else uint16). If residual
 * is not NULL, residual[i] = vecs[i] - centroids[code] (float32); residual
 * may equal vecs (in place) but must not overlap it otherwise. 1 <= M <= 8,
 * 0 <= m < M, n >= 1 (n == 0: no-op).
 */
AQLM_API int aqlm_encode_assign(const float *vecs, int64_t n, int32_t g, const float *centroids,
                                int32_t K, void *codes, int32_t M, int32_t m, float *residual,
                                void *stream);

/*
 * Centroid update: every centroid c with at least one vector whose code
 * (codes[i * M + m]) is c moves to the mean of those vectors; the others keep
 * their value (a stored code >= K moves nothing). The mean is exact in 24-bit
 * fixed point: each component is
 * rounded to a multiple of 2^-24 (nearest, ties to even), summed as a 64-bit
 * integer, and sum * 2^-24 / count is rounded once to float32. workspace is
 * caller-owned device scratch of K * (g + 1) int64 values; the call
 * overwrites it (no state is carried between calls). n <= 2^31.
 */
AQLM_API int aqlm_encode_update(const float *vecs, int64_t n, int32_t g, const void *codes,
                                int32_t K, int32_t M, int32_t m, float *centroids,
                                int64_t *workspace, void *stream);

/*
 * Codebook in the packed precision: books[i] = float16(centroids[i]) (round
 * to nearest even) and, if rounded is not NULL, rounded[i] = float(books[i]),
 * for i < count. rounded may equal centroids.
 */
AQLM_API int aqlm_encode_round(const float *centroids, int64_t count, uint16_t *books,
                               float *rounded, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* AQLM_ENCODE_H */
