// Internal declarations shared by the HIP translation units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aqlm {

// The three codebook schemes (M codebooks, B-bit codes, codeword length g).
enum class Scheme : int {
  k2x8 = 0,     // M = 2, B = 8,  g = 8
  k1x16 = 1,    // M = 1, B = 16, g = 8
  k1x16g16 = 2  // M = 1, B = 16, g = 16
};

struct LayerDesc {
  int64_t out;           // output rows
  int64_t in;            // input columns
  int64_t groups;        // in / g
  Scheme scheme;
  const void *codes;     // [out][groups][M], 2 bytes per group in every scheme
  const uint16_t *books; // [M][2^B][g] fp16 bits
  const uint16_t *scales;// [out] fp16 bits
};

constexpr int group_size(Scheme s) { return s == Scheme::k1x16g16 ? 16 : 8; }

// Every supported scheme stores exactly two bytes of codes per group.
constexpr int kCodeBytesPerGroup = 2;

hipError_t launch_dequant(const LayerDesc &L, uint16_t *W, hipStream_t stream);
hipError_t launch_gemv(const LayerDesc &L, const uint16_t *x, int batch, uint16_t *y,
                       hipStream_t stream);
hipError_t launch_gemm(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                       hipStream_t stream);
hipError_t launch_gemv_batched(const LayerDesc *Ls, const uint16_t *const *xs,
                               uint16_t *const *ys, int n, int batch, hipStream_t stream);

}  // namespace aqlm
