// Internal declarations shared by the HIP translation units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aqlm {

// The three codebook schemes (M codebooks, B-bit codes, codeword length g).
enum class Scheme : int {
  k2x8 = 0,      // M = 2, B = 8,  g = 8
  k1x16 = 1,     // M = 1, B = 16, g = 8
  k1x16g16 = 2,  // M = 1, B = 16, g = 16
  kGeneral = 3   // any other M = 1..8, B = 8..16, g = 8 or 16
};

struct LayerDesc {
  int64_t out;           // output rows
  int64_t in;            // input columns
  int64_t groups;        // in / g
  Scheme scheme;
  int M, B, g;           // codebooks, code bits, codeword length
  bool packed;           // codes bit-packed into 32-bit words (B bits each)
  const void *codes;     // [out][groups][M]; uint8 codes when B == 8, uint16 when B > 8,
                         // or the bit-packed stream
  const uint16_t *books; // [M][2^B][g] fp16 bits
  const uint16_t *scales;// [out] fp16 bits
};

constexpr int group_size(Scheme s) { return s == Scheme::k1x16g16 ? 16 : 8; }

// The three dedicated schemes store exactly two bytes of codes per group.
constexpr int kCodeBytesPerGroup = 2;

hipError_t launch_dequant(const LayerDesc &L, uint16_t *W, hipStream_t stream);
hipError_t launch_gemv(const LayerDesc &L, const uint16_t *x, int batch, uint16_t *y,
                       hipStream_t stream);
hipError_t launch_gemm(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                       hipStream_t stream);
// GEMV calls that the skinny matrix-core GEMM tiles (gemm.hip) serve faster
// than the GEMV kernels, and their launch.
bool gemv_uses_gemm_tiles(const LayerDesc &L, int batch);
hipError_t launch_gemv_as_gemm(const LayerDesc &L, const uint16_t *x, int batch, uint16_t *y,
                               hipStream_t stream);
// Batched product with a caller-owned workspace (gemm_mid.hip): bytes the
// workspace needs for this layer and batch (0: none, the call then runs
// launch_gemm), and the launch itself.
int64_t gemm_ws_bytes(const LayerDesc &L, int64_t batch);
// The same form at one activation tile (1..16 rows) where it needs no
// workspace at all (activations read in place, K not split); launch_gemm and
// the GEMV route to it when true, through launch_gemm_ws with no workspace.
bool gemm_mid_direct(const LayerDesc &L, int64_t batch);
hipError_t launch_gemm_ws(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                          void *ws, hipStream_t stream);
// Product for many activation rows with the weight tile decoded once into LDS
// per 256 activation rows (gemm_tile.hip, the three dedicated schemes):
// whether it serves the layer at this batch, its modelled duration (us),
// whether aqlm_gemm takes it over the wide tiles, and its launch.
bool gemm_tile_fits(const LayerDesc &L, int64_t batch);
double gemm_tile_cost_us(const LayerDesc &L, int64_t batch);
bool gemm_tile_preferred(const LayerDesc &L, int64_t batch);
hipError_t launch_gemm_tile(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                            hipStream_t stream);
// Kernels for Scheme::kGeneral (general.hip).
hipError_t launch_dequant_general(const LayerDesc &L, uint16_t *W, hipStream_t stream);
hipError_t launch_gemv_general(const LayerDesc &L, const uint16_t *x, int batch, uint16_t *y,
                               hipStream_t stream);
hipError_t launch_gemm_general(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                               hipStream_t stream);
// Matrix-core 2x8 GEMV for 1..8 activation rows (gemv_mfma.hip).
bool gemv_2x8_mfma_fits(const LayerDesc &L, int batch);
hipError_t launch_gemv_2x8_mfma(const LayerDesc &L, const uint16_t *x, int batch, uint16_t *y,
                                hipStream_t stream);
// Grouped form: launches every layer that gemv_2x8_mfma_fits accepts and sets
// done[i] for it; the caller launches the rest.
hipError_t launch_gemv_2x8_mfma_batched(const LayerDesc *Ls, const uint16_t *const *xs,
                                        uint16_t *const *ys, int n, int batch, bool *done,
                                        hipStream_t stream);
hipError_t launch_gemv_batched(const LayerDesc *Ls, const uint16_t *const *xs,
                               uint16_t *const *ys, int n, int batch, hipStream_t stream);
// Codebook-sliced 1x16 GEMV for one activation row (gemv_slice.hip): whether
// it serves a layer, the workspace it needs there (float32 member sums), and
// a launch of up to 16 such layers (plus the launch that adds the sums).
bool gemv_slice_fits(const LayerDesc &L, int batch);
int64_t gemv_slice_ws_bytes(const LayerDesc &L);
hipError_t launch_gemv_slice(const LayerDesc *const *Ls, const uint16_t *const *xs,
                             uint16_t *const *ys, float *const *parts, int n, hipStream_t stream);
// Workspace form of the grouped GEMV: the layers gemv_slice_fits accepts run
// the sliced kernel on workspace parts laid out in layer order; the others
// run as in launch_gemv_batched.
int64_t gemv_ws_bytes(const LayerDesc *Ls, int n, int batch);
hipError_t launch_gemv_batched_ws(const LayerDesc *Ls, const uint16_t *const *xs,
                                  uint16_t *const *ys, int n, int batch, void *ws,
                                  hipStream_t stream);

}  // namespace aqlm
