/*
 * aqlm.h - C ABI of the MI355X (gfx950) library for additive multi-codebook
 * quantized linear layers (AQLM).
 *
 * The operation. A linear layer y = x . W^T whose weight matrix W [out, in]
 * is stored as sums of learned codebook vectors: every weight vector is the
 * sum of one codeword from each of M codebooks ("Additive quantization that
 * actually survives one-bit weights", section "What it does"; "AQLM
 * (additive / multi-codebook quantization)", field "Activation scheme").
 * Activations stay float16; only the weights are quantized ("AQLM (additive
 * / multi-codebook quantization)", field "Bits").
 *
 * Packed format (all arrays dense, row-major, little-endian):
 *   codes      [out][in/g][M]   uint8 when B == 8, uint16 when B > 8 (one
 *                               code per element); an entry is an unsigned
 *                               codeword index < 2^B
 *   codebooks  [M][2^B][g]      float16 bit patterns
 *   scales     [out]            float16 bit patterns, one per output row
 * Bit-packed codes (flags = AQLM_CODES_PACKED): codes is instead a stream of
 * ceil(out * (in/g) * M * B / 32) little-endian 32-bit words, and code m of
 * group j of row o occupies bits p .. p + B - 1 of the stream, with
 * p = ((o * (in/g) + j) * M + m) * B and bit p being bit p % 32 of word
 * p / 32 (least significant first). The codes then cost exactly M * B / g
 * bits per weight for every B; for B = 8 and B = 16 the stream holds the
 * same bytes as the uint8 / uint16 arrays above.
 * Group j of output row o covers input columns j*g .. j*g+g-1, and
 *   W[o][j*g+k] = fp16_rne( float(scales[o]) *
 *                           (float(C_0[c_0][k]) + ... + float(C_{M-1}[c_{M-1}][k])) )
 * with c_m = codes[o][j][m], the float32 sum taken in ascending m starting
 * from the m = 0 codeword, a float32 multiply, and one round to nearest-even
 * float16 (subnormals kept, overflow to infinity). The pages leave the
 * group-to-column map, the scale and the rounding unstated; this is the
 * library's reading of them.
 *
 * Supported schemes: 1 <= M <= 8 codebooks, 8 <= B <= 16 code bits and
 * codeword length g = 8 or 16 -- the 8- and 16-dimensional codebooks of
 * "Additive quantization that actually survives one-bit weights", sections
 * "Key highlights" and "Caveats", with the number of codebooks and the group
 * size free as in the ablation of the "Extreme Compression of Large Language
 * Models via Additive Quantization" summary (table "Measured effects reported
 * in the paper"). (2, 8, 8) "2x8", (1, 16, 8) "1x16" and (1, 16, 16)
 * "1x16 g16" run dedicated kernels; every other scheme runs general ones.
 * Any in_features that is a multiple of g is accepted.
 *
 * Pointers. Every array pointer is a DEVICE pointer on the current HIP
 * device; codes, codebooks, scales, x, y and W must each be 16-byte aligned.
 * The caller owns every buffer: the library allocates nothing, frees
 * nothing and keeps no pointer after a call returns. Outputs must not alias
 * inputs.
 *
 * Streams and errors. `stream` is a hipStream_t (NULL = the default stream).
 * Each entry point validates its arguments on the host, then enqueues its
 * kernels on `stream` and returns without synchronising; buffers must stay
 * alive until that stream's work is done. On a validation failure nothing is
 * enqueued and a status below is returned. A launch failure reported by the
 * HIP runtime returns AQLM_ERR_HIP. Faults inside a kernel surface at the
 * caller's next synchronisation. All entry points are reentrant and keep no
 * state, except aqlm_gemm_noalloc, which keeps the address of its static
 * scratch array per device and whose overlapping calls on one GPU race (see
 * there). Results are deterministic: the same inputs give bit-identical
 * outputs on every call.
 */
#ifndef AQLM_MI355X_H
#define AQLM_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AQLM_ABI_VERSION 5

/* aqlm_layer.flags: codes are bit-packed (see the format above). */
#define AQLM_CODES_PACKED 1

#if defined(__GNUC__) || defined(__clang__)
#define AQLM_API __attribute__((visibility("default")))
#else
#define AQLM_API
#endif

typedef enum aqlm_status {
  AQLM_OK = 0,
  AQLM_ERR_NULL = 1,   /* a required pointer is NULL */
  AQLM_ERR_SHAPE = 2,  /* out < 1, in < 1, in % g != 0, a size overflows, or
                          unknown flags */
  AQLM_ERR_SCHEME = 3, /* (M, B, g) is not a supported scheme */
  AQLM_ERR_ALIGN = 4,  /* a pointer is not 16-byte aligned */
  AQLM_ERR_BATCH = 5,  /* batch outside the entry point's range */
  AQLM_ERR_HIP = 6,    /* the HIP runtime reported an error at launch */
  AQLM_ERR_WORKSPACE = 7, /* the workspace is smaller than aqlm_gemm_workspace_size */
  AQLM_ERR_SCRATCH = 8    /* aqlm_gemm_noalloc: the call needs more than
                             AQLM_STATIC_SCRATCH_BYTES of scratch memory */
} aqlm_status;

/* Size of the static device scratch array behind aqlm_gemm_noalloc (64 MiB;
   one copy per GPU the library runs on, held until the process ends). */
#define AQLM_STATIC_SCRATCH_BYTES (64ll << 20)

/* One quantized layer: sizes plus device pointers to the packed arrays. */
typedef struct aqlm_layer {
  int64_t out_features;      /* rows of W, >= 1 */
  int64_t in_features;       /* columns of W, >= 1, multiple of group_size */
  int32_t num_codebooks;     /* M */
  int32_t nbits;             /* B: codebook size is 2^B */
  int32_t group_size;        /* g: codeword length */
  int32_t flags;             /* 0 or AQLM_CODES_PACKED */
  const void *codes;         /* device, [out][in/g][M] uint8 (B=8) / uint16 (B>8),
                                or the bit-packed word stream */
  const uint16_t *codebooks; /* device, [M][2^B][g] float16 bits */
  const uint16_t *scales;    /* device, [out] float16 bits */
} aqlm_layer;

/*
 * aqlm_dequant: materialise W [out][in] float16 (row-major) from the packed
 * layer, bit-exact to the decode rule above. W is written in full; it is
 * the dequantize-to-float16 step that precedes a dense float16 matrix
 * product ("AQLM (additive / multi-codebook quantization)", notes).
 */
AQLM_API int aqlm_dequant(const aqlm_layer *layer, uint16_t *W, void *stream);

/*
 * aqlm_gemv: y[b][o] = sum_i x[b][i] * W[o][i] for b < batch, 1 <= batch <= 8,
 * without materialising W: codes are streamed once and every group is
 * decoded by codebook lookup inside the kernel (the token-generation path
 * of "AQLM (additive / multi-codebook quantization)", field "Kernels").
 * x is [batch][in] float16, y is [batch][out] float16 (round to nearest
 * from a float32 accumulation). batch == 0 is a no-op returning AQLM_OK.
 * Where a 16-row matrix-core tile of aqlm_gemm is faster for the batch
 * (1x16 codes at several rows, 2x8 rows too long to stage 3..8 activation
 * rows on chip) the call runs that tile; W is still never written.
 */
AQLM_API int aqlm_gemv(const aqlm_layer *layer, const uint16_t *x, int64_t batch,
              uint16_t *y, void *stream);

/*
 * aqlm_gemm: the same product for any batch >= 1 (batch == 0: no-op). Tiles
 * of W are decoded on chip and fed to float16 matrix-core (MFMA)
 * instructions with float32 accumulation; W is never written to memory
 * ("AQLM (additive / multi-codebook quantization)", notes: dequantize to
 * float16, then a float16 matrix-engine product). x is [batch][in], y is
 * [batch][out], both float16. Up to 8 rows the call runs aqlm_gemv's
 * routes (the fastest form there) and gives its bits. Above 128 rows, for the
 * three dedicated schemes with in a multiple of 64 (1x16 and 1x16 g16 at any
 * such batch; 2x8 from 512 rows where blocks of 128 output rows x 256
 * activation rows number at least 160), each 128 x 64 weight tile is decoded
 * once into on-chip memory and shared by all 256 activation rows of its
 * block; other calls above 128 rows run tiles of 256 output rows.
 */
AQLM_API int aqlm_gemm(const aqlm_layer *layer, const uint16_t *x, int64_t batch,
              uint16_t *y, void *stream);

/*
 * aqlm_gemm_workspace_size: bytes of device workspace that aqlm_gemm_ws needs
 * for this layer and batch, written to *bytes (0 when that call needs none
 * and runs exactly as aqlm_gemm). The size depends only on the layer's shape
 * and scheme and on batch. Validation and status codes as for aqlm_gemm;
 * *bytes is 0 on error.
 */
AQLM_API int aqlm_gemm_workspace_size(const aqlm_layer *layer, int64_t batch, int64_t *bytes);

/*
 * aqlm_gemm_ws: the product of aqlm_gemm with a caller-owned device
 * workspace, which lets the three dedicated schemes (2x8, 1x16 and 1x16 with
 * g = 16; element or bit-packed codes, in / g a multiple of 8) run the
 * workspace form of the matrix-core path from 17 rows up to 128, and above
 * that up to 4096 rows wherever the workspace stays within 64 MiB and, if
 * aqlm_gemm would run its decoded-tile kernel, the library's timing model of
 * the workspace form is below that kernel's. (At 1..16 rows, on layers whose row blocks fill half
 * the chip without splitting K, the same form reads x in place and needs no
 * workspace; aqlm_gemm and aqlm_gemv run it there themselves.) From 17 rows
 * the activations are first re-laid into blocks of 8 inputs so that every
 * MFMA operand load is contiguous, rows beyond 128 go to blocks of 128, and
 * K may be split across workgroups whose float32 partial sums meet in the
 * workspace. Every other case runs as aqlm_gemm and ignores the workspace.
 *   workspace        device pointer, 16-byte aligned, at least
 *                    aqlm_gemm_workspace_size bytes (NULL allowed when that
 *                    size is 0); overwritten by the call; must not overlap
 *                    x or y
 *   workspace_bytes  its size in bytes
 * The result is deterministic for a given layer shape and batch (the split
 * parts are added in a fixed order whatever order they finish in) but is
 * not bit-identical to aqlm_gemm, which sums in another order; both meet the
 * same tolerance. Calls on different streams need different workspaces.
 * Returns AQLM_ERR_WORKSPACE if workspace_bytes is too small, AQLM_ERR_NULL
 * if the workspace is needed and NULL, AQLM_ERR_ALIGN if it is misaligned;
 * otherwise as aqlm_gemm.
 */
AQLM_API int aqlm_gemm_ws(const aqlm_layer *layer, const uint16_t *x, int64_t batch, uint16_t *y,
                          void *workspace, int64_t workspace_bytes, void *stream);

/*
 * aqlm_gemv_workspace_size: bytes of device workspace that aqlm_gemv_ws needs
 * for these num_layers layers (a HOST array) at this batch, written to
 * *bytes (0 when the call needs none and runs exactly as aqlm_gemv_batched).
 * It depends only on the layers' shapes and schemes and on batch: 32 * out
 * bytes, rounded up to 256, for each 1x16 layer (g = 8) that the
 * codebook-sliced kernel serves at one activation row (in / 8 a multiple of
 * 8, at most 4096 groups per row, at least 2^19 codes), provided those layers
 * hold at least 2^22 codes together (below that the call runs the gather
 * kernel of aqlm_gemv_batched and needs nothing). Validation and status codes
 * as for aqlm_gemv_batched; *bytes is 0 on error.
 */
AQLM_API int aqlm_gemv_workspace_size(const aqlm_layer *layers, int32_t num_layers, int64_t batch,
                                      int64_t *bytes);

/*
 * aqlm_gemv_ws: aqlm_gemv_batched with a caller-owned device workspace (one
 * layer: num_layers = 1). Where aqlm_gemv_workspace_size counts a layer, that
 * layer runs the codebook-sliced 1x16 kernel: its 1 MiB codebook is split
 * over the LDS of a team of eight workgroups (four 16384-codeword slices by
 * the top two code bits, times two halves of each codeword), every member
 * reads all of the team's codes and looks up those of its slice, and a
 * second launch adds the eight members' float32 partial sums in a fixed
 * order, scales and rounds ("AQLM (additive / multi-codebook quantization)",
 * field "Kernels": lookup without per-element dequantization). Such layers
 * with the same row length (in 1 KiB code chunks) share one launch. Every
 * other layer runs exactly as in aqlm_gemv_batched (same kernels, same bits).
 *   workspace        device pointer, 16-byte aligned, at least
 *                    aqlm_gemv_workspace_size bytes (NULL allowed when that
 *                    size is 0); overwritten by the call; must not overlap x
 *                    or y
 *   workspace_bytes  its size in bytes
 * Results are deterministic (the same call gives the same bits) and meet the
 * product tolerance. For the layers the sliced kernel serves they differ in
 * the last bits from aqlm_gemv, which sums in another order; since the
 * kernel is chosen per call (by the codes of its eligible layers), a 1x16
 * layer may give different last bits alone and in a larger call. Calls on
 * different streams need different workspaces. Returns AQLM_ERR_WORKSPACE if workspace_bytes is too small,
 * AQLM_ERR_NULL if the workspace is needed and NULL, AQLM_ERR_ALIGN if it is
 * misaligned; otherwise as aqlm_gemv_batched.
 */
AQLM_API int aqlm_gemv_ws(const aqlm_layer *layers, const uint16_t *const *x, uint16_t *const *y,
                          int32_t num_layers, int64_t batch, void *workspace,
                          int64_t workspace_bytes, void *stream);

/*
 * aqlm_gemm_noalloc: aqlm_gemm_ws with no workspace argument and no device
 * allocation of any kind, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The scratch memory that aqlm_gemm_ws takes from its workspace
 * comes from a static device array of AQLM_STATIC_SCRATCH_BYTES inside the
 * library, one per GPU; its address on the current device is looked up on
 * the first call made on that device (hipGetSymbolAddress) and kept.
 * Results are bit-identical to aqlm_gemm_ws for the same layer and batch
 * (the same kernels run). Every call on one GPU shares that GPU's array and
 * leaves its contents behind: calls on one GPU that may overlap in time
 * (different streams, or different host threads without ordering) race on
 * it and must be serialised by the caller. Nothing in the array needs to
 * start at zero: each call writes every scratch byte it reads. Returns
 * AQLM_ERR_SCRATCH, with nothing enqueued, when aqlm_gemm_workspace_size for
 * the layer and batch exceeds AQLM_STATIC_SCRATCH_BYTES (call aqlm_gemm_ws
 * with a workspace, or aqlm_gemm, instead), AQLM_ERR_HIP if the array's
 * address cannot be obtained; otherwise as aqlm_gemm. Device ordinals must
 * be below 64.
 */
AQLM_API int aqlm_gemm_noalloc(const aqlm_layer *layer, const uint16_t *x, int64_t batch,
                               uint16_t *y, void *stream);

/*
 * aqlm_gemv_batched: aqlm_gemv for num_layers independent layers in one call:
 * y[i] = x[i] . W_i^T for i < num_layers, with the same batch (0..8) for all.
 * layers, x and y are HOST arrays of num_layers entries; x[i] and y[i] are
 * device pointers laid out as for aqlm_gemv (x[i] may be shared between
 * layers of equal in_features, as for the query/key/value projections).
 * Layers that the grouped kernel serves run in a single launch whose
 * workgroups are split across the layers in proportion to their code bytes,
 * so the per-launch start-up cost is paid once rather than once per layer;
 * any other layer gets its own launch. The pages credit launch-overhead
 * removal (CUDA graphs) with about a 3x inference speedup ("Additive
 * quantization that actually survives one-bit weights", "Key highlights").
 * Every layer is validated as in aqlm_gemv before anything is launched; the
 * outputs must be pairwise disjoint and must not alias any input. Results are
 * bit-identical to calling aqlm_gemv on each layer. num_layers == 0 or
 * batch == 0 is a no-op; num_layers must not exceed 4096.
 */
AQLM_API int aqlm_gemv_batched(const aqlm_layer *layers, const uint16_t *const *x,
                               uint16_t *const *y, int32_t num_layers, int64_t batch,
                               void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
AQLM_API const char *aqlm_status_string(int status);

/* AQLM_ABI_VERSION of the built library. */
AQLM_API int aqlm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* AQLM_MI355X_H */
