// General additive schemes: M = 1..8 codebooks of 2^B codewords each
// (B = 8..16), codeword length g = 8 or 16. The pages describe weights as sums
// of one codeword per codebook ("Additive quantization that actually survives
// one-bit weights", section "What it does"), name 8- and 16-dimensional
// codewords ("Key highlights", "Caveats"), and the number of codebooks and
// the group size are varied in an ablation ("Extreme Compression of Large
// Language Models via Additive Quantization" summary, table "Measured effects
// reported in the paper"). Codes are stored one per
// element, in uint8 when B = 8 and in uint16 when B > 8, laid out
// [out][in/g][M], or bit-packed (B bits each, least significant first, in
// 32-bit words); codebooks [M][2^B][g] fp16; one fp16 scale per output row.
//
// These kernels serve every scheme other than 2x8, 1x16 and 1x16 g16, which
// have dedicated kernels. Each lane decodes whole groups exactly: the M
// codewords widened to float32 and added in ascending m starting from the
// m = 0 codeword.
//   * dequant: the sum times the row scale in float32, one round to float16;
//   * GEMV (1..8 activation rows): float32 dot of the sum with x, scale once
//     per row, wavefront reduction in a fixed order;
//   * GEMM (any batch): each 64 x 64 weight tile is decoded exactly as in
//     dequant into LDS, then multiplied with the activation tile on the
//     matrix cores (v_mfma_f32_32x32x16_f16, float32 accumulation), i.e. the
//     product of x with the float16 weights that dequant would write.
// Codebooks are read through the cache hierarchy (8 KiB to 16 MiB).
#include "aqlm_device.hpp"

namespace aqlm {
namespace {

constexpr int kGenBlock = 256;

// Where a layer's codes are: one per uint8 (CB = 1) or uint16 (CB = 2)
// element, or bit-packed (CB = 0): B bits per code, least significant first,
// in a stream of 32-bit words read through a buffer resource (a window past
// the last word reads zero).
struct Codes {
  const uint8_t *p;
  uint32_t bytes;  // of a bit-packed stream
};

__host__ __device__ inline uint32_t packed_stream_bytes(int64_t ncodes, int B) {
  return (uint32_t)(((ncodes * B + 31) / 32) * 4);
}

// Code m of group gidx (the group's index in [out][in/g] order).
template <int CB>
__device__ __forceinline__ uint32_t code_at(const Codes &c, int64_t gidx, int M, int B, int m) {
  const int64_t i = gidx * M + m;
  if constexpr (CB == 1) {
    return c.p[i];
  } else if constexpr (CB == 2) {
    return reinterpret_cast<const uint16_t *>(c.p)[i];
  } else {
    const uint64_t bit = (uint64_t)i * (uint64_t)B;
    const uint32_t word = (uint32_t)(bit >> 5), sh = (uint32_t)(bit & 31u);
    const Rsrc rc = make_rsrc(c.p, c.bytes);
    const uint64_t win = (uint64_t)buf_load4(rc, word * 4u) |
                         ((uint64_t)buf_load4(rc, word * 4u + 4u) << 32);
    return (uint32_t)(win >> sh) & ((1u << B) - 1u);
  }
}

// Float32 sum of the group's M codewords in ascending m, starting from the
// m = 0 codeword (so -0 + -0 stays -0).
template <int G, int CB>
__device__ __forceinline__ void group_sum(const Codes &cs, int64_t gidx, const uint4 *books, int M,
                                          int B, float (&acc)[G]) {
  {
    const uint4 *cw = books + (size_t)code_at<CB>(cs, gidx, M, B, 0) * (G / 8);
#pragma unroll
    for (int v = 0; v < G / 8; ++v) {
      const uint4 w = cw[v];
      const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[v * 8 + 2 * i] = h2f(words[i] & 0xFFFFu);
        acc[v * 8 + 2 * i + 1] = h2f(words[i] >> 16);
      }
    }
  }
  for (int m = 1; m < M; ++m) {
    const uint4 *cw = books + (((size_t)m << B) + code_at<CB>(cs, gidx, M, B, m)) * (G / 8);
#pragma unroll
    for (int v = 0; v < G / 8; ++v) {
      const uint4 w = cw[v];
      const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[v * 8 + 2 * i] = materialize(acc[v * 8 + 2 * i] + h2f(words[i] & 0xFFFFu));
        acc[v * 8 + 2 * i + 1] = materialize(acc[v * 8 + 2 * i + 1] + h2f(words[i] >> 16));
      }
    }
  }
}

// Exact float16 weights of a group: float32 sum times float32 scale, one round
// (kept in registers before the conversion so that no fused form is used).
template <int G>
__device__ __forceinline__ void scale_round(const float (&acc)[G], float s, uint4 (&w)[G / 8]) {
#pragma unroll
  for (int v = 0; v < G / 8; ++v) {
    uint32_t words[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = f2h(materialize(materialize(acc[v * 8 + 2 * i]) * s));
      const uint32_t hi = f2h(materialize(materialize(acc[v * 8 + 2 * i + 1]) * s));
      words[i] = lo | (hi << 16);
    }
    w[v] = make_uint4(words[0], words[1], words[2], words[3]);
  }
}

template <int G, int CB>
__global__ __launch_bounds__(kGenBlock) void dequant_general_kernel(
    Codes codes, const uint16_t *__restrict__ books,
    const uint16_t *__restrict__ scales, uint16_t *__restrict__ W, int64_t groups, int64_t total,
    int M, int B) {
  const uint4 *gb = reinterpret_cast<const uint4 *>(books);
  for (int64_t idx = (int64_t)blockIdx.x * kGenBlock + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * kGenBlock) {
    const int64_t o = idx / groups;
    float acc[G];
    group_sum<G, CB>(codes, idx, gb, M, B, acc);
    uint4 w[G / 8];
    scale_round<G>(acc, h2f(scales[o]), w);
    // W[o][j*G ..] with idx = o * groups + j, and in = groups * G
    uint4 *dst = reinterpret_cast<uint4 *>(W + idx * G);
#pragma unroll
    for (int v = 0; v < G / 8; ++v) store_nt16(dst + v, w[v]);
  }
}

// One wavefront per output row (rows strided over the grid); lane l takes
// groups l, l + 64, ... of the row.
template <int G, int CB, int MAXB>
__global__ __launch_bounds__(kGenBlock) void gemv_general_kernel(
    Codes codes, const uint16_t *__restrict__ books,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y, int out, int in, int groups, int batch, int M, int B) {
  const uint4 *gb = reinterpret_cast<const uint4 *>(books);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int row = blockIdx.x * (kGenBlock / 64) + wave; row < out;
       row += gridDim.x * (kGenBlock / 64)) {
    float dot[MAXB];
#pragma unroll
    for (int b = 0; b < MAXB; ++b) dot[b] = 0.0f;
    for (int j = lane; j < groups; j += 64) {
      float acc[G];
      group_sum<G, CB>(codes, (int64_t)row * groups + j, gb, M, B, acc);
#pragma unroll
      for (int b = 0; b < MAXB; ++b) {
        if (b < batch) {
          const uint4 *xv = reinterpret_cast<const uint4 *>(x + (int64_t)b * in + (int64_t)j * G);
#pragma unroll
          for (int v = 0; v < G / 8; ++v) {
            const uint4 w = xv[v];
            const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              dot[b] = fmaf(acc[v * 8 + 2 * i], h2f(words[i] & 0xFFFFu), dot[b]);
              dot[b] = fmaf(acc[v * 8 + 2 * i + 1], h2f(words[i] >> 16), dot[b]);
            }
          }
        }
      }
    }
    const float s = h2f(scales[row]);
#pragma unroll
    for (int b = 0; b < MAXB; ++b) {
      if (b < batch) {
        const float v = wave_sum_to_lane63(dot[b]);
        if (lane == 63) y[(int64_t)b * out + row] = (uint16_t)f2h(v * s);
      }
    }
  }
}

// 64 x 64 output tiles, four wavefronts each owning a 32 x 32 quarter; the K
// loop walks 64 inputs at a time: decode the 64 x 64 weight tile (exact
// float16) and stage the 64 x 64 activation tile in LDS, then four MFMA steps.
constexpr int kGenTile = 64;
constexpr int kGenLd = kGenTile + 8;  // padded LDS row (halves): conflict-free fragment reads

template <int G, int CB>
__global__ __launch_bounds__(kGenBlock) void gemm_general_kernel(
    Codes codes, const uint16_t *__restrict__ books,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y, int out, int in, int groups, int batch, int M, int B) {
  constexpr int GPT = kGenTile / G;  // groups per tile row
  __shared__ __attribute__((aligned(16))) uint16_t wt[kGenTile * kGenLd];
  __shared__ __attribute__((aligned(16))) uint16_t xt[kGenTile * kGenLd];
  const uint4 *gb = reinterpret_cast<const uint4 *>(books);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int row0 = blockIdx.x * kGenTile, tok0 = blockIdx.y * kGenTile;
  const int nk = (in + kGenTile - 1) / kGenTile;

  float16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

  for (int kb = 0; kb < nk; ++kb) {
    for (int e = tid; e < kGenTile * GPT; e += kGenBlock) {
      const int r = e / GPT, jj = e - r * GPT;
      const int row = row0 + r, j = kb * GPT + jj;
      uint4 w[G / 8];
      if (row < out && j < groups) {
        float a[G];
        group_sum<G, CB>(codes, (int64_t)row * groups + j, gb, M, B, a);
        scale_round<G>(a, h2f(scales[row]), w);
      } else {
#pragma unroll
        for (int v = 0; v < G / 8; ++v) w[v] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < G / 8; ++v)
        *reinterpret_cast<uint4 *>(&wt[r * kGenLd + jj * G + v * 8]) = w[v];
    }
    for (int e = tid; e < kGenTile * kGenTile / 8; e += kGenBlock) {
      const int t = e >> 3, kv = e & 7;
      const int tok = tok0 + t, col = kb * kGenTile + kv * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tok < batch && col < in)
        v = *reinterpret_cast<const uint4 *>(x + (int64_t)tok * in + col);
      *reinterpret_cast<uint4 *>(&xt[t * kGenLd + kv * 8]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGenTile; kk += 16) {
      const int k = kk + 8 * (lane >> 5);
      const uint4 a = *reinterpret_cast<const uint4 *>(&wt[(wr * 32 + (lane & 31)) * kGenLd + k]);
      const uint4 b = *reinterpret_cast<const uint4 *>(&xt[(wc * 32 + (lane & 31)) * kGenLd + k]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                   __builtin_bit_cast(half8_t, b), acc, 0, 0, 0);
    }
    __syncthreads();
  }

  // lane holds activation row (lane % 32) of the quarter; register r is
  // weight row 8 * (r / 4) + 4 * (lane / 32) + r % 4
  const int tok = tok0 + wc * 32 + (lane & 31);
  if (tok < batch) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = row0 + wr * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row < out) y[(int64_t)tok * out + row] = (uint16_t)f2h(acc[r]);
    }
  }
}

Codes codes_of(const LayerDesc &L) {
  const uint8_t *p = static_cast<const uint8_t *>(L.codes);
  const uint32_t bytes = L.packed ? packed_stream_bytes(L.out * L.groups * L.M, L.B) : 0u;
  return Codes{p, bytes};
}

// Bytes per stored code: 1 (B = 8), 2 (B > 8), or 0 for a bit-packed stream
// of B < 16 bits (for B = 8 and 16 the stream is the element layout).
int code_bytes(const LayerDesc &L) {
  if (L.B == 8) return 1;
  if (L.B == 16 || !L.packed) return 2;
  return 0;
}

int grid_cap(int64_t n, int per_block) {
  const int64_t blocks = (n + per_block - 1) / per_block;
  return (int)(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

template <int G, int CB>
hipError_t dequant_gc(const LayerDesc &L, uint16_t *W, hipStream_t stream) {
  const int64_t total = L.out * L.groups;
  hipLaunchKernelGGL((dequant_general_kernel<G, CB>), dim3(grid_cap(total, kGenBlock)),
                     dim3(kGenBlock), 0, stream, codes_of(L), L.books, L.scales, W, L.groups,
                     total, L.M, L.B);
  return hipGetLastError();
}

template <int G, int CB, int MAXB>
hipError_t gemv_gc(const LayerDesc &L, const uint16_t *x, int batch, uint16_t *y,
                   hipStream_t stream) {
  hipLaunchKernelGGL((gemv_general_kernel<G, CB, MAXB>),
                     dim3(grid_cap(L.out, kGenBlock / 64)), dim3(kGenBlock), 0, stream,
                     codes_of(L), L.books, L.scales, x, y, (int)L.out, (int)L.in, (int)L.groups,
                     batch, L.M, L.B);
  return hipGetLastError();
}

template <int G, int CB>
hipError_t gemv_g(const LayerDesc &L, const uint16_t *x, int batch, uint16_t *y,
                  hipStream_t stream) {
  if (batch <= 1) return gemv_gc<G, CB, 1>(L, x, batch, y, stream);
  if (batch <= 2) return gemv_gc<G, CB, 2>(L, x, batch, y, stream);
  if (batch <= 4) return gemv_gc<G, CB, 4>(L, x, batch, y, stream);
  return gemv_gc<G, CB, 8>(L, x, batch, y, stream);
}

template <int G, int CB>
hipError_t gemm_gc(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                   hipStream_t stream) {
  const dim3 grid((unsigned)((L.out + kGenTile - 1) / kGenTile),
                  (unsigned)((batch + kGenTile - 1) / kGenTile));
  hipLaunchKernelGGL((gemm_general_kernel<G, CB>), grid, dim3(kGenBlock), 0, stream,
                     codes_of(L), L.books, L.scales, x, y, (int)L.out, (int)L.in, (int)L.groups,
                     (int)batch, L.M, L.B);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant_general(const LayerDesc &L, uint16_t *W, hipStream_t stream) {
  const int cb = code_bytes(L);
  if (L.g == 8)
    return cb == 1 ? dequant_gc<8, 1>(L, W, stream)
                   : (cb == 2 ? dequant_gc<8, 2>(L, W, stream) : dequant_gc<8, 0>(L, W, stream));
  return cb == 1 ? dequant_gc<16, 1>(L, W, stream)
                 : (cb == 2 ? dequant_gc<16, 2>(L, W, stream) : dequant_gc<16, 0>(L, W, stream));
}

hipError_t launch_gemv_general(const LayerDesc &L, const uint16_t *x, int batch, uint16_t *y,
                               hipStream_t stream) {
  const int cb = code_bytes(L);
  if (L.g == 8)
    return cb == 1 ? gemv_g<8, 1>(L, x, batch, y, stream)
                   : (cb == 2 ? gemv_g<8, 2>(L, x, batch, y, stream)
                              : gemv_g<8, 0>(L, x, batch, y, stream));
  return cb == 1 ? gemv_g<16, 1>(L, x, batch, y, stream)
                 : (cb == 2 ? gemv_g<16, 2>(L, x, batch, y, stream)
                            : gemv_g<16, 0>(L, x, batch, y, stream));
}

hipError_t launch_gemm_general(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                               hipStream_t stream) {
  const int cb = code_bytes(L);
  if (L.g == 8)
    return cb == 1 ? gemm_gc<8, 1>(L, x, batch, y, stream)
                   : (cb == 2 ? gemm_gc<8, 2>(L, x, batch, y, stream)
                              : gemm_gc<8, 0>(L, x, batch, y, stream));
  return cb == 1 ? gemm_gc<16, 1>(L, x, batch, y, stream)
                 : (cb == 2 ? gemm_gc<16, 2>(L, x, batch, y, stream)
                            : gemm_gc<16, 0>(L, x, batch, y, stream));
}

}  // namespace aqlm
