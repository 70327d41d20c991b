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
//   * GEMM: the product of x with the float16 weights that dequant would
//     write, on the matrix cores with float32 accumulation. Up to 128
//     activation rows, each lane decodes its 8 weights of an MFMA step
//     exactly into the A operand of v_mfma_f32_16x16x32_f16 (workgroups of 16
//     output rows, wavefronts interleaved over K, codes and codewords loaded
//     two and one steps ahead); above, each 64 x 64 weight tile is decoded
//     into LDS and multiplied with the staged activation tile
//     (v_mfma_f32_32x32x16_f16).
// Codebooks are read through the cache hierarchy (8 KiB to 16 MiB).
#include <type_traits>

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

// Up to 128 activation rows (NT tiles of 16): a workgroup of kGenSkWaves
// wavefronts owns 16 output rows; wavefront w takes the K blocks of 32 inputs
// w, w + kGenSkWaves, ... In MFMA step kb, lane (r, q) = (lane % 16, lane / 16)
// decodes weights 8q .. 8q+7 of K block kb of row r exactly (the M codewords,
// or their halves for g = 16, summed in float32 in ascending m, times the row
// scale, one round) into the A operand, and loads the matching 16 bytes of
// activation row 16 j + r as the B operand of tile j. The wavefronts' float32
// tiles are added in LDS in wavefront order. Codes are loaded two steps ahead
// and codewords and activations one step ahead, from registers rings indexed
// statically (the step loop is unrolled by two).
constexpr int kGenSkWaves = 8;
constexpr int kGenMaxM = 8;
constexpr int kGenSkMaxTiles = 8;  // up to 128 activation rows

template <int G, int CB, int NT>
__global__ __launch_bounds__(64 * kGenSkWaves) void gemm_general_skinny_kernel(
    Codes codes, const uint16_t *__restrict__ books, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ x, uint16_t *__restrict__ y, int out, int in, int groups,
    int batch, int M, int B) {
  __shared__ float4_t red[kGenSkWaves * NT * 64];
  const uint4 *gb = reinterpret_cast<const uint4 *>(books);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int row = blockIdx.x * 16 + r;
  const bool row_ok = row < out;
  const int nkb = (in + 31) / 32;
  const float s = row_ok ? h2f(scales[row]) : 0.0f;
  const Rsrc xr = make_rsrc(x, (uint32_t)((int64_t)batch * in * 2));
  constexpr uint32_t kOOB = 0x80000000u;

  // group and codeword part (g = 16: which half) of this lane in K block kb
  auto group_of = [&](int kb) { return G == 8 ? kb * 4 + q : kb * 2 + (q >> 1); };
  constexpr int kHalfOff = G == 8 ? 0 : 1;  // uint4 index step of the second half
  auto load_codes = [&](int kb, uint32_t (&c)[kGenMaxM]) __attribute__((always_inline)) {
    const int j = group_of(kb);
    const bool ok = row_ok && kb < nkb && j < groups;
#pragma unroll
    for (int m = 0; m < kGenMaxM; ++m)
      c[m] = (ok && m < M) ? code_at<CB>(codes, (int64_t)row * groups + j, M, B, m) : 0u;
  };
  auto load_words = [&](const uint32_t (&c)[kGenMaxM], uint4 (&cw)[kGenMaxM])
                        __attribute__((always_inline)) {
    const int half = G == 8 ? 0 : (q & 1);
#pragma unroll
    for (int m = 0; m < kGenMaxM; ++m)
      if (m < M)
        cw[m] = gb[(((size_t)m << B) + c[m]) * (G / 8) + (size_t)(half * kHalfOff)];
  };
  auto load_x = [&](int kb, uint4 (&bx)[NT]) __attribute__((always_inline)) {
    const int col = kb * 32 + 8 * q;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int tok = j * 16 + r;
      const bool ok = kb < nkb && tok < batch && col < in;
      bx[j] = buf_load16(xr, ok ? (uint32_t)(((int64_t)tok * in + col) * 2) : kOOB);
    }
  };
  // the exact float16 weights of this lane's 8 inputs (zero past the row end)
  auto decode = [&](int kb, const uint4 (&cw)[kGenMaxM]) __attribute__((always_inline)) {
    float acc[8];
    {
      const uint32_t wd[4] = {cw[0].x, cw[0].y, cw[0].z, cw[0].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = h2f(wd[i] & 0xFFFFu);
        acc[2 * i + 1] = h2f(wd[i] >> 16);
      }
    }
#pragma unroll
    for (int m = 1; m < kGenMaxM; ++m) {
      if (m < M) {
        const uint32_t wd[4] = {cw[m].x, cw[m].y, cw[m].z, cw[m].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = materialize(acc[2 * i] + h2f(wd[i] & 0xFFFFu));
          acc[2 * i + 1] = materialize(acc[2 * i + 1] + h2f(wd[i] >> 16));
        }
      }
    }
    const bool ok = row_ok && kb < nkb && group_of(kb) < groups;
    uint32_t words[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = f2h(materialize(materialize(acc[2 * i]) * s));
      const uint32_t hi = f2h(materialize(materialize(acc[2 * i + 1]) * s));
      words[i] = ok ? (lo | (hi << 16)) : 0u;
    }
    return make_uint4(words[0], words[1], words[2], words[3]);
  };

  float4_t acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t c[2][kGenMaxM];
  uint4 cw[2][kGenMaxM];
  uint4 bx[2][NT];
  int kb = w;
  constexpr int KS = kGenSkWaves;
  load_codes(kb, c[0]);
  load_codes(kb + KS, c[1]);
  load_words(c[0], cw[0]);
  load_x(kb, bx[0]);
  // step kb with ring slot K: codewords and activations of the next step,
  // codes of the step after it, then decode and multiply
  auto step = [&](auto kc) __attribute__((always_inline)) {
    constexpr int K = decltype(kc)::value;
    load_words(c[K ^ 1], cw[K ^ 1]);
    load_x(kb + KS, bx[K ^ 1]);
    load_codes(kb + 2 * KS, c[K]);
    const uint4 a = decode(kb, cw[K]);
#pragma unroll
    for (int j = 0; j < NT; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                     __builtin_bit_cast(half8_t, bx[K][j]), acc[j],
                                                     0, 0, 0);
    kb += KS;
  };
  while (kb < nkb) {
    step(std::integral_constant<int, 0>{});
    if (kb >= nkb) break;
    step(std::integral_constant<int, 1>{});
  }

#pragma unroll
  for (int j = 0; j < NT; ++j) red[(w * NT + j) * 64 + lane] = acc[j];
  __syncthreads();
  // element e = tile j * 64 + lane l: rows 4 (l / 16) .. + 3, activation row 16 j + l % 16
  for (int e = tid; e < NT * 64; e += 64 * kGenSkWaves) {
    float4_t v = red[e];
#pragma unroll
    for (int w2 = 1; w2 < kGenSkWaves; ++w2) v += red[w2 * NT * 64 + e];
    const int j = e >> 6, l = e & 63;
    const int tok = j * 16 + (l & 15);
    if (tok >= batch) continue;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = blockIdx.x * 16 + 4 * (l >> 4) + k;
      if (rr < out) y[(int64_t)tok * out + rr] = (uint16_t)f2h(v[k]);
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
  // bit-packed codes keep a two-word window per code in flight: at most four
  // activation tiles fit in registers
  constexpr int kMaxTiles = CB == 0 ? 4 : kGenSkMaxTiles;
  if (batch <= 16 * kMaxTiles && L.M <= kGenMaxM && L.in * batch * 2 < ((int64_t)1 << 31)) {
    const dim3 g((unsigned)((L.out + 15) / 16));
    auto k = batch <= 16   ? gemm_general_skinny_kernel<G, CB, 1>
             : batch <= 32 ? gemm_general_skinny_kernel<G, CB, 2>
                           : gemm_general_skinny_kernel<G, CB, 4>;
    if constexpr (kMaxTiles == 8)
      if (batch > 64) k = gemm_general_skinny_kernel<G, CB, 8>;
    hipLaunchKernelGGL(k, g, dim3(64 * kGenSkWaves), 0, stream, codes_of(L), L.books, L.scales, x,
                       y, (int)L.out, (int)L.in, (int)L.groups, (int)batch, L.M, L.B);
    return hipGetLastError();
  }
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
  // 6..8 activation rows with at most three codebooks in element layout (one
  // with bit-packed codes): the skinny GEMM's 16-row tile, which gathers each
  // group's codewords once for all rows, beats the GEMV, whose cost grows by
  // ~1.3 us per row on a 4096 x 4096 layer (measured on 1x8, 3x8 and 1x12
  // g8, 2x12 g16 and 2x16 g8: 8 rows 21-29% faster; packed 1x12 g8 20%).
  // With more codebooks the tile's exact per-lane decode costs more and the
  // GEMV stays ahead up to 8 rows.
  if (batch >= 6 && L.M <= (L.packed ? 1 : 3) && L.in * batch * 2 < ((int64_t)1 << 31))
    return launch_gemm_general(L, x, batch, y, stream);
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
