// Host (CPU) matrix-vector product for additive multi-codebook layers: the
// entry point of aqlm_host.h. Plain C++17 with OpenMP threads; the inner
// loops have an AVX2 + FMA + F16C form chosen at run time and a scalar form.
//
// Two methods, both accumulating in float32 with one final round to float16:
//   * 8-bit codebooks: per call, a float32 table T[b][j][m][c] = <x_b[j], C_m[c]>
//     for every activation row b, group j, codebook m and code c; a row then
//     costs M table reads and adds per group (the lookup form the pages give
//     for token generation, "AQLM (additive / multi-codebook quantization)",
//     field "Kernels");
//   * wider codes: the group's codewords are converted to float32, summed in
//     ascending m from the m = 0 codeword, and dotted with the activations.
// Each output row is summed by one thread in a fixed order, so the result does
// not depend on the number of threads.
#include <immintrin.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>
#include <vector>

#include "../../include/aqlm_host.h"

namespace {

struct HostLayer {
  int64_t out, in, groups;
  int M, B, g;
  bool packed;       // B-bit codes in 32-bit words, least significant first
  int64_t nwords;    // words of a packed stream
  const void *codes;
  const uint16_t *books;
  const uint16_t *scales;
};

int check_layer(const aqlm_layer *layer, HostLayer *d) {
  if (!layer) return AQLM_ERR_NULL;
  if (!layer->codes || !layer->codebooks || !layer->scales) return AQLM_ERR_NULL;
  const int M = layer->num_codebooks, B = layer->nbits, g = layer->group_size;
  if (!(M >= 1 && M <= 8 && B >= 8 && B <= 16 && (g == 8 || g == 16))) return AQLM_ERR_SCHEME;
  if (layer->flags != 0 && layer->flags != AQLM_CODES_PACKED) return AQLM_ERR_SHAPE;
  if (layer->out_features < 1 || layer->in_features < 1) return AQLM_ERR_SHAPE;
  if (layer->in_features % g) return AQLM_ERR_SHAPE;
  if (layer->out_features > (int64_t(1) << 30) || layer->in_features > (int64_t(1) << 30))
    return AQLM_ERR_SHAPE;
  d->out = layer->out_features;
  d->in = layer->in_features;
  d->groups = layer->in_features / g;
  d->M = M;
  d->B = B;
  d->g = g;
  d->packed = layer->flags == AQLM_CODES_PACKED && B != 8 && B != 16;
  d->nwords = (d->out * d->groups * M * B + 31) / 32;
  d->codes = layer->codes;
  d->books = layer->codebooks;
  d->scales = layer->scales;
  return AQLM_OK;
}

// float16 bits -> float32, exact (subnormals, infinities and NaNs included).
inline float half_to_float(uint16_t h) {
  const uint32_t sign = uint32_t(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu, bits;
  if (e == 0) {
    if (m == 0) {
      bits = sign;
    } else {  // subnormal: normalise the mantissa
      e = 113;
      while (!(m & 0x400u)) {
        m <<= 1;
        --e;
      }
      bits = sign | (e << 23) | ((m & 0x3FFu) << 13);
    }
  } else if (e == 31) {
    bits = sign | 0x7F800000u | (m << 13);
  } else {
    bits = sign | ((e + 112) << 23) | (m << 13);
  }
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

// float32 -> float16 bits, round to nearest even, overflow to infinity.
inline uint16_t float_to_half(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  const uint16_t sign = uint16_t((x >> 16) & 0x8000u);
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return sign | (ax > 0x7F800000u ? 0x7E00u : 0x7C00u);
  if (ax >= 0x477FF000u) return sign | 0x7C00u;  // at least 65520: rounds to infinity
  if (ax < 0x38800000u) {                        // below 2^-14: a multiple of 2^-24
    float v;
    memcpy(&v, &ax, 4);
    return sign | uint16_t(std::nearbyint(v * 16777216.0f));  // exact scaling, ties to even
  }
  uint32_t h = ((ax >> 23) - 112) << 10 | ((ax & 0x7FFFFFu) >> 13);
  const uint32_t rem = ax & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;  // a carry may reach infinity: right
  return sign | uint16_t(h);
}

inline uint32_t code_at(const HostLayer &L, int64_t o, int64_t j, int m) {
  const int64_t i = (o * L.groups + j) * L.M + m;
  if (L.packed) {
    const uint32_t *w = static_cast<const uint32_t *>(L.codes);
    const uint64_t bit = (uint64_t)i * (uint64_t)L.B;
    const int64_t k = (int64_t)(bit >> 5);
    const uint64_t win = (uint64_t)w[k] | (k + 1 < L.nwords ? (uint64_t)w[k + 1] << 32 : 0);
    return (uint32_t)(win >> (bit & 31)) & ((1u << L.B) - 1u);
  }
  return L.B == 8 ? static_cast<const uint8_t *>(L.codes)[i]
                  : static_cast<const uint16_t *>(L.codes)[i];
}

bool use_avx2() {
  const char *force = getenv("AQLM_HOST_ISA");
  if (force && strcmp(force, "scalar") == 0) return false;
  __builtin_cpu_init();
  return __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") &&
         __builtin_cpu_supports("f16c");
}

// ---- lookup tables (B == 8) ------------------------------------------------

// T[(b * groups + j) * M * 256 + m * 256 + c] = sum_k x[b][j*g+k] * C_m[c][k],
// k ascending. CT holds the codebooks transposed as float32: [m][k][256].
void build_tables_scalar(const HostLayer &L, const float *xf, int batch, const float *CT, float *T,
                         int nt) {
  const int64_t n = (int64_t)batch * L.groups;
#pragma omp parallel for num_threads(nt) schedule(static)
  for (int64_t bj = 0; bj < n; ++bj) {
    const int64_t b = bj / L.groups, j = bj % L.groups;
    const float *xg = xf + b * L.in + j * L.g;
    for (int m = 0; m < L.M; ++m) {
      float *t = T + (bj * L.M + m) * 256;
      for (int c = 0; c < 256; ++c) {
        float acc = 0.0f;
        for (int k = 0; k < L.g; ++k) acc = std::fma(xg[k], CT[(m * L.g + k) * 256 + c], acc);
        t[c] = acc;
      }
    }
  }
}

__attribute__((target("avx2,fma"))) void build_tables_avx2(const HostLayer &L, const float *xf,
                                                           int batch, const float *CT, float *T,
                                                           int nt) {
  const int64_t n = (int64_t)batch * L.groups;
#pragma omp parallel for num_threads(nt) schedule(static)
  for (int64_t bj = 0; bj < n; ++bj) {
    const int64_t b = bj / L.groups, j = bj % L.groups;
    const float *xg = xf + b * L.in + j * L.g;
    for (int m = 0; m < L.M; ++m) {
      float *t = T + (bj * L.M + m) * 256;
      for (int c = 0; c < 256; c += 8) {
        __m256 acc = _mm256_setzero_ps();
        for (int k = 0; k < L.g; ++k)
          acc = _mm256_fmadd_ps(_mm256_set1_ps(xg[k]),
                                _mm256_loadu_ps(CT + (m * L.g + k) * 256 + c), acc);
        _mm256_storeu_ps(t + c, acc);
      }
    }
  }
}

// Rows from the tables. Each output keeps four partial sums over groups
// (j mod 4), added in a fixed order at the end. Rows are taken in blocks of
// kRowBlock and groups in slices whose tables fit in a core's private cache,
// so each slice of the tables is read from cache for a whole block of rows;
// the slicing does not change the order in which an output's terms are added.
constexpr int64_t kRowBlock = 64;
constexpr int64_t kSliceBytes = 96 << 10;

void rows_from_tables(const HostLayer &L, const float *T, int batch, uint16_t *y, int nt) {
  const int M = L.M;
  const int64_t tstride = L.groups * M * 256;  // floats per activation row
  int64_t js = kSliceBytes / ((int64_t)M * 256 * 4 * batch);
  if (js < 4) js = 4;
  const int64_t nblk = (L.out + kRowBlock - 1) / kRowBlock;
#pragma omp parallel for num_threads(nt) schedule(static)
  for (int64_t blk = 0; blk < nblk; ++blk) {
    const int64_t o0 = blk * kRowBlock, o1 = o0 + kRowBlock < L.out ? o0 + kRowBlock : L.out;
    float p[kRowBlock][8][4];
    for (int64_t r = 0; r < o1 - o0; ++r)
      for (int b = 0; b < batch; ++b) p[r][b][0] = p[r][b][1] = p[r][b][2] = p[r][b][3] = 0.0f;
    for (int64_t j0 = 0; j0 < L.groups; j0 += js) {
      const int64_t j1 = j0 + js < L.groups ? j0 + js : L.groups;
      for (int64_t o = o0; o < o1; ++o) {
        const uint8_t *co = static_cast<const uint8_t *>(L.codes) + o * L.groups * M;
        for (int b = 0; b < batch; ++b) {
          const float *tb = T + b * tstride;
          float *pr = p[o - o0][b];
          for (int64_t j = j0; j < j1; ++j) {
            const float *tj = tb + j * M * 256;
            const uint8_t *cj = co + j * M;
            float v = tj[cj[0]];
            for (int m = 1; m < M; ++m) v += tj[m * 256 + cj[m]];
            pr[j & 3] += v;
          }
        }
      }
    }
    for (int64_t o = o0; o < o1; ++o) {
      const float s = half_to_float(L.scales[o]);
      for (int b = 0; b < batch; ++b) {
        const float *pr = p[o - o0][b];
        y[(int64_t)b * L.out + o] = float_to_half(((pr[0] + pr[1]) + (pr[2] + pr[3])) * s);
      }
    }
  }
}

// ---- direct decode (any B) -------------------------------------------------

void rows_direct_scalar(const HostLayer &L, const float *xf, int batch, uint16_t *y, int nt) {
  const int64_t nb = int64_t(1) << L.B;
#pragma omp parallel for num_threads(nt) schedule(static)
  for (int64_t o = 0; o < L.out; ++o) {
    const float s = half_to_float(L.scales[o]);
    float acc[8][16];
    for (int b = 0; b < batch; ++b)
      for (int k = 0; k < 16; ++k) acc[b][k] = 0.0f;
    for (int64_t j = 0; j < L.groups; ++j) {
      float v[16];
      const uint16_t *c0 = L.books + (int64_t)code_at(L, o, j, 0) * L.g;
      for (int k = 0; k < L.g; ++k) v[k] = half_to_float(c0[k]);
      for (int m = 1; m < L.M; ++m) {
        const uint16_t *cm = L.books + ((int64_t)m * nb + code_at(L, o, j, m)) * L.g;
        for (int k = 0; k < L.g; ++k) v[k] += half_to_float(cm[k]);
      }
      for (int b = 0; b < batch; ++b) {
        const float *xg = xf + b * L.in + j * L.g;
        for (int k = 0; k < L.g; ++k) acc[b][k] = std::fma(v[k], xg[k], acc[b][k]);
      }
    }
    for (int b = 0; b < batch; ++b) {
      float t = 0.0f;
      for (int k = 0; k < L.g; ++k) t += acc[b][k];
      y[(int64_t)b * L.out + o] = float_to_half(t * s);
    }
  }
}

__attribute__((target("avx2,fma,f16c"))) inline __m256 load_codeword8(const uint16_t *p) {
  return _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i *>(p)));
}

__attribute__((target("avx2,fma"))) inline float hsum8(__m256 v) {
  alignas(32) float t[8];
  _mm256_store_ps(t, v);
  return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
}

template <int G>
__attribute__((target("avx2,fma,f16c"))) void rows_direct_avx2(const HostLayer &L, const float *xf,
                                                                int batch, uint16_t *y, int nt) {
  constexpr int V = G / 8;  // 8-float vectors per group
  const int64_t nb = int64_t(1) << L.B;
#pragma omp parallel for num_threads(nt) schedule(static)
  for (int64_t o = 0; o < L.out; ++o) {
    const float s = half_to_float(L.scales[o]);
    __m256 acc[8][V];
    for (int b = 0; b < batch; ++b)
      for (int u = 0; u < V; ++u) acc[b][u] = _mm256_setzero_ps();
    for (int64_t j = 0; j < L.groups; ++j) {
      __m256 v[V];
      const uint16_t *c0 = L.books + (int64_t)code_at(L, o, j, 0) * G;
      for (int u = 0; u < V; ++u) v[u] = load_codeword8(c0 + 8 * u);
      for (int m = 1; m < L.M; ++m) {
        const uint16_t *cm = L.books + ((int64_t)m * nb + code_at(L, o, j, m)) * G;
        for (int u = 0; u < V; ++u) v[u] = _mm256_add_ps(v[u], load_codeword8(cm + 8 * u));
      }
      for (int b = 0; b < batch; ++b) {
        const float *xg = xf + b * L.in + j * G;
        for (int u = 0; u < V; ++u)
          acc[b][u] = _mm256_fmadd_ps(v[u], _mm256_loadu_ps(xg + 8 * u), acc[b][u]);
      }
    }
    for (int b = 0; b < batch; ++b) {
      float t = hsum8(acc[b][0]);
      if (V == 2) t += hsum8(acc[b][V - 1]);
      y[(int64_t)b * L.out + o] = float_to_half(t * s);
    }
  }
}

// Tables larger than this use the direct method instead.
constexpr int64_t kMaxTableBytes = int64_t(256) << 20;

}  // namespace

extern "C" {

const char *aqlm_host_isa(void) { return use_avx2() ? "avx2" : "scalar"; }

int aqlm_host_gemv(const aqlm_layer *layer, const uint16_t *x, int64_t batch, uint16_t *y,
                   int32_t threads) {
  HostLayer L;
  const int st = check_layer(layer, &L);
  if (st != AQLM_OK) return st;
  if (batch < 0 || batch > 8) return AQLM_ERR_BATCH;
  if (batch == 0) return AQLM_OK;
  if (!x || !y) return AQLM_ERR_NULL;
  const int nt = threads > 0 ? threads : omp_get_max_threads();
  const bool avx2 = use_avx2();
  const int nbatch = (int)batch;

  std::vector<float> xf((size_t)nbatch * L.in);
  for (size_t i = 0; i < xf.size(); ++i) xf[i] = half_to_float(x[i]);

  const int64_t table_bytes = (int64_t)nbatch * L.groups * L.M * 256 * 4;
  if (L.B == 8 && table_bytes <= kMaxTableBytes) {
    std::vector<float> CT((size_t)L.M * L.g * 256);
    for (int m = 0; m < L.M; ++m)
      for (int c = 0; c < 256; ++c)
        for (int k = 0; k < L.g; ++k)
          CT[((size_t)m * L.g + k) * 256 + c] = half_to_float(L.books[((size_t)m * 256 + c) * L.g + k]);
    std::vector<float> T((size_t)(table_bytes / 4));
    if (avx2)
      build_tables_avx2(L, xf.data(), nbatch, CT.data(), T.data(), nt);
    else
      build_tables_scalar(L, xf.data(), nbatch, CT.data(), T.data(), nt);
    rows_from_tables(L, T.data(), nbatch, y, nt);
    return AQLM_OK;
  }
  if (avx2) {
    if (L.g == 8)
      rows_direct_avx2<8>(L, xf.data(), nbatch, y, nt);
    else
      rows_direct_avx2<16>(L, xf.data(), nbatch, y, nt);
  } else {
    rows_direct_scalar(L, xf.data(), nbatch, y, nt);
  }
  return AQLM_OK;
}

}  // extern "C"
