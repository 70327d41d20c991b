// Toy encoder kernels (aqlm_encode.h): row scales, residual k-means codebooks
// and greedy nearest-codeword codes under the plain squared error.
//
// Every decision these kernels take (a code) must match the CPU oracle bit
// for bit, so the arithmetic is pinned: no fused multiply-add in this file,
// squared errors summed in ascending k in float32, the first (lowest) code
// kept on a tie, and centroid means summed exactly as 64-bit integers in
// 24-bit fixed point, which makes them independent of the order in which the
// atomics land.
#include <limits.h>
#include <stdint.h>

#include "../../include/aqlm_encode.h"
#include "aqlm_device.hpp"

#pragma clang fp contract(off)

namespace aqlm {
namespace {

constexpr int kEncBlock = 256;
constexpr int kAssignTileBytes = 16 * 1024;  // centroids staged in LDS per pass
constexpr float kFixedScale = 16777216.0f;   // 2^24
constexpr double kFixedInv = 1.0 / 16777216.0;

// --- normalisation: one workgroup per row ----------------------------------

__global__ __launch_bounds__(kEncBlock) void normalize_kernel(const uint16_t *__restrict__ W,
                                                              int64_t in,
                                                              uint16_t *__restrict__ scales,
                                                              float *__restrict__ vecs) {
  __shared__ uint32_t wave_max[kEncBlock / 64];
  const int64_t o = blockIdx.x;
  const uint16_t *w = W + o * in;
  // the largest magnitude: for finite float16 values the magnitude orders like
  // the bit pattern with the sign cleared
  uint32_t mx = 0;
  for (int64_t k = threadIdx.x; k < in; k += kEncBlock) mx = max(mx, (uint32_t)(w[k] & 0x7FFFu));
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = wave_max[0];
#pragma unroll
  for (int i = 1; i < kEncBlock / 64; ++i) mx = max(mx, wave_max[i]);
  const uint32_t s16 = mx == 0 ? 0x3C00u : mx;
  if (threadIdx.x == 0) scales[o] = (uint16_t)s16;
  const float s = h2f(s16);
  float *v = vecs + o * in;
  for (int64_t k = threadIdx.x; k < in; k += kEncBlock) v[k] = h2f(w[k]) / s;
}

// --- starting centroids -----------------------------------------------------

__global__ __launch_bounds__(kEncBlock) void init_kernel(const float *__restrict__ vecs, int64_t n,
                                                         int g, const int64_t *__restrict__ idx,
                                                         int K, float *__restrict__ cents) {
  const int64_t e = (int64_t)blockIdx.x * kEncBlock + threadIdx.x;
  if (e >= (int64_t)K * g) return;
  const int64_t c = e / g, k = e - c * g;
  const int64_t i = idx[c];
  cents[e] = (i >= 0 && i < n) ? vecs[i * g + k] : 0.0f;
}

// --- nearest centroid -------------------------------------------------------

// Each thread owns kVPT vectors (independent dependency chains for the VALU,
// and each centroid read from LDS serves all of them); centroids stream
// through LDS in 16 KiB tiles so that eight workgroups fit on a CU. Every lane
// of a wavefront reads the same centroid (a broadcast).
constexpr int kVPT = 2;

template <int G, typename CodeT>
__global__ __launch_bounds__(kEncBlock) void assign_kernel(const float *__restrict__ vecs, int64_t n,
                                                           const float *__restrict__ cents, int K,
                                                           CodeT *__restrict__ codes, int M, int m,
                                                           float *residual) {
  constexpr int kTile = kAssignTileBytes / (G * 4);
  __shared__ __attribute__((aligned(16))) float tile[kTile * G];
  const int64_t i0 = ((int64_t)blockIdx.x * kEncBlock + threadIdx.x) * kVPT;
  float v[kVPT][G];
#pragma unroll
  for (int p = 0; p < kVPT; ++p) {
    const bool live = i0 + p < n;
#pragma unroll
    for (int u = 0; u < G / 4; ++u) {
      const float4 t =
          live ? reinterpret_cast<const float4 *>(vecs + (i0 + p) * G)[u] : make_float4(0, 0, 0, 0);
      v[p][4 * u] = t.x;
      v[p][4 * u + 1] = t.y;
      v[p][4 * u + 2] = t.z;
      v[p][4 * u + 3] = t.w;
    }
  }
  float best[kVPT];
  int bi[kVPT];
#pragma unroll
  for (int p = 0; p < kVPT; ++p) {
    best[p] = __builtin_inff();
    bi[p] = 0;
  }
  for (int c0 = 0; c0 < K; c0 += kTile) {
    const int nt = min(kTile, K - c0);
    __syncthreads();
    for (int e = threadIdx.x; e < nt * G / 4; e += kEncBlock)
      reinterpret_cast<float4 *>(tile)[e] = reinterpret_cast<const float4 *>(cents + (int64_t)c0 * G)[e];
    __syncthreads();
    for (int c = 0; c < nt; ++c) {
      const float *cc = tile + c * G;
#pragma unroll
      for (int p = 0; p < kVPT; ++p) {
        float t = v[p][0] - cc[0];
        float d = t * t;
#pragma unroll
        for (int k = 1; k < G; ++k) {
          t = v[p][k] - cc[k];
          d = d + t * t;
        }
        if (d < best[p]) {  // strict: the lowest code wins a tie
          best[p] = d;
          bi[p] = c0 + c;
        }
      }
    }
  }
#pragma unroll
  for (int p = 0; p < kVPT; ++p) {
    const int64_t i = i0 + p;
    if (i >= n) break;
    codes[i * M + m] = (CodeT)bi[p];
    if (residual) {
      const float *cb = cents + (int64_t)bi[p] * G;
#pragma unroll
      for (int k = 0; k < G; ++k) residual[i * G + k] = v[p][k] - cb[k];
    }
  }
}

// --- centroid update ----------------------------------------------------------

__global__ __launch_bounds__(kEncBlock) void fill_zero_kernel(unsigned long long *p, int64_t count) {
  const int64_t e = (int64_t)blockIdx.x * kEncBlock + threadIdx.x;
  if (e < count) p[e] = 0ull;
}

__device__ __forceinline__ unsigned long long to_fixed(float x) {
  // x * 2^24 is exact in float32; rint rounds to nearest even
  return (unsigned long long)(long long)__builtin_rintf(x * kFixedScale);
}

// Sums (two's-complement 64-bit, so unsigned atomics add signed values
// correctly) and counts per centroid. With LDS = true the workgroup first
// gathers its vectors' sums in LDS and adds each nonzero entry to memory once.
template <int G, typename CodeT, bool LDS>
__global__ __launch_bounds__(kEncBlock) void accumulate_kernel(const float *__restrict__ vecs,
                                                               int64_t n,
                                                               const CodeT *__restrict__ codes,
                                                               int M, int m, int K,
                                                               unsigned long long *__restrict__ ws) {
  extern __shared__ unsigned long long lsum[];  // K * (G + 1) when LDS
  unsigned long long *gsum = ws, *gcnt = ws + (int64_t)K * G;
  if constexpr (LDS) {
    for (int e = threadIdx.x; e < K * (G + 1); e += kEncBlock) lsum[e] = 0ull;
    __syncthreads();
  }
  for (int64_t i = (int64_t)blockIdx.x * kEncBlock + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kEncBlock) {
    const int c = (int)codes[i * M + m];
    if (c >= K) continue;  // not a code of this codebook: no centroid to move
    const float *v = vecs + i * G;
    if constexpr (LDS) {
#pragma unroll
      for (int k = 0; k < G; ++k) atomicAdd(&lsum[c * G + k], to_fixed(v[k]));
      atomicAdd(&lsum[K * G + c], 1ull);
    } else {
#pragma unroll
      for (int k = 0; k < G; ++k) atomicAdd(&gsum[(int64_t)c * G + k], to_fixed(v[k]));
      atomicAdd(&gcnt[c], 1ull);
    }
  }
  if constexpr (LDS) {
    __syncthreads();
    for (int e = threadIdx.x; e < K * (G + 1); e += kEncBlock)
      if (lsum[e] != 0ull) atomicAdd(&ws[e], lsum[e]);
  }
}

__global__ __launch_bounds__(kEncBlock) void finalize_kernel(const long long *__restrict__ ws,
                                                             int K, int g,
                                                             float *__restrict__ cents) {
  const int64_t e = (int64_t)blockIdx.x * kEncBlock + threadIdx.x;
  if (e >= (int64_t)K * g) return;
  const long long cnt = ws[(int64_t)K * g + e / g];
  if (cnt > 0) cents[e] = (float)(((double)ws[e] * kFixedInv) / (double)cnt);
}

// --- float16 codebook ---------------------------------------------------------

__global__ __launch_bounds__(kEncBlock) void round_kernel(const float *cents, int64_t count,
                                                          uint16_t *__restrict__ books,
                                                          float *rounded) {
  const int64_t e = (int64_t)blockIdx.x * kEncBlock + threadIdx.x;
  if (e >= count) return;
  const uint32_t h = f2h(cents[e]);
  books[e] = (uint16_t)h;
  if (rounded) rounded[e] = h2f(h);
}

unsigned grid_for(int64_t count) { return (unsigned)((count + kEncBlock - 1) / kEncBlock); }

template <int G, typename CodeT>
hipError_t launch_assign_t(const float *vecs, int64_t n, const float *cents, int K, void *codes,
                           int M, int m, float *residual, hipStream_t stream) {
  const int64_t threads = (n + kVPT - 1) / kVPT;
  hipLaunchKernelGGL((assign_kernel<G, CodeT>), dim3(grid_for(threads)), dim3(kEncBlock), 0, stream, vecs,
                     n, cents, K, static_cast<CodeT *>(codes), M, m, residual);
  return hipGetLastError();
}

template <int G, typename CodeT>
hipError_t launch_update_t(const float *vecs, int64_t n, const void *codes, int K, int M, int m,
                           float *cents, unsigned long long *ws, hipStream_t stream) {
  const int64_t wsn = (int64_t)K * (G + 1);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(wsn)), dim3(kEncBlock), 0, stream, ws, wsn);
  // two workgroups per CU; each folds many vectors in LDS, which keeps the
  // number of atomics per memory word near the workgroup count
  int64_t blocks = (n + kEncBlock - 1) / kEncBlock;
  if (blocks > 512) blocks = 512;
  const size_t lds = (size_t)wsn * 8;
  if (lds <= 48 * 1024)
    hipLaunchKernelGGL((accumulate_kernel<G, CodeT, true>), dim3((unsigned)blocks), dim3(kEncBlock),
                       lds, stream, vecs, n, static_cast<const CodeT *>(codes), M, m, K, ws);
  else
    hipLaunchKernelGGL((accumulate_kernel<G, CodeT, false>), dim3((unsigned)blocks),
                       dim3(kEncBlock), 0, stream, vecs, n, static_cast<const CodeT *>(codes), M, m,
                       K, ws);
  hipLaunchKernelGGL(finalize_kernel, dim3(grid_for((int64_t)K * G)), dim3(kEncBlock), 0, stream,
                     reinterpret_cast<const long long *>(ws), K, G, cents);
  return hipGetLastError();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_k(int32_t K) { return K >= 256 && K <= 65536 && (K & (K - 1)) == 0; }
bool valid_g(int32_t g) { return g == 8 || g == 16; }
bool overlap(const void *a, const void *b, int64_t bytes) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)bytes && y < x + (uintptr_t)bytes;
}
int from_hip(hipError_t e) { return e == hipSuccess ? AQLM_OK : AQLM_ERR_HIP; }

}  // namespace
}  // namespace aqlm

using namespace aqlm;

extern "C" {

int aqlm_encode_normalize(const uint16_t *W, int64_t out, int64_t in, uint16_t *scales, float *vecs,
                          void *stream) {
  if (!W || !scales || !vecs) return AQLM_ERR_NULL;
  if (out < 1 || in < 1 || out > INT_MAX || in > ((int64_t)1 << 30)) return AQLM_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(scales) || !aligned16(vecs)) return AQLM_ERR_ALIGN;
  hipLaunchKernelGGL(normalize_kernel, dim3((unsigned)out), dim3(kEncBlock), 0,
                     static_cast<hipStream_t>(stream), W, in, scales, vecs);
  return from_hip(hipGetLastError());
}

int aqlm_encode_init(const float *vecs, int64_t n, int32_t g, const int64_t *indices, int32_t K,
                     float *centroids, void *stream) {
  if (!vecs || !indices || !centroids) return AQLM_ERR_NULL;
  if (!valid_g(g) || !valid_k(K)) return AQLM_ERR_SCHEME;
  if (n < 1 || n > ((int64_t)1 << 31)) return AQLM_ERR_SHAPE;
  if (!aligned16(vecs) || !aligned16(indices) || !aligned16(centroids)) return AQLM_ERR_ALIGN;
  hipLaunchKernelGGL(init_kernel, dim3(grid_for((int64_t)K * g)), dim3(kEncBlock), 0,
                     static_cast<hipStream_t>(stream), vecs, n, (int)g, indices, (int)K, centroids);
  return from_hip(hipGetLastError());
}

int aqlm_encode_assign(const float *vecs, int64_t n, int32_t g, const float *centroids, int32_t K,
                       void *codes, int32_t M, int32_t m, float *residual, void *stream) {
  if (!valid_g(g) || !valid_k(K)) return AQLM_ERR_SCHEME;
  if (M < 1 || M > 8 || m < 0 || m >= M || n < 0 || n > ((int64_t)1 << 31)) return AQLM_ERR_SHAPE;
  if (n == 0) return AQLM_OK;
  if (!vecs || !centroids || !codes) return AQLM_ERR_NULL;
  if (!aligned16(vecs) || !aligned16(centroids) || !aligned16(codes) ||
      (residual && !aligned16(residual)))
    return AQLM_ERR_ALIGN;
  if (residual && residual != vecs && overlap(residual, vecs, n * g * 4)) return AQLM_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (K == 256)
    e = g == 8 ? launch_assign_t<8, uint8_t>(vecs, n, centroids, K, codes, M, m, residual, s)
               : launch_assign_t<16, uint8_t>(vecs, n, centroids, K, codes, M, m, residual, s);
  else
    e = g == 8 ? launch_assign_t<8, uint16_t>(vecs, n, centroids, K, codes, M, m, residual, s)
               : launch_assign_t<16, uint16_t>(vecs, n, centroids, K, codes, M, m, residual, s);
  return from_hip(e);
}

int aqlm_encode_update(const float *vecs, int64_t n, int32_t g, const void *codes, int32_t K,
                       int32_t M, int32_t m, float *centroids, int64_t *workspace, void *stream) {
  if (!valid_g(g) || !valid_k(K)) return AQLM_ERR_SCHEME;
  if (M < 1 || M > 8 || m < 0 || m >= M || n < 1 || n > ((int64_t)1 << 31)) return AQLM_ERR_SHAPE;
  if (!vecs || !codes || !centroids || !workspace) return AQLM_ERR_NULL;
  if (!aligned16(vecs) || !aligned16(codes) || !aligned16(centroids) || !aligned16(workspace))
    return AQLM_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto *ws = reinterpret_cast<unsigned long long *>(workspace);
  hipError_t e;
  if (K == 256)
    e = g == 8 ? launch_update_t<8, uint8_t>(vecs, n, codes, K, M, m, centroids, ws, s)
               : launch_update_t<16, uint8_t>(vecs, n, codes, K, M, m, centroids, ws, s);
  else
    e = g == 8 ? launch_update_t<8, uint16_t>(vecs, n, codes, K, M, m, centroids, ws, s)
               : launch_update_t<16, uint16_t>(vecs, n, codes, K, M, m, centroids, ws, s);
  return from_hip(e);
}

int aqlm_encode_round(const float *centroids, int64_t count, uint16_t *books, float *rounded,
                      void *stream) {
  if (count < 0 || count > ((int64_t)1 << 31)) return AQLM_ERR_SHAPE;
  if (count == 0) return AQLM_OK;
  if (!centroids || !books) return AQLM_ERR_NULL;
  if (!aligned16(centroids) || !aligned16(books) || (rounded && !aligned16(rounded)))
    return AQLM_ERR_ALIGN;
  hipLaunchKernelGGL(round_kernel, dim3(grid_for(count)), dim3(kEncBlock), 0,
                     static_cast<hipStream_t>(stream), centroids, count, books, rounded);
  return from_hip(hipGetLastError());
}

}  // extern "C"
