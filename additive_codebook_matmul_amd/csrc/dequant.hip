// Dequantization: W[o][j*g + k] for every group (o, j), bit-exact to the
// decode rule (float32 codeword sum in codebook order, float32 row scale,
// one round to nearest-even float16).
//
// The kernel writes 2*out*in bytes and reads 2 bytes of codes per g weights,
// so it is bound by HBM writes. One thread decodes one group: two code bytes
// (2x8) or one 16-bit code (1x16) in, g float16 (16 or 32 bytes) out, stored
// with 16-byte vector stores that are contiguous across the wavefront. The
// 2x8 codebooks (8 KiB) are staged in LDS; the 1x16 codebooks (1 or 2 MiB)
// are read through the L2 cache. The grid is at most eight blocks per CU and
// each thread loops over groups: one block per 256 groups made every block
// stage the 8 KiB table, twice the bytes of W in L2 reads. Group indices are
// 32-bit whenever they fit, so the row of a group is a short division.
#include "aqlm_device.hpp"

namespace aqlm {
namespace {

constexpr int kBlock = 256;

// 2x8 groups per thread and loop pass: their code and scale loads are all
// issued before the first is used, so a wavefront has four loads in flight
// instead of one. With the codes cold in HBM (rotated copies of 64 layers)
// 4096x4096 took 10.0 -> 9.0 us and 11008x4096 26.0 -> 22.8 us (2 per pass:
// 9.5 / 23.8, 8: 9.3 / 24.1). The 1x16 kernels, bound by the codeword
// gathers, gained nothing from it (1x16 g16 lost 1-6 %) and keep one group
// per pass.
constexpr int kDqU = 4;

template <typename I>
__global__ __launch_bounds__(kBlock) void dequant_2x8_kernel(
    const uint16_t *__restrict__ codes, const uint16_t *__restrict__ books,
    const uint16_t *__restrict__ scales, uint16_t *__restrict__ W, I groups_per_row,
    I total_groups) {
  __shared__ uint4 lds_books[2 * 256];  // [m][code] -> 8 halves
  const uint4 *gbooks = reinterpret_cast<const uint4 *>(books);
  for (int i = threadIdx.x; i < 2 * 256; i += kBlock) lds_books[i] = gbooks[i];
  __syncthreads();

  uint4 *W4 = reinterpret_cast<uint4 *>(W);
  const I stride = (I)gridDim.x * kBlock;
  for (I gid0 = (I)blockIdx.x * kBlock + threadIdx.x; gid0 < total_groups;
       gid0 += kDqU * stride) {
    uint32_t pair[kDqU];
    uint32_t sc[kDqU];
#pragma unroll
    for (int u = 0; u < kDqU; ++u) {
      const I gid = gid0 + (I)u * stride;
      const bool ok = gid < total_groups;
      // low byte: codebook 0, high byte: codebook 1
      pair[u] = ok ? codes[gid] : 0u;
      sc[u] = ok ? scales[gid / groups_per_row] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kDqU; ++u) {
      const I gid = gid0 + (I)u * stride;
      if (gid < total_groups) {
        const uint4 a = lds_books[pair[u] & 0xFF];
        const uint4 b = lds_books[256 + (pair[u] >> 8)];
        const float s = h2f(sc[u]);
        uint4 w;
        w.x = decode_word2(a.x, b.x, s);
        w.y = decode_word2(a.y, b.y, s);
        w.z = decode_word2(a.z, b.z, s);
        w.w = decode_word2(a.w, b.w, s);
        store_nt16(W4 + gid, w);
      }
    }
  }
}

template <int G, typename I>
__global__ __launch_bounds__(kBlock) void dequant_1x16_kernel(
    const uint16_t *__restrict__ codes, const uint16_t *__restrict__ books,
    const uint16_t *__restrict__ scales, uint16_t *__restrict__ W, I groups_per_row,
    I total_groups) {
  constexpr int V = G / 8;  // 16-byte vectors per codeword
  const uint4 *gbooks = reinterpret_cast<const uint4 *>(books);
  uint4 *W4 = reinterpret_cast<uint4 *>(W);
  const I stride = (I)gridDim.x * kBlock;
  for (I gid = (I)blockIdx.x * kBlock + threadIdx.x; gid < total_groups; gid += stride) {
    const I o = gid / groups_per_row;
    const uint32_t c = codes[gid];
    const float s = h2f(scales[o]);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const uint4 a = gbooks[c * V + v];
      uint4 w;
      w.x = decode_word1(a.x, s);
      w.y = decode_word1(a.y, s);
      w.z = decode_word1(a.z, s);
      w.w = decode_word1(a.w, s);
      store_nt16(W4 + (int64_t)gid * V + v, w);
    }
  }
}

int grid_for(int64_t work) {
  int64_t blocks = (work + kBlock - 1) / kBlock;
  const int64_t cap = 256 * 8;  // eight blocks per CU; the kernels loop over the rest
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

}  // namespace

hipError_t launch_dequant(const LayerDesc &L, uint16_t *W, hipStream_t stream) {
  const int64_t total = L.out * L.groups;
  const uint16_t *codes = static_cast<const uint16_t *>(L.codes);
  const int grid = grid_for(total);
  // 32-bit indices (a short division per group) while every group index and
  // its grid-stride successor fit
  const bool narrow = total + (int64_t)grid * kBlock < ((int64_t)1 << 32);
  switch (L.scheme) {
    case Scheme::k2x8:
      if (narrow)
        hipLaunchKernelGGL(dequant_2x8_kernel<uint32_t>, dim3(grid), dim3(kBlock), 0, stream, codes,
                           L.books, L.scales, W, (uint32_t)L.groups, (uint32_t)total);
      else
        hipLaunchKernelGGL(dequant_2x8_kernel<int64_t>, dim3(grid), dim3(kBlock), 0, stream, codes,
                           L.books, L.scales, W, L.groups, total);
      break;
    case Scheme::k1x16:
      if (narrow)
        hipLaunchKernelGGL((dequant_1x16_kernel<8, uint32_t>), dim3(grid), dim3(kBlock), 0, stream,
                           codes, L.books, L.scales, W, (uint32_t)L.groups, (uint32_t)total);
      else
        hipLaunchKernelGGL((dequant_1x16_kernel<8, int64_t>), dim3(grid), dim3(kBlock), 0, stream,
                           codes, L.books, L.scales, W, L.groups, total);
      break;
    case Scheme::k1x16g16:
      if (narrow)
        hipLaunchKernelGGL((dequant_1x16_kernel<16, uint32_t>), dim3(grid), dim3(kBlock), 0, stream,
                           codes, L.books, L.scales, W, (uint32_t)L.groups, (uint32_t)total);
      else
        hipLaunchKernelGGL((dequant_1x16_kernel<16, int64_t>), dim3(grid), dim3(kBlock), 0, stream,
                           codes, L.books, L.scales, W, L.groups, total);
      break;
    case Scheme::kGeneral:
      return launch_dequant_general(L, W, stream);
  }
  return hipGetLastError();
}

}  // namespace aqlm
