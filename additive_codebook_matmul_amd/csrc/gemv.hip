// Matrix-vector products y = x . W^T for 1..8 activation rows, decoding W on
// the fly from the packed codes (no dequantized copy of W is ever written).
//
// Each group's contribution is the dot product of g activations with the sum
// of its codewords, so y[b][o] = scale[o] * sum_j sum_m <x_b[j], C_m[c_ojm]>,
// accumulated in float32 with fp16 x fp16 -> fp32 dot2 instructions, the
// scale applied once per row in float32 and y rounded to float16.
//
// Fast path (codes rows a multiple of 16 bytes): a wavefront owns RPW output
// rows; each lane streams 16-byte code chunks (8 groups) of those rows with
// coalesced loads, looks the codewords up (2x8: codebooks staged in LDS;
// 1x16: read through L2), takes the activations of its chunk from an LDS
// slice of x, and the per-lane partial sums are reduced across the
// wavefront with DPP in a fixed order. Generic path: one group per lane per
// step, for rows whose code bytes are not a multiple of 16.
#include "aqlm_device.hpp"

namespace aqlm {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kXLdsHalves = 16384;  // 32 KiB of activations staged per slice

template <Scheme S, int BATCH, int RPW>
__global__ __launch_bounds__(kBlock) void gemv_fast_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ books,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y, int out, int in, int row_chunks, int slice_chunks) {
  constexpr int G = group_size(S);
  constexpr int IPC = 8 * G;  // activations covered by one 16-byte code chunk
  constexpr int XV = G / 8;   // 16-byte activation vectors per group
  __shared__ uint4 lds_books[S == Scheme::k2x8 ? 512 : 1];
  __shared__ uint4 lds_x[kXLdsHalves / 8];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row_bytes = (int64_t)row_chunks * 16;
  const uint4 *gbooks = reinterpret_cast<const uint4 *>(books);

  if constexpr (S == Scheme::k2x8) {
    for (int i = threadIdx.x; i < 512; i += kBlock) lds_books[i] = gbooks[i];
  }

  const int row_base = (blockIdx.x * kWaves + wave) * RPW;
  float acc[RPW][BATCH];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < BATCH; ++b) acc[r][b] = 0.0f;

  for (int c0 = 0; c0 < row_chunks; c0 += slice_chunks) {
    const int nc = min(slice_chunks, row_chunks - c0);
    const int nvec = nc * IPC / 8;  // 16-byte activation vectors per batch row
    __syncthreads();
    for (int i = threadIdx.x; i < BATCH * nvec; i += kBlock) {
      const int b = i / nvec, v = i - b * nvec;
      lds_x[i] = *reinterpret_cast<const uint4 *>(x + (int64_t)b * in + (int64_t)c0 * IPC + v * 8);
    }
    __syncthreads();

    for (int c = lane; c < nc; c += 64) {
      uint4 cw[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int row = row_base + r;
        if (row < out)
          cw[r] = load_nt16(codes + (int64_t)row * row_bytes + (int64_t)(c0 + c) * 16);
        else
          cw[r] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const uint32_t words[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
#pragma unroll
        for (int gi = 0; gi < 8; ++gi) {
          const uint32_t code = (words[gi >> 1] >> ((gi & 1) * 16)) & 0xFFFFu;
          const int xv = (c * 8 + gi) * XV;  // activation vector index within the slice row
          if constexpr (S == Scheme::k2x8) {
            const uint4 a = lds_books[code & 0xFF];
            const uint4 bb = lds_books[256 + (code >> 8)];
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
              const uint4 xx = lds_x[b * nvec + xv];
              acc[r][b] = dot8(xx, bb, dot8(xx, a, acc[r][b]));
            }
          } else if constexpr (S == Scheme::k1x16) {
            const uint4 a = gbooks[code];
#pragma unroll
            for (int b = 0; b < BATCH; ++b) acc[r][b] = dot8(lds_x[b * nvec + xv], a, acc[r][b]);
          } else {
            const uint4 a0 = gbooks[2 * code];
            const uint4 a1 = gbooks[2 * code + 1];
#pragma unroll
            for (int b = 0; b < BATCH; ++b)
              acc[r][b] = dot8(lds_x[b * nvec + xv + 1], a1, dot8(lds_x[b * nvec + xv], a0, acc[r][b]));
          }
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = row_base + r;
    const float s = row < out ? h2f(scales[row]) : 0.0f;
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const float v = wave_sum_to_lane63(acc[r][b]);
      if (lane == 63 && row < out) y[(int64_t)b * out + row] = (uint16_t)f2h(v * s);
    }
  }
}

template <Scheme S, int BATCH>
__global__ __launch_bounds__(kBlock) void gemv_generic_kernel(
    const uint16_t *__restrict__ codes, const uint16_t *__restrict__ books,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y, int out, int in, int groups) {
  constexpr int G = group_size(S);
  constexpr int XV = G / 8;
  const int lane = threadIdx.x & 63;
  const int gwave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * kWaves;
  const uint4 *gbooks = reinterpret_cast<const uint4 *>(books);
  for (int row = gwave; row < out; row += nwaves) {
    float acc[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) acc[b] = 0.0f;
    for (int j = lane; j < groups; j += 64) {
      const uint32_t code = codes[(int64_t)row * groups + j];
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const uint4 *xp = reinterpret_cast<const uint4 *>(x + (int64_t)b * in + (int64_t)j * G);
        if constexpr (S == Scheme::k2x8) {
          const uint4 a = gbooks[code & 0xFF];
          const uint4 bb = gbooks[256 + (code >> 8)];
          acc[b] = dot8(xp[0], bb, dot8(xp[0], a, acc[b]));
        } else {
#pragma unroll
          for (int v = 0; v < XV; ++v) acc[b] = dot8(xp[v], gbooks[(int64_t)code * XV + v], acc[b]);
        }
      }
    }
    const float s = h2f(scales[row]);
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const float v = wave_sum_to_lane63(acc[b]);
      if (lane == 63) y[(int64_t)b * out + row] = (uint16_t)f2h(v * s);
    }
  }
}

template <Scheme S, int BATCH>
hipError_t launch_batch(const LayerDesc &L, const uint16_t *x, uint16_t *y, hipStream_t stream) {
  constexpr int G = group_size(S);
  const int out = (int)L.out, in = (int)L.in, groups = (int)L.groups;
  if (groups % 8 == 0) {
    constexpr int RPW = BATCH <= 2 ? 4 : 2;
    const int row_chunks = groups / 8;
    int slice_chunks = kXLdsHalves / (BATCH * 8 * G);
    if (slice_chunks < 1) slice_chunks = 1;
    const int rows_per_block = kWaves * RPW;
    const int grid = (out + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((gemv_fast_kernel<S, BATCH, RPW>), dim3(grid), dim3(kBlock), 0, stream,
                       static_cast<const uint8_t *>(L.codes), L.books, L.scales, x, y, out, in,
                       row_chunks, slice_chunks);
  } else {
    int grid = (out + kWaves - 1) / kWaves;
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL((gemv_generic_kernel<S, BATCH>), dim3(grid), dim3(kBlock), 0, stream,
                       static_cast<const uint16_t *>(L.codes), L.books, L.scales, x, y, out, in,
                       groups);
  }
  return hipGetLastError();
}

template <Scheme S>
hipError_t launch_scheme(const LayerDesc &L, const uint16_t *x, int batch, uint16_t *y,
                         hipStream_t stream) {
  switch (batch) {
    case 1: return launch_batch<S, 1>(L, x, y, stream);
    case 2: return launch_batch<S, 2>(L, x, y, stream);
    case 3: return launch_batch<S, 3>(L, x, y, stream);
    case 4: return launch_batch<S, 4>(L, x, y, stream);
    case 5: return launch_batch<S, 5>(L, x, y, stream);
    case 6: return launch_batch<S, 6>(L, x, y, stream);
    case 7: return launch_batch<S, 7>(L, x, y, stream);
    case 8: return launch_batch<S, 8>(L, x, y, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemv(const LayerDesc &L, const uint16_t *x, int batch, uint16_t *y,
                       hipStream_t stream) {
  switch (L.scheme) {
    case Scheme::k2x8: return launch_scheme<Scheme::k2x8>(L, x, batch, y, stream);
    case Scheme::k1x16: return launch_scheme<Scheme::k1x16>(L, x, batch, y, stream);
    case Scheme::k1x16g16: return launch_scheme<Scheme::k1x16g16>(L, x, batch, y, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace aqlm
