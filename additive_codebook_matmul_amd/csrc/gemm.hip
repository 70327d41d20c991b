// Batched product y = x . W^T on the matrix cores: tiles of W are decoded on
// chip straight into MFMA operand registers and multiplied with float16
// activations by v_mfma_f32_32x32x16_f16 (float32 accumulation). W is never
// written to memory.
//
// Block: 4 wavefronts. Each wavefront owns 64 output rows (two 32-row MFMA
// tiles) and the block's BN = 64 activation rows (two 32-column tiles), so a
// block covers 256 x 64 outputs. The K loop walks 8 groups at a time (64
// inputs for g = 8, 128 for g = 16):
//   * activations for the next K block are loaded from HBM into registers
//     and then written to a double-buffered LDS tile (rows padded by 16 bytes
//     so that 32 lanes reading one column hit distinct banks);
//   * each lane decodes its rows' groups into an 8-half A operand: the sum of
//     the codewords in packed fp16 (2x8: the two codewords come from LDS;
//     1x16: one 16-byte gather from the L2-resident codebook);
//   * the row scale multiplies the float32 accumulator in the epilogue.
// The MFMA K index of every lane element is paired identically in A and B, so
// any assignment of groups to MFMA steps gives the same sum; for g = 8 the two
// lane halves take groups s and s + 4 of the K block in step s.
#include "aqlm_device.hpp"

namespace aqlm {
namespace {

constexpr int kBlock = 256;
constexpr int kBM = 256;  // output rows per block
constexpr int kBN = 64;   // activation rows per block
constexpr int kKG = 8;    // groups per K block

template <Scheme S>
struct GemmCfg {
  static constexpr int G = group_size(S);
  static constexpr int KI = kKG * G;         // inputs per K block
  static constexpr int ROW_HALVES = KI + 8;  // padded LDS row of the activation tile
  static constexpr int TILE_HALVES = kBN * ROW_HALVES;
  static constexpr int XVEC = kBN * KI / 8;  // 16-byte vectors per activation tile
  static constexpr int XPT = XVEC / kBlock;  // vectors staged per thread
};

template <Scheme S, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void gemm_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ books,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y, int out, int in, int groups, int batch) {
  using C = GemmCfg<S>;
  __shared__ uint4 lds_books[S == Scheme::k2x8 ? 512 : 1];
  __shared__ __attribute__((aligned(16))) uint16_t lds_x[2][C::TILE_HALVES];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;  // which 8 K values of the MFMA step this lane feeds
  const int l32 = lane & 31;
  const int row0 = blockIdx.x * kBM + wave * 64;
  const int tok0 = blockIdx.y * kBN;
  const int64_t row_bytes = (int64_t)groups * 2;
  const uint4 *gbooks = reinterpret_cast<const uint4 *>(books);

  if constexpr (S == Scheme::k2x8) {
    for (int i = threadIdx.x; i < 512; i += kBlock) lds_books[i] = gbooks[i];
  }

  const int nkb = (groups + kKG - 1) / kKG;

  // Activation staging: thread t moves vectors t, t + 256, ... of the tile.
  uint4 xr[C::XPT];
  auto load_x = [&](int kb) {
#pragma unroll
    for (int i = 0; i < C::XPT; ++i) {
      const int v = threadIdx.x + i * kBlock;
      const int t = v / (C::KI / 8);
      const int kv = v - t * (C::KI / 8);
      const int tok = tok0 + t;
      const int col = kb * C::KI + kv * 8;
      if (tok < batch && col < in)
        xr[i] = *reinterpret_cast<const uint4 *>(x + (int64_t)tok * in + col);
      else
        xr[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::XPT; ++i) {
      const int v = threadIdx.x + i * kBlock;
      const int t = v / (C::KI / 8);
      const int kv = v - t * (C::KI / 8);
      *reinterpret_cast<uint4 *>(&lds_x[buf][t * C::ROW_HALVES + kv * 8]) = xr[i];
    }
  };

  // Codes of the lane's two rows for one K block: g = 8 lanes need 4 groups
  // (8 bytes) each, g = 16 lanes need all 8 groups (16 bytes).
  auto load_codes = [&](int kb, int mi, uint32_t (&cw)[4]) {
    const int row = row0 + mi * 32 + l32;
    cw[0] = cw[1] = cw[2] = cw[3] = 0;
    if (row >= out) return;
    const uint8_t *rp = codes + (int64_t)row * row_bytes;
    if constexpr (ALIGNED) {
      if constexpr (C::G == 8) {
        const uint2 v = *reinterpret_cast<const uint2 *>(rp + (int64_t)kb * 16 + half * 8);
        cw[0] = v.x;
        cw[1] = v.y;
      } else {
        const uint4 v = *reinterpret_cast<const uint4 *>(rp + (int64_t)kb * 16);
        cw[0] = v.x;
        cw[1] = v.y;
        cw[2] = v.z;
        cw[3] = v.w;
      }
    } else {
      const uint16_t *rp16 = reinterpret_cast<const uint16_t *>(rp);
      if constexpr (C::G == 8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int gidx = kb * kKG + half * 4 + q;
          const uint32_t c = gidx < groups ? rp16[gidx] : 0u;
          cw[q >> 1] |= c << ((q & 1) * 16);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int gidx = kb * kKG + q;
          const uint32_t c = gidx < groups ? rp16[gidx] : 0u;
          cw[q >> 1] |= c << ((q & 1) * 16);
        }
      }
    }
  };

  float16_t acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  load_x(0);
  store_x(0);
  __syncthreads();

  uint32_t cw[2][4];
  load_codes(0, 0, cw[0]);
  load_codes(0, 1, cw[1]);

  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load_x(kb + 1);
    uint32_t cwn[2][4];
    if (kb + 1 < nkb) {
      load_codes(kb + 1, 0, cwn[0]);
      load_codes(kb + 1, 1, cwn[1]);
    }
    const uint16_t *xt = lds_x[buf];
    constexpr int STEPS = C::G == 8 ? 4 : 8;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      // K columns of this step for this lane half, within the K block
      const int kcol = C::G == 8 ? (half * 4 + s) * 8 : s * 16 + half * 8;
      uint4 a[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int q = C::G == 8 ? s : s;  // index of the group within the lane's code words
        const uint32_t code = (cw[mi][q >> 1] >> ((q & 1) * 16)) & 0xFFFFu;
        if constexpr (S == Scheme::k2x8) {
          a[mi] = hadd8(lds_books[code & 0xFF], lds_books[256 + (code >> 8)]);
        } else if constexpr (S == Scheme::k1x16) {
          a[mi] = gbooks[code];
        } else {
          a[mi] = gbooks[2 * code + half];
        }
      }
      uint4 bx[2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bx[ni] = *reinterpret_cast<const uint4 *>(&xt[(ni * 32 + l32) * C::ROW_HALVES + kcol]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(half8_t, a[mi]), __builtin_bit_cast(half8_t, bx[ni]),
              acc[mi][ni], 0, 0, 0);
    }
    if (kb + 1 < nkb) {
      store_x(buf ^ 1);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q) cw[mi][q] = cwn[mi][q];
    }
    __syncthreads();
  }

  // Epilogue: lane holds column l32 of each 32x32 tile; register r is row
  // 8*(r/4) + 4*half + r%4.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int tok = tok0 + ni * 32 + l32;
      if (tok >= batch) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + mi * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < out)
          y[(int64_t)tok * out + row] = (uint16_t)f2h(acc[mi][ni][r] * h2f(scales[row]));
      }
    }
  }
}

template <Scheme S>
hipError_t launch_scheme(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                         hipStream_t stream) {
  const int out = (int)L.out, in = (int)L.in, groups = (int)L.groups;
  const dim3 grid((out + kBM - 1) / kBM, (unsigned)((batch + kBN - 1) / kBN));
  const uint8_t *codes = static_cast<const uint8_t *>(L.codes);
  if (groups % kKG == 0)
    hipLaunchKernelGGL((gemm_kernel<S, true>), grid, dim3(kBlock), 0, stream, codes, L.books,
                       L.scales, x, y, out, in, groups, (int)batch);
  else
    hipLaunchKernelGGL((gemm_kernel<S, false>), grid, dim3(kBlock), 0, stream, codes, L.books,
                       L.scales, x, y, out, in, groups, (int)batch);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                       hipStream_t stream) {
  switch (L.scheme) {
    case Scheme::k2x8: return launch_scheme<Scheme::k2x8>(L, x, batch, y, stream);
    case Scheme::k1x16: return launch_scheme<Scheme::k1x16>(L, x, batch, y, stream);
    case Scheme::k1x16g16: return launch_scheme<Scheme::k1x16g16>(L, x, batch, y, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace aqlm
