// Batched 2x8 product for many activation rows, with each weight tile decoded
// once into LDS and shared by all wavefronts of the block.
//
// The wide kernel (gemm.hip) decodes every wavefront's own rows straight into
// MFMA operand registers and reuses each decoded operand for the block's
// 32 * NI activation rows, so at 2048 rows every weight is decoded 32 times
// and the random codeword reads of the decode keep the LDS busier than the
// matrix cores. Here a block owns 128 output rows and 256 activation rows:
//   * per K block of 8 groups (64 inputs) the block's 256 threads decode the
//     128 x 64 weight tile once (thread t: row t / 2, groups 4 (t % 2) ..
//     4 (t % 2) + 3; the fp16 sum of the two codewords from an 8 KiB LDS copy
//     of the codebooks, as in every 2x8 matrix-core tile) into an LDS tile, and
//     stage the 256 x 64 activation tile next to it; both are double-buffered
//     and filled for K block kb + 1 while the matrix cores work on kb;
//   * wavefront w multiplies all 128 rows with activation rows 64 w .. 64 w +
//     63: 4 x 2 tiles of v_mfma_f32_32x32x16_f16 per 16-input step, both
//     operands read from LDS (one 16-byte read per lane and tile);
//   * tile rows are 128 bytes; 16-byte chunk j of row r is stored at chunk
//     j ^ ((r >> 1) & 7), so the 16 lanes of an LDS pass (16 consecutive rows,
//     one chunk) and the decode and staging writes touch 16 distinct 16-byte
//     bank groups;
//   * codes are loaded four K blocks ahead (8 bytes per thread and K block),
//     activations two K blocks ahead, with unconditional buffer loads (out of
//     range offsets read zero: rows past the end decode to codeword sums that
//     are never stored, activation rows past the end are zero);
//   * the row scale multiplies the float32 accumulator in the epilogue; the
//     overflow guard of the fp16 codeword sum is the one of the other tiles.
// A weight is decoded once per 256 activation rows (the wide kernel: per 64),
// and the LDS traffic per MFMA is about 1.1 conflict-free 16-byte reads.
#include <atomic>
#include <type_traits>

#include "aqlm_device.hpp"

namespace aqlm {
namespace {

constexpr int kTThreads = 256;
constexpr int kTWaves = kTThreads / 64;
constexpr int kTBM = 128;          // output rows per block
constexpr int kTBN = 256;          // activation rows per block (64 per wavefront)
constexpr int kTKG = 8;            // groups per K block: 64 inputs
constexpr int kTCodeDepth = 4;     // K blocks of codes in flight; the loop is unrolled to match
constexpr uint32_t kTOOB = 0x80000000u;
constexpr int kTBooksBytes = 512 * 16;
constexpr int kTWBytes = kTBM * 128;  // 128 rows x 64 halves
constexpr int kTXBytes = kTBN * 128;  // 256 activation rows x 64 halves
constexpr int kTLdsBytes = kTBooksBytes + 2 * kTWBytes + 2 * kTXBytes + kTWaves * 4;

// Byte offset of 16-byte chunk j of tile row r.
__device__ __forceinline__ uint32_t tile_off(int r, int j) {
  return (uint32_t)r * 128u + (uint32_t)((j ^ ((r >> 1) & 7)) << 4);
}

__global__ __launch_bounds__(kTThreads) void gemm_tile_2x8_kernel(
    const uint8_t *__restrict__ codes, const uint4 *__restrict__ books,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x, uint16_t *__restrict__ y,
    int out, int in, int groups, int batch, uint32_t codes_bytes, uint32_t x_bytes) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint4 *lbooks = reinterpret_cast<uint4 *>(lds);
  uint8_t *wt = lds + kTBooksBytes;  // [2][kTWBytes]
  uint8_t *xt = wt + 2 * kTWBytes;   // [2][kTXBytes]
  uint32_t *big_flags = reinterpret_cast<uint32_t *>(xt + 2 * kTXBytes);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int row0 = blockIdx.x * kTBM;
  const int tok0 = blockIdx.y * kTBN;
  const uint32_t row_bytes = (uint32_t)groups * 2u;
  const Rsrc crs = make_rsrc(codes, codes_bytes);
  const Rsrc xrs = make_rsrc(x, x_bytes);
  const int nkb = groups / kTKG;

  // decode role: row dr of the tile, groups 4 dh .. 4 dh + 3 of the K block
  const int dr = tid >> 1, dh = tid & 1;
  const bool dr_ok = row0 + dr < out;
  const uint32_t coff = (uint32_t)(row0 + dr) * row_bytes + (uint32_t)dh * 8u;
  auto load_codes = [&](int kb) -> uint2 {
    return buf_load8(crs, (dr_ok && kb < nkb) ? coff + (uint32_t)kb * 16u : kTOOB);
  };
  // staging role: chunks c = tid + 256 i of the activation tile, activation
  // row c / 8, 16-byte chunk c % 8 (a row's 128 bytes by 8 consecutive lanes)
  auto load_x = [&](int kb, uint4 (&xr)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + i * kTThreads;
      const int t = c >> 3, j = c & 7;
      const bool ok = tok0 + t < batch && kb < nkb;
      xr[i] = buf_load16(
          xrs, ok ? (uint32_t)(tok0 + t) * (uint32_t)in * 2u + (uint32_t)(kb * 64 + j * 8) * 2u
                  : kTOOB);
    }
  };
  auto store_x = [&](int buf, const uint4 (&xr)[8]) {
    uint8_t *dst = xt + buf * kTXBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + i * kTThreads;
      *reinterpret_cast<uint4 *>(dst + tile_off(c >> 3, c & 7)) = xr[i];
    }
  };
  auto decode = [&](int buf, uint2 cw) {
    uint8_t *dst = wt + buf * kTWBytes;
    const uint32_t w[2] = {cw.x, cw.y};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t code = (w[g >> 1] >> ((g & 1) * 16)) & 0xFFFFu;
      const uint4 v = hadd8(lbooks[code & 0xFFu], lbooks[256 + (code >> 8)]);
      *reinterpret_cast<uint4 *>(dst + tile_off(dr, dh * 4 + g)) = v;
    }
  };

  float16_t acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  // the MFMAs of one K block from LDS buffer buf: in step s the lane half hl
  // feeds chunk 2 s + hl of the K block, in A and in B alike; step s + 1's
  // operand reads are issued before step s's MFMAs. (Spreading the next K
  // block's decode and staging between these MFMAs measured the same.)
  auto compute = [&](int buf) {
    const uint8_t *W = wt + buf * kTWBytes;
    const uint8_t *X = xt + buf * kTXBytes;
    uint4 a[2][4], b[2][2];
    auto reads = [&](int s, int slot) __attribute__((always_inline)) {
      const int j = 2 * s + hl;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        a[slot][mi] = *reinterpret_cast<const uint4 *>(W + tile_off(mi * 32 + l32, j));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        b[slot][ni] = *reinterpret_cast<const uint4 *>(X + tile_off(wave * 64 + ni * 32 + l32, j));
    };
    reads(0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int cur = s & 1;
      if (s + 1 < 4) reads(s + 1, cur ^ 1);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(half8_t, a[cur][mi]), __builtin_bit_cast(half8_t, b[cur][ni]),
              acc[mi][ni], 0, 0, 0);
      if (s + 1 < 4) {
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // next step's LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // then this step's MFMAs
      }
    }
  };

  // Prologue: codes of K blocks 0 .. 3, activations of K blocks 0 and 1, the
  // codebooks into LDS, K block 0's activations into LDS, then K block 0's
  // weight tile.
  uint2 cq[kTCodeDepth];
#pragma unroll
  for (int i = 0; i < kTCodeDepth; ++i) cq[i] = load_codes(i);
  uint4 xr[2][8];
  load_x(0, xr[0]);
  load_x(1, xr[1]);
  bool large = false;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint4 v = books[tid + i * kTThreads];
    large |= has_large_half(v);
    lbooks[tid + i * kTThreads] = v;
  }
  publish_flag(big_flags, large);
  store_x(0, xr[0]);
  __syncthreads();
  // codebooks large enough for the fp16 codeword sum to overflow: halve the
  // table, double the totals (overflow guard, aqlm_device.hpp)
  float total_mul = 1.0f;
  if (read_flag(big_flags, kTWaves)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) lbooks[tid + i * kTThreads] = hhalf8(lbooks[tid + i * kTThreads]);
    __syncthreads();
    total_mul = 2.0f;
  }
  decode(0, cq[0]);
  cq[0] = load_codes(kTCodeDepth);
  __syncthreads();

  // K block kb: prefetch the activations of kb + 2, multiply kb, fill the
  // other buffers with kb + 1 (decode from code slot (kb + 1) % 4, then refill
  // that slot with kb + 5), barrier.
  auto iter = [&](int kb, auto kc) {
    constexpr int K = decltype(kc)::value;  // kb % 4
    constexpr int N = (K + 1) % kTCodeDepth;
    load_x(kb + 2, xr[K & 1]);
    compute(K & 1);
    // the last K block also fills the other buffers, with the zeros of the
    // out-of-range loads; nothing reads them
    decode((K + 1) & 1, cq[N]);
    store_x((K + 1) & 1, xr[(K + 1) & 1]);
    cq[N] = load_codes(kb + 1 + kTCodeDepth);
    __syncthreads();
  };
  int kb = 0;
  for (; kb + 4 <= nkb; kb += 4) {
    iter(kb, std::integral_constant<int, 0>{});
    iter(kb + 1, std::integral_constant<int, 1>{});
    iter(kb + 2, std::integral_constant<int, 2>{});
    iter(kb + 3, std::integral_constant<int, 3>{});
  }
  if (kb < nkb) iter(kb, std::integral_constant<int, 0>{});
  if (kb + 1 < nkb) iter(kb + 1, std::integral_constant<int, 1>{});
  if (kb + 2 < nkb) iter(kb + 2, std::integral_constant<int, 2>{});

  // Epilogue: lane holds activation row l32 of each 32 x 32 tile; register r
  // is output row 8 (r / 4) + 4 hl + r % 4, so registers 4 q .. 4 q + 3 are
  // four consecutive rows (one 8-byte store when out is a multiple of 4).
  const bool packed = (out & 3) == 0;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int tok = tok0 + wave * 64 + ni * 32 + l32;
      if (tok >= batch) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rb = row0 + mi * 32 + 8 * q + 4 * hl;
        if (packed && rb + 3 < out) {
          uint32_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h[e] = f2h((acc[mi][ni][4 * q + e] * total_mul) * h2f(scales[rb + e]));
          *reinterpret_cast<uint2 *>(y + (int64_t)tok * out + rb) =
              make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (rb + e < out)
              y[(int64_t)tok * out + rb + e] =
                  (uint16_t)f2h((acc[mi][ni][4 * q + e] * total_mul) * h2f(scales[rb + e]));
        }
      }
    }
  }
}

}  // namespace

// True when the decoded-tile kernel serves this 2x8 layer and batch: whole
// K blocks (groups a multiple of 8) and 32-bit byte offsets for the codes
// (rows of one block past the end) and the activations (one block past the
// end).
bool gemm_tile_fits(const LayerDesc &L, int64_t batch) {
  if (L.scheme != Scheme::k2x8 || L.groups % kTKG != 0) return false;
  const int64_t row_bytes = L.groups * kCodeBytesPerGroup;
  return (L.out + kTBM) * row_bytes + 4096 < (int64_t(1) << 31) &&
         (batch + kTBN) * L.in * 2 + 4096 < (int64_t(1) << 31);
}

// Where it runs instead of the wide tiles: from 1536 activation rows, when
// its grid gives every CU a block at least once. Same-box timings of the
// binding's gemm (2x8, wide tiles -> this kernel): 11008x4096 at 2048 rows
// 329-332 -> 293-295 us, 4096x11008 at 2048 rows 273 -> 254-257 us; at 1024
// rows 11008x4096 is even (172 -> 176 us) and 4096x11008, on 128 blocks,
// slower (157 -> 203 us), at 256 rows 11008x4096 slower (67 -> 84 us).
bool gemm_tile_preferred(const LayerDesc &L, int64_t batch) {
  if (batch < 1536 || !gemm_tile_fits(L, batch)) return false;
  return ((L.out + kTBM - 1) / kTBM) * ((batch + kTBN - 1) / kTBN) >= 256;
}

hipError_t launch_gemm_tile(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                            hipStream_t stream) {
  static std::atomic<uint64_t> raised{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (dev >= 64 || !(raised.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_tile_2x8_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kTLdsBytes);
    if (e != hipSuccess) return e;
    raised.fetch_or(bit, std::memory_order_acq_rel);
  }
  const dim3 grid((unsigned)((L.out + kTBM - 1) / kTBM), (unsigned)((batch + kTBN - 1) / kTBN));
  hipLaunchKernelGGL(gemm_tile_2x8_kernel, grid, dim3(kTThreads), kTLdsBytes, stream,
                     static_cast<const uint8_t *>(L.codes), reinterpret_cast<const uint4 *>(L.books),
                     L.scales, x, y, (int)L.out, (int)L.in, (int)L.groups, (int)batch,
                     (uint32_t)(L.out * L.groups * kCodeBytesPerGroup), (uint32_t)(batch * L.in * 2));
  return hipGetLastError();
}

}  // namespace aqlm
