// Batched product for many activation rows, with each weight tile decoded
// once into LDS and shared by all wavefronts of the block (the dedicated
// schemes 2x8, 1x16 and 1x16 g16).
//
// The wide kernel (gemm.hip) decodes every wavefront's own rows straight into
// MFMA operand registers and reuses each decoded operand for the block's
// 32 * NI activation rows, so at 2048 rows every weight is decoded 16 to 32
// times: for 2x8 the random codeword reads of the decode keep the LDS busier
// than the matrix cores, for 1x16 the codeword gathers from L2 bound the
// kernel. Here a block of 512 threads owns 128 output rows and 256
// activation rows, and its wavefronts split into two roles that meet at one
// barrier per K block of 64 inputs:
//   * four filling wavefronts decode K block kb + 1's 128 x 64 weight tile
//     once (thread p: row p / 2, inputs 32 (p % 2) .. + 31, i.e. four
//     16-byte chunks) into one of two LDS tiles and stage its 256 x 64
//     activation tile next to it, while the matrix cores work on kb. A 2x8
//     chunk is the fp16 sum of the two codewords read from an 8 KiB LDS copy
//     of the codebooks, as in every 2x8 matrix-core tile; a 1x16 chunk is the
//     codeword (g 8) or half of it (g 16), gathered from the L2-resident
//     codebook two K blocks ahead. Codes and activations are loaded four K
//     blocks ahead, all with unconditional buffer loads (out of range
//     offsets read zero: rows past the end decode to codeword 0 or codeword
//     sums that are never stored, activation rows past the end are zero);
//   * four multiplying wavefronts, one per SIMD next to a filling one: wave
//     w multiplies all 128 rows with activation rows 64 w .. 64 w + 63,
//     4 x 2 tiles of v_mfma_f32_32x32x16_f16 per 16-input step, both
//     operands read from LDS (one 16-byte read per lane and tile);
//   * tile rows are 128 bytes; 16-byte chunk j of row r is stored at chunk
//     j ^ ((r >> 1) & 7), so the 16 lanes of an LDS pass (16 consecutive rows,
//     one chunk) and the decode and staging writes touch 16 distinct 16-byte
//     bank groups;
//   * the row scale multiplies the float32 accumulator in the epilogue; the
//     overflow guard of the 2x8 fp16 codeword sum is the one of the other
//     tiles (a single 1x16 codeword is an fp16 value already).
// A weight is decoded once per 256 activation rows, and the LDS traffic per
// MFMA is about 1.1 conflict-free 16-byte reads.
//
// Where the time goes (2x8, 11008 x 4096 at 2048 rows, same-box timings of
// copies with parts of the work removed): the MFMAs alone 135 us, with their
// LDS operand reads 176 us, the filling wavefronts alone 157-185 us, all of
// it 261-276 us; 1x16 g16: the gathers alone 155 us (the L2 gather rate).
// Measured and not kept: the activation operand loaded by the multiplying
// wavefronts from global memory one K block ahead (no LDS staging; the
// fill drops to 108 us, the multiply stalls on the loads: 291 us), operand
// reads pinned two steps ahead of their MFMAs (no gain), the 2x8 codebooks
// in a 64 KiB bank-spread table (conflict-free decode reads; no gain), one
// role for all 256 threads of a four-wavefront block (301 us).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "aqlm_device.hpp"

namespace aqlm {
namespace {

constexpr int kTThreads = 512;     // 4 multiplying + 4 filling wavefronts
constexpr int kTWaves = kTThreads / 64;
constexpr int kTFill = 256;        // threads of the filling wavefronts
constexpr int kTBM = 128;          // output rows per block
constexpr int kTBN = 256;          // activation rows per block (64 per multiplying wavefront)
constexpr int kTKIn = 64;          // inputs per K block
constexpr int kTCodeDepth = 4;     // K blocks of codes in flight; the fill loop is unrolled to match
constexpr uint32_t kTOOB = 0x80000000u;
constexpr int kTWBytes = kTBM * 128;  // 128 rows x 64 halves
constexpr int kTXBytes = kTBN * 128;  // 256 activation rows x 64 halves

// Per scheme: codeword length, code bytes a fill thread takes per K block
// (half of a row's), bytes of the LDS codebook copy.
template <Scheme S> struct TileScheme {
  static constexpr int G = S == Scheme::k1x16g16 ? 16 : 8;
  static constexpr int KG = kTKIn / G;                 // groups per K block
  static constexpr int CB = KG * kCodeBytesPerGroup / 2;
  static constexpr int BOOKS = S == Scheme::k2x8 ? 512 * 16 : 0;
  static constexpr int LDS = BOOKS + 2 * kTWBytes + 2 * kTXBytes + kTWaves * 4;
};

// Byte offset of 16-byte chunk j of tile row r.
__device__ __forceinline__ uint32_t tile_off(int r, int j) {
  return (uint32_t)r * 128u + (uint32_t)((j ^ ((r >> 1) & 7)) << 4);
}

// The filling wavefronts (threads p = 0 .. 255 of them): decode K block
// kb + 1's weight tile and stage its activation tile into the LDS buffers
// the multiplying wavefronts are not reading, one barrier per K block.
template <Scheme S>
__device__ __forceinline__ void tile_fill(const int p, uint8_t *__restrict__ wt,
                                          uint8_t *__restrict__ xt, const uint4 *lbooks,
                                          const Rsrc crs, const Rsrc xrs, const Rsrc brs,
                                          int row0, int tok0, int out, int in, int groups,
                                          int batch) {
  using C = TileScheme<S>;
  const uint32_t row_bytes = (uint32_t)groups * 2u;
  const int nkb = groups / C::KG;
  // decode role: row dr of the tile, inputs 32 dh .. 32 dh + 31 of the K
  // block (tile chunks 4 dh .. 4 dh + 3): 2x8 and 1x16 four groups, 1x16 g16
  // two
  const int dr = p >> 1, dh = p & 1;
  const bool dr_ok = row0 + dr < out;
  const uint32_t coff = (uint32_t)(row0 + dr) * row_bytes + (uint32_t)dh * C::CB;
  auto load_codes = [&](int kb) -> uint2 {
    const uint32_t off = (dr_ok && kb < nkb) ? coff + (uint32_t)kb * (2 * C::CB) : kTOOB;
    if constexpr (C::CB == 8) return buf_load8(crs, off);
    else return make_uint2(buf_load4(crs, off), 0u);
  };
  // staging role: chunks c = p + 256 i of the activation tile, activation
  // row c / 8, 16-byte chunk c % 8 (a row's 128 bytes by 8 consecutive lanes)
  auto load_x = [&](int kb, uint4 (&xr)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = p + i * kTFill;
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
      const int c = p + i * kTFill;
      *reinterpret_cast<uint4 *>(dst + tile_off(c >> 3, c & 7)) = xr[i];
    }
  };
  // 2x8: the eight codewords of four groups read from the LDS codebooks at
  // the start of a K block's fill, summed into the tile at its end
  auto read_books = [&](uint2 cw, uint4 (&bk)[8]) {
    const uint32_t w[2] = {cw.x, cw.y};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t code = (w[g >> 1] >> ((g & 1) * 16)) & 0xFFFFu;
      bk[2 * g] = lbooks[code & 0xFFu];
      bk[2 * g + 1] = lbooks[256 + (code >> 8)];
    }
  };
  auto put_sums = [&](int buf, const uint4 (&bk)[8]) {
    uint8_t *dst = wt + buf * kTWBytes;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<uint4 *>(dst + tile_off(dr, dh * 4 + g)) = hadd8(bk[2 * g], bk[2 * g + 1]);
  };
  // 1x16: the four chunks gathered from the codebook (16 bytes per codeword
  // for g 8, 32 for g 16) two K blocks ahead, then written into the tile
  auto gather = [&](uint2 cw, uint4 (&gv)[4]) {
    const uint32_t w[2] = {cw.x, cw.y};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if constexpr (C::G == 8) {
        const uint32_t code = (w[g >> 1] >> ((g & 1) * 16)) & 0xFFFFu;
        gv[g] = buf_load16(brs, code * 16u);
      } else {
        const uint32_t code = (w[0] >> ((g >> 1) * 16)) & 0xFFFFu;
        gv[g] = buf_load16(brs, code * 32u + (uint32_t)(g & 1) * 16u);
      }
    }
  };
  auto put = [&](int buf, const uint4 (&gv)[4]) {
    uint8_t *dst = wt + buf * kTWBytes;
#pragma unroll
    for (int g = 0; g < 4; ++g) *reinterpret_cast<uint4 *>(dst + tile_off(dr, dh * 4 + g)) = gv[g];
  };

  // One filling wavefront per SIMD has nothing to hide its load latency
  // behind but its own later work, so the activation loads run four K
  // blocks ahead (K blocks kb + 1 .. kb + 4 in flight, slot k % 4) and the
  // 1x16 codeword gathers two. Codes come four K blocks before their first
  // use.
  uint2 cq[kTCodeDepth];
#pragma unroll
  for (int i = 0; i < kTCodeDepth; ++i) cq[i] = load_codes(i);
  uint4 xr[4][8];
  uint4 gv[2][4];
  if constexpr (S != Scheme::k2x8) {
    gather(cq[0], gv[0]);
    gather(cq[1], gv[1]);
    cq[0] = load_codes(4);
    cq[1] = load_codes(5);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) load_x(i, xr[i]);
  if constexpr (S == Scheme::k2x8) {
    uint4 bk[8];
    read_books(cq[0], bk);
    cq[0] = load_codes(4);
    put_sums(0, bk);
  } else {
    put(0, gv[0]);
  }
  store_x(0, xr[0]);
  __syncthreads();

  // K block kb (the multiply of kb runs meanwhile): fill the other buffers
  // with kb + 1, issuing the loads of later K blocks into the slots K block
  // kb has left, barrier. The last K blocks fill buffers with the zeros of
  // out-of-range loads (codeword 0 for 1x16); nothing reads them.
  auto iter = [&](int kb, auto kc) {
    constexpr int K = decltype(kc)::value;  // kb % 4
    if constexpr (S == Scheme::k2x8) {
      constexpr int N = (K + 1) % kTCodeDepth;
      uint4 bk[8];
      read_books(cq[N], bk);  // K block kb + 1
      cq[N] = load_codes(kb + 5);
      load_x(kb + 4, xr[K]);
      store_x((K + 1) & 1, xr[(K + 1) % 4]);
      put_sums((K + 1) & 1, bk);
    } else {
      constexpr int N = (K + 2) % kTCodeDepth;
      gather(cq[N], gv[K & 1]);  // K block kb + 2
      cq[N] = load_codes(kb + 6);
      load_x(kb + 4, xr[K]);
      put((K + 1) & 1, gv[(K + 1) & 1]);
      store_x((K + 1) & 1, xr[(K + 1) % 4]);
    }
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
}

// The multiplying wavefronts (w = 0 .. 3): all 128 rows of the block times
// activation rows 64 w .. 64 w + 63, one barrier per K block, then y.
__device__ __forceinline__ void tile_multiply(const int w, const int lane, const uint8_t *wt,
                                              const uint8_t *xt, const uint16_t *__restrict__ scales,
                                              uint16_t *__restrict__ y, int row0, int tok0,
                                              int out, int batch, int nkb, float total_mul) {
  const int l32 = lane & 31, hl = lane >> 5;
  float16_t acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  // the MFMAs of one K block from LDS buffer buf: in step s the lane half hl
  // feeds chunk 2 s + hl of the K block, in A and in B alike; step s + 1's
  // operand reads are issued before step s's MFMAs.
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
        b[slot][ni] = *reinterpret_cast<const uint4 *>(X + tile_off(w * 64 + ni * 32 + l32, j));
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

  __syncthreads();  // K block 0's tiles
  int kb = 0;
  for (; kb + 2 <= nkb; kb += 2) {
    compute(0);
    __syncthreads();
    compute(1);
    __syncthreads();
  }
  if (kb < nkb) {
    compute(0);
    __syncthreads();
  }

  // Epilogue: lane holds activation row l32 of each 32 x 32 tile; register r
  // is output row 8 (r / 4) + 4 hl + r % 4, so registers 4 q .. 4 q + 3 are
  // four consecutive rows (one 8-byte store when out is a multiple of 4).
  // The scales of the lane's sixteen groups of four rows are all loaded
  // before the first store: stores count against the same wait counter as
  // loads, so a scale load after a store would wait for that store too, and
  // the stores would take one memory round trip each.
  const Rsrc rsc = make_rsrc(scales, (uint32_t)out * 2u);
  constexpr uint32_t kOOB = 0x80000000u;  // past the buffer: reads zero
  auto epilogue = [&](auto packed_c) {
    constexpr bool packed = decltype(packed_c)::value;
    uint2 sc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rb = row0 + mi * 32 + 8 * q + 4 * hl;
        if constexpr (packed) {  // rb and out multiples of 4: the four rows are all in or all out
          sc[mi][q] = buf_load8(rsc, rb < out ? (uint32_t)rb * 2u : kOOB);
        } else {
          uint32_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h[e] = buf_load_u16(rsc, rb + e < out ? (uint32_t)(rb + e) * 2u : kOOB);
          sc[mi][q] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        }
      }
    auto scale_of = [&](int mi, int q, int e) {
      const uint32_t v = (e >> 1) ? sc[mi][q].y : sc[mi][q].x;
      return h2f((e & 1) ? v >> 16 : v & 0xFFFFu);
    };
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int tok = tok0 + w * 64 + ni * 32 + l32;
        if (tok >= batch) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rb = row0 + mi * 32 + 8 * q + 4 * hl;
          if constexpr (packed) {
            if (rb < out) {
              uint32_t h[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                h[e] = f2h((acc[mi][ni][4 * q + e] * total_mul) * scale_of(mi, q, e));
              *reinterpret_cast<uint2 *>(y + (int64_t)tok * out + rb) =
                  make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (rb + e < out)
                y[(int64_t)tok * out + rb + e] =
                    (uint16_t)f2h((acc[mi][ni][4 * q + e] * total_mul) * scale_of(mi, q, e));
          }
        }
      }
    }
  };
  if ((out & 3) == 0)
    epilogue(std::true_type{});
  else
    epilogue(std::false_type{});
}

template <Scheme S>
__global__ __launch_bounds__(kTThreads) void gemm_tile_kernel(
    const uint8_t *__restrict__ codes, const uint4 *__restrict__ books,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x, uint16_t *__restrict__ y,
    int out, int in, int groups, int batch, uint32_t codes_bytes, uint32_t x_bytes) {
  using C = TileScheme<S>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint4 *lbooks = reinterpret_cast<uint4 *>(lds);
  uint8_t *wt = lds + C::BOOKS;      // [2][kTWBytes]
  uint8_t *xt = wt + 2 * kTWBytes;   // [2][kTXBytes]
  uint32_t *big_flags = reinterpret_cast<uint32_t *>(xt + 2 * kTXBytes);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = blockIdx.x * kTBM;
  const int tok0 = blockIdx.y * kTBN;

  // 2x8: the codebooks into LDS, one 16-byte entry per thread; codebooks
  // large enough for the fp16 codeword sum to overflow are halved and the
  // totals doubled (overflow guard, aqlm_device.hpp)
  float total_mul = 1.0f;
  if constexpr (S == Scheme::k2x8) {
    const uint4 v = books[tid];
    lbooks[tid] = v;
    publish_flag(big_flags, has_large_half(v));
    __syncthreads();
    if (read_flag(big_flags, kTWaves)) {
      lbooks[tid] = hhalf8(v);
      total_mul = 2.0f;
    }
    __syncthreads();
  }
  // Both roles pass the same barriers: one after K block 0's tiles, one per
  // K block after that.
  if (wave >= kTWaves / 2) {
    tile_fill<S>(tid - kTFill, wt, xt, lbooks, make_rsrc(codes, codes_bytes), make_rsrc(x, x_bytes),
                 make_rsrc(books, (uint32_t)(65536 * C::G * 2)), row0, tok0, out, in, groups,
                 batch);
  } else {
    tile_multiply(wave, tid & 63, wt, xt, scales, y, row0, tok0, out, batch, groups / C::KG,
                  total_mul);
  }
}

}  // namespace

// True when the decoded-tile kernel serves this layer and batch: a dedicated
// scheme (element or bit-packed codes: for 8- and 16-bit codes the packed
// stream holds the element layout's bytes), whole K blocks (in a multiple of
// 64) and 32-bit byte offsets for the codes (rows of one block past the end)
// and the activations (one block past the end).
bool gemm_tile_fits(const LayerDesc &L, int64_t batch) {
  if (L.scheme == Scheme::kGeneral || L.in % kTKIn != 0) return false;
  const int64_t row_bytes = L.groups * kCodeBytesPerGroup;
  return (L.out + kTBM) * row_bytes + 4096 < (int64_t(1) << 31) &&
         (batch + kTBN) * L.in * 2 + 4096 < (int64_t(1) << 31);
}

// Modelled duration in microseconds. One block per CU, so the grid runs in
// rounds of up to 256 blocks; a round costs a + b * (its blocks / 256) per K
// block of 64 inputs (the b term: HBM and L2 contention as the round fills).
// a and b per scheme are fitted to kernel times on 11008x4096 and 4096x11008
// layers from 129 to 2048 rows (one round of 32..256 blocks, and two or
// three rounds), which the model follows to within 10 %.
double gemm_tile_cost_us(const LayerDesc &L, int64_t batch) {
  const double a = L.scheme == Scheme::k2x8 ? 0.83 : L.scheme == Scheme::k1x16g16 ? 0.83 : 0.93;
  const double b = L.scheme == Scheme::k2x8 ? 0.51 : L.scheme == Scheme::k1x16g16 ? 0.85 : 1.05;
  int64_t blocks = ((L.out + kTBM - 1) / kTBM) * ((batch + kTBN - 1) / kTBN);
  double per_kb = 0.0;
  while (blocks > 0) {
    const int64_t round = std::min<int64_t>(blocks, 256);
    per_kb += a + b * (double)round / 256.0;
    blocks -= round;
  }
  return per_kb * (double)(L.in / kTKIn);
}

// The route of aqlm_gemm (no workspace) above 128 rows, against the wide
// tiles. 1x16 and 1x16 g16: wherever the kernel fits; the codeword gathers
// of the wide tiles cost more at every size measured (11008x4096 and
// 4096x11008, 129..2048 rows: 1.0-1.6x this kernel's time, 1.5-2.4x on the
// 4096-row layer). 2x8: from 512 rows when the grid has at least 160 blocks;
// below that the wide tiles' 64-row blocks keep more CUs busy (11008x4096 at
// 129..320 rows: wide 63-69 us, this kernel 68-76 us; 4096x11008 is faster
// in the wide tiles up to 1024 rows: 123-156 us against 154-174 us).
bool gemm_tile_preferred(const LayerDesc &L, int64_t batch) {
  if (batch <= 128 || !gemm_tile_fits(L, batch)) return false;
  if (L.scheme != Scheme::k2x8) return true;
  return batch >= 512 && ((L.out + kTBM - 1) / kTBM) * ((batch + kTBN - 1) / kTBN) >= 160;
}

namespace {
template <Scheme S>
hipError_t launch_tile(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                       hipStream_t stream) {
  static std::atomic<uint64_t> raised{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (dev >= 64 || !(raised.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_tile_kernel<S>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, TileScheme<S>::LDS);
    if (e != hipSuccess) return e;
    raised.fetch_or(bit, std::memory_order_acq_rel);
  }
  const dim3 grid((unsigned)((L.out + kTBM - 1) / kTBM), (unsigned)((batch + kTBN - 1) / kTBN));
  hipLaunchKernelGGL(gemm_tile_kernel<S>, grid, dim3(kTThreads), TileScheme<S>::LDS, stream,
                     static_cast<const uint8_t *>(L.codes), reinterpret_cast<const uint4 *>(L.books),
                     L.scales, x, y, (int)L.out, (int)L.in, (int)L.groups, (int)batch,
                     (uint32_t)(L.out * L.groups * kCodeBytesPerGroup), (uint32_t)(batch * L.in * 2));
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_tile(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                            hipStream_t stream) {
  switch (L.scheme) {
    case Scheme::k2x8: return launch_tile<Scheme::k2x8>(L, x, batch, y, stream);
    case Scheme::k1x16: return launch_tile<Scheme::k1x16>(L, x, batch, y, stream);
    case Scheme::k1x16g16: return launch_tile<Scheme::k1x16g16>(L, x, batch, y, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace aqlm
