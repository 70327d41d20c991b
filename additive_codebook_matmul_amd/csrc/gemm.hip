// Batched product y = x . W^T on the matrix cores: tiles of W are decoded on
// chip straight into MFMA operand registers and multiplied with float16
// activations (float32 accumulation). W is never written to memory.
//
// Wide tiles (more than kSkinnyMaxBatch activation rows, gemm_wide_kernel):
// 4 wavefronts, each owning 64 output rows (two 32-row tiles of
// v_mfma_f32_32x32x16_f16) and the block's 32*NI activation rows (NI 32-column
// tiles), so a block covers 256 x 32*NI outputs and every decoded operand is
// used NI times. The K loop walks 8 groups at a time (64 inputs for g = 8,
// 128 for g = 16):
//   * codes are loaded kWideCodeDepth K blocks ahead (a static register ring,
//     the loop being unrolled to match), activations two K blocks ahead into
//     registers, then written to a double-buffered LDS tile (rows padded by 16
//     bytes so that 32 lanes reading one column hit distinct banks). Every
//     load is an unconditional buffer load (out-of-range offsets read zero),
//     so the compiler keeps exact wait counts;
//   * each lane decodes its rows' groups into an 8-half A operand: the sum of
//     the codewords in packed fp16 (2x8: the two codewords come from an 8 KiB
//     LDS copy; 1x16: one 16-byte gather from the L2-resident codebook);
//   * the row scale multiplies the float32 accumulator in the epilogue.
// The MFMA K index of every lane element is paired identically in A and B, so
// any assignment of groups to MFMA steps gives the same sum; for g = 8 the two
// lane halves take groups s and s + 4 of the K block in step s.
#include <atomic>
#include <type_traits>

#include "aqlm_device.hpp"

namespace aqlm {
namespace {

constexpr int kBlock = 256;
constexpr int kBM = 256;  // output rows per block
constexpr int kKG = 8;    // groups per K block
constexpr int kWideCodeDepth = 4;
constexpr uint32_t kWideOOB = 0x80000000u;

template <Scheme S, int NI>
struct WideCfg {
  static constexpr int G = group_size(S);
  static constexpr int BN = 32 * NI;            // activation rows per block
  static constexpr int KI = kKG * G;            // inputs per K block
  static constexpr int ROW_HALVES = KI + 8;     // padded LDS row of the activation tile
  static constexpr int TILE_HALVES = BN * ROW_HALVES;
  static constexpr int XPT = BN * KI / 8 / kBlock;  // 16-byte activation vectors per thread
  static constexpr int CWORDS = G == 8 ? 2 : 4;     // code words per lane, row tile and K block
};

template <Scheme S, bool ALIGNED, int NI>
__global__ __launch_bounds__(kBlock) void gemm_wide_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ books,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y, int out, int in, int groups, int batch, uint32_t codes_bytes,
    uint32_t x_bytes) {
  using C = WideCfg<S, NI>;
  constexpr int KD = kWideCodeDepth;
  __shared__ uint4 lds_books[S == Scheme::k2x8 ? 512 : 1];
  __shared__ __attribute__((aligned(16))) uint16_t lds_x[2][C::TILE_HALVES];
  __shared__ uint32_t big_flags[kBlock / 64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;  // which 8 K values of the MFMA step this lane feeds
  const int l32 = lane & 31;
  const int row0 = blockIdx.x * kBM + wave * 64;
  const int tok0 = blockIdx.y * C::BN;
  const uint32_t row_bytes = (uint32_t)groups * 2u;
  const uint4 *gbooks = reinterpret_cast<const uint4 *>(books);
  const Rsrc crs = make_rsrc(codes, codes_bytes);
  const Rsrc xrs = make_rsrc(x, x_bytes);
  const int nkb = (groups + kKG - 1) / kKG;

  // Codes of the lane's two row tiles for K block kb: g = 8 lanes need 4
  // groups (8 bytes) each, g = 16 lanes all 8 groups (16 bytes).
  auto load_codes = [&](int kb, uint32_t (&cw)[2][C::CWORDS]) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const uint32_t rowoff = (uint32_t)(row0 + mi * 32 + l32) * row_bytes;
      const bool ok = kb < nkb;
      if constexpr (ALIGNED) {
        if constexpr (C::G == 8) {
          const uint2 v = buf_load8(crs, ok ? rowoff + (uint32_t)kb * 16u + half * 8u : kWideOOB);
          cw[mi][0] = v.x;
          cw[mi][1] = v.y;
        } else {
          const uint4 v = buf_load16(crs, ok ? rowoff + (uint32_t)kb * 16u : kWideOOB);
          cw[mi][0] = v.x;
          cw[mi][1] = v.y;
          cw[mi][2] = v.z;
          cw[mi][3] = v.w;
        }
      } else {
        // rows whose codes are not 16-byte aligned: one 16-bit code at a time
        constexpr int NQ = C::G == 8 ? 4 : 8;
#pragma unroll
        for (int w = 0; w < C::CWORDS; ++w) cw[mi][w] = 0;
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) {
          const int gidx = kb * kKG + (C::G == 8 ? half * 4 : 0) + qq;
          const uint32_t c =
              buf_load_u16(crs, (ok && gidx < groups) ? rowoff + (uint32_t)gidx * 2u : kWideOOB);
          cw[mi][qq >> 1] |= c << ((qq & 1) * 16);
        }
      }
    }
  };
  // Activations of K block kb: thread t moves vectors t, t + 256, ... of the tile.
  auto load_x = [&](int kb, uint4 (&xr)[C::XPT]) {
#pragma unroll
    for (int i = 0; i < C::XPT; ++i) {
      const int v = threadIdx.x + i * kBlock;
      const int t = v / (C::KI / 8);
      const int kv = v - t * (C::KI / 8);
      const int col = kb * C::KI + kv * 8;
      const uint32_t off = (uint32_t)(tok0 + t) * (uint32_t)in * 2u + (uint32_t)col * 2u;
      xr[i] = buf_load16(xrs, col < in ? off : kWideOOB);
    }
  };
  auto store_x = [&](int buf, const uint4 (&xr)[C::XPT]) {
#pragma unroll
    for (int i = 0; i < C::XPT; ++i) {
      const int v = threadIdx.x + i * kBlock;
      const int t = v / (C::KI / 8);
      const int kv = v - t * (C::KI / 8);
      *reinterpret_cast<uint4 *>(&lds_x[buf][t * C::ROW_HALVES + kv * 8]) = xr[i];
    }
  };

  float16_t acc[2][NI];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  // one K block from LDS tile `buf` with codes cw; MASK zeroes the operands of
  // groups past the end of the row (a partial last K block)
  auto compute = [&](auto masked, int kb, int buf, const uint32_t (&cw)[2][C::CWORDS]) {
    constexpr bool MASK = decltype(masked)::value;
    const uint16_t *xt = lds_x[buf];
    constexpr int STEPS = C::G == 8 ? 4 : 8;
    if constexpr (S == Scheme::k2x8) {
      // 2x8: the LDS reads of step s + 1 (two codeword pairs, NI activation
      // fragments) are issued before the MFMAs of step s and the codeword
      // sums taken after them, so LDS latency (bank conflicts included:
      // random codes) overlaps the matrix cores instead of preceding them
      uint4 c0[2][2], c1[2][2], bx[2][NI];
      auto reads = [&](int s, int slot) __attribute__((always_inline)) {
        const int kcol = (half * 4 + s) * 8;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          const uint32_t code = (cw[mi][s >> 1] >> ((s & 1) * 16)) & 0xFFFFu;
          c0[slot][mi] = lds_books[code & 0xFF];
          c1[slot][mi] = lds_books[256 + (code >> 8)];
        }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          bx[slot][ni] =
              *reinterpret_cast<const uint4 *>(&xt[(ni * 32 + l32) * C::ROW_HALVES + kcol]);
      };
      reads(0, 0);
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        const int cur = s & 1;
        uint4 a[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          a[mi] = hadd8(c0[cur][mi], c1[cur][mi]);
          if constexpr (MASK) {
            if (kb * kKG + half * 4 + s >= groups) a[mi] = make_uint4(0, 0, 0, 0);
          }
        }
        if (s + 1 < STEPS) reads(s + 1, cur ^ 1);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(half8_t, a[mi]), __builtin_bit_cast(half8_t, bx[cur][ni]),
                acc[mi][ni], 0, 0, 0);
        if (s + 1 < STEPS) {
          __builtin_amdgcn_sched_group_barrier(0x100, 4 + NI, 0);  // next step's LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * NI, 0);  // then this step's MFMAs
        }
      }
      return;
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      // K columns of this step for this lane half, within the K block
      const int kcol = C::G == 8 ? (half * 4 + s) * 8 : s * 16 + half * 8;
      uint4 a[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const uint32_t code = (cw[mi][s >> 1] >> ((s & 1) * 16)) & 0xFFFFu;
        if constexpr (S == Scheme::k2x8) {
          a[mi] = hadd8(lds_books[code & 0xFF], lds_books[256 + (code >> 8)]);
        } else if constexpr (S == Scheme::k1x16) {
          a[mi] = gbooks[code];
        } else {
          a[mi] = gbooks[2 * code + half];
        }
        if constexpr (MASK) {
          const int gidx = kb * kKG + (C::G == 8 ? half * 4 + s : s);
          if (gidx >= groups) a[mi] = make_uint4(0, 0, 0, 0);
        }
      }
      uint4 bx[NI];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        bx[ni] = *reinterpret_cast<const uint4 *>(&xt[(ni * 32 + l32) * C::ROW_HALVES + kcol]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(half8_t, a[mi]), __builtin_bit_cast(half8_t, bx[ni]),
              acc[mi][ni], 0, 0, 0);
    }
  };

  // Prologue: codes of K blocks 0 .. KD-1, activations of K blocks 0 and 1,
  // the 2x8 codebooks, then K block 0's activations into LDS.
  uint32_t cw[KD][2][C::CWORDS];
  uint4 xr[2][C::XPT];
#pragma unroll
  for (int i = 0; i < KD; ++i) load_codes(i, cw[i]);
  load_x(0, xr[0]);
  load_x(1, xr[1]);
  if constexpr (S == Scheme::k2x8) {
    bool large = false;
    for (int i = threadIdx.x; i < 512; i += kBlock) {
      const uint4 v = gbooks[i];
      large |= has_large_half(v);
      lds_books[i] = v;
    }
    publish_flag(big_flags, large);
  }
  store_x(0, xr[0]);
  __syncthreads();
  // codebooks large enough for the fp16 codeword sum to overflow: halve the
  // table, double the totals (overflow guard, aqlm_device.hpp)
  float total_mul = 1.0f;
  if constexpr (S == Scheme::k2x8) {
    if (read_flag(big_flags, kBlock / 64)) {
      for (int i = threadIdx.x; i < 512; i += kBlock) lds_books[i] = hhalf8(lds_books[i]);
      __syncthreads();
      total_mul = 2.0f;
    }
  }

  const bool tail_partial = groups % kKG != 0;
  // K block kb (code slot K = kb % KD, activation slot kb % 2): prefetch
  // activations of kb + 2, compute, write kb + 1's activations to the other
  // LDS buffer, refill code slot K with kb + KD.
  auto iter = [&](int kb, auto kc) {
    constexpr int K = decltype(kc)::value;
    load_x(kb + 2, xr[K & 1]);
    if (tail_partial && kb == nkb - 1)
      compute(std::true_type{}, kb, K & 1, cw[K]);
    else
      compute(std::false_type{}, kb, K & 1, cw[K]);
    store_x((K + 1) & 1, xr[(K + 1) & 1]);
    load_codes(kb + KD, cw[K]);
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

  // Epilogue: lane holds column l32 of each 32x32 tile; register r is row
  // 8*(r/4) + 4*half + r%4. The lane's 32 row scales are loaded before the
  // first store: stores count against the same wait counter as loads, so a
  // scale load after a store would wait for that store.
  const Rsrc rsc = make_rsrc(scales, (uint32_t)out * 2u);
  uint32_t sh[2][16];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = row0 + mi * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      sh[mi][r] = buf_load_u16(rsc, row < out ? (uint32_t)row * 2u : kWideOOB);
    }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int tok = tok0 + ni * 32 + l32;
      if (tok >= batch) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + mi * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < out)
          y[(int64_t)tok * out + row] =
              (uint16_t)f2h((acc[mi][ni][r] * total_mul) * h2f(sh[mi][r]));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Skinny tiles for few activation rows: v_mfma_f32_16x16x32_f16 on 16 output
// rows x 16 activation rows. Lane l feeds row (A) or activation row (B)
// l % 16 and K slice l / 16 of eight inputs; it holds output rows
// 4 * (l / 16) .. + 3 of activation row l % 16 in its accumulator.
//
// A block owns 16 output rows and NT tiles of 16 activation rows; its waves
// split the input dimension into contiguous ranges of chunks, and their
// float32 partial sums are added in LDS in wave order (deterministic). A chunk
// is one 16-byte code load per lane (8 groups): 32 groups (256 inputs) for
// g = 8, 16 groups for g = 16, consumed in 8 MFMA steps.
//
// K order: in step s, lane quarter q takes the 16-byte column block 4s + q of
// the chunk's 512 activation bytes: group 4s + q (g = 8), or half q % 2 of
// group 2s + q / 2 (g = 16). A and B use the same map, so the MFMA's K order
// is a permutation of the inputs and the sum is unchanged. A lane loads 8
// consecutive codes of its row; a per-wave LDS transpose puts them in step
// order.
//
// Activations: the B layout gives the four 16-byte pieces of one activation
// row to lanes l, l + 16, l + 32, l + 48, so loading fragments directly would
// never coalesce (the L1 then serves one lane per clock). Each wave instead
// loads its chunk's activations with fully coalesced 16-byte loads into
// registers, writes them to a private LDS slot (column block XOR activation
// row, so fragment reads are free of bank conflicts) and reads its B fragments
// from there. Codes are loaded kSkinnyCodeDepth chunks ahead, activations (and
// 1x16 codewords) one chunk ahead.
constexpr int kSkinnyMaxWaves = 8;
constexpr int kSkinnyCodeDepth = 4;  // the step loop below is unrolled to match
constexpr int64_t kSkinnyMaxBatch = 128;  // above this the wide tiles take over
constexpr int kSkinnyXSlotBytes = 16 * 512;  // one 16-row activation tile of a chunk

// Dynamic LDS of one block: [2x8 codebooks 8 KiB, overflow-guard flags 64 B]
// [code transpose 1 KiB per wave][activation slots NT x 8 KiB per wave]; the
// final reduction reuses the activation slots.
constexpr int kSkinnyBooksBytes = 8192 + 64;
constexpr int skinny_lds_bytes(bool lut, int nt, int waves) {
  return (lut ? kSkinnyBooksBytes : 0) + waves * 1024 + waves * nt * kSkinnyXSlotBytes;
}

template <Scheme S, int NT, bool ALIGNED>
__global__ __launch_bounds__(64 * kSkinnyMaxWaves) void gemm_skinny_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ books,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y, int out, int in, int groups, int batch, uint32_t codes_bytes,
    uint32_t x_bytes) {
  constexpr int G = group_size(S);
  constexpr int GPC = G == 8 ? 32 : 16;  // groups per chunk
  constexpr bool LUT = S == Scheme::k2x8;
  constexpr int CD = kSkinnyCodeDepth;
  // steps between transposing a chunk's codes and computing it: the 1x16
  // codeword gathers need them a step earlier
  constexpr int SA = LUT ? 1 : 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int lane = threadIdx.x & 63, waves = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int r = lane & 15, q = lane >> 4;
  const int row0 = blockIdx.x * 16, tok0 = blockIdx.y * (16 * NT);
  const uint32_t row_bytes = (uint32_t)groups * 2u;
  const int piece = G == 8 ? q : (q >> 1);  // which 8 codes of the chunk the lane loads
  const uint4 *gbooks = reinterpret_cast<const uint4 *>(books);

  uint4 *lds_books = reinterpret_cast<uint4 *>(lds);
  uint32_t *big_flags = reinterpret_cast<uint32_t *>(lds + 8192);
  uint8_t *lds_codes = lds + (LUT ? kSkinnyBooksBytes : 0);
  uint8_t *lds_xall = lds_codes + waves * 1024;
  uint4 *xslot = reinterpret_cast<uint4 *>(lds_xall + wave * NT * kSkinnyXSlotBytes);
  uint16_t *cslot = reinterpret_cast<uint16_t *>(lds_codes + wave * 1024) + r * 32;

  // Rows >= out and activation rows >= batch start past the end of their
  // buffers, so their loads return zero.
  const Rsrc crs = make_rsrc(codes, codes_bytes);
  const Rsrc xrs = make_rsrc(x, x_bytes);
  const uint32_t crow = (uint32_t)(row0 + r) * row_bytes;
  // coalesced activation loads: load j of tile t brings activation rows
  // 2j + lane / 32 of the tile, 16-byte column block lane % 32
  const int xl_row = lane >> 5, xl_blk = lane & 31;
  uint32_t xl_off[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    xl_off[t] = (uint32_t)(tok0 + 16 * t + xl_row) * (uint32_t)in * 2u + (uint32_t)xl_blk * 16u;
  const uint32_t x_pair_stride = 2u * (uint32_t)in * 2u;  // two activation rows

  const int nchunks = (groups + GPC - 1) / GPC;
  const int nfull = groups / GPC;
  const int cb = wave * nchunks / waves, ce = (wave + 1) * nchunks / waves;
  // full chunks run in the pipelined loop; a partial last chunk runs after it
  const int nmain = max(0, min(ce, nfull) - cb);
  // Chunk of step i; steps past the loop repeat its last chunk (a cache hit),
  // so prefetching never streams extra code bytes.
  auto chunk_of = [&](int i) { return cb + min(i, nmain - 1); };

  auto load_codes = [&](int c, uint32_t (&cw)[4]) {
    const uint32_t off = crow + (uint32_t)(c * GPC + piece * 8) * 2u;
    if constexpr (ALIGNED) {
      const uint4 v = buf_load16(crs, off);
      cw[0] = v.x;
      cw[1] = v.y;
      cw[2] = v.z;
      cw[3] = v.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        cw[i] = buf_load_u16(crs, off + 4u * i) | (buf_load_u16(crs, off + 4u * i + 2u) << 16);
    }
  };
  auto load_x = [&](int c, uint4 (&xr)[NT][8]) {
    const uint32_t cbyte = (uint32_t)c * 512u;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j) xr[t][j] = buf_load16(xrs, xl_off[t] + j * x_pair_stride + cbyte);
  };
  auto store_x = [&](const uint4 (&xr)[NT][8]) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = 2 * j + xl_row;
        xslot[t * 512 + row * 32 + (xl_blk ^ row)] = xr[t][j];
      }
  };
  auto frag = [&](int t, int s) { return xslot[t * 512 + r * 32 + ((4 * s + q) ^ r)]; };

  // Transpose the row's chunk codes through this wave's LDS slot so that
  // sc holds the lane's codes in step order (two per register).
  auto stage = [&](const uint32_t (&cw)[4], uint32_t (&sc)[4]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = piece * 8 + i;  // code index within the chunk row
      const int pos = G == 8 ? (k & 3) * 8 + (k >> 2) : (k & 1) * 8 + (k >> 1);
      cslot[pos] = (uint16_t)(cw[i >> 1] >> ((i & 1) * 16));
    }
    const uint4 v = *reinterpret_cast<const uint4 *>(cslot + (G == 8 ? q : (q >> 1)) * 8);
    sc[0] = v.x;
    sc[1] = v.y;
    sc[2] = v.z;
    sc[3] = v.w;
  };
  auto code_of = [](const uint32_t (&sc)[4], int s) {
    return (sc[s >> 1] >> ((s & 1) * 16)) & 0xFFFFu;
  };
  auto gather = [&](const uint32_t (&sc)[4], uint4 (&ga)[8]) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t code = code_of(sc, s);
      ga[s] = gbooks[G == 8 ? code : 2u * code + (uint32_t)(q & 1)];
    }
  };

  float4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Four MFMA steps at a time: every LDS read of the four is issued before
  // the first add, so their latencies overlap instead of adding up.
  auto compute = [&](auto masked, int c, const uint32_t (&sc)[4], const uint4 (&ga)[8]) {
    constexpr bool MASK = decltype(masked)::value;
#pragma unroll
    for (int h = 0; h < 8; h += 4) {
      uint4 c0[4], c1[4], b[4][NT];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = h + u;
        if constexpr (LUT) {
          const uint32_t code = code_of(sc, s);
          c0[u] = lds_books[code & 0xFFu];
          c1[u] = lds_books[256u + (code >> 8)];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) b[u][t] = frag(t, s);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = h + u;
        uint4 a = LUT ? hadd8(c0[u], c1[u]) : ga[s];
        if constexpr (MASK) {
          // 16-byte column blocks past the end of the row: zero both operands
          if (c * 512 + (4 * s + q) * 16 >= in * 2) {
            a = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < NT; ++t) b[u][t] = make_uint4(0, 0, 0, 0);
          }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                         __builtin_bit_cast(half8_t, b[u][t]),
                                                         acc[t], 0, 0, 0);
      }
    }
  };

  // Register rings indexed statically (the step loop is unrolled CD times):
  // moving a register whose load is still in flight would stall on it.
  uint32_t cw[CD][4];  // raw codes, CD chunks ahead
  uint32_t sc[4][4];   // codes in step order
  uint4 xr[NT][8];     // next chunk's activations on their way to LDS
  uint4 ga[2][8];      // 1x16 codewords (unused by the LDS lookup)
  if (nmain > 0) {
    load_x(chunk_of(0), xr);
#pragma unroll
    for (int i = 0; i < CD; ++i) load_codes(chunk_of(i), cw[i]);
  }
  bool halved = false;
  if constexpr (LUT) {
    // issued after the first chunk's loads so that the latencies overlap
    bool large = false;
    for (int i = threadIdx.x; i < 512; i += blockDim.x) {
      const uint4 v = gbooks[i];
      large |= has_large_half(v);
      lds_books[i] = v;
    }
    publish_flag(big_flags, large);
    __syncthreads();
    // codebooks large enough for the fp16 codeword sum to overflow: halve the
    // table, double the totals (overflow guard, aqlm_device.hpp)
    halved = read_flag(big_flags, waves);
    if (halved) {
      for (int i = threadIdx.x; i < 512; i += blockDim.x) lds_books[i] = hhalf8(lds_books[i]);
      __syncthreads();
    }
  }
  if (nmain > 0) {
    store_x(xr);
#pragma unroll
    for (int i = 0; i < SA; ++i) stage(cw[i], sc[i]);
    if constexpr (!LUT) gather(sc[0], ga[0]);
  }

  // Step i (code slot K = i % CD). Loads are issued in the order activations,
  // codewords, codes, so that waiting for the first two never waits for the
  // codes fetched CD steps ahead (vmcnt retires in order).
  auto step = [&](int i, auto kc) {
    constexpr int K = decltype(kc)::value;
    load_x(chunk_of(i + 1), xr);
    stage(cw[(K + SA) % CD], sc[(K + SA) & 3]);
    if constexpr (!LUT) gather(sc[(K + 1) & 3], ga[(K + 1) & 1]);
    load_codes(chunk_of(i + CD), cw[K]);
    compute(std::false_type{}, chunk_of(i), sc[K], ga[K & 1]);
    // overwrites this chunk's activations: the fragment reads above are
    // ahead of these writes in the wave's LDS queue
    store_x(xr);
  };
  int i = 0;
  for (; i + CD <= nmain; i += CD) {
    step(i, std::integral_constant<int, 0>{});
    step(i + 1, std::integral_constant<int, 1>{});
    step(i + 2, std::integral_constant<int, 2>{});
    step(i + 3, std::integral_constant<int, 3>{});
  }
  if (i < nmain) step(i, std::integral_constant<int, 0>{});
  if (i + 1 < nmain) step(i + 1, std::integral_constant<int, 1>{});
  if (i + 2 < nmain) step(i + 2, std::integral_constant<int, 2>{});

  if (ce > nfull) {
    // the partial last chunk (only the last wave has one), unpipelined
    const int c = nfull;
    uint32_t tcw[4], tsc[4];
    load_codes(c, tcw);
    load_x(c, xr);
    stage(tcw, tsc);
    if constexpr (!LUT) gather(tsc, ga[0]);
    store_x(xr);
    compute(std::true_type{}, c, tsc, ga[0]);
  }

  if (halved) {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = acc[t] * 2.0f;
  }
  // Epilogue: add the waves' partial sums in wave order, scale, round. The
  // rows of an element depend on its lane only; their scales are loaded
  // before its stores (stores count against the same wait counter as loads).
  const Rsrc rsc = make_rsrc(scales, (uint32_t)out * 2u);
  auto row_scales = [&](int l, uint32_t (&sh)[4]) {
    const int rb = row0 + 4 * (l >> 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) sh[k] = buf_load_u16(rsc, rb + k < out ? (uint32_t)(rb + k) * 2u : kWideOOB);
  };
  auto write = [&](int t, int l, const float4_t &v, const uint32_t (&sh)[4]) {
    const int tok = tok0 + 16 * t + (l & 15);
    if (tok >= batch) return;
    const int rb = row0 + 4 * (l >> 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int row = rb + k;
      if (row < out) y[(int64_t)tok * out + row] = (uint16_t)f2h(v[k] * h2f(sh[k]));
    }
  };
  if (waves == 1) {
    uint32_t sh[4];
    row_scales(lane, sh);
#pragma unroll
    for (int t = 0; t < NT; ++t) write(t, lane, acc[t], sh);
    return;
  }
  float4_t *red = reinterpret_cast<float4_t *>(lds_xall);
  __syncthreads();  // every wave is done with its activation slot
#pragma unroll
  for (int t = 0; t < NT; ++t) red[(wave * NT + t) * 64 + lane] = acc[t];
  __syncthreads();
  for (int e = threadIdx.x; e < NT * 64; e += blockDim.x) {
    const int t = e >> 6, l = e & 63;
    float4_t v = red[t * 64 + l];
    for (int w = 1; w < waves; ++w) v += red[(w * NT + t) * 64 + l];
    uint32_t sh[4];
    row_scales(l, sh);
    write(t, l, v, sh);
  }
}

template <Scheme S, int NT>
hipError_t launch_skinny(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                         hipStream_t stream) {
  const int out = (int)L.out, in = (int)L.in, groups = (int)L.groups;
  constexpr bool LUT = S == Scheme::k2x8;
  constexpr int GPC = group_size(S) == 8 ? 32 : 16;
  const int nchunks = (groups + GPC - 1) / GPC;
  const int row_tiles = (out + 15) / 16;
  const int tok_blocks = (int)((batch + 16 * NT - 1) / (16 * NT));
  // enough wavefronts to cover the chip about eight times, at least one chunk each
  const int64_t wgs = (int64_t)row_tiles * tok_blocks;
  int waves = 1;
  while (waves < kSkinnyMaxWaves && wgs * waves < 2048 && waves * 2 <= nchunks) waves *= 2;
  const dim3 grid(row_tiles, tok_blocks);
  const uint32_t codes_bytes = (uint32_t)(L.out * L.groups * kCodeBytesPerGroup);
  const uint32_t x_bytes = (uint32_t)(batch * L.in * 2);
  const uint8_t *codes = static_cast<const uint8_t *>(L.codes);
  const size_t lds = skinny_lds_bytes(LUT, NT, waves);
  const bool aligned = groups % 8 == 0;
  auto k = aligned ? gemm_skinny_kernel<S, NT, true> : gemm_skinny_kernel<S, NT, false>;
  static_assert(skinny_lds_bytes(LUT, NT, kSkinnyMaxWaves) <= 160 * 1024, "LDS budget");
  if (lds > 64 * 1024) {
    // more than the default dynamic LDS limit: raise it once per device
    static std::atomic<uint64_t> raised[2]{};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = uint64_t(1) << (dev & 63);
    if (dev >= 64 || !(raised[aligned].load(std::memory_order_acquire) & bit)) {
      e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              skinny_lds_bytes(LUT, NT, kSkinnyMaxWaves));
      if (e != hipSuccess) return e;
      raised[aligned].fetch_or(bit, std::memory_order_acq_rel);
    }
  }
  hipLaunchKernelGGL(k, grid, dim3(64 * waves), lds, stream, codes, L.books, L.scales, x, y, out,
                     in, groups, (int)batch, codes_bytes, x_bytes);
  return hipGetLastError();
}

// Byte offsets of the skinny kernel are 32-bit: rows past the end (up to 15)
// and chunks read ahead must stay below 2^32.
bool skinny_fits(const LayerDesc &L, int64_t batch, int nt) {
  const int64_t row_bytes = L.groups * kCodeBytesPerGroup;
  const int64_t code_span = (L.out + 16) * row_bytes + 4096;
  const int64_t x_span = (batch + 16 * nt) * L.in * 2 + 4096;
  return code_span < (int64_t(1) << 32) && x_span < (int64_t(1) << 32);
}

// Activation rows per wide block, 32 * NI. The 1x16 schemes gather their
// codewords from L2, so a wider block (each gather feeding more MFMAs) pays;
// 2x8 decodes from LDS and prefers the smaller register footprint (two waves
// per SIMD instead of one).
template <Scheme S>
constexpr int wide_ni() { return S == Scheme::k2x8 ? 2 : 4; }



// 32-bit byte offsets of the wide kernel: codes of 256 rows past the end and
// activations of a whole block past the end must stay below 2^32.
bool wide_fits(const LayerDesc &L, int64_t batch, int ni) {
  const int64_t row_bytes = L.groups * kCodeBytesPerGroup;
  return (L.out + kBM) * row_bytes + 4096 < (int64_t(1) << 31) &&
         (batch + 32 * ni) * L.in * 2 + 4096 < (int64_t(1) << 31);
}

template <Scheme S, int NI>
hipError_t launch_wide(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                       hipStream_t stream) {
  const int out = (int)L.out, in = (int)L.in, groups = (int)L.groups;
  const dim3 grid((out + kBM - 1) / kBM, (unsigned)((batch + 32 * NI - 1) / (32 * NI)));
  const uint8_t *codes = static_cast<const uint8_t *>(L.codes);
  const uint32_t codes_bytes = (uint32_t)(L.out * L.groups * kCodeBytesPerGroup);
  const uint32_t x_bytes = (uint32_t)(batch * L.in * 2);
  if (groups % kKG == 0)
    hipLaunchKernelGGL((gemm_wide_kernel<S, true, NI>), grid, dim3(kBlock), 0, stream, codes,
                       L.books, L.scales, x, y, out, in, groups, (int)batch, codes_bytes, x_bytes);
  else
    hipLaunchKernelGGL((gemm_wide_kernel<S, false, NI>), grid, dim3(kBlock), 0, stream, codes,
                       L.books, L.scales, x, y, out, in, groups, (int)batch, codes_bytes, x_bytes);
  return hipGetLastError();
}

template <Scheme S>
hipError_t launch_scheme(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                         hipStream_t stream) {
  // one activation tile of the workspace form, where it needs no workspace
  if (gemm_mid_direct(L, batch)) return launch_gemm_ws(L, x, batch, y, nullptr, stream);
  if (batch <= 16 && skinny_fits(L, batch, 1)) return launch_skinny<S, 1>(L, x, batch, y, stream);
  if (batch <= kSkinnyMaxBatch && skinny_fits(L, batch, 2))
    return launch_skinny<S, 2>(L, x, batch, y, stream);
  if (gemm_tile_preferred(L, batch)) return launch_gemm_tile(L, x, batch, y, stream);
  if (wide_fits(L, batch, wide_ni<S>())) return launch_wide<S, wide_ni<S>()>(L, x, batch, y, stream);
  // sizes past the 32-bit offsets of the tiled kernels: the general kernel
  // (64-bit indexing, exact fp16 weight tiles)
  return launch_gemm_general(L, x, batch, y, stream);
}

}  // namespace

hipError_t launch_gemm(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                       hipStream_t stream) {
  // Up to 8 rows the token-generation routes (matrix-core or lookup GEMV, or a
  // 16-row GEMM tile where that measured faster) are the fastest form of the
  // same product for every scheme: the call runs them, bit-identical to
  // aqlm_gemv.
  if (batch <= 8) return launch_gemv(L, x, (int)batch, y, stream);
  switch (L.scheme) {
    case Scheme::k2x8: return launch_scheme<Scheme::k2x8>(L, x, batch, y, stream);
    case Scheme::k1x16: return launch_scheme<Scheme::k1x16>(L, x, batch, y, stream);
    case Scheme::k1x16g16: return launch_scheme<Scheme::k1x16g16>(L, x, batch, y, stream);
    case Scheme::kGeneral: return launch_gemm_general(L, x, batch, y, stream);
  }
  return hipErrorInvalidValue;
}

// Token-generation calls (1..8 activation rows) that a 16-row GEMM tile
// serves faster than the GEMV kernels, measured per scheme on 4096 x 4096,
// 11008 x 4096 and 4096 x 11008 layers. The tile is the workspace form's
// one activation tile read in place where that applies (layers with enough
// row blocks to fill half the chip unsplit), else the skinny tile. A 1x16
// GEMV reads the activations once per output row, so its cost grows with
// batch x in; the 1x16 g16 GEMV (two 16-byte gathers per group and lane)
// loses from two rows, and from one row against the in-place tile; 2x8
// takes a tile only when its matrix-core GEMV cannot stage the activations
// in LDS (the lookup kernel then costs 3x the tile at 5..8 rows of 11008
// inputs).
bool gemv_uses_gemm_tiles(const LayerDesc &L, int batch) {
  if (batch < 1 || batch > 8 || !skinny_fits(L, batch, 1)) return false;
  const bool in_place = L.scheme != Scheme::k2x8 && gemm_mid_direct(L, batch);
  switch (L.scheme) {
    case Scheme::k2x8: return batch >= 3 && !gemv_2x8_mfma_fits(L, batch);
    case Scheme::k1x16: return in_place ? batch >= 5 : (int64_t)batch * L.in >= 32768;
    case Scheme::k1x16g16: return in_place || batch >= 2;
    default: return false;
  }
}

hipError_t launch_gemv_as_gemm(const LayerDesc &L, const uint16_t *x, int batch, uint16_t *y,
                               hipStream_t stream) {
  if (gemm_mid_direct(L, batch)) return launch_gemm_ws(L, x, batch, y, nullptr, stream);
  switch (L.scheme) {
    case Scheme::k2x8: return launch_skinny<Scheme::k2x8, 1>(L, x, batch, y, stream);
    case Scheme::k1x16: return launch_skinny<Scheme::k1x16, 1>(L, x, batch, y, stream);
    case Scheme::k1x16g16: return launch_skinny<Scheme::k1x16g16, 1>(L, x, batch, y, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace aqlm
