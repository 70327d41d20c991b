// 2x8 products for 1..8 activation rows on the matrix cores.
//
// The lookup GEMV spends twelve VALU operations per group (four address
// permutes, eight fp16 dot2), so it is issue-bound far below HBM speed. Here
// the dot products run on v_mfma_f32_16x16x32_f16 instead: the two codewords
// of a group are read from LDS, added in fp16 (one packed add per pair of
// weights, as in the batched GEMM's tiles) and fed to one MFMA as A operand;
// the sum over groups is accumulated in float32 and the row scale applied to
// it. The activation rows are the B operand (16 MFMA columns, the first BATCH
// of them used). A group then costs 2/64 of an address permute per lane, two
// 16-byte LDS reads and half an MFMA step; the kernel is bound by LDS and HBM
// bandwidth rather than by VALU issue.
//
// Layout of the work:
//   * a workgroup (8 wavefronts) owns tiles of 16 output rows; its
//     wavefronts split the row's 32-group chunks into contiguous ranges and
//     add their float32 partial sums in LDS in wave order (deterministic);
//   * in MFMA step s of chunk c, lane (r = lane % 16, q = lane / 16) feeds
//     group c*32 + 8q + s of row r, so each lane's codes for a chunk are one
//     16-byte load (8 consecutive groups of its row);
//   * codebooks live in a 64 KiB bank-spread LDS table: the 256-byte stripe
//     of code value c holds eight 16-byte copies of C_0[c] (slots 0..7) and
//     eight of C_1[c] (slots 8..15). Lane r reads slot r in its first read
//     (codebook r / 8) and slot r ^ 8 in its second (the other codebook), so
//     the 16 lanes of every 16-byte LDS pass touch 16 distinct slots, i.e. all
//     64 banks once, whatever the codes;
//   * the activations are copied to LDS once per workgroup (rows padded by 16
//     bytes); B fragment reads of one activation row are broadcasts;
//   * codes of NBUF tiles ahead are in flight (buffer loads, non-temporal).
//     When every block has at most two tiles (and they fit in registers),
//     all of a block's tiles are loaded in the prologue and nothing is
//     refilled (ALL): the second tile does not wait for a load issued after
//     the first, and no prefetch runs past the last tile (a load with an
//     out-of-range offset returns zero but still occupies the texture-address
//     unit that the real loads of every wave on the CU queue behind).
#include "aqlm_device.hpp"

#include <atomic>
#include <type_traits>

namespace aqlm {
namespace {

constexpr int kMBlock = 512;
constexpr int kMWaves = kMBlock / 64;
constexpr int kMTable = 65536;
constexpr int kMaxTilesPerBlock = 64;  // row scales of a block's tiles are staged in LDS
constexpr uint32_t kMOOB = 0x80000000u;

// LDS: the 64 KiB table is a static array (its addresses then fold into the
// read instructions); the dynamic part holds the activations (BATCH rows of
// in + 8 halves), the row scales, the reduction buffers (two of waves x 16
// rows x BATCH floats) and one overflow-guard flag per wavefront.
constexpr size_t mfma_dyn_lds_bytes(int batch, int in) {
  return (size_t)batch * (in + 8) * 2 + kMaxTilesPerBlock * 16 * 2 + 2 * kMWaves * 16 * batch * 4 +
         kMWaves * 4;
}
constexpr size_t mfma_lds_bytes(int batch, int in) { return kMTable + mfma_dyn_lds_bytes(batch, in); }

struct MfmaLayer {
  const uint8_t *codes;
  const uint16_t *books;
  const uint16_t *scales;
  const uint16_t *x;
  uint16_t *y;
  int out, in, groups;
  int batch;                 // activation rows, 1 .. BATCH
  int blk_begin, blk_count;  // blocks [blk_begin, blk_begin + blk_count) serve this layer
};

template <int BATCH, int MAXC, int NBUF, bool ALL>
__device__ __forceinline__ void gemv_2x8_mfma_body(const MfmaLayer &L, int blk) {
  __shared__ __attribute__((aligned(16))) uint8_t table[kMTable];
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int xstride = L.in + 8;  // halves per staged activation row
  uint16_t *xs = reinterpret_cast<uint16_t *>(lds);
  uint16_t *sc_lds = xs + BATCH * xstride;
  float *red = reinterpret_cast<float *>(sc_lds + kMaxTilesPerBlock * 16);
  uint32_t *big_flags = reinterpret_cast<uint32_t *>(red + 2 * kMWaves * 16 * BATCH);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int out = L.out, in = L.in, groups = L.groups;
  const int nch = groups / 32;
  const int cb = wave * nch / kMWaves;
  const int nw = (wave + 1) * nch / kMWaves - cb;  // this wave's chunks, <= MAXC
  const int ntiles = (out + 15) / 16;
  const int my_tiles = blk < ntiles ? (ntiles - blk + L.blk_count - 1) / L.blk_count : 0;
  const uint32_t row_bytes = (uint32_t)groups * 2u;

  // Prologue. Every load from L2 (one codeword per thread, the activations,
  // the row scales) is issued first, then the code loads of the first NBUF
  // tiles (HBM), then the LDS writes: waiting for the L2 data never waits for
  // the codes, since the vector-memory counter retires in order.
  const int batch = L.batch;
  const int tm = (tid >> 3) & 1;                  // this thread's table entry: codebook tm,
  const int tc = (tid & 7) | ((tid >> 4) << 3);   // code value tc
  const uint4 book_v = reinterpret_cast<const uint4 *>(L.books)[tm * 256 + tc];
  const int nxv = batch * (in / 8);  // 16-byte activation vectors
  const Rsrc rx = make_rsrc(L.x, (uint32_t)nxv * 16u);
  // activation vectors per thread and pass: enough for BATCH rows of the
  // longest input the class serves (MAXC * 8 waves * 32 groups), at most 4
  constexpr int kXPT = BATCH * MAXC / 2 < 1 ? 1 : (BATCH * MAXC / 2 > 4 ? 4 : BATCH * MAXC / 2);
  uint4 xv[kXPT];
#pragma unroll
  for (int j = 0; j < kXPT; ++j) xv[j] = buf_load16(rx, (uint32_t)(tid + j * kMBlock) * 16u);
  const Rsrc rs = make_rsrc(L.scales, (uint32_t)out * 2u);
  uint32_t sv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = tid + j * kMBlock;
    const int row = (blk + (e >> 4) * L.blk_count) * 16 + (e & 15);
    sv[j] = buf_load_u16(rs, (e < my_tiles * 16 && row < out) ? (uint32_t)row * 2u : kMOOB);
  }

  // keep the L2 loads above ahead of the code loads below (the scheduler may
  // otherwise sink them past the HBM loads, and the LDS writes would then
  // wait for the codes)
  __builtin_amdgcn_sched_barrier(0);

  const Rsrc rc = make_rsrc(L.codes, (uint32_t)out * row_bytes);
  const uint32_t lane_off = (uint32_t)r * row_bytes + (uint32_t)(cb * 32 + q * 8) * 2u;
  const uint32_t tile_bytes = 16u * row_bytes;
  uint4 cw[NBUF][MAXC];
  auto load_tile = [&](int i, uint4 (&dst)[MAXC]) {
    const bool ok = i < my_tiles;
    const uint32_t toff = (uint32_t)(blk + i * L.blk_count) * tile_bytes + lane_off;
#pragma unroll
    for (int k = 0; k < MAXC; ++k)
      dst[k] = buf_load16_nt(rc, (ok && k < nw) ? toff + (uint32_t)k * 64u : kMOOB);
  };
#pragma unroll
  for (int u = 0; u < NBUF; ++u) load_tile(u, cw[u]);
  __builtin_amdgcn_sched_barrier(0);

  // The table: each thread writes the 8 copies of its codeword, copy
  // (j + tid) % 8 in write j, so that the 16 lanes of a pass hit 16 distinct
  // 16-byte slots (lanes 8 apart hold the two codebooks).
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<uint4 *>(table + tc * 256 + tm * 128 + ((j + tid) & 7) * 16) = book_v;
  // first pass of activations and the scales (their loads precede the code
  // loads, so these writes wait for L2 only)
#pragma unroll
  for (int j = 0; j < kXPT; ++j) {
    const int e = tid + j * kMBlock;
    if (e < nxv) {
      const int b = e / (in / 8), v = e - b * (in / 8);
      *reinterpret_cast<uint4 *>(xs + b * xstride + v * 8) = xv[j];
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = tid + j * kMBlock;
    if (e < my_tiles * 16) sc_lds[e] = (uint16_t)sv[j];
  }
  // further passes (long rows or several activation rows)
  for (int base = kXPT * kMBlock; base < nxv; base += kXPT * kMBlock) {
#pragma unroll
    for (int j = 0; j < kXPT; ++j) xv[j] = buf_load16(rx, (uint32_t)(base + tid + j * kMBlock) * 16u);
#pragma unroll
    for (int j = 0; j < kXPT; ++j) {
      const int e = base + tid + j * kMBlock;
      if (e < nxv) {
        const int b = e / (in / 8), v = e - b * (in / 8);
        *reinterpret_cast<uint4 *>(xs + b * xstride + v * 8) = xv[j];
      }
    }
  }

  // address of a codeword copy: byte 1 = the code, byte 0 = slot * 16
  const uint32_t baseA = (uint32_t)r * 16u, baseB = (uint32_t)(r ^ 8) * 16u;
  const uint32_t mA = (uint32_t)(r >> 3), mB = mA ^ 1u;
  const uint32_t selA[2] = {0x0C0C0000u | ((4u + mA) << 8), 0x0C0C0000u | ((6u + mA) << 8)};
  const uint32_t selB[2] = {0x0C0C0000u | ((4u + mB) << 8), 0x0C0C0000u | ((6u + mB) << 8)};
  // B fragments: activation row min(r, batch - 1) (columns past the batch
  // repeat the last row and are never stored)
  const uint16_t *xrow = xs + (r < batch ? r : batch - 1) * xstride + (cb * 32 + q * 8) * 8;
  publish_flag(big_flags, has_large_half(book_v));
  __syncthreads();
  // codebooks large enough for the fp16 codeword sum to overflow: halve the
  // table, double the row totals (overflow guard, aqlm_device.hpp)
  const bool halved = read_flag(big_flags, kMWaves);
  if (halved) {
    const uint4 hv = hhalf8(book_v);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<uint4 *>(table + tc * 256 + tm * 128 + ((j + tid) & 7) * 16) = hv;
    __syncthreads();
  }
  const float total_mul = halved ? 2.0f : 1.0f;

  // B fragments do not depend on the tile. In the two-chunk class a
  // wavefront's 16 fragments (64 registers) read by its first tile are kept
  // for its later ones: a four-address 16-byte LDS read costs as much LDS
  // time as a conflict-free one (about 4.3 clocks per wavefront), a third of
  // a tile's LDS reads (q,k,v call, two tiles per block, 7.9 -> 7.7 us).
  // Reading them all before the first tile instead delays that tile (o,
  // one tile per block: 4.05 -> 4.2 us).
  constexpr bool kKeepB = MAXC <= 2 && (!ALL || NBUF == 2);
  uint4 bh[kKeepB ? MAXC : 1][8];

  // bmode 0: fragments read from LDS; 1: read from LDS and kept in bh;
  // 2: taken from bh
  auto tile = [&](int i, const uint4 (&c)[MAXC], auto bmode) {
    constexpr int BM = decltype(bmode)::value;
    float4_t acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
      if (k < nw) {
        const uint32_t w[4] = {c[k].x, c[k].y, c[k].z, c[k].w};
#pragma unroll
        for (int h = 0; h < 8; h += 4) {
          uint4 a0[4], a1[4], b[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int s = h + u;
            const uint32_t addrA = __builtin_amdgcn_perm(w[s >> 1], baseA, selA[s & 1]);
            const uint32_t addrB = __builtin_amdgcn_perm(w[s >> 1], baseB, selB[s & 1]);
            a0[u] = *reinterpret_cast<const uint4 *>(table + addrA);
            a1[u] = *reinterpret_cast<const uint4 *>(table + addrB);
            if constexpr (BM == 2)
              b[u] = bh[kKeepB ? k : 0][s];
            else
              b[u] = *reinterpret_cast<const uint4 *>(xrow + (k * 32 + s) * 8);
            if constexpr (BM == 1) bh[kKeepB ? k : 0][s] = b[u];
          }
          // two accumulators so that consecutive MFMAs are independent
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const half8_t w = __builtin_bit_cast(half8_t, hadd8(a0[u], a1[u]));
            if (u & 1)
              acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(w, __builtin_bit_cast(half8_t, b[u]),
                                                            acc1, 0, 0, 0);
            else
              acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(w, __builtin_bit_cast(half8_t, b[u]),
                                                            acc0, 0, 0, 0);
          }
        }
      }
    }
    // partial sums of rows 4q .. 4q+3 for activation row r -> LDS, then the
    // first 16 * BATCH threads add the waves' parts in order
    const float4_t acc = acc0 + acc1;
    float *rb = red + (i & 1) * (kMWaves * 16 * BATCH);
    if (r < BATCH) {
#pragma unroll
      for (int e = 0; e < 4; ++e) rb[(wave * 16 + 4 * q + e) * BATCH + r] = acc[e];
    }
    __syncthreads();
    if (tid < 16 * BATCH) {
      const int row16 = tid / BATCH, b = tid - row16 * BATCH;
      float v = rb[row16 * BATCH + b];
#pragma unroll
      for (int w2 = 1; w2 < kMWaves; ++w2) v += rb[(w2 * 16 + row16) * BATCH + b];
      const int row = (blk + i * L.blk_count) * 16 + row16;
      if (row < out && b < batch)
        L.y[(int64_t)b * out + row] = (uint16_t)f2h((v * total_mul) * h2f(sc_lds[i * 16 + row16]));
    }
  };

  using keep_first = std::integral_constant<int, kKeepB ? 1 : 0>;
  using keep_rest = std::integral_constant<int, kKeepB ? 2 : 0>;
  if constexpr (ALL) {
    // my_tiles <= NBUF: every tile was loaded in the prologue
    if (my_tiles > 0) tile(0, cw[0], keep_first{});
#pragma unroll
    for (int u = 1; u < NBUF; ++u)
      if (u < my_tiles) tile(u, cw[u], keep_rest{});
  } else if (my_tiles > 0) {
    // NBUF tiles per loop pass so that every code buffer index is static;
    // each buffer is refilled with the codes NBUF tiles ahead right after its
    // tile (the first pass is peeled off: its first tile keeps the fragments)
    tile(0, cw[0], keep_first{});
    load_tile(NBUF, cw[0]);
#pragma unroll
    for (int u = 1; u < NBUF; ++u) {
      if (u < my_tiles) {
        tile(u, cw[u], keep_rest{});
        load_tile(u + NBUF, cw[u]);
      }
    }
    for (int i0 = NBUF; i0 < my_tiles; i0 += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        if (i0 + u < my_tiles) {
          tile(i0 + u, cw[u], keep_rest{});
          load_tile(i0 + u + NBUF, cw[u]);
        }
      }
    }
  }
}

template <int BATCH, int MAXC, int NBUF, bool ALL>
__global__ __launch_bounds__(kMBlock) void gemv_2x8_mfma_kernel(MfmaLayer L) {
  gemv_2x8_mfma_body<BATCH, MAXC, NBUF, ALL>(L, blockIdx.x);
}

constexpr int kMaxMfmaGroup = 16;
struct MfmaGroup {
  MfmaLayer layer[kMaxMfmaGroup];
  int n;
};

template <int BATCH, int MAXC, int NBUF, bool ALL>
__global__ __launch_bounds__(kMBlock) void gemv_2x8_mfma_group_kernel(MfmaGroup G) {
  int l = 0;
#pragma unroll 1
  for (int i = 1; i < G.n; ++i)
    if ((int)blockIdx.x >= G.layer[i].blk_begin) l = i;
  gemv_2x8_mfma_body<BATCH, MAXC, NBUF, ALL>(G.layer[l], blockIdx.x - G.layer[l].blk_begin);
}

// Raise the dynamic LDS limit of a kernel once per device.
template <typename K>
hipError_t allow_lds(K kernel, size_t bytes, std::atomic<uint64_t> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (dev < 64 && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

constexpr size_t kMaxLds = 160 * 1024;

template <int BATCH, int MAXC, int NBUF, bool ALL>
hipError_t launch_one(const MfmaLayer &L, hipStream_t stream) {
  static std::atomic<uint64_t> done{0};
  auto k = gemv_2x8_mfma_kernel<BATCH, MAXC, NBUF, ALL>;
  hipError_t e = allow_lds(k, kMaxLds - kMTable, done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(L.blk_count), dim3(kMBlock), mfma_dyn_lds_bytes(BATCH, L.in), stream,
                     L);
  return hipGetLastError();
}

template <int BATCH, int MAXC, int NBUF, bool ALL>
hipError_t launch_group(const MfmaGroup &G, int blocks, size_t lds, hipStream_t stream) {
  static std::atomic<uint64_t> done{0};
  auto k = gemv_2x8_mfma_group_kernel<BATCH, MAXC, NBUF, ALL>;
  hipError_t e = allow_lds(k, kMaxLds - kMTable, done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(blocks), dim3(kMBlock), lds - kMTable, stream, G);
  return hipGetLastError();
}

// The launches for the NBUF code that nbuf_for returns (-NBUF: ALL).
template <int BATCH, int MAXC>
hipError_t launch_one_nb(const MfmaLayer &L, int code, hipStream_t stream) {
  switch (code) {
    case -1: return launch_one<BATCH, MAXC, 1, true>(L, stream);
    case -2: if constexpr (2 * MAXC <= 16) return launch_one<BATCH, MAXC, 2, true>(L, stream); break;
    case 2: return launch_one<BATCH, MAXC, 2, false>(L, stream);
  }
  return hipErrorInvalidValue;
}

template <int BATCH, int MAXC>
hipError_t launch_group_nb(const MfmaGroup &G, int blocks, size_t lds, int code,
                           hipStream_t stream) {
  switch (code) {
    case -1: return launch_group<BATCH, MAXC, 1, true>(G, blocks, lds, stream);
    case -2:
      if constexpr (2 * MAXC <= 16) return launch_group<BATCH, MAXC, 2, true>(G, blocks, lds, stream);
      break;
    case 2: return launch_group<BATCH, MAXC, 2, false>(G, blocks, lds, stream);
  }
  return hipErrorInvalidValue;
}

// Chunk-per-wave class: MAXC >= ceil(chunks / 8).
int mfma_class(int64_t nch) {
  if (nch <= 16) return 0;   // MAXC 2
  if (nch <= 32) return 1;   // MAXC 4
  if (nch <= 64) return 2;   // MAXC 8
  if (nch <= 128) return 3;  // MAXC 16
  return -1;
}

// Tiles of codes in flight per wave: every tile of the block (ALL) when a
// block has at most two (q,k,v call 8.8 -> 8.1 us, o 4.2 -> 4.0, down
// 8.0 -> 7.6 against one tile ahead), else two, refilled after each tile
// (three-tile blocks: all three up front took the gate,up call from 10.8 to
// 11.3 us). Returns NBUF, or -NBUF for ALL.
constexpr int nbuf_for(int max_tiles_per_block, int maxc) {
  if (max_tiles_per_block <= 2 && max_tiles_per_block * maxc <= 16) return -max_tiles_per_block;
  return 2;
}

int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return cus;
}


// ---------------------------------------------------------------------------
// One activation row, rows of at most 2048 groups (in <= 16384): one output
// row per wavefront at a time.
//
// The matrix core's 16 A rows are 16 segments of ONE output row. In step t
// (t = 0..7) lane L = 16 q + r feeds group g(L, t) = 8 r + 128 q + t of the
// row: the fp16 sum of the group's two codewords as its A operand and the
// group's 8 activations as its B operand (row r of A, column r of B). The
// result's diagonal element D[r][r] then collects the products of exactly
// the groups of segment r, and the row's total is the sum of the diagonal;
// over the 8 steps and 64 lanes every group of the row is taken once
// (8 r + t runs over 0..127, 128 q over the four quarters). Against the tile
// form above:
//   * a lane's codes for the whole row are one 16-byte load (groups 8 r +
//     128 q .. + 7, at byte 16 r + 256 q), so the wavefront's 64 loads are
//     the row's 1 KiB in order, whole cache lines (the tile form reads 64
//     bytes of each of 16 rows per load instruction, which costs the
//     texture-address unit about three times as long per instruction, and
//     every wavefront of a CU issues its code loads at once at the start);
//   * a lane's activation fragments do not depend on the row: its 8
//     fragments (32 registers) are read from LDS once and serve every row,
//     so a row costs two 16-byte LDS reads per step instead of three;
//   * a row needs no other wavefront: no partial sums in LDS and no barrier
//     after the prologue. The diagonal is gathered by quad broadcasts (the
//     four diagonal elements of a quad sit in its four lanes) and the four
//     diagonal quads are added in a fixed order, so a row's result does not
//     depend on which wavefront or workgroup computes it.
// The staged activations keep 16 bytes of padding after every 8 groups, so
// the 16 lanes of a 16-byte LDS pass (consecutive r) hit distinct banks.
constexpr int kRThreads = 1024;
constexpr int kRWaves = kRThreads / 64;
constexpr int kRGroups = 512;                   // groups of one pass over a row
constexpr int kRMaxPasses = 4;                  // rows of up to 2048 groups (in <= 16384)
constexpr int kRXBytes = kRGroups / 8 * 144;    // staged activations of one pass, with padding

__device__ __forceinline__ uint32_t rows_x_off(uint32_t g) { return g * 16u + (g >> 3) * 16u; }

// An LDS word read as one value for the whole wavefront.
__device__ __forceinline__ uint32_t lds_read_word(uint32_t *w) {
  return __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}
// Waits until an LDS counter of the workgroup reaches n. The wait is bounded
// (about 0.1 s) so that a kernel always ends; the counters it serves reach n
// within microseconds, because every wavefront adds its count unconditionally.
// LDS operations that follow in program order are issued after it returns.
__device__ __forceinline__ void lds_wait_count(uint32_t *w, uint32_t n) {
#pragma unroll 1
  for (int i = 0; i < (1 << 22); ++i) {
    if (lds_read_word(w) >= n) break;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}

struct RowsLayer {
  const uint8_t *codes;
  const uint16_t *books;
  const uint16_t *scales;
  const uint16_t *x;
  uint16_t *y;
  int out, groups;
  int blk_begin, blk_count;  // blocks [blk_begin, blk_begin + blk_count) serve this layer
};

struct RowsGroup {
  RowsLayer layer[kMaxMfmaGroup];
  int n;
};

// RD: rows of codes in flight per wavefront; NP: passes of 512 groups per
// row (a row of more than 512 groups is taken pass by pass, each pass as
// above; the activation fragments of a lane are then read from LDS in every
// step rather than kept, since NP x 32 registers would not fit).
template <int RD, int NP>
__global__ __launch_bounds__(kRThreads) void gemv_2x8_rows_kernel(RowsGroup G) {
  __shared__ __attribute__((aligned(16))) uint8_t table[kMTable];
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t *xs = lds;
  // hand-over words: [0] the overflow guard (set if any codebook entry has a
  // large half), [1] table-building wavefronts that have published their
  // part of it, [2] wavefronts whose LDS writes are done
  uint32_t *sy = reinterpret_cast<uint32_t *>(lds + NP * kRXBytes);
  if (threadIdx.x < 3) sy[threadIdx.x] = 0u;
  // the wavefronts of a workgroup start together: this barrier is short, and
  // it is the only one
  __syncthreads();

  int l = 0;
#pragma unroll 1
  for (int i = 1; i < G.n; ++i)
    if ((int)blockIdx.x >= G.layer[i].blk_begin) l = i;
  const RowsLayer &L = G.layer[l];
  const int blk = (int)blockIdx.x - L.blk_begin;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const uint32_t row_bytes = (uint32_t)L.groups * 2u;
  // this workgroup's rows [r0, r1); wavefront w takes r0 + w, r0 + w + 16, ...
  const int r0 = (int)((int64_t)L.out * blk / L.blk_count);
  const int r1 = (int)((int64_t)L.out * (blk + 1) / L.blk_count);
  const int nrows = r1 > r0 + wave ? (r1 - r0 - wave + kRWaves - 1) / kRWaves : 0;

  // Prologue. Wavefronts 0..7 build the codebook table and stage the
  // activations; 8..15 write nothing to LDS. A wavefront stalls at a vector
  // load until the texture-address unit accepts it, and a CU's code loads
  // keep that unit busy for a microsecond or more, so the builders queue
  // their codes only after their LDS writes, while the others queue theirs at
  // once. There is no barrier: each wavefront counts itself done in LDS (after
  // its LDS writes, if any) and waits for all sixteen counts before its first
  // table read.
  const bool builder = wave < 8;
  const int tm = (tid >> 3) & 1;                  // table entry: codebook tm,
  const int tc = (tid & 7) | ((tid >> 4) << 3);   // code value tc (builders)
  const Rsrc rc = make_rsrc(L.codes, (uint32_t)L.out * row_bytes);
  const Rsrc rs = make_rsrc(L.scales, (uint32_t)L.out * 2u);
  const uint32_t lane_g = (uint32_t)(8 * r + 128 * q);  // the first of the lane's 8 groups in a pass
  if (builder) {
    // activation vectors (one group's 8 values each): groups tid + 512 i,
    // zero past the row's groups
    const Rsrc rx = make_rsrc(L.x, (uint32_t)L.groups * 16u);
    const uint4 book_v = reinterpret_cast<const uint4 *>(L.books)[tm * 256 + tc];
    uint4 xv[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) xv[i] = buf_load16(rx, (uint32_t)(tid + i * 512) * 16u);
    // the overflow guard is known once all eight builders have published
    const bool big = __ballot(has_large_half(book_v)) != 0;
    if (lane == 0) {
      if (big) __hip_atomic_fetch_or(&sy[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      asm volatile("" ::: "memory");
      __hip_atomic_fetch_add(&sy[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    lds_wait_count(&sy[1], 8u);
    // codebooks large enough for the fp16 codeword sum to overflow: a halved
    // table, doubled row totals (overflow guard, aqlm_device.hpp)
    const uint4 tv = lds_read_word(&sy[0]) != 0u ? hhalf8(book_v) : book_v;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<uint4 *>(table + tc * 256 + tm * 128 + ((j + tid) & 7) * 16) = tv;
#pragma unroll
    for (int i = 0; i < NP; ++i)
      *reinterpret_cast<uint4 *>(xs + rows_x_off((uint32_t)(tid + i * 512))) = xv[i];
  }
  // LDS operations of a wavefront complete in order: the count follows its writes
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane == 0) __hip_atomic_fetch_add(&sy[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);

  uint4 cw[RD][NP];
  uint32_t sv[RD];
  auto load_row = [&](int k, uint4 (&c)[NP], uint32_t &sc) {
    const bool ok = k < nrows;
    const uint32_t row = (uint32_t)(r0 + wave + k * kRWaves);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t g = lane_g + (uint32_t)(p * kRGroups);
      // groups is a multiple of 8: a lane's 8 groups are all in the row or all past it
      c[p] = buf_load16_nt(rc, (ok && g < (uint32_t)L.groups) ? row * row_bytes + g * 2u : kMOOB);
    }
    sc = buf_load_u16(rs, ok ? row * 2u : kMOOB);
  };
#pragma unroll
  for (int u = 0; u < RD; ++u) load_row(u, cw[u], sv[u]);
  lds_wait_count(&sy[2], (uint32_t)kRWaves);
  const bool halved = lds_read_word(&sy[0]) != 0u;
  const float total_mul = halved ? 2.0f : 1.0f;

  // this lane's activation fragments, the same for every row (kept in
  // registers for one-pass rows)
  uint4 b[NP == 1 ? 8 : 1];
  if constexpr (NP == 1) {
#pragma unroll
    for (int t = 0; t < 8; ++t) b[t] = *reinterpret_cast<const uint4 *>(xs + rows_x_off(lane_g + t));
  }

  const uint32_t baseA = (uint32_t)r * 16u, baseB = (uint32_t)(r ^ 8) * 16u;
  const uint32_t mA = (uint32_t)(r >> 3), mB = mA ^ 1u;
  const uint32_t selA[2] = {0x0C0C0000u | ((4u + mA) << 8), 0x0C0C0000u | ((6u + mA) << 8)};
  const uint32_t selB[2] = {0x0C0C0000u | ((4u + mB) << 8), 0x0C0C0000u | ((6u + mB) << 8)};
  const bool diag_quad = ((lane >> 2) >> 2) == ((lane >> 2) & 3);

  // The row's total (in lane 63): 8 steps, two accumulators so that
  // consecutive MFMAs are independent, then the diagonal.
  auto row_total = [&](const uint4 (&c)[NP]) {
    float4_t acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t w[4] = {c[p].x, c[p].y, c[p].z, c[p].w};
#pragma unroll
      for (int h = 0; h < 8; h += 4) {
        uint4 a0[4], a1[4], bb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int s = h + u;
          const uint32_t addrA = __builtin_amdgcn_perm(w[s >> 1], baseA, selA[s & 1]);
          const uint32_t addrB = __builtin_amdgcn_perm(w[s >> 1], baseB, selB[s & 1]);
          a0[u] = *reinterpret_cast<const uint4 *>(table + addrA);
          a1[u] = *reinterpret_cast<const uint4 *>(table + addrB);
          if constexpr (NP == 1)
            bb[u] = b[s];
          else
            bb[u] = *reinterpret_cast<const uint4 *>(
                xs + rows_x_off(lane_g + (uint32_t)(p * kRGroups + s)));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const half8_t wv = __builtin_bit_cast(half8_t, hadd8(a0[u], a1[u]));
          if (u & 1)
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, __builtin_bit_cast(half8_t, bb[u]),
                                                          acc1, 0, 0, 0);
          else
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, __builtin_bit_cast(half8_t, bb[u]),
                                                          acc0, 0, 0, 0);
        }
        // keep each half-pass's LDS reads next to its MFMAs (hoisting the
        // reads of later passes costs registers and spills)
        if constexpr (NP > 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
    const float4_t acc = acc0 + acc1;
    // lane 4 j + e of a diagonal quad j holds D[4 k + e][4 k + e] (k = j / 5)
    // in element e
    float v = dpp<kDppQuadBcast0>(acc[0]) + dpp<kDppQuadBcast1>(acc[1]);
    v += dpp<kDppQuadBcast2>(acc[2]);
    v += dpp<kDppQuadBcast3>(acc[3]);
    return quads_sum_to_lane63(diag_quad ? v : 0.0f);
  };

  // rows k, k + 1, ...: row k's codes are in ring slot k % RD, refilled with
  // row k + RD once its total is taken. Every slot issues the same vector
  // memory operations whether or not its row exists (loads past the
  // wavefront's rows and the result store of every lane but 63 fall out of
  // range), so the compiler can count them exactly and a row waits only for
  // its own codes, not for the whole ring.
  const Rsrc ry = make_rsrc(L.y, (uint32_t)L.out * 2u);
  for (int k0 = 0; k0 < nrows; k0 += RD) {
#pragma unroll
    for (int u = 0; u < RD; ++u) {
      const int k = k0 + u;
      float v = 0.0f;
      if (k < nrows) v = row_total(cw[u]);
      const uint32_t sc = sv[u];
      load_row(k + RD, cw[u], sv[u]);
      const uint32_t row = (uint32_t)(r0 + wave + k * kRWaves);
      buf_store_u16(ry, (lane == 63 && k < nrows) ? row * 2u : kMOOB,
                    (uint16_t)f2h((v * total_mul) * h2f(sc)));
    }
  }
}

template <int RD, int NP>
hipError_t launch_rows(const RowsGroup &G, int blocks, hipStream_t stream) {
  static std::atomic<uint64_t> done{0};
  auto k = gemv_2x8_rows_kernel<RD, NP>;
  constexpr size_t dyn = NP * kRXBytes + kRWaves * 4;
  hipError_t e = allow_lds(k, kMaxLds - kMTable, done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(blocks), dim3(kRThreads), dyn, stream, G);
  return hipGetLastError();
}

// The layers (all accepted by gemv_2x8_rows_fits, all with the same number of
// 512-group passes), one launch: workgroups
// split over the layers in proportion to their rows, one workgroup per CU
// in all, at most one per 16 rows.
hipError_t launch_rows_group(const LayerDesc *const *Ls, const uint16_t *const *xs,
                             uint16_t *const *ys, int n, hipStream_t stream) {
  RowsGroup G;
  G.n = n;
  const int cus = device_cus();
  double total = 0;
  for (int i = 0; i < n; ++i) total += (double)Ls[i]->out;
  int begin = 0, max_rpw = 1;
  for (int i = 0; i < n; ++i) {
    const LayerDesc &L = *Ls[i];
    const int most = (int)((L.out + kRWaves - 1) / kRWaves);
    int blocks = (int)((double)cus * (double)L.out / total + 0.5);
    if (blocks > most) blocks = most;
    if (blocks < 1) blocks = 1;
    // rows per wavefront: the longest share of any workgroup of this layer
    const int rows_per_block = (int)((L.out + blocks - 1) / blocks);
    const int rpw = (rows_per_block + kRWaves - 1) / kRWaves;
    if (rpw > max_rpw) max_rpw = rpw;
    G.layer[i] = RowsLayer{static_cast<const uint8_t *>(L.codes), L.books, L.scales, xs[i], ys[i],
                           (int)L.out, (int)L.groups, begin, blocks};
    begin += blocks;
  }
  // every layer of the launch has the same pass count
  switch ((int)((Ls[0]->groups + kRGroups - 1) / kRGroups)) {
    case 1:
      if (max_rpw <= 1) return launch_rows<1, 1>(G, begin, stream);
      if (max_rpw <= 2) return launch_rows<2, 1>(G, begin, stream);
      if (max_rpw <= 3) return launch_rows<3, 1>(G, begin, stream);
      // five or six rows per wavefront: all of them in flight (gate,up call
      // 10.65-11.10 -> 10.46-10.57 us against four); more rows stream
      // through a ring of four (eight in flight made the ten-row
      // whole-block call slower, 23.7-24.2 -> 25.2-25.8 us)
      if (max_rpw == 5 || max_rpw == 6) return launch_rows<6, 1>(G, begin, stream);
      return launch_rows<4, 1>(G, begin, stream);
    case 2: return launch_rows<1, 2>(G, begin, stream);
    case 3: return launch_rows<1, 3>(G, begin, stream);
    case 4: return launch_rows<1, 4>(G, begin, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// True when the one-row-per-wavefront form serves this layer: one
// activation row, rows of at most 2048 groups in whole 8-group lane pieces,
// 32-bit byte offsets.
bool gemv_2x8_rows_fits(const LayerDesc &L, int batch) {
  if (L.scheme != Scheme::k2x8 || batch != 1) return false;
  if (L.groups % 8 != 0 || L.groups > kRMaxPasses * kRGroups) return false;
  return (L.out + 1) * L.groups * 2 < ((int64_t)1 << 31);
}

// True when the matrix-core GEMV serves this layer and batch.
bool gemv_2x8_mfma_fits(const LayerDesc &L, int batch) {
  if (L.scheme != Scheme::k2x8 || batch < 1 || batch > 8) return false;
  if (gemv_2x8_rows_fits(L, batch)) return true;
  if (L.groups % 32 != 0 || mfma_class(L.groups / 32) < 0) return false;
  const int rows = batch <= 1 ? 1 : (batch <= 2 ? 2 : (batch <= 4 ? 4 : 8));
  if (mfma_lds_bytes(rows, (int)L.in) > kMaxLds) return false;
  // 32-bit byte offsets, including 16 rows past the end
  return (L.out + 16) * L.groups * 2 < ((int64_t)1 << 31);
}

namespace {

template <int BATCH>
hipError_t launch_mfma_batch(const LayerDesc &L, const uint16_t *x, int batch, uint16_t *y,
                             hipStream_t stream) {
  const int ntiles = (int)((L.out + 15) / 16);
  const size_t lds = mfma_lds_bytes(BATCH, (int)L.in);
  const int cus = device_cus();
  // as many blocks as fit on the chip at once
  int blocks = lds <= kMaxLds / 2 ? 2 * cus : cus;
  if (blocks > ntiles) blocks = ntiles;
  const int min_blocks = (ntiles + kMaxTilesPerBlock - 1) / kMaxTilesPerBlock;
  if (blocks < min_blocks) blocks = min_blocks;
  MfmaLayer M{static_cast<const uint8_t *>(L.codes), L.books, L.scales, x, y, (int)L.out, (int)L.in,
              (int)L.groups, batch, 0, blocks};
  const int per_block = (ntiles + blocks - 1) / blocks;
  switch (mfma_class(L.groups / 32)) {
    case 0: return launch_one_nb<BATCH, 2>(M, nbuf_for(per_block, 2), stream);
    case 1: return launch_one_nb<BATCH, 4>(M, nbuf_for(per_block, 4), stream);
    case 2: return launch_one_nb<BATCH, 8>(M, nbuf_for(per_block, 8), stream);
    case 3: return launch_one_nb<BATCH, 16>(M, nbuf_for(per_block, 16), stream);
  }
  return hipErrorInvalidValue;
}

// Several layers in one launch, one class (chunks per wave) at a time: blocks
// are split over the layers in proportion to their code bytes, at least one
// tile per block and at most kMaxTilesPerBlock tiles per block.
template <int BATCH, int MAXC>
hipError_t launch_mfma_group(const LayerDesc *const *Ls, const uint16_t *const *xs,
                             uint16_t *const *ys, int n, int batch, hipStream_t stream) {
  MfmaGroup G;
  G.n = n;
  size_t lds = 0;
  for (int i = 0; i < n; ++i) {
    const size_t b = mfma_lds_bytes(BATCH, (int)Ls[i]->in);
    if (b > lds) lds = b;
  }
  const int cus = device_cus();
  const int budget = lds <= kMaxLds / 2 ? 2 * cus : cus;
  // tiles per block from the layers' total work (one tile costs the same in
  // every layer of a class up to its chunk count), the same for all layers
  double tile_work = 0;
  for (int i = 0; i < n; ++i) tile_work += (double)((Ls[i]->out + 15) / 16) * (double)Ls[i]->groups;
  int begin = 0, max_per_block = 1;
  for (int i = 0; i < n; ++i) {
    const LayerDesc &L = *Ls[i];
    const int ntiles = (int)((L.out + 15) / 16);
    // this layer's share of the budget, then an even split of its tiles
    const double share = budget * ((double)ntiles * (double)L.groups) / tile_work;
    int per_block = (int)((ntiles + share - 1) / (share > 1 ? share : 1));
    if (per_block < 1) per_block = 1;
    if (per_block > kMaxTilesPerBlock) per_block = kMaxTilesPerBlock;
    const int blocks = (ntiles + per_block - 1) / per_block;
    if (per_block > max_per_block) max_per_block = per_block;
    G.layer[i] = MfmaLayer{static_cast<const uint8_t *>(L.codes), L.books, L.scales, xs[i], ys[i],
                           (int)L.out, (int)L.in, (int)L.groups, batch, begin, blocks};
    begin += blocks;
  }
  return launch_group_nb<BATCH, MAXC>(G, begin, lds, nbuf_for(max_per_block, MAXC), stream);
}

template <int BATCH>
hipError_t mfma_group_batch(const LayerDesc *const *Ls, const uint16_t *const *xs,
                            uint16_t *const *ys, int n, int batch, int cls, hipStream_t stream) {
  switch (cls) {
    case 0: return launch_mfma_group<BATCH, 2>(Ls, xs, ys, n, batch, stream);
    case 1: return launch_mfma_group<BATCH, 4>(Ls, xs, ys, n, batch, stream);
    case 2: return launch_mfma_group<BATCH, 8>(Ls, xs, ys, n, batch, stream);
    case 3: return launch_mfma_group<BATCH, 16>(Ls, xs, ys, n, batch, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Grouped launches of the layers that gemv_2x8_mfma_fits accepts; marks them
// in `done` and leaves the others to the caller.
hipError_t launch_gemv_2x8_mfma_batched(const LayerDesc *Ls, const uint16_t *const *xs,
                                        uint16_t *const *ys, int n, int batch, bool *done,
                                        hipStream_t stream) {
  {
    // one activation row, rows of at most 2048 groups: the one-row-per-wavefront
    // form, one launch per pass count
    const LayerDesc *sel[kMaxMfmaGroup];
    const uint16_t *sx[kMaxMfmaGroup];
    uint16_t *sy[kMaxMfmaGroup];
    int m = 0;
    for (int np = 1; np <= kRMaxPasses; ++np)
    for (int i = 0; i <= n; ++i) {
      const bool take = i < n && !done[i] && gemv_2x8_rows_fits(Ls[i], batch) &&
                        (Ls[i].groups + kRGroups - 1) / kRGroups == np;
      if (take) {
        sel[m] = &Ls[i];
        sx[m] = xs[i];
        sy[m] = ys[i];
        ++m;
        done[i] = true;
      }
      if (m == kMaxMfmaGroup || (i == n && m > 0)) {
        const hipError_t e = launch_rows_group(sel, sx, sy, m, stream);
        if (e != hipSuccess) return e;
        m = 0;
      }
    }
  }
  for (int cls = 0; cls < 4; ++cls) {
    const LayerDesc *sel[kMaxMfmaGroup];
    const uint16_t *sx[kMaxMfmaGroup];
    uint16_t *sy[kMaxMfmaGroup];
    int m = 0;
    for (int i = 0; i <= n; ++i) {
      const bool take = i < n && !done[i] && gemv_2x8_mfma_fits(Ls[i], batch) &&
                        mfma_class(Ls[i].groups / 32) == cls;
      if (take) {
        sel[m] = &Ls[i];
        sx[m] = xs[i];
        sy[m] = ys[i];
        ++m;
        done[i] = true;
      }
      if (m == kMaxMfmaGroup || (i == n && m > 0)) {
        hipError_t e = batch <= 1   ? mfma_group_batch<1>(sel, sx, sy, m, batch, cls, stream)
                       : batch <= 2 ? mfma_group_batch<2>(sel, sx, sy, m, batch, cls, stream)
                       : batch <= 4 ? mfma_group_batch<4>(sel, sx, sy, m, batch, cls, stream)
                                    : mfma_group_batch<8>(sel, sx, sy, m, batch, cls, stream);
        if (e != hipSuccess) return e;
        m = 0;
      }
    }
  }
  return hipSuccess;
}

hipError_t launch_gemv_2x8_mfma(const LayerDesc &L, const uint16_t *x, int batch, uint16_t *y,
                                hipStream_t stream) {
  if (gemv_2x8_rows_fits(L, batch)) {
    const LayerDesc *ls[1] = {&L};
    const uint16_t *xs[1] = {x};
    uint16_t *ys[1] = {y};
    return launch_rows_group(ls, xs, ys, 1, stream);
  }
  if (batch <= 1) return launch_mfma_batch<1>(L, x, batch, y, stream);
  if (batch <= 2) return launch_mfma_batch<2>(L, x, batch, y, stream);
  if (batch <= 4) return launch_mfma_batch<4>(L, x, batch, y, stream);
  return launch_mfma_batch<8>(L, x, batch, y, stream);
}

}  // namespace aqlm
