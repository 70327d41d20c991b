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
//     NBUF is 1 when no block has more than two tiles: a prefetch past the
//     last tile is a load with an out-of-range offset, which returns zero but
//     still occupies the texture-address unit that the real loads of every
//     wave on the CU queue behind.
#include "aqlm_device.hpp"

#include <atomic>

namespace aqlm {
namespace {

constexpr int kMBlock = 512;
constexpr int kMWaves = kMBlock / 64;
constexpr int kMTable = 65536;
constexpr int kMaxTilesPerBlock = 64;  // row scales of a block's tiles are staged in LDS
constexpr uint32_t kMOOB = 0x80000000u;

// LDS: the 64 KiB table is a static array (its addresses then fold into the
// read instructions); the dynamic part holds the activations (BATCH rows of
// in + 8 halves), the row scales and the reduction buffers (two of waves x 16
// rows x BATCH floats).
constexpr size_t mfma_dyn_lds_bytes(int batch, int in) {
  return (size_t)batch * (in + 8) * 2 + kMaxTilesPerBlock * 16 * 2 + 2 * kMWaves * 16 * batch * 4;
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

template <int BATCH, int MAXC, int NBUF>
__device__ __forceinline__ void gemv_2x8_mfma_body(const MfmaLayer &L, int blk) {
  __shared__ __attribute__((aligned(16))) uint8_t table[kMTable];
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int xstride = L.in + 8;  // halves per staged activation row
  uint16_t *xs = reinterpret_cast<uint16_t *>(lds);
  uint16_t *sc_lds = xs + BATCH * xstride;
  float *red = reinterpret_cast<float *>(sc_lds + kMaxTilesPerBlock * 16);

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
  __syncthreads();

  auto tile = [&](int i, const uint4 (&c)[MAXC]) {
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
            b[u] = *reinterpret_cast<const uint4 *>(xrow + (k * 32 + s) * 8);
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
        L.y[(int64_t)b * out + row] = (uint16_t)f2h(v * h2f(sc_lds[i * 16 + row16]));
    }
  };

  // NBUF tiles per loop pass so that every code buffer index is static; each
  // buffer is refilled with the codes NBUF tiles ahead right after its tile.
  for (int i0 = 0; i0 < my_tiles; i0 += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      if (i0 + u < my_tiles) {
        tile(i0 + u, cw[u]);
        load_tile(i0 + u + NBUF, cw[u]);
      }
    }
  }
}

template <int BATCH, int MAXC, int NBUF>
__global__ __launch_bounds__(kMBlock) void gemv_2x8_mfma_kernel(MfmaLayer L) {
  gemv_2x8_mfma_body<BATCH, MAXC, NBUF>(L, blockIdx.x);
}

constexpr int kMaxMfmaGroup = 16;
struct MfmaGroup {
  MfmaLayer layer[kMaxMfmaGroup];
  int n;
};

template <int BATCH, int MAXC, int NBUF>
__global__ __launch_bounds__(kMBlock) void gemv_2x8_mfma_group_kernel(MfmaGroup G) {
  int l = 0;
#pragma unroll 1
  for (int i = 1; i < G.n; ++i)
    if ((int)blockIdx.x >= G.layer[i].blk_begin) l = i;
  gemv_2x8_mfma_body<BATCH, MAXC, NBUF>(G.layer[l], blockIdx.x - G.layer[l].blk_begin);
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

template <int BATCH, int MAXC, int NBUF>
hipError_t launch_one(const MfmaLayer &L, hipStream_t stream) {
  static std::atomic<uint64_t> done{0};
  auto k = gemv_2x8_mfma_kernel<BATCH, MAXC, NBUF>;
  hipError_t e = allow_lds(k, kMaxLds - kMTable, done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(L.blk_count), dim3(kMBlock), mfma_dyn_lds_bytes(BATCH, L.in), stream,
                     L);
  return hipGetLastError();
}

template <int BATCH, int MAXC, int NBUF>
hipError_t launch_group(const MfmaGroup &G, int blocks, size_t lds, hipStream_t stream) {
  static std::atomic<uint64_t> done{0};
  auto k = gemv_2x8_mfma_group_kernel<BATCH, MAXC, NBUF>;
  hipError_t e = allow_lds(k, kMaxLds - kMTable, done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(blocks), dim3(kMBlock), lds - kMTable, stream, G);
  return hipGetLastError();
}

// Chunk-per-wave class: MAXC >= ceil(chunks / 8).
int mfma_class(int64_t nch) {
  if (nch <= 16) return 0;   // MAXC 2
  if (nch <= 32) return 1;   // MAXC 4
  if (nch <= 64) return 2;   // MAXC 8
  if (nch <= 128) return 3;  // MAXC 16
  return -1;
}

// Tiles of codes in flight per wave: one when no block has more than two
// tiles (a deeper prefetch would only issue out-of-range loads), else two.
constexpr int nbuf_for(int max_tiles_per_block) { return max_tiles_per_block <= 2 ? 1 : 2; }

int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return cus;
}

}  // namespace

// True when the matrix-core GEMV serves this layer and batch.
bool gemv_2x8_mfma_fits(const LayerDesc &L, int batch) {
  if (L.scheme != Scheme::k2x8 || batch < 1 || batch > 8) return false;
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
  const bool deep = nbuf_for((ntiles + blocks - 1) / blocks) == 2;
  switch (mfma_class(L.groups / 32)) {
    case 0: return deep ? launch_one<BATCH, 2, 2>(M, stream) : launch_one<BATCH, 2, 1>(M, stream);
    case 1: return deep ? launch_one<BATCH, 4, 2>(M, stream) : launch_one<BATCH, 4, 1>(M, stream);
    case 2: return deep ? launch_one<BATCH, 8, 2>(M, stream) : launch_one<BATCH, 8, 1>(M, stream);
    case 3: return deep ? launch_one<BATCH, 16, 2>(M, stream) : launch_one<BATCH, 16, 1>(M, stream);
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
  return nbuf_for(max_per_block) == 2 ? launch_group<BATCH, MAXC, 2>(G, begin, lds, stream)
                                      : launch_group<BATCH, MAXC, 1>(G, begin, lds, stream);
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
  if (batch <= 1) return launch_mfma_batch<1>(L, x, batch, y, stream);
  if (batch <= 2) return launch_mfma_batch<2>(L, x, batch, y, stream);
  if (batch <= 4) return launch_mfma_batch<4>(L, x, batch, y, stream);
  return launch_mfma_batch<8>(L, x, batch, y, stream);
}

}  // namespace aqlm
