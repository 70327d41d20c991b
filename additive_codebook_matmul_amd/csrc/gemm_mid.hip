// Batched product y = x . W^T for any number of activation rows with a caller-owned
// device workspace (aqlm_gemm_ws). The weights are decoded on chip straight
// into the A operand of v_mfma_f32_16x16x32_f16 (float32 accumulation) and
// are never written to memory.
//
// Why a workspace. In the MFMA operand layout a lane holds 16 bytes of one
// activation row, and the 16 lanes that hold one k-slice hold 16 different
// rows. Loaded straight from x [batch][in], every lane of a wavefront touches
// its own cache line and the vector L1 serves about one lane per clock. The
// first launch (gemm_xblock_kernel) therefore re-lays x into k-blocks of 8
// inputs, one slab per block of BP = 16 NT activation rows,
//   xb[tb][kb][t][0..7] = x[tb BP + t][8 kb .. 8 kb + 7]    (zero past batch),
// after which the B operand of one MFMA step for 16 activation rows is one
// contiguous 256-byte run, and the k-block stride is a compile-time constant.
// The workspace also holds the float32 partial tiles of the split-K form
// below. With one activation tile (NT = 1, up to 16 rows) there is no
// re-layout: a lane's 16-byte pieces of its activation row stay in one
// 128-byte line for the steps that use them, so the B operands are loaded
// from x in place, and with K unsplit the form needs no workspace at all.
//
// Tiles. A workgroup of four wavefronts owns RT (2, 3 or 4) tiles of 16
// output rows and all BP activation rows (NT tiles of 16): each decoded A
// operand feeds NT MFMAs and each B operand RT MFMAs. K is walked in
// super-chunks of 32 groups (256 inputs for g = 8, 512 for g = 16). Within a
// super-chunk, lane quarter q owns groups 8q .. 8q+7 -- one 16-byte load of
// codes per row tile -- and in MFMA step s it feeds k-block g q + s of the
// super-chunk, in A and in B alike, so the sum is unchanged. (1x16 g16 pairs
// the quarters instead: 2p and 2p + 1 take the two halves of group 16p + s
// in step s; see PAIR below.) The four wavefronts take every fourth
// super-chunk of the workgroup's K range and add their float32 partial tiles
// in LDS in wavefront order at the end.
//
// Split-K. When the row blocks alone are too few to fill the chip, the K
// range is cut into `splits` parts (workgroup = row block * splits + part).
// Every workgroup then writes its float32 partial tile to the workspace and a
// third launch (gemm_mid_reduce_kernel) adds the parts of each output in part
// order, scales and writes y: deterministic, and free of cross-workgroup
// synchronisation (a device-scope release inside the kernel would write back
// the whole L2 of the XCD once per workgroup). Workgroups are dispatched to
// the XCDs in turn, so with splits dividing 8 the parts of one block of
// activation rows land on fixed XCDs and each XCD's L2 holds only its share
// of xb.
//
// Pipelining: codes one super-chunk ahead; B operands (and the 1x16 codewords,
// gathered from the L2-resident codebook) D steps ahead in register rings; the
// 2x8 A operands one step ahead from LDS. Every load of codes and activations
// is an unconditional buffer load whose out-of-range offsets read zero
// (codeword 0 times zero activations adds 0).
//
// 2x8 codebooks in LDS: a 64 KiB bank-spread table. The 256-byte stripe of
// code value c holds eight 16-byte copies of C_0[c] (slots 0..7) and eight of
// C_1[c] (slots 8..15); lane r of a 16-lane LDS pass reads slot r first
// (codebook r / 8) and slot r ^ 8 second, so every pass touches all 64 banks
// once whatever the codes. The fp16 sum does not depend on the order of its
// two terms. After the K loop the same LDS holds the partial tiles.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "aqlm_device.hpp"

namespace aqlm {
namespace {

constexpr int kMidWaves = 4;
constexpr int kMidThreads = 64 * kMidWaves;
constexpr int kGroupsPerSc = 32;  // groups per super-chunk
constexpr uint32_t kMidOOB = 0x80000000u;
constexpr int64_t kMidMinBatch = 1;
constexpr int64_t kMidMaxBatch = 4096;
constexpr int kMidCus = 256;
constexpr int kMidOccupancy = 1;  // wavefronts per SIMD the kernel is built for
constexpr int kMidMaxTiles = 32;  // largest RT * NT (accumulator tiles per wavefront)

template <Scheme S>
struct MidCfg {
  static constexpr int G = group_size(S);
  static constexpr int STEPS = G;          // MFMA steps per super-chunk
  static constexpr int SC_BLOCKS = 4 * G;  // k-blocks of 8 inputs per super-chunk
};

// B-ring depth: enough steps ahead to cover ~1000 clocks of MFMA work.
constexpr int ring_depth(int rt, int nt) { return rt * nt >= 16 ? 2 : rt * nt >= 8 ? 4 : 8; }

// LDS: the 2x8 table (reused for the partial tiles after the K loop), then
// the row scales, then one overflow-guard flag per wavefront
constexpr size_t mid_red_bytes(int rt, int nt) { return (size_t)kMidWaves * rt * nt * 1024; }
constexpr size_t mid_lds_bytes(bool lut, int rt, int nt) {
  return ((lut && mid_red_bytes(rt, nt) < 65536) ? 65536 : mid_red_bytes(rt, nt)) + 64 * 4 +
         kMidWaves * 4;
}

// Code of step s (a compile-time constant) from a lane's 16 code bytes: g = 8
// steps walk the 8 groups, g = 16 steps take each group twice.
template <int G>
__device__ __forceinline__ uint32_t code_of(const uint4 &cw, int s) {
  const int gi = G == 8 ? s : s >> 1;
  const int d = gi >> 1;
  const uint32_t word = d == 0 ? cw.x : d == 1 ? cw.y : d == 2 ? cw.z : cw.w;
  return (gi & 1) ? word >> 16 : word & 0xFFFFu;
}

__global__ __launch_bounds__(256) void gemm_xblock_kernel(const uint4 *__restrict__ x,
                                                          uint4 *__restrict__ xb, int nkb,
                                                          int batch, int bp_block) {
  // 16 activation rows x 16 k-blocks through LDS: rows are read and k-blocks
  // written as 256-byte runs (the +1 column keeps the transposed read free of
  // bank conflicts)
  __shared__ uint4 tile[16][17];
  const int i = threadIdx.x;
  const int kb0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
  {
    const int t = t0 + (i >> 4), kb = kb0 + (i & 15);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (t < batch && kb < nkb) v = x[(size_t)t * nkb + kb];
    tile[i >> 4][i & 15] = v;
  }
  __syncthreads();
  {
    // t0 and bp_block are multiples of 16: the 16 rows share one slab
    const int tb = t0 / bp_block, t = t0 - tb * bp_block + (i & 15);
    const int kb = kb0 + (i >> 4);
    if (kb < nkb) xb[((size_t)tb * nkb + kb) * bp_block + t] = tile[i & 15][i >> 4];
  }
}

// Output element e of row block rb: accumulator (t, j) = e / 64 of the
// 16 x 16 tiles, lane e % 64 (rows 4 (lane / 16) .. + 3, activation row lane % 16).
template <int NT>
__device__ __forceinline__ void store_out(uint16_t *__restrict__ y,
                                          const uint16_t *__restrict__ scales, int out, int batch,
                                          int row0, int e, float4_t v) {
  const int tj = e >> 6, l = e & 63;
  const int t = tj / NT, j = tj - t * NT;
  const int tok = j * 16 + (l & 15);
  if (tok >= batch) return;
  const int row = row0 + t * 16 + 4 * (l >> 4);
  uint16_t *dst = y + (int64_t)tok * out + row;
  if ((out & 3) == 0 && row + 3 < out) {
    const uint32_t h0 = f2h(v[0] * h2f(scales[row])) | (f2h(v[1] * h2f(scales[row + 1])) << 16);
    const uint32_t h1 = f2h(v[2] * h2f(scales[row + 2])) | (f2h(v[3] * h2f(scales[row + 3])) << 16);
    *reinterpret_cast<uint2 *>(dst) = make_uint2(h0, h1);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (row + k < out) dst[k] = (uint16_t)f2h(v[k] * h2f(scales[row + k]));
  }
}

// Split-K epilogue: the parts of each element added in part order.
template <int RT, int NT>
__global__ __launch_bounds__(256) void gemm_mid_reduce_kernel(const float4_t *__restrict__ part,
                                                              const uint16_t *__restrict__ scales,
                                                              uint16_t *__restrict__ y, int out,
                                                              int batch, int splits) {
  constexpr int E = RT * NT * 64;
  const int rb = blockIdx.y, tb = blockIdx.z;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const float4_t *p = part + ((size_t)tb * gridDim.y + rb) * splits * E + e;
  float4_t v = p[0];
  for (int k = 1; k < splits; ++k) v += p[(size_t)k * E];
  const int tok0 = tb * 16 * NT;
  store_out<NT>(y + (int64_t)tok0 * out, scales, out, batch - tok0, rb * 16 * RT, e, v);
}

// A lane's codes of one super-chunk under 1x16 g16: 16 groups, two loads.
struct CodePair {
  uint4 lo, hi;
};

template <Scheme S, int RT, int NT>
__global__ __launch_bounds__(kMidThreads)
__attribute__((amdgpu_waves_per_eu(kMidOccupancy, kMidOccupancy)))
void gemm_mid_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ books,
                     const uint16_t *__restrict__ scales, const uint4 *__restrict__ xb,
                     uint16_t *__restrict__ y, float4_t *__restrict__ part, int out, int groups,
                     int batch, int splits, uint32_t codes_bytes, uint32_t slab_bytes) {
  using C = MidCfg<S>;
  constexpr int G = C::G, STEPS = C::STEPS;
  constexpr bool LUT = S == Scheme::k2x8;
  // 1x16 g16: lane quarters 2p and 2p + 1 take the two 16-byte halves of the
  // same codeword in every step (pair p walks groups 16p .. 16p + 15 of the
  // super-chunk, one per step), so one gather instruction fetches both halves
  constexpr bool PAIR = S == Scheme::k1x16g16;
  using CW = std::conditional_t<PAIR, CodePair, uint4>;
  // one activation tile: B fragments straight from x [batch][in] (a lane's
  // 16-byte pieces of one row stay in one 128-byte line for the 8 steps that
  // use them, so the L1 serves all but the first); xb is then x itself and
  // slab_bytes its size
  constexpr bool DIRECT = NT == 1;
  constexpr int BP = 16 * NT;      // activation rows of a workgroup (one slab of xb)
  constexpr int E = RT * NT * 64;  // float4 accumulators of a workgroup tile
  constexpr int D = ring_depth(RT, NT);
  static_assert(STEPS % D == 0, "the ring depth divides the steps of a super-chunk");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t *table = lds;
  float4_t *red = reinterpret_cast<float4_t *>(lds);
  uint32_t *big_flags = reinterpret_cast<uint32_t *>(lds + mid_lds_bytes(LUT, RT, NT) -
                                                     kMidWaves * 4);
  float *lds_scale = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(big_flags) - 64 * 4);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int sp = (int)(blockIdx.x % (unsigned)splits), rb = (int)(blockIdx.x / (unsigned)splits);
  // activation block: rows tok0 .. tok0 + BP - 1 of the batch, slab blockIdx.y of xb
  const int tok0 = blockIdx.y * BP;
  const int nb = batch - tok0;
  const int row0 = rb * 16 * RT;
  const int nsc = (groups + kGroupsPerSc - 1) / kGroupsPerSc;
  const int sc_end = (int)((int64_t)(sp + 1) * nsc / splits);
  const uint32_t row_bytes = (uint32_t)groups * 2u;
  const Rsrc crs = make_rsrc(codes, codes_bytes);
  const Rsrc xrs = make_rsrc(DIRECT ? xb : xb + (size_t)blockIdx.y * (slab_bytes / 16u), slab_bytes);
  const uint4 *gbooks = reinterpret_cast<const uint4 *>(books);

  // the row scales for the epilogue (read after the barriers that end the K loop)
  if (tid < 16 * RT) lds_scale[tid] = row0 + tid < out ? h2f(scales[row0 + tid]) : 0.0f;

  const uint32_t code_lane = (uint32_t)(row0 + r) * row_bytes + (uint32_t)q * 16u;
  const uint32_t x_lane = ((uint32_t)(q * G * BP) + (uint32_t)r) * 16u;
  constexpr uint32_t kBlockBytes = BP * 16u;  // one k-block of the slab
  constexpr uint32_t kScXBytes = C::SC_BLOCKS * kBlockBytes;
  // paired form: pair p = q / 2 reads codes 32 p .. 32 p + 31 of the
  // super-chunk's 64 code bytes; in step s lane quarter q feeds k-block
  // 2 (16 p + s) + q % 2, in A and in B alike
  const int pq = q >> 1, hq = q & 1;
  const uint32_t code_pair = (uint32_t)(row0 + r) * row_bytes + (uint32_t)pq * 32u;
  const uint32_t x_pair = ((uint32_t)((32 * pq + hq) * BP) + (uint32_t)r) * 16u;

  // this lane's code bytes of super-chunk sc for every row tile
  auto load_codes = [&](int sc, CW (&cw)[RT]) __attribute__((always_inline)) {
    if constexpr (PAIR) {
      const int g0 = sc * kGroupsPerSc + 16 * pq;
      const uint32_t b = code_pair + (uint32_t)sc * (kGroupsPerSc * 2u);
      const uint32_t blo = sc < sc_end && g0 < groups ? b : kMidOOB;
      const uint32_t bhi = sc < sc_end && g0 + 8 < groups ? b + 16u : kMidOOB;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        cw[t].lo = buf_load16(crs, blo + (uint32_t)t * 16u * row_bytes);
        cw[t].hi = buf_load16(crs, bhi + (uint32_t)t * 16u * row_bytes);
      }
    } else {
      const bool ok = sc < sc_end && sc * kGroupsPerSc + 8 * q < groups;
      const uint32_t base = ok ? code_lane + (uint32_t)sc * (kGroupsPerSc * 2u) : kMidOOB;
#pragma unroll
      for (int t = 0; t < RT; ++t) cw[t] = buf_load16(crs, base + (uint32_t)t * 16u * row_bytes);
    }
  };
  // B operands of step s of super-chunk sc (k-block g q + s, or the paired
  // form's, rows 16 j + r)
  const int nkb = groups * (G / 8);                       // k-blocks of a row
  const uint32_t x_row = (uint32_t)r * (uint32_t)nkb * 16u;  // row r of x (past batch: out of range)
  auto x_at = [&](int sc, int s) __attribute__((always_inline)) {
    if constexpr (DIRECT) {
      const int kb = sc * C::SC_BLOCKS + (PAIR ? 32 * pq + hq + 2 * s : G * q + s);
      return sc < sc_end && kb < nkb ? x_row + (uint32_t)kb * 16u : kMidOOB;
    } else if constexpr (PAIR)
      return sc < sc_end ? x_pair + (uint32_t)sc * kScXBytes + (uint32_t)s * 2u * kBlockBytes
                         : kMidOOB;
    else
      return sc < sc_end ? x_lane + (uint32_t)sc * kScXBytes + (uint32_t)s * kBlockBytes : kMidOOB;
  };
  auto load_x = [&](int sc, int s, uint4 (&bx)[NT]) __attribute__((always_inline)) {
    const uint32_t base = x_at(sc, s);
#pragma unroll
    for (int j = 0; j < NT; ++j) bx[j] = buf_load16(xrs, base + (uint32_t)j * 256u);
  };
  auto load_x1 = [&](int sc, int s, int j) __attribute__((always_inline)) {
    return buf_load16(xrs, x_at(sc, s) + (uint32_t)j * 256u);
  };
  // 1x16: this lane's codeword (half, for g = 16) of step s
  auto gather1 = [&](const CW &c, int s) __attribute__((always_inline)) {
    if constexpr (PAIR) {
      const uint32_t code = code_of<8>(s < 8 ? c.lo : c.hi, s & 7);
      return gbooks[2u * code + (uint32_t)hq];
    } else {
      const uint32_t code = code_of<G>(c, s);
      return gbooks[G == 8 ? code : 2u * code + (uint32_t)(s & 1)];
    }
  };
  auto gather = [&](const CW (&cw)[RT], int s, uint4 (&ga)[RT]) __attribute__((always_inline)) {
    if constexpr (PAIR) {
#pragma unroll
      for (int t = 0; t < RT; ++t) ga[t] = gather1(cw[t], s);
    } else {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const uint32_t code = code_of<G>(cw[t], s);
        ga[t] = gbooks[G == 8 ? code : 2u * code + (uint32_t)(s & 1)];
      }
    }
  };
  // 2x8: the fp16 sum of the two codewords of step s. A table address is
  // (code << 8) | (slot * 16): one byte permute per read picks the code byte
  // of this lane's codebook (r / 8 first, the other second).
  const uint32_t baseA = (uint32_t)r * 16u, baseB = (uint32_t)(r ^ 8) * 16u;
  const uint32_t mA = (uint32_t)(r >> 3), mB = mA ^ 1u;
  const uint32_t selA[2] = {0x0C0C0000u | ((4u + mA) << 8), 0x0C0C0000u | ((6u + mA) << 8)};
  const uint32_t selB[2] = {0x0C0C0000u | ((4u + mB) << 8), 0x0C0C0000u | ((6u + mB) << 8)};
  auto decode = [&](const auto &cw, int s, uint4 (&a)[RT]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const uint32_t word = (s >> 1) == 0 ? cw[t].x : (s >> 1) == 1 ? cw[t].y
                          : (s >> 1) == 2 ? cw[t].z : cw[t].w;
      const uint32_t addrA = __builtin_amdgcn_perm(word, baseA, selA[s & 1]);
      const uint32_t addrB = __builtin_amdgcn_perm(word, baseB, selB[s & 1]);
      a[t] = hadd8(*reinterpret_cast<const uint4 *>(table + addrA),
                   *reinterpret_cast<const uint4 *>(table + addrB));
    }
  };

  float4_t acc[RT][NT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[t][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  int sc = (int)((int64_t)sp * nsc / splits) + w;
  CW cw[2][RT];  // codes of this and of the wave's next super-chunk (static ring)
  uint4 bx[D][NT];
  uint4 ga[LUT ? 1 : D][RT];
  uint4 a[2][RT];
  bool halved = false;  // overflow guard of the 2x8 codeword sum
  load_codes(sc, cw[0]);
  load_codes(sc + kMidWaves, cw[1]);
#pragma unroll
  for (int i = 0; i < D; ++i) load_x(sc, i, bx[i]);
  if constexpr (LUT) {
    // each thread writes the 8 copies of two codewords, copy (j + tid) % 8 in
    // write j: the 16 lanes of a pass hit 16 distinct slots (lanes 8 apart
    // hold the two codebooks)
    const int tm = (tid >> 3) & 1;
    const int tc = (tid & 7) | ((tid >> 4) << 3);
    const uint4 v0 = gbooks[tm * 256 + tc], v1 = gbooks[tm * 256 + tc + 128];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int slot = ((j + tid) & 7) * 16;
      *reinterpret_cast<uint4 *>(table + tc * 256 + tm * 128 + slot) = v0;
      *reinterpret_cast<uint4 *>(table + (tc + 128) * 256 + tm * 128 + slot) = v1;
    }
    publish_flag(big_flags, has_large_half(v0) || has_large_half(v1));
    __syncthreads();
    // codebooks large enough for the fp16 codeword sum to overflow: halve the
    // table, double the totals (overflow guard, aqlm_device.hpp)
    halved = read_flag(big_flags, kMidWaves);
    if (halved) {
      const uint4 h0 = hhalf8(v0), h1 = hhalf8(v1);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int slot = ((j + tid) & 7) * 16;
        *reinterpret_cast<uint4 *>(table + tc * 256 + tm * 128 + slot) = h0;
        *reinterpret_cast<uint4 *>(table + (tc + 128) * 256 + tm * 128 + slot) = h1;
      }
      __syncthreads();
    }
    decode(cw[0], 0, a[0]);
  } else {
#pragma unroll
    for (int i = 0; i < D; ++i) gather(cw[0], i, ga[i]);
  }

  // one super-chunk whose codes are in cw[K] (the next one's in cw[K ^ 1]);
  // the refilled code slot is cw[K], for the super-chunk after the next
  auto super_chunk = [&](auto kc) __attribute__((always_inline)) {
    constexpr int K = decltype(kc)::value;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const int slot = s % D;
      if constexpr (LUT) {
        // A operands of the next step first, so their LDS reads overlap this step's MFMAs
        if (s + 1 < STEPS)
          decode(cw[K], s + 1, a[(s + 1) & 1]);
        else
          decode(cw[K ^ 1], 0, a[(s + 1) & 1]);
      }
      // the slot is refilled with step s + D (in the wave's next super-chunk
      // past the end of this one)
      const int sn = s + D < STEPS ? s + D : s + D - STEPS;
      const int scn = s + D < STEPS ? sc : sc + kMidWaves;
      if constexpr (LUT) {
        // activation tile by activation tile: its RT MFMAs, then the refill
        // of its B register, pinned in that order (left to itself the
        // scheduler sinks the refills next to their use a step later, and
        // every step then waits out the L2 latency)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
#pragma unroll
          for (int t = 0; t < RT; ++t)
            acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(half8_t, a[s & 1][t]), __builtin_bit_cast(half8_t, bx[slot][j]),
                acc[t][j], 0, 0, 0);
          bx[slot][j] = load_x1(scn, sn, j);
          __builtin_amdgcn_sched_group_barrier(0x008, RT, 0);  // RT MFMAs
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // then one vector-memory read
        }
      } else {
        // 1x16: each gathered A operand feeds its NT MFMAs in a row (the
        // tile-by-tile order measured slower here). Up to 64 activation rows
        // each row tile's next codeword gather is pinned right after its
        // MFMAs and the activation refills after the last tile; with more
        // rows the L2 gather rate bounds the loop and pinning gains nothing.
#pragma unroll
        for (int t = 0; t < RT; ++t) {
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(half8_t, ga[slot][t]), __builtin_bit_cast(half8_t, bx[slot][j]),
                acc[t][j], 0, 0, 0);
          if constexpr (NT <= 4) {
            ga[slot][t] = gather1(cw[s + D < STEPS ? K : K ^ 1][t], sn);
            __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);  // NT MFMAs
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // then the gather
          }
        }
        load_x(scn, sn, bx[slot]);
        if constexpr (NT <= 4)
          __builtin_amdgcn_sched_group_barrier(0x020, NT, 0);  // then the activations
        else
          gather(cw[s + D < STEPS ? K : K ^ 1], sn, ga[slot]);
      }
    }
    load_codes(sc + 2 * kMidWaves, cw[K]);
    sc += kMidWaves;
  };
  while (sc < sc_end) {
    super_chunk(std::integral_constant<int, 0>{});
    if (sc >= sc_end) break;
    super_chunk(std::integral_constant<int, 1>{});
  }

  if (halved) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[t][j] = acc[t][j] * 2.0f;
  }
  // the four wavefronts' partial tiles, added in wavefront order (the 2x8
  // table is dead once every wavefront has left the K loop)
  if constexpr (LUT) __syncthreads();
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int j = 0; j < NT; ++j) red[((w * RT + t) * NT + j) * 64 + lane] = acc[t][j];
  __syncthreads();

  auto wave_sum = [&](int e) __attribute__((always_inline)) {
    float4_t v = red[e] + red[E + e];
    v += red[2 * E + e];
    v += red[3 * E + e];
    return v;
  };
  if (splits == 1) {
    for (int e = tid; e < E; e += kMidThreads) {
      const float4_t v = wave_sum(e);
      const int tj = e >> 6, l = e & 63;
      const int t = tj / NT, j = tj - t * NT;
      const int tok = j * 16 + (l & 15);
      if (tok >= nb) continue;
      const int rr = t * 16 + 4 * (l >> 4);
      const int row = row0 + rr;
      uint16_t *dst = y + (int64_t)(tok0 + tok) * out + row;
      const float s0 = lds_scale[rr], s1 = lds_scale[rr + 1];
      const float s2 = lds_scale[rr + 2], s3 = lds_scale[rr + 3];
      if ((out & 3) == 0 && row + 3 < out) {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(f2h(v[0] * s0) | (f2h(v[1] * s1) << 16),
                                                     f2h(v[2] * s2) | (f2h(v[3] * s3) << 16));
      } else {
        const float sv[4] = {s0, s1, s2, s3};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (row + k < out) dst[k] = (uint16_t)f2h(v[k] * sv[k]);
      }
    }
  } else {
    float4_t *mine = part + ((size_t)blockIdx.y * gridDim.x + blockIdx.x) * E;
    for (int e = tid; e < E; e += kMidThreads) mine[e] = wave_sum(e);
  }
}

// ---------------------------------------------------------------------------
// Plan: activation tiles, row tiles per workgroup and K parts, chosen by a
// clock model of one workgroup step round (four wavefronts, one MFMA step
// each) -- MFMA issue, L1 accesses (one per 64-byte run a lane quad touches),
// LDS codebook reads (2x8) or L2 codeword gathers (1x16) -- times the steps
// per wavefront, times the rounds of workgroups over the CUs. Three row
// tiles exist for layers such as 11008 outputs, where four leave a third of
// the CUs idle and two need a second round.
struct MidPlan {
  int nt = 0, ntb = 0, rt = 0, splits = 0, nrb = 0;
  size_t xb_bytes = 0, part_off = 0, total = 0;
};

constexpr size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int mid_nt(int64_t batch) {
  const int n = (int)((batch + 15) / 16);
  return n <= 4 ? n : n <= 6 ? 6 : 8;
}

// Above 128 rows this form (blocks of 128 activation rows) takes every call
// it can plan, up to 4096 rows, except
//   * where aqlm_gemm would run the decoded-tile kernel (gemm_tile.hip) and
//     that kernel's timing model is below this form's: the clock model of
//     mid_plan times mid_us_per_unit, the mean ratio of measured kernel times
//     to the model on 11008x4096 and 4096x11008 layers at 129..2048 rows
//     (within 20 % at every point);
//   * where the workspace would pass 64 MiB, the static scratch of
//     aqlm_gemm_noalloc: such calls keep a route that needs none.
// Those calls run as aqlm_gemm. Measured times on those layers (us):
//                        rows   this form   tile kernel   wide tiles
//   2x8      11008x4096   384       57          77            91
//                         640       93         141           104
//                        2048      286         269           331
//            4096x11008   640       98         164           136
//                        1536      175         196           235
//   1x16 g16 11008x4096   448      122          84           123
//            4096x11008   512      106         202           314
//   1x16     4096x11008   256       82         187           284
//                        1024      268         229           350
// The wide tiles are slower than one of the other two at nearly every size.
double mid_us_per_unit(Scheme s) {
  return s == Scheme::k2x8 ? 1.15e-3 : s == Scheme::k1x16g16 ? 0.53e-3 : 0.72e-3;
}
constexpr size_t kMidMaxWsAbove128 = size_t(64) << 20;

bool mid_plan(const LayerDesc &L, int64_t batch, MidPlan *p) {
  // (bit-packed 8- and 16-bit codes are the element layout's bytes)
  if (L.scheme == Scheme::kGeneral || batch < kMidMinBatch || batch > kMidMaxBatch) return false;
  if (L.groups % 8 != 0) return false;  // a lane's 16 code bytes never straddle a row end
  const int G = group_size(L.scheme);
  const int steps = G;
  // above 128 rows: blocks of 128 activation rows, one more grid dimension
  const int nt = batch <= 128 ? mid_nt(batch) : 8;
  const int ntb = (int)((batch + 16 * nt - 1) / (16 * nt));
  const int64_t bp = 16 * nt * ntb;
  const int64_t row_bytes = L.groups * kCodeBytesPerGroup;
  const int64_t nsc = (L.groups + kGroupsPerSc - 1) / kGroupsPerSc;
  // one activation tile reads x directly: no re-laid copy
  const int64_t xb_bytes = nt == 1 ? 0 : L.in * bp * 2;
  // 32-bit buffer offsets, with room for the out-of-range marker
  if ((L.out + 64) * row_bytes >= (int64_t(1) << 31) || L.in * bp * 2 + 4 * 65536 >= (int64_t(1) << 31))
    return false;
  double best = 0;
  for (int rt : {4, 3, 2}) {
    if (rt * nt > kMidMaxTiles) continue;
    const int64_t nrb = (L.out + 16 * rt - 1) / (16 * rt);
    const double mfma = 16.0 * rt * nt;
    const double l1 = kMidWaves * (16.0 * nt + 64.0 * rt / steps);
    const double dec = L.scheme == Scheme::k2x8 ? kMidWaves * 40.0 * rt : kMidWaves * 150.0 * rt;
    const double round = std::max(std::max(mfma, l1), dec);
    for (int splits : {1, 2, 4, 8}) {
      if (splits > 1 && splits * 2 > nsc) break;
      const int64_t sc_per_wave = ((nsc + splits - 1) / splits + kMidWaves - 1) / kMidWaves;
      const double wg = sc_per_wave * steps * round +
                        (splits > 1 ? 2000.0 + 16.0 * rt * nt : 0.0);
      const int64_t rounds =
          (nrb * splits * ntb + kMidCus * kMidOccupancy - 1) / (kMidCus * kMidOccupancy);
      const double t = rounds * wg;
      if (p->nt == 0 || t < best) {
        best = t;
        p->nt = nt;
        p->ntb = ntb;
        p->rt = rt;
        p->splits = splits;
        p->nrb = (int)nrb;
      }
    }
  }
  if (p->nt == 0) return false;
  // Up to 16 rows aqlm_gemm's skinny tile is as fast as this form once K has
  // to be split (the reduce launch then costs what the tile saves) or when
  // the row blocks leave most CUs idle anyway (the re-layout launch is then
  // pure overhead); with neither, this form is 20-28% faster (11008 x 4096,
  // 1..16 rows).
  if (batch <= 16 && (p->splits > 1 || p->nrb * p->ntb < kMidCus / 2)) return false;
  p->xb_bytes = (size_t)xb_bytes;
  p->part_off = align256((size_t)xb_bytes);
  p->total = p->part_off +
             (p->splits > 1 ? (size_t)p->nrb * p->splits * p->ntb * p->rt * p->nt * 1024 : 0);
  if (batch > 128) {
    if (p->total > kMidMaxWsAbove128) return false;
    // the call then runs as aqlm_gemm, which takes the decoded-tile kernel
    if (gemm_tile_preferred(L, batch) &&
        gemm_tile_cost_us(L, batch) < best * mid_us_per_unit(L.scheme))
      return false;
  }
  return p->total < (size_t(1) << 40);
}

template <Scheme S, int RT, int NT>
hipError_t launch_mid_t(const LayerDesc &L, const MidPlan &P, const uint16_t *x, int64_t batch,
                        uint16_t *y, uint8_t *ws, hipStream_t stream) {
  constexpr bool LUT = S == Scheme::k2x8;
  constexpr size_t lds = mid_lds_bytes(LUT, RT, NT);
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto k = gemm_mid_kernel<S, RT, NT>;
  if (lds > 64 * 1024) {
    // more than the default dynamic LDS limit: raise it once per device
    static std::atomic<uint64_t> raised{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = uint64_t(1) << (dev & 63);
    if (dev >= 64 || !(raised.load(std::memory_order_acquire) & bit)) {
      e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      raised.fetch_or(bit, std::memory_order_acq_rel);
    }
  }
  float4_t *part = reinterpret_cast<float4_t *>(ws + P.part_off);
  const uint4 *xb = reinterpret_cast<const uint4 *>(ws);
  uint32_t slab = (uint32_t)(P.xb_bytes / P.ntb);
  if constexpr (NT == 1) {
    // one activation tile reads x in place
    xb = reinterpret_cast<const uint4 *>(x);
    slab = (uint32_t)(batch * L.in * 2);
  } else {
    const int nkb = (int)(L.in / 8);
    hipLaunchKernelGGL(gemm_xblock_kernel, dim3((unsigned)((nkb + 15) / 16), (unsigned)(NT * P.ntb)),
                       dim3(256), 0, stream, reinterpret_cast<const uint4 *>(x),
                       reinterpret_cast<uint4 *>(ws), nkb, (int)batch, 16 * NT);
    const hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  hipLaunchKernelGGL(k, dim3((unsigned)(P.nrb * P.splits), (unsigned)P.ntb), dim3(kMidThreads), lds,
                     stream, static_cast<const uint8_t *>(L.codes), L.books, L.scales, xb, y, part,
                     (int)L.out, (int)L.groups, (int)batch, P.splits,
                     (uint32_t)(L.out * L.groups * kCodeBytesPerGroup), slab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P.splits == 1) return e;
  constexpr int E = RT * NT * 64;
  hipLaunchKernelGGL((gemm_mid_reduce_kernel<RT, NT>),
                     dim3((unsigned)((E + 255) / 256), (unsigned)P.nrb, (unsigned)P.ntb), dim3(256),
                     0, stream, part, L.scales, y, (int)L.out, (int)batch, P.splits);
  return hipGetLastError();
}

template <Scheme S, int NT>
hipError_t launch_mid_nt(const LayerDesc &L, const MidPlan &P, const uint16_t *x, int64_t batch,
                         uint16_t *y, uint8_t *ws, hipStream_t stream) {
  switch (P.rt) {
    case 4: return launch_mid_t<S, 4, NT>(L, P, x, batch, y, ws, stream);
    case 3: return launch_mid_t<S, 3, NT>(L, P, x, batch, y, ws, stream);
    default: return launch_mid_t<S, 2, NT>(L, P, x, batch, y, ws, stream);
  }
}

template <Scheme S>
hipError_t launch_mid_s(const LayerDesc &L, const MidPlan &P, const uint16_t *x, int64_t batch,
                        uint16_t *y, uint8_t *ws, hipStream_t stream) {
  switch (P.nt) {
    case 1: return launch_mid_nt<S, 1>(L, P, x, batch, y, ws, stream);
    case 2: return launch_mid_nt<S, 2>(L, P, x, batch, y, ws, stream);
    case 3: return launch_mid_nt<S, 3>(L, P, x, batch, y, ws, stream);
    case 4: return launch_mid_nt<S, 4>(L, P, x, batch, y, ws, stream);
    case 6: return launch_mid_nt<S, 6>(L, P, x, batch, y, ws, stream);
    default: return launch_mid_nt<S, 8>(L, P, x, batch, y, ws, stream);
  }
}

}  // namespace

bool gemm_mid_direct(const LayerDesc &L, int64_t batch) {
  MidPlan p;
  return batch <= 16 && mid_plan(L, batch, &p) && p.total == 0;
}

int64_t gemm_ws_bytes(const LayerDesc &L, int64_t batch) {
  MidPlan p;
  return mid_plan(L, batch, &p) ? (int64_t)p.total : 0;
}

hipError_t launch_gemm_ws(const LayerDesc &L, const uint16_t *x, int64_t batch, uint16_t *y,
                          void *ws, hipStream_t stream) {
  MidPlan p;
  if (!mid_plan(L, batch, &p)) return launch_gemm(L, x, batch, y, stream);
  uint8_t *w = static_cast<uint8_t *>(ws);
  switch (L.scheme) {
    case Scheme::k2x8: return launch_mid_s<Scheme::k2x8>(L, p, x, batch, y, w, stream);
    case Scheme::k1x16: return launch_mid_s<Scheme::k1x16>(L, p, x, batch, y, w, stream);
    default: return launch_mid_s<Scheme::k1x16g16>(L, p, x, batch, y, w, stream);
  }
}

}  // namespace aqlm
