// 1x16 products for one activation row with the codebook held in LDS.
//
// The 1 MiB codebook of a 1x16 layer (65536 codewords of 8 float16 values)
// does not fit in one CU's LDS, and fetching one random 16-byte codeword per
// code through the cache hierarchy runs at about 0.43 fetches per clock per
// CU, whatever the cache policy: one cache line moves per 2-byte code. Here
// the codebook is split over a team of eight workgroups, one per CU: member
// (slice v, half h) holds half h (values 4h .. 4h+3) of the 16384 codewords
// whose top two code bits are v, 128 KiB of LDS. Every member reads all codes
// of the team's rows (coalesced 16-byte loads; the other seven members read
// the same lines, mostly from L2), looks up only the codes of its slice (an
// 8-byte LDS read; other codes read a zero entry) and takes the dot product of
// that half-codeword with the matching four activations on the matrix cores
// (4x4x4 products, whose diagonals hold the lanes' own dot products). A row's eight member
// sums go to the workspace, and a second launch adds them in member order,
// applies the row scale and rounds to float16. Random 8-byte LDS reads cost
// about a third of a clock per lane, against several clocks per L2 codeword
// fetch, so the kernel is bound by LDS lookups rather than by the L2 path.
//
// Layout of the work:
//   * workgroup w is member (w / 8) % 8 of team (w / 64) * 8 + w % 8: the
//     members of a team are eight consecutive-in-XCD workgroups, which the
//     dispatcher places on one XCD (workgroups go to the XCDs in turn), so
//     their shared code lines meet in one L2. Correctness does not depend on
//     the placement;
//   * teams are split over the layers of a call in proportion to their code
//     bytes; a team owns a contiguous range of one layer's rows, and its
//     eight wavefronts take the rows in turn;
//   * a wavefront reads a row as 1 KiB chunks, lane l taking groups
//     512c + 8l .. 512c + 8l + 7 of chunk c, so every lane keeps the
//     activations of its groups (its half of each) in registers for the whole
//     kernel; the codes of the next D rows are in flight;
//   * the slice test and entry indexes of a word of two codes take two VALU
//     operations: t = w ^ (v << 14 | v << 30) clears the top two bits of each
//     16-bit half of a slice-v code, so a packed 16-bit min(t, 16384) gives
//     the entry index of a hit and the zero entry 16384 of a miss, per half.
#include <atomic>

#include "aqlm_device.hpp"

namespace aqlm {
namespace {

constexpr int kSlMembers = 8;                          // 4 value slices x 2 halves
constexpr int kSlEntries = 16384;                      // codewords per value slice
constexpr int kSlTableBytes = (kSlEntries + 2) * 8;    // half-codewords + zero entry (+ pad)
constexpr int kSlMaxChunks = 8;                        // 1 KiB code chunks per row
constexpr int kSlMaxGroup = 16;
constexpr uint32_t kSlOOB = 0x80000000u;

struct SliceLayer {
  const uint8_t *codes;   // [out][groups] uint16 codes
  const uint16_t *books;  // [65536][8] float16
  const uint16_t *x;      // [groups * 8] float16, one activation row
  float *part;            // [8][out] member sums
  int out, groups;
  int team_begin, team_count;  // teams [team_begin, team_begin + team_count)
};

struct SliceArgs {
  SliceLayer layer[kSlMaxGroup];
  int n;
};

// LDS byte address of the entry whose index is the low (high) 16 bits of m:
// index * 8 + base in one v_mad_u32_u16 (op_sel picks the high half).
__device__ __forceinline__ uint32_t entry_addr_lo(uint32_t m, uint32_t base) {
  uint32_t r;
  asm("v_mad_u32_u16 %0, %1, 8, %2" : "=v"(r) : "v"(m), "s"(base));
  return r;
}
__device__ __forceinline__ uint32_t entry_addr_hi(uint32_t m, uint32_t base) {
  uint32_t r;
  asm("v_mad_u32_u16 %0, %1, 8, %2 op_sel:[1,0,0,0]" : "=v"(r) : "v"(m), "s"(base));
  return r;
}
__device__ __forceinline__ uint2 lds_load8(uint32_t addr) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = *reinterpret_cast<__attribute__((address_space(3))) const u32x2 *>((uintptr_t)addr);
  return make_uint2(v.x, v.y);
}

// NCH: 1 KiB code chunks per row; D: rows a wavefront handles at once; G:
// groups of D rows whose codes are in flight; T: threads per workgroup.
template <int NCH, int D, int G, int T>
__global__ __launch_bounds__(T) void gemv_1x16_slice_kernel(SliceArgs A) {
  constexpr int W = T / 64;  // wavefronts per workgroup
  extern __shared__ __attribute__((aligned(16))) uint8_t table[];
  const int w = blockIdx.x;
  const int member = (w >> 3) & 7;
  const int team = (w >> 6) * 8 + (w & 7);
  int li = 0;
#pragma unroll 1
  for (int i = 1; i < A.n; ++i)
    if (team >= A.layer[i].team_begin) li = i;
  const SliceLayer &L = A.layer[li];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t slice = (uint32_t)(member >> 1), half = (uint32_t)(member & 1);
  const int tl = team - L.team_begin;
  const int r0 = (int)((int64_t)L.out * tl / L.team_count);
  const int r1 = (int)((int64_t)L.out * (tl + 1) / L.team_count);
  const uint32_t row_bytes = (uint32_t)L.groups * 2u;

  // Prologue, in issue order: this member's half-codewords (entry e =
  // codeword (slice << 14) + e, bytes 8 * half .. 8 * half + 7; thread t moves
  // entries t + T i), this lane's activations, then the codes of the first G
  // row groups. Vector loads retire in issue order, so writing the staged
  // entries to LDS waits for L2 only, and at the row loop only code loads are
  // still in flight.
  const Rsrc rb = make_rsrc(L.books, 65536u * 16u);
  constexpr int kPer = kSlEntries / T / 2;  // entries per thread and round
  auto stage_load = [&](int round, uint2 (&st)[kPer]) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const uint32_t e = (uint32_t)(tid + (round * kPer + i) * T);
      st[i] = buf_load8(rb, (((slice << 14) + e) << 4) + (half << 3));
    }
  };
  auto stage_store = [&](int round, const uint2 (&st)[kPer]) {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      *reinterpret_cast<uint2 *>(table + (size_t)(tid + (round * kPer + i) * T) * 8) = st[i];
  };
  uint2 st0[kPer], st1[kPer];
  stage_load(0, st0);

  // this lane's activations: half `half` of groups 512c + 8 lane + p
  const Rsrc rx = make_rsrc(L.x, row_bytes * 8u);
  uint2 xf[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t g = (uint32_t)c * 512u + (uint32_t)lane * 8u + (uint32_t)p;
      xf[c][p] = buf_load8(rx, g < (uint32_t)L.groups ? g * 16u + half * 8u : kSlOOB);
    }
  stage_load(1, st1);

  // Codes: row group k of this wavefront is rows r0 + wave + W (D k + d),
  // d < D. Rows at or past r1 load from an out-of-range offset (zeros), so
  // every load of the loop below is unconditional and the wait counts exact.
  const Rsrc rc = make_rsrc(L.codes, (uint32_t)L.out * row_bytes);
  const uint32_t lane_off = (uint32_t)lane * 16u;
  const int first = r0 + wave;
  uint4 cw[G][D][NCH];
  auto load_group = [&](int k, uint4 (&dst)[D][NCH]) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int row = first + W * (D * k + d);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t in_row = (uint32_t)c * 1024u + lane_off;
        // cached loads: the other seven members of the team read the same
        // lines, which must stay in L2 for them
        dst[d][c] = buf_load16(
            rc, (row < r1 && in_row < row_bytes) ? (uint32_t)row * row_bytes + in_row : kSlOOB);
      }
    }
  };
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < G; ++k) load_group(k, cw[k]);
  __builtin_amdgcn_sched_barrier(0);

  stage_store(0, st0);
  stage_store(1, st1);
  if (tid < 2) *reinterpret_cast<uint2 *>(table + (size_t)(kSlEntries + tid) * 8) = make_uint2(0, 0);
  __syncthreads();

  // lanes past the end of a row read no codes (zero words): their key is all
  // ones, so their t = w ^ key sends both halves to the zero entry
  const uint32_t key = (slice << 14) | (slice << 30);
  uint32_t keyc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) keyc[c] = (uint32_t)c * 1024u + lane_off < row_bytes ? key : ~0u;
  const uint32_t tbase = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t *)table);
  float *const part = L.part + (size_t)member * L.out;

  // The D row sums of a group, reduced over the wavefront (totals in lane 63).
  // Entry indexes: a packed 16-bit min of t; addresses: each half times 8
  // plus the table's base, one multiply-add per half.
  // Products: each looked-up half-codeword and the lane's four activations
  // go into a 4x4x4 matrix-core product; lane 4q + j gives row j of block q's
  // A and column j of its B, so element j of that lane's accumulator (the
  // block's diagonal) collects exactly the lane's own dot products. The other
  // elements hold cross products of neighbouring lanes and are not read.
  auto group_sums = [&](const uint4 (&c4)[D][NCH], float (&sum)[D]) {
    float4_t acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      uint2 e[D][8];
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const uint32_t wd[4] = {c4[d][c].x, c4[d][c].y, c4[d][c].z, c4[d][c].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t m = __builtin_bit_cast(
              uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, wd[k] ^ keyc[c]),
                                                  u16x2_t{(uint16_t)kSlEntries, (uint16_t)kSlEntries}));
          e[d][2 * k] = lds_load8(entry_addr_lo(m, tbase));
          e[d][2 * k + 1] = lds_load8(entry_addr_hi(m, tbase));
        }
      }
#pragma unroll
      for (int d = 0; d < D; ++d)
#pragma unroll
        for (int p = 0; p < 8; ++p)
          acc[d] = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, e[d][p]),
                                                      __builtin_bit_cast(half4_t, xf[c][p]), acc[d],
                                                      0, 0, 0);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      // the quad's four diagonal elements, then the sum over the 16 quads
      float v = dpp<kDppQuadBcast0>(acc[d][0]) + dpp<kDppQuadBcast1>(acc[d][1]);
      v += dpp<kDppQuadBcast2>(acc[d][2]);
      v += dpp<kDppQuadBcast3>(acc[d][3]);
      sum[d] = quads_sum_to_lane63(v);
    }
  };
  auto store_group = [&](int k, const float (&sum)[D]) {
    if (lane == 63) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int row = first + W * (D * k + d);
        if (row < r1) part[row] = sum[d];
      }
    }
  };

  // groups k, k + 1, ...: group k's codes are in ring slot k % G; after its
  // sums are taken the slot is refilled with group k + G
  const int rows_here = r1 > first ? (r1 - first + W - 1) / W : 0;  // rows of this wavefront
  const int groups = (rows_here + D - 1) / D;
  int k = 0;
  for (; k + G <= groups; k += G) {
#pragma unroll
    for (int s = 0; s < G; ++s) {
      float sum[D];
      group_sums(cw[s], sum);
      // keep the next slots' waits below this refill (G groups stay in flight)
      __builtin_amdgcn_sched_barrier(0);
      load_group(k + s + G, cw[s]);
      store_group(k + s, sum);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int s = 0; s < G; ++s) {
    if (k + s < groups) {
      float sum[D];
      group_sums(cw[s], sum);
      store_group(k + s, sum);
    }
  }
}

// y[o] = fp16(scale[o] * (((p_0 + p_1) + p_2) + ... + p_7)) for every row of
// every layer of the call. Each layer has blocks of its own (blocks
// [blk_begin, blk_begin + ceil(out / 256)) of the launch), so the layer is a
// function of the block index: its descriptor is read with scalar loads
// rather than fetched per lane from memory before the partial sums.
struct SliceReduceLayer {
  const float *part;
  const uint16_t *scales;
  uint16_t *y;
  int out, blk_begin;
};
struct SliceReduceArgs {
  SliceReduceLayer layer[kSlMaxGroup];
  int n;
};

__global__ __launch_bounds__(256) void gemv_1x16_slice_reduce(SliceReduceArgs A) {
  const int blk = blockIdx.x;
  int li = 0;
#pragma unroll 1
  for (int i = 1; i < A.n; ++i)
    if (blk >= A.layer[i].blk_begin) li = i;
  const SliceReduceLayer &L = A.layer[li];
  const int o = (blk - L.blk_begin) * 256 + (int)threadIdx.x;
  if (o >= L.out) return;
  float v = L.part[o];
#pragma unroll
  for (int m = 1; m < kSlMembers; ++m) v += L.part[(size_t)m * L.out + o];
  L.y[o] = (uint16_t)f2h(v * h2f(L.scales[o]));
}

int slice_chunks(const LayerDesc &L) { return (int)((L.groups * 2 + 1023) / 1024); }

int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return cus;
}

template <int NCH>
hipError_t launch_slice_t(const SliceArgs &A, int teams, hipStream_t stream) {
  // rows per wavefront step and groups in flight: codes of G * D rows ahead;
  // 1024 threads while the registers allow four wavefronts per SIMD
  constexpr int D = NCH <= 2 ? 4 : NCH <= 4 ? 2 : 1;
  constexpr int G = 2;
  constexpr int T = NCH <= 1 ? 1024 : 512;
  auto k = gemv_1x16_slice_kernel<NCH, D, G, T>;
  static std::atomic<uint64_t> raised{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (dev >= 64 || !(raised.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kSlTableBytes);
    if (e != hipSuccess) return e;
    raised.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL(k, dim3((unsigned)(teams * kSlMembers)), dim3(T), kSlTableBytes, stream, A);
  return hipGetLastError();
}

}  // namespace

// True when the codebook-sliced kernel serves this layer at this batch (it
// needs a workspace of gemv_slice_ws_bytes).
bool gemv_slice_fits(const LayerDesc &L, int batch) {
  if (L.scheme != Scheme::k1x16 || batch != 1) return false;
  if (L.groups % 8 != 0 || slice_chunks(L) > kSlMaxChunks) return false;
  // smaller layers: the staging of the slices costs more than it saves
  if (L.out * L.groups < (int64_t(1) << 19)) return false;
  // 32-bit byte offsets (codes, out-of-range marker)
  return L.out * L.groups * 2 < (int64_t(1) << 31);
}

int64_t gemv_slice_ws_bytes(const LayerDesc &L) {
  return ((int64_t)kSlMembers * L.out * 4 + 255) / 256 * 256;
}

// The layers (all accepted by gemv_slice_fits, at most kSlMaxGroup of them,
// each with its workspace part): one launch per row length class (1 KiB
// chunks per row), whose teams are split over its layers, then one launch
// that adds the member sums of every layer.
hipError_t launch_gemv_slice(const LayerDesc *const *Ls, const uint16_t *const *xs,
                             uint16_t *const *ys, float *const *parts, int n,
                             hipStream_t stream) {
  if (n < 1 || n > kSlMaxGroup) return hipErrorInvalidValue;
  for (int nch = 1; nch <= kSlMaxChunks; ++nch) {
    int idx[kSlMaxGroup], m = 0;
    double total = 0;
    for (int i = 0; i < n; ++i)
      if (slice_chunks(*Ls[i]) == nch) {
        idx[m++] = i;
        total += (double)Ls[i]->out * (double)Ls[i]->groups;
      }
    if (m == 0) continue;
    // a multiple of 8 teams: workgroup w maps to (team, member) one to one
    // only then (w = 64 a + 8 member + x, team = 8 a + x)
    int teams = device_cus() / 64 * 8;
    if (teams < 8 * ((m + 7) / 8)) teams = 8 * ((m + 7) / 8);
    SliceArgs A;
    A.n = m;
    int begin = 0;
    for (int j = 0; j < m; ++j) {
      const LayerDesc &L = *Ls[idx[j]];
      // teams in proportion to the layers' codes, at least one each
      int cnt = j + 1 == m ? teams - begin
                           : (int)((double)teams * (double)L.out * (double)L.groups / total + 0.5);
      const int left = teams - begin - (m - 1 - j);
      if (cnt > left) cnt = left;
      if (cnt < 1) cnt = 1;
      A.layer[j] = SliceLayer{static_cast<const uint8_t *>(L.codes), L.books, xs[idx[j]],
                              parts[idx[j]], (int)L.out, (int)L.groups, begin, cnt};
      begin += cnt;
    }
    hipError_t e;
    switch (nch) {
      case 1: e = launch_slice_t<1>(A, teams, stream); break;
      case 2: e = launch_slice_t<2>(A, teams, stream); break;
      case 3: e = launch_slice_t<3>(A, teams, stream); break;
      case 4: e = launch_slice_t<4>(A, teams, stream); break;
      case 5: e = launch_slice_t<5>(A, teams, stream); break;
      case 6: e = launch_slice_t<6>(A, teams, stream); break;
      case 7: e = launch_slice_t<7>(A, teams, stream); break;
      default: e = launch_slice_t<8>(A, teams, stream); break;
    }
    if (e != hipSuccess) return e;
  }
  SliceReduceArgs R;
  R.n = n;
  int blocks = 0;
  for (int i = 0; i < n; ++i) {
    R.layer[i] = SliceReduceLayer{parts[i], Ls[i]->scales, ys[i], (int)Ls[i]->out, blocks};
    blocks += (int)((Ls[i]->out + 255) / 256);
  }
  hipLaunchKernelGGL(gemv_1x16_slice_reduce, dim3((unsigned)blocks), dim3(256), 0, stream, R);
  return hipGetLastError();
}

}  // namespace aqlm
