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
#include <vector>

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

// ---------------------------------------------------------------------------
// 2x8 lookup GEMV for one or two activation rows.
//
// LDS holds both 8-bit codebooks in a 64 KiB bank-spread table: the entry of
// code value c is a 256-byte stripe of sixteen 16-byte slots; slots 0..7 hold
// copies of codeword C_0[c], slots 8..15 copies of C_1[c]:
//   byte address of half h (0, 1) of copy k of C_m[c] = c*256 + m*128 + k*16 + h*8.
// Within a 32-lane LDS pass, lane group q = (lane % 32) / 8 reads combination
// (m, h) = ((q + i) % 4) / 2, (q + i) % 2 in read i (i = 0..3) from copy
// k = lane % 8, so the 32 lanes of every read touch 32 distinct 8-byte bank
// pairs whatever the codes are. Each address is one v_perm_b32: the code byte
// becomes bits 8..15 and a per-lane constant supplies bits 0..7. Reads are
// ds_read_b64 (on gfx950 16-byte LDS reads run at about a third of the
// 8-byte rate). The table is filled straight from memory with 16-byte
// global-to-LDS loads, one whole codeword per lane. Every lane keeps the
// activations of its code chunks in registers, in the half order its reads
// return, so a group costs four address permutes and eight dot2.
// ---------------------------------------------------------------------------
constexpr int kTable2x8Bytes = 256 * 256;

// The work of one workgroup on one layer; gw / waves_total number this
// workgroup's wavefronts among all wavefronts assigned to the layer.
template <int BLOCK, int LPR, int CPL, int BATCH, int DEPTH>
__device__ __forceinline__ void gemv_2x8_body(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ books,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y, int out, int in, int row_chunks, int gw, int waves_total) {
  constexpr int WAVES = BLOCK / 64;
  constexpr int RPI = 64 / LPR;  // rows per wave iteration
  __shared__ __attribute__((aligned(16))) uint8_t table[kTable2x8Bytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lq = (lane & 31) >> 3;
  const int kslot = lane & 7;
  const int lane_in_row = lane % LPR;
  const int row_slot = lane / LPR;
  const uint32_t row_bytes = (uint32_t)row_chunks * 16;
  const int row_groups = (out + RPI - 1) / RPI;
  const int my_iters = gw < row_groups ? (row_groups - gw + waves_total - 1) / waves_total : 0;
  constexpr uint32_t kOOB = 0x80000000u;  // past every buffer: reads return zero

  // Buffer resources: loads outside [0, num_records) return 0, so every load
  // below is unconditional and the compiler can keep precise wait counts.
  const Rsrc rc = make_rsrc(codes, (uint32_t)out * row_bytes);
  const Rsrc rx = make_rsrc(x, (uint32_t)BATCH * (uint32_t)in * 2u);
  const Rsrc rs = make_rsrc(scales, (uint32_t)out * 2u);

  // 1. codebooks straight into the LDS table: load f fills stripes
  //    4f .. 4f+3 (1 KiB), lane l supplying slot l % 16 of stripe 4f + l / 16
  static_assert(64 % WAVES == 0, "fill loads must split evenly over the waves");
  {
    const int m = (lane & 15) >> 3;
    const uint4 *gb = reinterpret_cast<const uint4 *>(books);
#pragma unroll
    for (int j = 0; j < 64 / WAVES; ++j) {
      const int f = wave * (64 / WAVES) + j;
      __builtin_amdgcn_global_load_lds(gb + m * 256 + 4 * f + (lane >> 4),
                                       table + f * 1024, 16, 0, 0);
    }
  }

  // 2. activations of this lane's chunks
  uint4 xv[BATCH][CPL][8];
#pragma unroll
  for (int b = 0; b < BATCH; ++b)
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const int p = lane_in_row + LPR * t;
#pragma unroll
      for (int gi = 0; gi < 8; ++gi) {
        const uint32_t off = p < row_chunks ? ((uint32_t)b * in + (uint32_t)p * 64 + gi * 8) * 2u : kOOB;
        xv[b][t][gi] = buf_load16(rx, off);
      }
    }

  // every row scale this wave will need: lane j holds the scale of iteration
  // j / RPI, row slot j % RPI (a wave owns at most 64 rows)
  uint32_t scale_reg;
  {
    const int j_it = lane / RPI, j_slot = lane % RPI;
    const int row = (gw + j_it * waves_total) * RPI + j_slot;
    scale_reg = buf_load_u16(rs, (j_it < my_iters && row < out) ? (uint32_t)row * 2u : kOOB);
  }

  // 3. the first DEPTH iterations of codes
  uint4 buf[DEPTH][CPL];
  // Offsets advance by a uniform step per iteration: row(it) = row0 + it * RPI * waves_total.
  const int row0 = gw * RPI + row_slot;
  const int row_step = RPI * waves_total;
  uint32_t lane_off[CPL];
#pragma unroll
  for (int t = 0; t < CPL; ++t)
    lane_off[t] = __umul24((uint32_t)row0, row_bytes) + (uint32_t)(lane_in_row + LPR * t) * 16u;
  const uint32_t off_step = __umul24((uint32_t)row_step, row_bytes);
  auto load_iter = [&](int it, uint4 (&dst)[CPL]) {
    const bool ok = it < my_iters && row0 + it * row_step < out;
    const uint32_t itoff = (uint32_t)it * off_step;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const bool in_row = lane_in_row + LPR * t < row_chunks;
      dst[t] = buf_load16_nt(rc, (ok && in_row) ? lane_off[t] + itoff : kOOB);
    }
  };
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) load_iter(s, buf[s]);

  // activation halves in read order: reads i = 0, 2 return half (lq & 1)
  uint2 xa[BATCH][CPL][8], xb[BATCH][CPL][8];
#pragma unroll
  for (int b = 0; b < BATCH; ++b)
#pragma unroll
    for (int t = 0; t < CPL; ++t)
#pragma unroll
      for (int gi = 0; gi < 8; ++gi) {
        const uint2 lo = make_uint2(xv[b][t][gi].x, xv[b][t][gi].y);
        const uint2 hi = make_uint2(xv[b][t][gi].z, xv[b][t][gi].w);
        xa[b][t][gi] = (lq & 1) ? hi : lo;
        xb[b][t][gi] = (lq & 1) ? lo : hi;
      }

  uint32_t base[4], sel[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int Q = (lq + i) & 3;
    const int m = Q >> 1;
    base[i] = (uint32_t)(m * 128 + kslot * 16 + (Q & 1) * 8);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
      sel[i][hi] = 0x0C0C0000u | ((uint32_t)(4 + 2 * hi + m) << 8);  // byte1 = code, byte0 = base
  }
  __syncthreads();

  // One row iteration: decode-and-dot over the lane's chunks, then reduce.
  auto compute = [&](const uint4 (&cw)[CPL], int it) {
    float acc0[BATCH], acc1[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) acc0[b] = acc1[b] = 0.0f;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const uint32_t words[4] = {cw[t].x, cw[t].y, cw[t].z, cw[t].w};
#pragma unroll
      for (int gi = 0; gi < 8; ++gi) {
        const uint32_t w = words[gi >> 1];
        const int hi = gi & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t addr = __builtin_amdgcn_perm(w, base[i], sel[i][hi]);
          const uint2 v = *reinterpret_cast<const uint2 *>(table + addr);
#pragma unroll
          for (int b = 0; b < BATCH; ++b) {
            const uint2 xx = (i & 1) ? xb[b][t][gi] : xa[b][t][gi];
            if (i & 1)
              acc1[b] = dot2(v.y, xx.y, dot2(v.x, xx.x, acc1[b]));
            else
              acc0[b] = dot2(v.y, xx.y, dot2(v.x, xx.x, acc0[b]));
          }
        }
      }
    }
    const int row = (gw + it * waves_total) * RPI + row_slot;
    // scale of this row: held by lane it * RPI + row_slot
    float sc;
    if constexpr (RPI == 1) {
      sc = low_half_to_float(__builtin_amdgcn_readlane(scale_reg, it));
    } else {
      uint32_t sb = __builtin_amdgcn_readlane(scale_reg, it * RPI);
#pragma unroll
      for (int r = 1; r < RPI; ++r) {
        const uint32_t v = __builtin_amdgcn_readlane(scale_reg, it * RPI + r);
        sb = row_slot == r ? v : sb;
      }
      sc = low_half_to_float(sb);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const float v = row_sum<LPR>(acc0[b] + acc1[b]);
      if (lane_in_row == LPR - 1 && row < out) y[(int64_t)b * out + row] = (uint16_t)f2h(v * sc);
    }
  };

  // Steady state: whole groups of DEPTH iterations, each slot refilled right
  // after use (past the wave's last row the refill reads zeros), so the wait
  // before a slot covers only that slot's loads.
  int it0 = 0;
  for (; it0 + DEPTH <= my_iters; it0 += DEPTH) {
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) {
      compute(buf[s], it0 + s);
      load_iter(it0 + s + DEPTH, buf[s]);
    }
  }
  // Tail: fewer than DEPTH iterations left, all already loaded.
#pragma unroll
  for (int s = 0; s < DEPTH - 1; ++s)
    if (it0 + s < my_iters) compute(buf[s], it0 + s);
}

template <int BLOCK, int LPR, int CPL, int BATCH, int DEPTH>
__global__ __launch_bounds__(BLOCK) void gemv_2x8_lds_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ books,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y, int out, int in, int row_chunks) {
  constexpr int WAVES = BLOCK / 64;
  gemv_2x8_body<BLOCK, LPR, CPL, BATCH, DEPTH>(codes, books, scales, x, y, out, in, row_chunks,
                                               blockIdx.x * WAVES + (threadIdx.x >> 6),
                                               gridDim.x * WAVES);
}

// Several independent layers in one launch: workgroup b serves the layer
// whose [wg_begin, wg_begin + wg_count) range holds b.
constexpr int kMaxGroup = 16;
struct GroupSlot {
  const uint8_t *codes;
  const uint16_t *books;
  const uint16_t *scales;
  const uint16_t *x;
  uint16_t *y;
  int out, in, row_chunks, wg_begin, wg_count;
};
struct GroupArgs {
  GroupSlot slot[kMaxGroup];
  int n;
};

template <int BLOCK, int LPR, int CPL, int BATCH, int DEPTH>
__global__ __launch_bounds__(BLOCK) void gemv_2x8_group_kernel(const GroupArgs args) {
  constexpr int WAVES = BLOCK / 64;
  int l = 0;
  for (int i = 1; i < args.n; ++i)
    if ((int)blockIdx.x >= args.slot[i].wg_begin) l = i;
  const GroupSlot &g = args.slot[l];
  gemv_2x8_body<BLOCK, LPR, CPL, BATCH, DEPTH>(
      g.codes, g.books, g.scales, g.x, g.y, g.out, g.in, g.row_chunks,
      ((int)blockIdx.x - g.wg_begin) * WAVES + (threadIdx.x >> 6), g.wg_count * WAVES);
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

template <int LPR, int CPL, int BATCH>
void launch_2x8_lds_cfg(const LayerDesc &L, const uint16_t *x, uint16_t *y, hipStream_t stream) {
  // One 512-thread workgroup per CU when the activations of a lane's chunks fit
  // in 256 registers; otherwise two 256-thread workgroups per CU.
  constexpr bool kWide = BATCH * CPL <= 3;
  constexpr int BLOCK = kWide ? 512 : 256;
  constexpr int DEPTH = CPL == 1 ? 4 : 2;
  const int out = (int)L.out, in = (int)L.in;
  const int row_chunks = (int)(L.groups / 8);
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int rows_per_iter = 64 / LPR;
  const int waves_needed = (out + rows_per_iter - 1) / rows_per_iter;
  int grid = kWide ? cus : 2 * cus;
  const int grid_needed = (waves_needed + BLOCK / 64 - 1) / (BLOCK / 64);
  // each wavefront keeps the scales of its rows in one register: <= 64 rows
  const int grid_min = (int)((out + 64LL * (BLOCK / 64) - 1) / (64LL * (BLOCK / 64)));
  if (grid < grid_min) grid = grid_min;
  if (grid > grid_needed) grid = grid_needed;
  hipLaunchKernelGGL((gemv_2x8_lds_kernel<BLOCK, LPR, CPL, BATCH, DEPTH>), dim3(grid), dim3(BLOCK), 0,
                     stream, static_cast<const uint8_t *>(L.codes), L.books, L.scales, x, y, out, in,
                     row_chunks);
}

// Returns false when the shape needs more code chunks per lane than the
// register-resident activations allow; the caller then uses the general kernel.
template <int BATCH>
bool launch_2x8_lds(const LayerDesc &L, const uint16_t *x, uint16_t *y, hipStream_t stream) {
  const int64_t chunks = L.groups / 8;
  // 32-bit buffer offsets: codes (with the prefetch overrun) and x must stay below 2 GiB
  if ((L.out + 4096) * chunks * 16 >= (int64_t)1 << 31 || L.in * 2 * BATCH >= ((int64_t)1 << 31))
    return false;
  if (chunks <= 16) { launch_2x8_lds_cfg<16, 1, BATCH>(L, x, y, stream); return true; }
  if (chunks <= 32) { launch_2x8_lds_cfg<32, 1, BATCH>(L, x, y, stream); return true; }
  if (chunks <= 64) { launch_2x8_lds_cfg<64, 1, BATCH>(L, x, y, stream); return true; }
  if (chunks <= 128) { launch_2x8_lds_cfg<64, 2, BATCH>(L, x, y, stream); return true; }
  if (chunks <= 192) { launch_2x8_lds_cfg<64, 3, BATCH>(L, x, y, stream); return true; }
  if constexpr (BATCH == 1) {
    if (chunks <= 256) { launch_2x8_lds_cfg<64, 4, BATCH>(L, x, y, stream); return true; }
  }
  return false;
}

// Grouped launches. Configuration index of a 2x8 layer's code-chunk count
// (16-byte chunks per row) for the register-resident kernel, or -1.
int config_2x8(int64_t chunks, int batch) {
  if (chunks <= 16) return 0;
  if (chunks <= 32) return 1;
  if (chunks <= 64) return 2;
  if (chunks <= 128) return 3;
  if (chunks <= 192) return 4;
  if (batch == 1 && chunks <= 256) return 5;
  return -1;
}

template <int LPR, int CPL, int BATCH>
hipError_t launch_group_cfg(GroupArgs &args, int cus, hipStream_t stream) {
  constexpr bool kWide = BATCH * CPL <= 3;
  constexpr int BLOCK = kWide ? 512 : 256;
  constexpr int WAVES = BLOCK / 64;
  constexpr int RPI = 64 / LPR;
  constexpr int DEPTH = CPL == 1 ? 4 : 2;
  const int budget = kWide ? cus : 2 * cus;
  double total = 0;
  for (int i = 0; i < args.n; ++i) total += (double)args.slot[i].out * args.slot[i].row_chunks;
  int begin = 0;
  for (int i = 0; i < args.n; ++i) {
    GroupSlot &g = args.slot[i];
    const int row_groups = (g.out + RPI - 1) / RPI;
    const int max_wg = (row_groups + WAVES - 1) / WAVES;            // one row group per wave
    const int min_wg = (g.out + 64 * WAVES - 1) / (64 * WAVES);     // <= 64 rows per wave
    int n = (int)(budget * ((double)g.out * g.row_chunks) / total + 0.5);
    if (n < min_wg) n = min_wg;
    if (n > max_wg) n = max_wg;
    if (n < 1) n = 1;
    g.wg_begin = begin;
    g.wg_count = n;
    begin += n;
  }
  hipLaunchKernelGGL((gemv_2x8_group_kernel<BLOCK, LPR, CPL, BATCH, DEPTH>), dim3(begin),
                     dim3(BLOCK), 0, stream, args);
  return hipGetLastError();
}

template <int BATCH>
hipError_t launch_group(int cfg, GroupArgs &args, int cus, hipStream_t stream) {
  switch (cfg) {
    case 0: return launch_group_cfg<16, 1, BATCH>(args, cus, stream);
    case 1: return launch_group_cfg<32, 1, BATCH>(args, cus, stream);
    case 2: return launch_group_cfg<64, 1, BATCH>(args, cus, stream);
    case 3: return launch_group_cfg<64, 2, BATCH>(args, cus, stream);
    case 4: return launch_group_cfg<64, 3, BATCH>(args, cus, stream);
    case 5:
      if constexpr (BATCH == 1) return launch_group_cfg<64, 4, BATCH>(args, cus, stream);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

// Rows per wavefront of gemv_fast_kernel for a layer of `out` rows whose
// lanes each take `passes` code chunks of a row: the largest of max_rpw, 2, 1
// for which workgroups x passes reaches 2 * kGemvCus, else 1. The kernel is
// bound by its codeword gathers per CU, so a short layer (1024 rows at four
// rows per wavefront is 64 workgroups) must spread its rows over every CU,
// while rows long enough to give each lane several chunks keep four.
constexpr int kGemvCus = 256;
inline int fast_rows_per_wave(int out, int max_rpw, int passes) {
  for (int r = max_rpw; r > 1; r /= 2)
    if ((int64_t)((out + kWaves * r - 1) / (kWaves * r)) * passes >= 2 * kGemvCus) return r;
  return 1;
}

template <Scheme S, int BATCH>
hipError_t launch_batch(const LayerDesc &L, const uint16_t *x, uint16_t *y, hipStream_t stream) {
  constexpr int G = group_size(S);
  const int out = (int)L.out, in = (int)L.in, groups = (int)L.groups;
  if constexpr (S == Scheme::k2x8 && BATCH <= 2) {
    if (groups % 8 == 0 && launch_2x8_lds<BATCH>(L, x, y, stream)) return hipGetLastError();
  }
  if (groups % 8 == 0) {
    const int row_chunks = groups / 8;
    int slice_chunks = kXLdsHalves / (BATCH * 8 * G);
    if (slice_chunks < 1) slice_chunks = 1;
    // Rows per wavefront: 4 (up to two activation rows, else 2), 2 or 1 as
    // above. A row's sum does not depend on it, so the result is the same
    // bits whichever is taken.
    const int rpw = fast_rows_per_wave(out, BATCH <= 2 ? 4 : 2, (row_chunks + 63) / 64);
    const int rows_per_block = kWaves * rpw;
    const int grid = (out + rows_per_block - 1) / rows_per_block;
    const uint8_t *codes = static_cast<const uint8_t *>(L.codes);
    if (rpw == 1)
      hipLaunchKernelGGL((gemv_fast_kernel<S, BATCH, 1>), dim3(grid), dim3(kBlock), 0, stream,
                         codes, L.books, L.scales, x, y, out, in, row_chunks, slice_chunks);
    else if (rpw == 2)
      hipLaunchKernelGGL((gemv_fast_kernel<S, BATCH, 2>), dim3(grid), dim3(kBlock), 0, stream,
                         codes, L.books, L.scales, x, y, out, in, row_chunks, slice_chunks);
    else if constexpr (BATCH <= 2)
      hipLaunchKernelGGL((gemv_fast_kernel<S, BATCH, 4>), dim3(grid), dim3(kBlock), 0, stream,
                         codes, L.books, L.scales, x, y, out, in, row_chunks, slice_chunks);
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
  if (gemv_2x8_mfma_fits(L, batch)) return launch_gemv_2x8_mfma(L, x, batch, y, stream);
  if (gemv_uses_gemm_tiles(L, batch)) return launch_gemv_as_gemm(L, x, batch, y, stream);
  switch (L.scheme) {
    case Scheme::k2x8: return launch_scheme<Scheme::k2x8>(L, x, batch, y, stream);
    case Scheme::k1x16: return launch_scheme<Scheme::k1x16>(L, x, batch, y, stream);
    case Scheme::k1x16g16: return launch_scheme<Scheme::k1x16g16>(L, x, batch, y, stream);
    case Scheme::kGeneral: return launch_gemv_general(L, x, batch, y, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_batched(const LayerDesc *Ls, const uint16_t *const *xs,
                               uint16_t *const *ys, int n, int batch, hipStream_t stream) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  // 2x8 layers the matrix-core kernel serves go to it, grouped
  bool done_fixed[64];
  std::vector<char> done_heap;
  bool *done = done_fixed;
  if (n > 64) {
    done_heap.assign(n, 0);
    done = reinterpret_cast<bool *>(done_heap.data());
  }
  for (int i = 0; i < n; ++i) done[i] = false;
  {
    const hipError_t e = launch_gemv_2x8_mfma_batched(Ls, xs, ys, n, batch, done, stream);
    if (e != hipSuccess) return e;
  }
  // other layers the grouped lookup kernel serves, bucketed by configuration;
  // the rest run alone
  GroupArgs buckets[6];
  for (int c = 0; c < 6; ++c) buckets[c].n = 0;
  for (int i = 0; i < n; ++i) {
    if (done[i]) continue;
    const LayerDesc &L = Ls[i];
    const int64_t chunks = L.groups / 8;
    const bool fits32 = (L.out + 4096) * chunks * 16 < ((int64_t)1 << 31) &&
                        L.in * 2 * batch < ((int64_t)1 << 31);
    const int cfg = (L.scheme == Scheme::k2x8 && batch <= 2 && L.groups % 8 == 0 && fits32)
                        ? config_2x8(chunks, batch) : -1;
    if (cfg < 0) {
      const hipError_t e = launch_gemv(L, xs[i], batch, ys[i], stream);
      if (e != hipSuccess) return e;
      continue;
    }
    GroupArgs &b = buckets[cfg];
    b.slot[b.n] = GroupSlot{static_cast<const uint8_t *>(L.codes), L.books, L.scales, xs[i], ys[i],
                            (int)L.out, (int)L.in, (int)chunks, 0, 0};
    if (++b.n == kMaxGroup) {
      const hipError_t e = batch == 1 ? launch_group<1>(cfg, b, cus, stream)
                                      : launch_group<2>(cfg, b, cus, stream);
      if (e != hipSuccess) return e;
      b.n = 0;
    }
  }
  for (int c = 0; c < 6; ++c) {
    if (buckets[c].n == 0) continue;
    const hipError_t e = batch == 1 ? launch_group<1>(c, buckets[c], cus, stream)
                                    : launch_group<2>(c, buckets[c], cus, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The codebook-sliced kernel pays a fixed cost per call (staging each
// member's 128 KiB of codewords, a second launch for the sums) and then runs
// about 1.5x faster per code than the gather kernel: it wins from about 2^22
// codes (8 MiB) in the call's eligible layers (a 4096x4096 layer alone is
// 2^21). Below that the call runs the gather kernel.
constexpr int64_t kSliceMinCallCodes = int64_t(1) << 22;

bool call_uses_slices(const LayerDesc *Ls, int n, int batch) {
  int64_t codes = 0;
  for (int i = 0; i < n; ++i)
    if (gemv_slice_fits(Ls[i], batch)) codes += Ls[i].out * Ls[i].groups;
  return codes >= kSliceMinCallCodes;
}

int64_t gemv_ws_bytes(const LayerDesc *Ls, int n, int batch) {
  if (!call_uses_slices(Ls, n, batch)) return 0;
  int64_t total = 0;
  for (int i = 0; i < n; ++i)
    if (gemv_slice_fits(Ls[i], batch)) total += gemv_slice_ws_bytes(Ls[i]);
  return total;
}

hipError_t launch_gemv_batched_ws(const LayerDesc *Ls, const uint16_t *const *xs,
                                  uint16_t *const *ys, int n, int batch, void *ws,
                                  hipStream_t stream) {
  if (!call_uses_slices(Ls, n, batch)) return launch_gemv_batched(Ls, xs, ys, n, batch, stream);
  // sliced layers: up to 16 per launch, each with its part of the workspace
  constexpr int kGroup = 16;
  const LayerDesc *sel[kGroup];
  const uint16_t *sx[kGroup];
  uint16_t *sy[kGroup];
  float *sp[kGroup];
  int m = 0;
  uint8_t *w = static_cast<uint8_t *>(ws);
  std::vector<LayerDesc> rest_l;
  std::vector<const uint16_t *> rest_x;
  std::vector<uint16_t *> rest_y;
  for (int i = 0; i < n; ++i) {
    if (!gemv_slice_fits(Ls[i], batch)) {
      rest_l.push_back(Ls[i]);
      rest_x.push_back(xs[i]);
      rest_y.push_back(ys[i]);
      continue;
    }
    sel[m] = &Ls[i];
    sx[m] = xs[i];
    sy[m] = ys[i];
    sp[m] = reinterpret_cast<float *>(w);
    w += gemv_slice_ws_bytes(Ls[i]);
    if (++m == kGroup) {
      const hipError_t e = launch_gemv_slice(sel, sx, sy, sp, m, stream);
      if (e != hipSuccess) return e;
      m = 0;
    }
  }
  if (m > 0) {
    const hipError_t e = launch_gemv_slice(sel, sx, sy, sp, m, stream);
    if (e != hipSuccess) return e;
  }
  if (rest_l.empty()) return hipSuccess;
  return launch_gemv_batched(rest_l.data(), rest_x.data(), rest_y.data(), (int)rest_l.size(),
                             batch, stream);
}

}  // namespace aqlm
