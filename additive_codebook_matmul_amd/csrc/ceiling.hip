// Measurement kernels of the benchmark (libaqlm_ceiling.so, not part of the
// product library): the on-chip and HBM ceilings that the GEMV kernels are
// judged against.
//
//   aqlm_ceiling_read    streams `bytes` from a buffer once with 16-byte
//                        non-temporal loads (the pure-read ceiling at a
//                        layer's byte count: what any kernel that reads its
//                        codes once can reach);
//   aqlm_ceiling_gather  random 16-byte loads from a table (the rate at which
//                        a kernel can fetch codewords through the cache
//                        hierarchy, one codeword per lane);
//   aqlm_ceiling_write   writes `bytes` of a buffer once with 16-byte
//                        non-temporal stores (the pure-write ceiling that
//                        the dequant kernel, which writes the dense float16
//                        W, is judged against);
//   aqlm_ceiling_lds     LDS access rates of the patterns the kernels use:
//                        conflict-free and four-address (broadcast) 16-byte
//                        reads, random 8-byte reads from 128 KiB, random
//                        16-byte reads from 8 KiB, conflict-free 16-byte
//                        writes; with the shader clock read inside the
//                        kernel (core-clock counter against the 100 MHz
//                        real-time counter), so rates come out per clock.
//
// Every load feeds a value that a (practically never taken) store to `sink`
// depends on, so nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define CEIL_API extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kThreads = 256;

// One word per block: the XOR of every thread's value.
__device__ __forceinline__ void fold_to_sink(uint32_t acc, uint32_t *sink) {
  __shared__ uint32_t word;
  if (threadIdx.x == 0) word = 0;
  __syncthreads();
  atomicXor(&word, acc);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = word;
}

// Block b reads vectors [b * 256 * U, (b + 1) * 256 * U) of the buffer, U
// coalesced 16-byte non-temporal loads per thread, all in flight before the
// first is used.
template <int U>
__global__ __launch_bounds__(kThreads) void read_kernel(const uint4 *__restrict__ buf, int64_t n16,
                                                        uint32_t *__restrict__ sink) {
  // the resource spans exactly the buffer (below 2 GiB), so offset
  // 0x80000000 is past its end: such a load returns zero and touches no memory
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4 *>(buf), (short)0, (int)(n16 * 16), 0x00020000);
  const int64_t base = (int64_t)blockIdx.x * kThreads * U + threadIdx.x;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, i < n16 ? (uint32_t)(i * 16) : 0x80000000u, 0,
                                                 2);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  // a store that depends on every load (and practically never happens)
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// Random 16-byte entries of a table of 2^log2_entries entries (an LCG per
// lane picks them; every offset is inside the table).
__global__ __launch_bounds__(kThreads) void gather_kernel(const uint4 *__restrict__ table,
                                                          int log2_entries, int per_lane,
                                                          uint32_t *__restrict__ sink) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4 *>(table), (short)0, (int)(16u << log2_entries), 0x00020000);
  const uint32_t mask = (1u << log2_entries) - 1u;
  uint32_t h = (blockIdx.x * kThreads + threadIdx.x) * 2654435761u + 12345u;
  uint32_t acc = 0;
  for (int i = 0; i < per_lane; i += 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      h = h * 1664525u + 1013904223u;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, ((h >> 8) & mask) * 16u, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x + v[u].w;
  }
  fold_to_sink(acc, sink);
}

// Block b writes vectors [b * 256 * U, (b + 1) * 256 * U) of the buffer, U
// coalesced 16-byte non-temporal stores per thread (the stores of the
// dequant kernel).
template <int U>
__global__ __launch_bounds__(kThreads) void write_kernel(uint4 *__restrict__ buf, int64_t n16,
                                                         uint32_t seed) {
  const int64_t base = (int64_t)blockIdx.x * kThreads * U + threadIdx.x;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    if (i < n16) {
      const u32x4 v = {seed ^ (uint32_t)i, seed + (uint32_t)i, (uint32_t)(i >> 32), ~seed};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(buf) + i);
    }
  }
}

// LDS patterns. Every lane keeps 16 offsets into the table in registers (a
// sample of its pattern; the random patterns draw theirs with an LCG at the
// start) and cycles through them; an empty asm statement marks each offset as changed before its use,
// so the accesses stay in the loop, and a read feeds one three-operand add
// per 8 bytes into the lane's fold (every byte of the read is used, so its
// width is kept).
//   0  16-byte reads, lane l at 16 l + 1024 k: the 16 lanes of every pass
//      cover all 64 banks once (the GEMV's A-operand table reads);
//   1  16-byte reads, four addresses per wavefront (lane / 16 picks one):
//      the GEMV's activation fragments at one activation row;
//   2  8-byte reads at random 8-byte entries of a 128 KiB table (the
//      codebook-sliced 1x16 GEMV's lookups);
//   3  16-byte reads at random 16-byte entries of an 8 KiB table (a 2x8
//      codebook copy read by a decode);
//   4  16-byte writes, lane l at 16 l + 1024 k (conflict-free).
constexpr int kLdsOffsets = 16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

template <int MODE>
__global__ __launch_bounds__(1024) void lds_kernel(int iters, uint32_t *__restrict__ sink,
                                                  unsigned long long *__restrict__ clocks) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr uint32_t kBytes = MODE == 2 ? 131072u : MODE == 3 ? 8192u : 65536u;
  const int tid = threadIdx.x, lane = tid & 63;
  for (uint32_t i = (uint32_t)tid * 16u; i < kBytes; i += 1024u * 16u)
    *reinterpret_cast<u32x4 *>(lds + i) = u32x4{i, i ^ 0x55u, i + 7u, ~i};
  const uint32_t base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t *)lds);
  uint32_t off[kLdsOffsets];
  uint32_t h = (blockIdx.x * 1024u + (uint32_t)tid) * 2654435761u + 977u;
  const uint32_t wv = (uint32_t)(tid >> 6);
#pragma unroll
  for (int k = 0; k < kLdsOffsets; ++k) {
    h = h * 1664525u + 1013904223u;
    uint32_t o;
    if (MODE == 0 || MODE == 4)
      o = ((uint32_t)lane * 16u + ((uint32_t)k * 16u + wv) * 1024u) & (kBytes - 1u);
    else if (MODE == 1)
      o = ((uint32_t)(lane >> 4) * 16u + ((uint32_t)k * 16u + wv) * 64u) & (kBytes - 1u);
    else if (MODE == 2)
      o = ((h >> 9) & 16383u) * 8u;
    else
      o = ((h >> 9) & 511u) * 16u;
    off[k] = base + o;
  }
  __syncthreads();
  unsigned long long c0 = 0, r0 = 0;
  if (tid == 0) {
    c0 = clock64();
    r0 = wall_clock64();
  }
  uint32_t acc = 0, acc2 = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kLdsOffsets; ++k) {
      uint32_t a = off[k];
      asm volatile("" : "+v"(a));
      if constexpr (MODE == 4) {
        *reinterpret_cast<lds_u32x4 *>((uintptr_t)a) = u32x4{acc, acc2, 0u, 1u};
        acc += 1u;
      } else if constexpr (MODE == 2) {
        const u32x2 v = *reinterpret_cast<const lds_u32x2 *>((uintptr_t)a);
        acc = v.x + v.y + acc;
      } else {
        const u32x4 v = *reinterpret_cast<const lds_u32x4 *>((uintptr_t)a);
        acc = v.x + v.y + acc;
        acc2 = v.z + v.w + acc2;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    clocks[2 * blockIdx.x] = clock64() - c0;
    clocks[2 * blockIdx.x + 1] = wall_clock64() - r0;
  }
  if ((acc ^ acc2) == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

int cus() {
  int dev = 0, n = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  return n;
}

}  // namespace

// Blocks (and sink words) of the gather launch.
CEIL_API int aqlm_ceiling_blocks(void) { return 8 * cus(); }

// Read `bytes` (a multiple of 16, below 2 GiB) from buf once, per_thread
// (1, 2, 4, 8 or 16) loads of 16 bytes per thread, ceil(bytes / (4096 *
// per_thread)) blocks; sink must hold that many words. 0 on success.
CEIL_API int aqlm_ceiling_read(const void *buf, int64_t bytes, int per_thread, uint32_t *sink,
                               void *stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 || bytes >= ((int64_t)1 << 31)) return 1;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = (n16 + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const uint4 *b = static_cast<const uint4 *>(buf);
  const dim3 grid((unsigned)blocks), block(kThreads);
  switch (per_thread) {
    case 1: hipLaunchKernelGGL(read_kernel<1>, grid, block, 0, st, b, n16, sink); break;
    case 2: hipLaunchKernelGGL(read_kernel<2>, grid, block, 0, st, b, n16, sink); break;
    case 4: hipLaunchKernelGGL(read_kernel<4>, grid, block, 0, st, b, n16, sink); break;
    case 8: hipLaunchKernelGGL(read_kernel<8>, grid, block, 0, st, b, n16, sink); break;
    case 16: hipLaunchKernelGGL(read_kernel<16>, grid, block, 0, st, b, n16, sink); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// per_lane random 16-byte loads (a multiple of 8) by each of
// aqlm_ceiling_blocks() * 256 lanes from a table of 2^log2_entries 16-byte
// entries (log2_entries 4..26). 0 on success.
CEIL_API int aqlm_ceiling_gather(const void *table, int log2_entries, int per_lane,
                                 uint32_t *sink, void *stream) {
  if (!table || !sink || log2_entries < 4 || log2_entries > 26 || per_lane <= 0 || per_lane % 8)
    return 1;
  hipLaunchKernelGGL(gather_kernel, dim3(8 * cus()), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4 *>(table),
                     log2_entries, per_lane, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Write `bytes` (a multiple of 16) of buf once, per_thread (1, 2, 4 or 8)
// stores of 16 bytes per thread, ceil(bytes / (4096 * per_thread)) blocks.
// 0 on success.
CEIL_API int aqlm_ceiling_write(void *buf, int64_t bytes, int per_thread, void *stream) {
  if (!buf || bytes <= 0 || bytes % 16) return 1;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = (n16 + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
  if (blocks >= ((int64_t)1 << 31)) return 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  uint4 *b = static_cast<uint4 *>(buf);
  const dim3 grid((unsigned)blocks), block(kThreads);
  const uint32_t seed = 0x2545F491u;
  switch (per_thread) {
    case 1: hipLaunchKernelGGL(write_kernel<1>, grid, block, 0, st, b, n16, seed); break;
    case 2: hipLaunchKernelGGL(write_kernel<2>, grid, block, 0, st, b, n16, seed); break;
    case 4: hipLaunchKernelGGL(write_kernel<4>, grid, block, 0, st, b, n16, seed); break;
    case 8: hipLaunchKernelGGL(write_kernel<8>, grid, block, 0, st, b, n16, seed); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Dynamic LDS bytes of an aqlm_ceiling_lds mode (0 .. 4), 0 for an unknown
// mode.
CEIL_API int aqlm_ceiling_lds_bytes(int mode) {
  return mode == 2 ? 131072 : mode == 3 ? 8192 : (mode >= 0 && mode <= 4) ? 65536 : 0;
}

// LDS access rate of `mode` (see lds_kernel): `blocks` workgroups of 1024
// threads (sixteen wavefronts; one per CU when `blocks` is the CU count),
// each lane issuing 16 * iters accesses. clocks receives, per block, the
// core-clock cycles and the 100 MHz real-time ticks from just before the
// access loop to the barrier after it (2 * blocks words); sink must hold
// `blocks` words. 0 on success.
CEIL_API int aqlm_ceiling_lds(int mode, int blocks, int iters, uint32_t *sink,
                              unsigned long long *clocks, void *stream) {
  const int bytes = aqlm_ceiling_lds_bytes(mode);
  if (!bytes || blocks <= 0 || iters <= 0 || !sink || !clocks) return 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)blocks), block(1024);
  hipError_t e = hipSuccess;
  switch (mode) {
#define CEIL_LDS_CASE(M)                                                                         \
  case M:                                                                                        \
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(lds_kernel<M>),                       \
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);                  \
    if (e != hipSuccess) return 2;                                                               \
    hipLaunchKernelGGL(lds_kernel<M>, grid, block, bytes, st, iters, sink, clocks);              \
    break;
    CEIL_LDS_CASE(0)
    CEIL_LDS_CASE(1)
    CEIL_LDS_CASE(2)
    CEIL_LDS_CASE(3)
    CEIL_LDS_CASE(4)
#undef CEIL_LDS_CASE
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
