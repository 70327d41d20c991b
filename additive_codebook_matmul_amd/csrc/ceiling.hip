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
//                        W, is judged against).
//
// Every load feeds a value that a (practically never taken) store to `sink`
// depends on, so nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define CEIL_API extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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
