// Streaming read of a device buffer: the read bandwidth this device reaches
// with 16-byte non-temporal loads and nothing else to do, reported beside
// the attention kernels as the ceiling their KV reads can approach ("Decode
// Phase" glossary: a decode step is bound by the time to read the KV cache,
// cache bytes / memory bandwidth).
//
// A grid of 12 waves per compute unit; wave w reads 1 KB units w, w + W,
// w + 2W, ... of the buffer (64 lanes x 16 bytes), two units per batch, so
// that at any moment the grid reads one contiguous window of the buffer.
// These settings read fastest in a sweep of 4 to 32 waves per compute unit,
// 2 to 8 units per batch and contiguous per-wave segments (a 2 GiB buffer:
// 7.29 TB/s; 7.06-7.18 TB/s for the next best settings; 5.4-6.5 TB/s with
// 16 or more waves and 4 or more units in flight per wave, where the
// requests in flight per compute unit exceed about 32 KB).  Each lane folds what it reads into an
// XOR so the loads cannot be dropped; lane 0 of each wave stores the wave's
// fold to sink[wave].

#include "pkv_internal.hpp"

namespace pkv {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeWavesPerCu = 12;
constexpr int kUnroll = 2;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ buf,
                                                                   size_t units, unsigned* sink) {
  const int lane = threadIdx.x & 63;
  const size_t wave = (size_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  const size_t waves = (size_t)gridDim.x * (kProbeThreads / 64);
  unsigned acc = 0;
  size_t u = wave;
  for (; u + (kUnroll - 1) * waves < units; u += kUnroll * waves) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k)
      v[k] = __builtin_nontemporal_load(buf + (u + k * waves) * 64 + lane);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (; u < units; u += waves) {
    const u32x4 v = __builtin_nontemporal_load(buf + u * 64 + lane);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // (fold the wave's lanes: the sink holds one word per wave)
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if (lane == 0) sink[wave] = acc;
}

}  // namespace

int read_probe_waves(int cu_count) {
  int blocks = 0;   // (the grid is resident at once: 3 workgroups per compute unit must fit)
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, read_probe_kernel, kProbeThreads, 0) !=
          hipSuccess ||
      blocks * (kProbeThreads / 64) < kProbeWavesPerCu)
    return 0;
  return cu_count * kProbeWavesPerCu;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, unsigned* sink, int waves,
                             hipStream_t stream) {
  const size_t units = bytes / 1024;
  if (units == 0 || waves <= 0) return hipSuccess;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)(waves / (kProbeThreads / 64))),
                     dim3(kProbeThreads), 0, stream, static_cast<const u32x4*>(buf), units, sink);
  return hipGetLastError();
}

}  // namespace pkv
