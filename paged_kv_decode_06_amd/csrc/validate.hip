// Check of the device-resident inputs of an attention call (a debug aid;
// the hot path trusts them).  The contract ("Decode Phase Attention Forward
// Pass", sections 2-3, for the paging walk): every sequence length L_b lies
// in [1, MBS * BS]; the block-table entries of the pages the history uses
// (j < ceil(L_b / BS)) lie in [0, NB); for fp8 / int8 caches the K and V
// scales of those (block, kv head) pairs are positive finite numbers.
//
// One thread per (sequence, page); the first violation in (sequence, kind,
// page) order is kept with a 64-bit atomic minimum in a word of the caller's
// workspace, which a one-thread kernel first sets to "none".

#include <math.h>

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {
namespace {

constexpr unsigned long long kNone = ~0ull;

__global__ void validate_init(unsigned long long* first) { *first = kNone; }

// key = b << 32 | kind << 28 | j  (kind: 0 length, 1 block id, 2 K scale,
// 3 V scale; j < 2^28 pages)
__global__ __launch_bounds__(256) void validate_kernel(
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, int B, int Hkv, int BS,
    int NB, int MBS, unsigned long long* first) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)B * MBS) return;
  const int b = (int)(i / MBS), j = (int)(i % MBS);
  const int L = context_lens[b];
  auto report = [&](unsigned kind, unsigned jj) {
    atomicMin(first, ((unsigned long long)b << 32) | ((unsigned long long)kind << 28) | jj);
  };
  if (L < 1 || (long long)L > (long long)MBS * BS) {
    if (j == 0) report(0, 0);
    return;
  }
  if ((long long)j * BS >= L) return;   // a page the history does not use
  const int blk = block_tables[(long long)b * MBS + j];
  if (blk < 0 || blk >= NB) {
    report(1, (unsigned)j);
    return;
  }
  if (k_scale != nullptr) {
    for (int g = 0; g < Hkv; ++g) {
      const float ks = k_scale[(long long)blk * Hkv + g];
      const float vs = v_scale[(long long)blk * Hkv + g];
      if (!(ks > 0.0f) || !isfinite(ks)) report(2, (unsigned)j);
      if (!(vs > 0.0f) || !isfinite(vs)) report(3, (unsigned)j);
    }
  }
}

}  // namespace

hipError_t launch_validate(const int32_t* block_tables, const int32_t* context_lens,
                           const float* k_scale, const float* v_scale, int B, int Hkv, int BS,
                           int NB, int MBS, unsigned long long* first, hipStream_t stream) {
  hipLaunchKernelGGL(validate_init, dim3(1), dim3(1), 0, stream, first);
  const long long n = (long long)B * MBS;
  if (n > 0) {
    const unsigned grid = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(validate_kernel, dim3(grid), dim3(256), 0, stream, block_tables,
                       context_lens, k_scale, v_scale, B, Hkv, BS, NB, MBS, first);
  }
  return hipGetLastError();
}

}  // namespace pkv
