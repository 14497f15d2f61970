// One-token KV append into the block-paged cache.
//
// The new token of each sequence goes to (block, offset) = (slot / BS,
// slot % BS), as in the decode-time K/V write of "tiny-vllm part 5"
// (section on scattering into blocks); the caller resolves the slot (or, for
// the decode step with the VALU partition kernel, the slot is position
// context_lens[i] - 1 through the block table) and one launch writes every
// sequence's K and V rows.  fp8 / int8: the token that opens a block
// (offset 0) sets that block's per-head scale to amax/448 (fp8) or amax/127
// (int8).

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {
namespace {

// Slot of token i: the caller's slot_mapping, or (slots == NULL) position
// context_lens[i] - 1 of sequence i through its block-table row.  -1 = skip.
__device__ __forceinline__ int64_t token_slot(int i, const int32_t* __restrict__ slots,
                                              const int32_t* __restrict__ block_tables,
                                              const int32_t* __restrict__ context_lens, int MBS,
                                              int BS, int NB) {
  if (slots != nullptr) {
    const int64_t s = slots[i];
    return (s >= 0 && s < (int64_t)NB * BS) ? s : -1;
  }
  const int L = context_lens[i];
  if (L < 1 || (int64_t)L > (int64_t)MBS * BS) return -1;
  const int blk = block_tables[(int64_t)i * MBS + (L - 1) / BS];
  if ((unsigned)blk >= (unsigned)NB) return -1;
  return (int64_t)blk * BS + (L - 1) % BS;
}

// bf16: one workgroup per token; each lane copies 16-byte pieces of the
// token's K row (Hkv*D values) or V row.  A bit copy, so trivially exact.
__global__ __launch_bounds__(256) void kv_append_bf16_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int32_t* __restrict__ slots, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int MBS, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, int row_vecs, int BS, int NB) {
  const int i = blockIdx.x;
  for (int c = threadIdx.x; c < 2 * row_vecs; c += blockDim.x) {
    // the row load does not wait for the slot: both latencies overlap
    const bool is_k = c < row_vecs;
    const int cc = is_k ? c : c - row_vecs;
    const uint4 v = (is_k ? k_new : v_new)[(int64_t)i * row_vecs + cc];
    const int64_t slot = token_slot(i, slots, block_tables, context_lens, MBS, BS, NB);
    if (slot < 0) return;
    (is_k ? k_cache : v_cache)[slot * row_vecs + cc] = v;
  }
}

// fp8 / int8: one wave per (token, kv head, K or V).  Lane l holds elements
// l, l + 64, ... of the head's D values.
template <int D, bool INT8>
__global__ __launch_bounds__(64) void kv_append_q8_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int MBS, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, float* __restrict__ k_scale, float* __restrict__ v_scale,
    int Hkv, int BS, int NB) {
  constexpr int PER = D / kWave;
  const int lane = threadIdx.x;
  const int which = blockIdx.x & 1;          // 0 = K, 1 = V
  const int g = (blockIdx.x >> 1) % Hkv;
  const int i = (blockIdx.x >> 1) / Hkv;
  const uint16_t* src = (which ? v_new : k_new) + ((int64_t)i * Hkv + g) * D;
  float x[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) x[k] = __uint_as_float((uint32_t)src[lane + k * kWave] << 16);
  const int64_t slot = token_slot(i, slots, block_tables, context_lens, MBS, BS, NB);
  if (slot < 0) return;
  const int64_t blk = slot / BS;
  const int off = (int)(slot % BS);
  uint8_t* dst = (which ? v_cache : k_cache) + (slot * Hkv + g) * D;
  float* scale_slot = (which ? v_scale : k_scale) + blk * Hkv + g;

  float sc;
  if (off == 0) {
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < PER; ++k) amax = fmaxf(amax, __builtin_fabsf(x[k]));
    amax = wave_max(amax);
    sc = INT8 ? int8_block_scale(amax) : fp8_block_scale(amax);
    if (lane == 0) *scale_slot = sc;
  } else {
    sc = *scale_slot;
  }
#pragma unroll
  for (int k = 0; k < PER; ++k)
    dst[lane + k * kWave] =
        (uint8_t)(INT8 ? int8_encode_scaled(x[k], sc) : fp8_encode_scaled(x[k], sc));
}

}  // namespace

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int32_t* slots,
                            const int32_t* block_tables, const int32_t* context_lens, int MBS,
                            void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                            int N, int Hkv, int D, int BS, int NB, int kind, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  if (kind == kKvBf16) {
    const int row_vecs = Hkv * D / 8;
    hipLaunchKernelGGL(kv_append_bf16_kernel, dim3(N), dim3(256), 0, stream,
                       (const uint4*)k_new, (const uint4*)v_new, slots, block_tables,
                       context_lens, MBS, (uint4*)k_cache, (uint4*)v_cache, row_vecs, BS, NB);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)N * Hkv * 2);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(64), 0, stream, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, slots, block_tables, context_lens, MBS,
                       (uint8_t*)k_cache, (uint8_t*)v_cache, k_scale, v_scale, Hkv, BS, NB);
  };
  const bool i8 = kind == kKvInt8;
  if (D == 128)
    i8 ? launch(kv_append_q8_kernel<128, true>) : launch(kv_append_q8_kernel<128, false>);
  else if (D == 64)
    i8 ? launch(kv_append_q8_kernel<64, true>) : launch(kv_append_q8_kernel<64, false>);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
