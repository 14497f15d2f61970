// RoPE fused with the one-token KV append.
//
// "tiny-vllm part 5", section "RoPE: one current position, recomputed on
// every call": each head's pairs (x[2i], x[2i+1]) are rotated by the angle
// pos * f_i, with f_i = theta^(-2i/D) and the Llama 3 scaling of the table
// path (frequencies whose wavelength 2 pi / f exceeds original_max /
// low_freq_factor are divided by `factor`; between that and original_max /
// high_freq_factor they are blended linearly in original_max / wavelength).
// The page notes that its decode path recomputes unscaled angles while its
// prefill table is scaled; here one rule serves both (factor = 1 turns the
// scaling off).
//
// The D / 2 frequencies are computed once per call on the host (they depend
// only on D and the parameters) and passed in the kernel arguments.  Grid
// (token, part): part 0 rotates the token's new key heads into LDS and
// appends the rotated key and the value row exactly as the stand-alone
// append does (a bf16 copy, or fp8 / int8 codes with a per-(block, kv head)
// scale); parts 1.. rotate kQHeads query heads each into q_out.  Every
// workgroup first tabulates the cos / sin of the token's D / 2 angles in LDS
// (rope_sincos, pkv_device.hpp; the decode step with RoPE uses the same
// function, so the two paths agree bit for bit).  The angle, cos / sin and
// the rotation are computed in fp64 and the result is rounded once, straight
// from fp64 to bf16 (nearest even).

#include <algorithm>
#include <cmath>

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kQHeads = 8;   // query heads per workgroup

template <int D, int KIND>
__global__ __launch_bounds__(kRopeThreads) void rope_append_kernel(
    const uint32_t* q, uint32_t* q_out, const uint32_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ slots, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ block_tables, int MBS, unsigned char* k_cache,
    unsigned char* v_cache, float* k_scale, float* v_scale, int Hq, int Hkv, int BS, int NB,
    const RopeParams rp) {
  constexpr int HP = D / 2;                   // pairs per head
  __shared__ uint32_t k_rot[8 * HP];          // the token's rotated key heads (Hkv <= 8)
  __shared__ double cs[HP][2];                // cos, sin of pair j's angle (every head's)
  const int i = blockIdx.x;
  const int part = blockIdx.y;
  const int tid = threadIdx.x;
  // positions / slots NULL: token i is the new token of sequence i, at
  // position context_lens[i] - 1 of the sequence ([N, MBS] block table); a
  // length outside [1, MBS * BS] skips its append (q is still rotated)
  const int L = positions == nullptr ? context_lens[i] : 0;
  const double pos = positions != nullptr ? (double)positions[i] : (double)L - 1.0;

  // the angle pos * f_j is one rounded fp64 product, as in the oracle
  for (int j = tid; j < HP; j += kRopeThreads) {
    double sn, c;
    rope_sincos(__dmul_rn(pos, rp.freq[j]), &sn, &c);
    cs[j][0] = c;
    cs[j][1] = sn;
  }
  __syncthreads();

  if (part > 0) {
    // query heads h0 .. h0 + kQHeads - 1 -> q_out (in place allowed: each
    // pair is read, then written)
    const int h0 = (part - 1) * kQHeads;
    const int n = min(kQHeads, Hq - h0) * HP;
    for (int t = tid; t < n; t += kRopeThreads) {
      const int64_t e = ((int64_t)i * Hq + h0) * HP + t;
      q_out[e] = rotate_pair(q[e], cs[t % HP][0], cs[t % HP][1]);
    }
    return;
  }
  // key heads -> LDS
  for (int t = tid; t < Hkv * HP; t += kRopeThreads) {
    k_rot[t] = rotate_pair(k_new[(int64_t)i * Hkv * HP + t], cs[t % HP][0], cs[t % HP][1]);
  }
  __syncthreads();

  int64_t slot = -1;
  if (slots != nullptr) {
    slot = slots[i];
  } else if (L >= 1 && L <= MBS * BS) {
    const int t = L - 1;
    slot = (int64_t)block_tables[(int64_t)i * MBS + t / BS] * BS + t % BS;
  }
  if (slot < 0 || slot >= (int64_t)NB * BS) return;
  const int64_t row = slot * Hkv * D;         // element offset of the slot's row
  if constexpr (KIND == kKvBf16) {
    uint32_t* kd = reinterpret_cast<uint32_t*>(k_cache) + row / 2;
    uint32_t* vd = reinterpret_cast<uint32_t*>(v_cache) + row / 2;
    const uint32_t* vs = reinterpret_cast<const uint32_t*>(v_new) + (int64_t)i * Hkv * HP;
    for (int t = tid; t < Hkv * HP; t += kRopeThreads) {
      kd[t] = k_rot[t];
      vd[t] = vs[t];
    }
  } else {
    // one wave per (kv head, K or V); lane l holds elements l, l + 64, ...
    constexpr int PER = D / kWave;
    const int lane = tid & (kWave - 1);
    const int64_t blk = slot / BS;
    const bool opens = slot % BS == 0;
    for (int job = tid >> 6; job < 2 * Hkv; job += kRopeThreads / kWave) {
      const int g = job >> 1;
      const bool is_v = job & 1;
      float x[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int d = lane + k * kWave;
        const uint32_t bits = is_v ? (uint32_t)v_new[((int64_t)i * Hkv + g) * D + d]
                                   : (k_rot[g * HP + d / 2] >> (16 * (d & 1))) & 0xffffu;
        x[k] = __uint_as_float(bits << 16);
      }
      float* scale_slot = (is_v ? v_scale : k_scale) + blk * Hkv + g;
      float sc;
      if (opens) {
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < PER; ++k) amax = fmaxf(amax, __builtin_fabsf(x[k]));
        amax = wave_max(amax);
        sc = KIND == kKvInt8 ? int8_block_scale(amax) : fp8_block_scale(amax);
        if (lane == 0) *scale_slot = sc;
      } else {
        sc = *scale_slot;
      }
      unsigned char* dst = (is_v ? v_cache : k_cache) + row + (int64_t)g * D;
#pragma unroll
      for (int k = 0; k < PER; ++k)
        dst[lane + k * kWave] = (unsigned char)(KIND == kKvInt8 ? int8_encode_scaled(x[k], sc)
                                                                : fp8_encode_scaled(x[k], sc));
    }
  }
}

}  // namespace

// f_i of pair i < D / 2 (fp64, on the host): theta^(-2i/D), then the Llama 3
// scaling.  Seen from the wavelength lambda = 2 pi / f: the slowdown
// 1 / factor applies in full to pairs whose wavelength is at least
// original_max / low_freq_factor, not at all to those at most original_max /
// high_freq_factor, and between the two the unscaled frequency's share grows
// linearly in original_max / lambda.
void rope_freqs(int D, RopeParams& rp) {
  const double pi = 3.14159265358979323846;
  for (int i = 0; i < D / 2; ++i) {
    const double f = std::pow(rp.theta, -(2.0 * i) / (double)D);
    const double lambda = 2.0 * pi / f;
    const double keep =
        std::min(1.0, std::max(0.0, (rp.original_max / lambda - rp.low_freq_factor) /
                                        (rp.high_freq_factor - rp.low_freq_factor)));
    const double slow = f / rp.factor;
    rp.freq[i] = slow + keep * (f - slow);
  }
}

hipError_t launch_rope_append(const void* q, void* q_out, const void* k_new, const void* v_new,
                              const int32_t* positions, const int32_t* slots, void* k_cache,
                              void* v_cache, float* k_scale, float* v_scale, int N, int Hq,
                              int Hkv, int D, int BS, int NB, int kind, const RopeParams& rp,
                              hipStream_t stream, const int32_t* context_lens,
                              const int32_t* block_tables, int MBS) {
  if (N == 0) return hipSuccess;
  if (Hkv > 8) return hipErrorInvalidValue;
  if ((positions == nullptr) != (slots == nullptr)) return hipErrorInvalidValue;
  if (positions == nullptr && (context_lens == nullptr || block_tables == nullptr || MBS < 1))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)N, 1u + (unsigned)((Hq + kQHeads - 1) / kQHeads));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kRopeThreads), 0, stream, (const uint32_t*)q,
                       (uint32_t*)q_out, (const uint32_t*)k_new, (const uint16_t*)v_new,
                       positions, slots, context_lens, block_tables, MBS,
                       (unsigned char*)k_cache, (unsigned char*)v_cache, k_scale, v_scale, Hq,
                       Hkv, BS, NB, rp);
  };
  if (D == 128) {
    if (kind == kKvBf16) go(rope_append_kernel<128, kKvBf16>);
    else if (kind == kKvFp8) go(rope_append_kernel<128, kKvFp8>);
    else go(rope_append_kernel<128, kKvInt8>);
  } else if (D == 64) {
    if (kind == kKvBf16) go(rope_append_kernel<64, kKvBf16>);
    else if (kind == kKvFp8) go(rope_append_kernel<64, kKvFp8>);
    else go(rope_append_kernel<64, kKvInt8>);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
