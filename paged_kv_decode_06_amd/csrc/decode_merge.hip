// Log-sum-exp merge of the partition kernel's per-wave shares.
//
// For a (sequence, query head) whose history was split over waves w0..w1,
// share p holds m_p (max score, exp2 domain), l_p = sum_t exp2(s_t - m_p)
// and o_p = sum_t exp2(s_t - m_p) v_t.  With M = max_p m_p:
//   out = sum_p exp2(m_p - M) o_p / sum_p exp2(m_p - M) l_p,
// which is the softmax over the whole history.

#include <float.h>

#include "decode_common.hpp"

namespace pkv {
namespace {

// Merge: one wave per (sequence, query head).  The rows of a (b, g) run are
// wave + segment for the consecutive waves w0..w1 whose pieces cover it.
template <int D>
__global__ __launch_bounds__(kAttnBlockThreads) void merge_kernel(const AttnParams p, int G) {
  constexpr int PER = D / kWave;               // head-dim elements per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t bh = (int64_t)blockIdx.x * (kAttnBlockThreads / kWave) + (threadIdx.x >> 6);
  if (bh >= (int64_t)p.B * p.Hq) return;
  const int b = (int)(bh / p.Hq);
  const int h = (int)(bh % p.Hq);
  const int g = h / G;
  const int jj = h % G;
  const int Hkv = p.Hkv;
  const int total = Hkv * p.ws_pre[p.B];
  const int n_b = p.ws_pre[b + 1] - p.ws_pre[b];
  uint16_t* op = static_cast<uint16_t*>(p.out) + bh * D;
  if (n_b == 0) {                              // empty history: defined as 0
#pragma unroll
    for (int k = 0; k < PER; ++k) op[lane * PER + k] = 0;
    return;
  }
  const int W = p.total_waves;
  const int Q = (total + W - 1) / W;
  const int start = Hkv * p.ws_pre[b] + g * n_b;
  const int w0 = start / Q;
  const int w1 = (start + n_b - 1) / Q;
  if (w0 == w1) return;                        // finished by the partition kernel
  const int seg = b * Hkv + g;
  const int P = w1 - w0 + 1;
  const int64_t row0 = (int64_t)w0 + seg;

  float M = -FLT_MAX;
  for (int i = lane; i < P; i += kWave) M = fmaxf(M, p.ws_ml[((row0 + i) * G + jj) * 2]);
  M = wave_max(M);

  float num[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) num[k] = 0.0f;
  float den = 0.0f;
  for (int i0 = 0; i0 < P; i0 += kWave) {
    const int n = min(kWave, P - i0);
    float wgt = 0.0f;
    if (lane < n) {
      const float2 ml = *reinterpret_cast<const float2*>(p.ws_ml + ((row0 + i0 + lane) * G + jj) * 2);
      wgt = fast_exp2(ml.x - M);
      den += wgt * ml.y;
    }
    for (int i = 0; i < n; ++i) {
      const float wi = __shfl(wgt, i);
      const float* src = p.ws_o + ((row0 + i0 + i) * G + jj) * D + lane * PER;
#pragma unroll
      for (int k = 0; k < PER; ++k) num[k] = fmaf(wi, src[k], num[k]);
    }
  }
  den = wave_sum(den);
  const float inv = 1.0f / den;
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(op + lane * 2) = pack_bf16x2(num[0] * inv, num[1] * inv);
  } else {
    op[lane] = (uint16_t)f32_to_bf16_rne(num[0] * inv);
  }
}

}  // namespace

hipError_t launch_merge(const AttnParams& p, int D, int G, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.Hq;
  const int waves_per_block = kAttnBlockThreads / kWave;
  const dim3 grid((unsigned)((rows + waves_per_block - 1) / waves_per_block));
  if (rows == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kAttnBlockThreads), 0, stream, p, G);
  else if (D == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(kAttnBlockThreads), 0, stream, p, G);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
