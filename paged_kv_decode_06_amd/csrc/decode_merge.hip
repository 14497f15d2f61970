// Log-sum-exp merge of the partition kernel's per-wave shares.
//
// For a (sequence, query token, query head) whose history was split over
// pieces k0..k1, share p holds m_p (max score, exp2 domain),
// l_p = sum_t exp2(s_t - m_p) and o_p = sum_t exp2(s_t - m_p) v_t over the
// keys the query sees in that piece.  With M = max_p m_p:
//   out = sum_p exp2(m_p - M) o_p / sum_p exp2(m_p - M) l_p,
// which is the softmax over every key the query sees (0 if it sees none).
// Output rows are (b, i, h) for query i < q_len_b.  The partition kernel's
// shares are per (sequence, unit) with a unit of hg adjacent kv heads (the
// UG = hg G query heads u UG .. u UG + UG - 1); the share column of query i,
// head h = u UG + jj is i UG + jj.

#include <float.h>

#include "decode_common.hpp"

namespace pkv {
namespace {

// Merge, one workgroup per (sequence, unit) run and 16 columns: the run's
// shares are rows k0 + seg .. k1 + seg, each holding the unit's `cols`
// columns (more than 16: a second workgroup, blockIdx.y = 1, takes columns
// 16..).  The workgroup is NGRP groups of wcols * TPR threads (TPR = D / DPT);
// in a group, thread t owns dims DPT (t % TPR) .. + DPT - 1 of column
// 16 blockIdx.y + t / TPR,
// and group g folds in shares g, g + NGRP, ..., kBatch at a time: each
// share's (m, l) and o are loaded together (one wait on memory per batch)
// and the running max is rescaled when a batch brings a larger m.  The
// groups then meet in LDS.  With NGRP groups a run of up to NGRP * kBatch
// shares takes one trip to memory after the prefix sums.  Runs of at most 8
// columns take two groups when the partition's waves wrote one share row
// each (the B64 Llama-shaped step's runs then have about 9 shares); with the
// workgroup combine they have about 3, and one group, without the meeting in
// LDS, is faster.
// The run's prefix sums and split are read once for all its columns.
// DPT: dims per thread, 4 or 8 (one group only).  With 8, a workgroup has
// half the threads, so twice as many are resident and a merge of many runs
// takes fewer rounds of its two trips to memory (70B-shaped mix, 1024 runs:
// 8.4 -> 6.5 us; with two column tiles, two workgroups a run: 24.2 -> 17.5
// us; the others level).  Each output element takes the same operations in
// the same order either way.
template <int D, int NGRP, int DPT = 4>
__global__ __launch_bounds__(NGRP * 8 * D / DPT > 16 * D / DPT ? NGRP * 8 * D / DPT : 16 * D / DPT)
void merge_seg_kernel(const AttnParams p, int G) {
  static_assert(DPT == 4 || (DPT == 8 && NGRP == 1), "8 dims per thread: one group");
  constexpr int TPR = D / DPT;                 // threads per column (DPT dims each)
  constexpr int NV = DPT / 4;                  // float4 vectors per thread
  constexpr int kBatch = 8;
  __shared__ float s_acc[NGRP > 1 ? NGRP : 1][NGRP > 1 ? 8 : 1][NGRP > 1 ? D : 1];
  __shared__ float s_den[NGRP > 1 ? NGRP : 1][NGRP > 1 ? 8 : 1];
  __shared__ float s_max[NGRP > 1 ? NGRP : 1][NGRP > 1 ? 8 : 1];
  const int gthreads = blockDim.x / NGRP;      // threads of one group (wcols * TPR)
  const int grp = threadIdx.x / gthreads;
  const int t = threadIdx.x % gthreads;
  const int U = p.Hkv / p.hg;
  const int seg = blockIdx.x;                  // b U + u
  const int b = seg / U, u = seg % U;
  const int cl = t / TPR;                      // column within the workgroup
  const int n = 16 * blockIdx.y + cl;          // column
  const int d4 = (t % TPR) * DPT;
  const int C = p.cols;
  const int UG = p.hg * G;
  const int qi = n / UG;
  const bool live = n < C && qi < seq_queries(p, b);
  const int h = u * UG + n % UG;
  const int32_t* __restrict__ pre = p.ws_pre;
  const int pre_B = pre[p.B], pre_b = pre[b], pre_b1 = pre[b + 1];
  const int n_b = pre_b1 - pre_b;
  const int r0 = p.q_start != nullptr ? p.q_start[b] : b;
  uint16_t* op = static_cast<uint16_t*>(p.out) + ((int64_t)(r0 + qi) * p.Hq + h) * D + d4;
  if (n_b == 0) {                              // empty history: defined as 0
    if (live && grp == 0) {
#pragma unroll
      for (int v = 0; v < NV; ++v) *reinterpret_cast<uint2*>(op + 4 * v) = make_uint2(0, 0);
    }
    return;                                    // (the whole workgroup)
  }
  // (pieces, or with the workgroup or chain combine the workgroups' ranges
  // of kAttnWavesPerBlock pieces, are the share rows' owners)
  const WorkSplit split = make_split(U * pre_B, p.total_waves);
  const int owner = p.wgc || p.chain ? kAttnWavesPerBlock : 1;
  // (n_b counts the run's slots: its pages start p.run_cost slots in)
  const int start = U * pre_b + u * n_b;
  const int k0 = piece_of(split, start + p.run_cost) / owner;
  const int k1 = piece_of(split, start + n_b - 1) / owner;
  if (k0 == k1) return;                        // finished by the partition kernel
  const int P = k1 - k0 + 1;
  const int64_t row0 = (int64_t)k0 + seg;
  const float* __restrict__ ml = p.ws_ml;
  const float* __restrict__ po = p.ws_o;

  float M = -FLT_MAX;
  float4 accv[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) accv[v] = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.0f;
  for (int i0 = grp; i0 < P; i0 += NGRP * kBatch) {
    float2 mlv[kBatch];
    float4 o[kBatch][NV];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = i0 + k * NGRP;
      mlv[k] = make_float2(-FLT_MAX, 0.0f);
#pragma unroll
      for (int v = 0; v < NV; ++v) o[k][v] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (live && i < P) {
        const int64_t row = (row0 + i) * C + n;
        mlv[k] = *reinterpret_cast<const float2*>(ml + row * 2);
#pragma unroll
        for (int v = 0; v < NV; ++v)
          o[k][v] = *reinterpret_cast<const float4*>(po + row * D + d4 + 4 * v);
      }
    }
    float mb = M;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) mb = fmaxf(mb, mlv[k].x);
    const float a = fast_exp2(M - mb);
    den *= a;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      accv[v].x *= a;
      accv[v].y *= a;
      accv[v].z *= a;
      accv[v].w *= a;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = fast_exp2(mlv[k].x - mb);
      den = fmaf(w, mlv[k].y, den);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        accv[v].x = fmaf(w, o[k][v].x, accv[v].x);
        accv[v].y = fmaf(w, o[k][v].y, accv[v].y);
        accv[v].z = fmaf(w, o[k][v].z, accv[v].z);
        accv[v].w = fmaf(w, o[k][v].w, accv[v].w);
      }
    }
    M = mb;
  }
  if constexpr (NGRP > 1) {   // the groups meet in LDS, each brought to the common max
    float4& acc = accv[0];     // (4 dims per thread)
    *reinterpret_cast<float4*>(&s_acc[grp][cl][d4]) = acc;
    if (d4 == 0) {
      s_den[grp][cl] = den;
      s_max[grp][cl] = M;
    }
    __syncthreads();
    if (grp != 0) return;
    float Mt = s_max[0][cl];
#pragma unroll
    for (int q = 1; q < NGRP; ++q) Mt = fmaxf(Mt, s_max[q][cl]);
    acc = make_float4(0.f, 0.f, 0.f, 0.f);
    den = 0.0f;
#pragma unroll
    for (int q = 0; q < NGRP; ++q) {
      const float a = fast_exp2(s_max[q][cl] - Mt);
      const float4 v = *reinterpret_cast<const float4*>(&s_acc[q][cl][d4]);
      acc.x = fmaf(a, v.x, acc.x);
      acc.y = fmaf(a, v.y, acc.y);
      acc.z = fmaf(a, v.z, acc.z);
      acc.w = fmaf(a, v.w, acc.w);
      den = fmaf(a, s_den[q][cl], den);
    }
  }
  if (!live) return;
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;   // 0: the query sees no key
#pragma unroll
  for (int v = 0; v < NV; ++v)
    *reinterpret_cast<uint2*>(op + 4 * v) =
        make_uint2(pack_bf16x2(accv[v].x * inv, accv[v].y * inv),
                   pack_bf16x2(accv[v].z * inv, accv[v].w * inv));
}

// Merge for few rows with many shares each (long contexts): one workgroup
// per (sequence, query head); thread t owns 4 head dims of every NGRP-th
// share, so NGRP shares are read at once, and the groups are combined
// through LDS.
template <int D>
__global__ __launch_bounds__(kAttnBlockThreads) void merge_wide_kernel(const AttnParams p, int G) {
  constexpr int TPR = D / 4;
  constexpr int NGRP = kAttnBlockThreads / TPR;
  __shared__ float s_acc[NGRP][D];
  __shared__ float s_den[NGRP];
  __shared__ float s_max[NGRP];
  const int t = threadIdx.x;
  const int grp = t / TPR;
  const int d4 = (t % TPR) * 4;
  const int64_t bqh = blockIdx.x;
  const int b = (int)(bqh / ((int64_t)p.max_q * p.Hq));
  const int qi = (int)(bqh / p.Hq % p.max_q);
  const int h = (int)(bqh % p.Hq);
  if (qi >= seq_queries(p, b)) return;
  const int UG = p.hg * G;
  const int u = h / UG;
  const int col = qi * UG + h % UG;
  const int C = p.cols;
  const int U = p.Hkv / p.hg;
  const int32_t* __restrict__ pre = p.ws_pre;
  const int pre_B = pre[p.B], pre_b = pre[b], pre_b1 = pre[b + 1];
  const int total = U * pre_B;
  const int n_b = pre_b1 - pre_b;
  const int r0 = p.q_start != nullptr ? p.q_start[b] : b;
  uint16_t* op = static_cast<uint16_t*>(p.out) + ((int64_t)(r0 + qi) * p.Hq + h) * D;
  if (n_b == 0) {
    if (t < TPR) *reinterpret_cast<uint2*>(op + d4) = make_uint2(0, 0);
    return;
  }
  const WorkSplit split = make_split(total, p.total_waves);
  const int owner = p.wgc || p.chain ? kAttnWavesPerBlock : 1;   // (share rows per workgroup: see above)
  // (n_b counts the run's slots: its pages start p.run_cost slots in)
  const int start = U * pre_b + u * n_b;
  const int k0 = piece_of(split, start + p.run_cost) / owner;
  const int k1 = piece_of(split, start + n_b - 1) / owner;
  if (k0 == k1) return;
  const int seg = b * U + u;
  const int P = k1 - k0 + 1;
  const int64_t row0 = (int64_t)k0 + seg;
  const float* __restrict__ ml = p.ws_ml;
  const float* __restrict__ po = p.ws_o;

  // One pass, as in merge_seg_kernel: group `grp` takes shares grp, grp + NGRP,
  // ..., kBatch at a time, with its own running max; the groups meet in LDS,
  // where each is brought to the common max.  (Few workgroups: registers for
  // a deep batch are free, and 16 covers a 128-share row in one trip.)
  constexpr int kBatch = 16;
  float Mg = -FLT_MAX;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.0f;
  for (int i0 = grp; i0 < P; i0 += NGRP * kBatch) {
    float2 mlv[kBatch];
    float4 o[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = i0 + k * NGRP;
      mlv[k] = make_float2(-FLT_MAX, 0.0f);
      o[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < P) {
        const int64_t row = (row0 + i) * C + col;
        mlv[k] = *reinterpret_cast<const float2*>(ml + row * 2);
        o[k] = *reinterpret_cast<const float4*>(po + row * D + d4);
      }
    }
    float mb = Mg;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) mb = fmaxf(mb, mlv[k].x);
    const float a = fast_exp2(Mg - mb);
    den *= a;
    acc.x *= a;
    acc.y *= a;
    acc.z *= a;
    acc.w *= a;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = fast_exp2(mlv[k].x - mb);
      den = fmaf(w, mlv[k].y, den);
      acc.x = fmaf(w, o[k].x, acc.x);
      acc.y = fmaf(w, o[k].y, acc.y);
      acc.z = fmaf(w, o[k].z, acc.z);
      acc.w = fmaf(w, o[k].w, acc.w);
    }
    Mg = mb;
  }
  *reinterpret_cast<float4*>(&s_acc[grp][d4]) = acc;
  if (d4 == 0) {
    s_den[grp] = den;
    s_max[grp] = Mg;
  }
  __syncthreads();
  if (t < TPR) {
    float M = s_max[0];
#pragma unroll
    for (int q = 1; q < NGRP; ++q) M = fmaxf(M, s_max[q]);
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    float dsum = 0.0f;
#pragma unroll
    for (int q = 0; q < NGRP; ++q) {
      const float a = fast_exp2(s_max[q] - M);
      const float4 v = *reinterpret_cast<const float4*>(&s_acc[q][d4]);
      sum.x = fmaf(a, v.x, sum.x);
      sum.y = fmaf(a, v.y, sum.y);
      sum.z = fmaf(a, v.z, sum.z);
      sum.w = fmaf(a, v.w, sum.w);
      dsum = fmaf(a, s_den[q], dsum);
    }
    const float inv = dsum > 0.0f ? 1.0f / dsum : 0.0f;   // 0: the query sees no key
    *reinterpret_cast<uint2*>(op + d4) =
        make_uint2(pack_bf16x2(sum.x * inv, sum.y * inv), pack_bf16x2(sum.z * inv, sum.w * inv));
  }
}

}  // namespace

// Fewer (sequence, query head) rows than this get a workgroup each (they
// are few and have many shares: long contexts); more are merged a run at a
// time.
constexpr int64_t kWideMergeRows = 1024;

hipError_t launch_merge(const AttnParams& p, int D, int G, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.max_q * p.Hq;
  if (rows == 0) return hipSuccess;
  if (rows < kWideMergeRows) {
    if (D == 128)
      hipLaunchKernelGGL(merge_wide_kernel<128>, dim3((unsigned)rows), dim3(kAttnBlockThreads), 0,
                         stream, p, G);
    else if (D == 64)
      hipLaunchKernelGGL(merge_wide_kernel<64>, dim3((unsigned)rows), dim3(kAttnBlockThreads), 0,
                         stream, p, G);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  // (a workgroup per run and 16 columns, D / 4 threads a column; runs of at
  // most 8 columns whose shares were not combined in the partition kernel
  // get two thread groups, which split the shares)
  if (p.cols < 1 || p.cols > 32) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((int64_t)p.B * (p.Hkv / p.hg)), (unsigned)((p.cols + 15) / 16));
  const int wcols = p.cols < 16 ? p.cols : 16;
  const bool two = wcols <= 8 && p.wgc == 0;
  // (one group: 8 dims per thread)
  if (D == 128) {
    if (two)
      hipLaunchKernelGGL((merge_seg_kernel<128, 2>), grid, dim3(2 * wcols * 32), 0, stream, p, G);
    else
      hipLaunchKernelGGL((merge_seg_kernel<128, 1, 8>), grid, dim3(wcols * 16), 0, stream, p, G);
  } else if (D == 64) {
    if (two)
      hipLaunchKernelGGL((merge_seg_kernel<64, 2>), grid, dim3(2 * wcols * 16), 0, stream, p, G);
    else
      hipLaunchKernelGGL((merge_seg_kernel<64, 1, 8>), grid, dim3(wcols * 8), 0, stream, p, G);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
