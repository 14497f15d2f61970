// Decode-phase paged attention: partition kernel + log-sum-exp merge kernel.
//
// Semantics ("Decode Phase Attention Forward Pass", sections 2-5): one query
// token per sequence attends, with no causal mask, over positions
// t < context_lens[b] of its history; position t lives at
// (block_tables[b][t / BS], t % BS); query head h reads kv head h / G.
// The pages' route gathers the history into a zero-padded dense tensor and
// calls a dense kernel; here nothing is gathered: each wave reads the pages
// in place through the block table and positions past the context length
// are selected away (never weighted by zero, so stale or NaN bytes in a
// block's tail cannot leak in).
//
// Work decomposition (flash-decoding style split of the context).  The work
// axis is every (sequence b, kv head g, page j) triple in that order:
// position Hkv*pre[b] + g*n_b + j, where n_b = ceil(L_b / BS) and pre is the
// prefix sum of n_b.  A persistent grid of W waves cuts this axis into equal
// pieces of Q = ceil(Hkv*pre[B] / W) pages, so every wave streams the same
// number of KV bytes whatever the length mix.  A (b, g) run that one wave
// covers completely is finished in place (out written as bf16); otherwise
// each wave that touches it leaves (m, l, o) for its share in workspace row
// wave + segment, and the merge kernel combines the rows of a segment,
// which are consecutive.
//
// Inside a wave (VALU path): lanes are laid out as TPW token rows of LPT
// lanes; a lane holds 8 consecutive head-dim elements of one token (one
// 16-byte load for bf16, 8 bytes for fp8).  q for the G heads of the group
// sits in registers, so each K/V byte is loaded once for the whole GQA group.
// Per page: partial dot products, a DPP reduction over the LPT lanes of a
// row, online softmax per row in the exp2 domain, PV accumulation.  The TPW
// rows are merged with cross-lane shuffles at the end of a piece.

#include <float.h>

#include <type_traits>

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {
namespace {

template <int D_, int BS_, int G_, bool FP8_>
struct Shape {
  static constexpr int D = D_;
  static constexpr int BS = BS_;
  static constexpr int G = G_;
  static constexpr bool FP8 = FP8_;
  static constexpr int VEC = 8;            // head-dim elements per lane per load
  static constexpr int LPT = D / VEC;      // lanes per token row
  static constexpr int TPW = kWave / LPT;  // token rows per wave-wide load
  static constexpr int LPP = BS / TPW;     // wave-wide loads per page
  static constexpr int EB = FP8 ? 1 : 2;   // bytes per cache element
  using Vec = typename std::conditional<FP8, uint2, uint4>::type;
  static_assert(LPP >= 1 && BS % TPW == 0, "page must hold whole token rows");
};

// Sequence page counts -> exclusive prefix sums in LDS (s_pre[0..B]).
__device__ void build_prefix(const int32_t* __restrict__ context_lens, int B, int BS, int MBS,
                             int32_t* s_pre, int32_t* s_tmp) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int per = (B + nt - 1) / nt;
  const int b0 = tid * per;
  const int b1 = min(B, b0 + per);
  const int max_len = MBS * BS;
  int sum = 0;
  for (int b = b0; b < b1; ++b) {
    const int L = min(max(context_lens[b], 0), max_len);
    sum += (L + BS - 1) / BS;
  }
  s_tmp[tid] = sum;
  __syncthreads();
  // Hillis-Steele inclusive scan of the per-thread sums
  for (int off = 1; off < nt; off <<= 1) {
    const int v = tid >= off ? s_tmp[tid - off] : 0;
    __syncthreads();
    s_tmp[tid] += v;
    __syncthreads();
  }
  int run = tid == 0 ? 0 : s_tmp[tid - 1];
  for (int b = b0; b < b1; ++b) {
    s_pre[b] = run;
    const int L = min(max(context_lens[b], 0), max_len);
    run += (L + BS - 1) / BS;
  }
  if (tid == nt - 1) s_pre[B] = s_tmp[nt - 1];
  __syncthreads();
}

// Last b in [0, B) with Hkv * pre[b] <= x (x < Hkv * pre[B]).
__device__ __forceinline__ int find_sequence(const int32_t* s_pre, int B, int Hkv, int x) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (Hkv * s_pre[mid] <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

template <class S>
__device__ __forceinline__ typename S::Vec load_row(const uint8_t* __restrict__ base) {
  return *reinterpret_cast<const typename S::Vec*>(base);
}

template <class S>
__global__ __launch_bounds__(kAttnBlockThreads) void partition_kernel(const AttnParams p) {
  constexpr int D = S::D, BS = S::BS, G = S::G, LPT = S::LPT, TPW = S::TPW, LPP = S::LPP;
  constexpr int EB = S::EB;
  using Vec = typename S::Vec;

  extern __shared__ int32_t s_pre[];           // [B + 1] then [blockDim] scratch
  int32_t* s_tmp = s_pre + p.B + 1;
  build_prefix(p.context_lens, p.B, BS, p.MBS, s_pre, s_tmp);

  const int Hkv = p.Hkv;
  const int total = Hkv * s_pre[p.B];          // pages over all (b, g)
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= p.B; i += blockDim.x) p.ws_pre[i] = s_pre[i];
  if (total == 0) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = blockIdx.x * (kAttnBlockThreads / kWave) + (threadIdx.x >> 6);
  const int W = p.total_waves;
  const int Q = (total + W - 1) / W;
  int x = wave * Q;
  const int x_end = min(total, x + Q);
  const int r = lane / LPT;                    // token row within a wave-wide load
  const int c = lane % LPT;                    // 8-element chunk of the head dim
  const int64_t row_bytes = (int64_t)Hkv * D * EB;   // one token, all kv heads
  const uint8_t* __restrict__ kc = static_cast<const uint8_t*>(p.k_cache);
  const uint8_t* __restrict__ vc = static_cast<const uint8_t*>(p.v_cache);
  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(p.q);

  while (x < x_end) {
    // ---- locate the (sequence, kv head) run containing x ----------------
    const int b = find_sequence(s_pre, p.B, Hkv, x);
    const int n_b = s_pre[b + 1] - s_pre[b];
    const int seg_start = Hkv * s_pre[b];
    const int g = (x - seg_start) / n_b;
    const int run_start = seg_start + g * n_b;
    const int j0 = x - run_start;
    const int j1 = min(n_b, x_end - run_start);
    const int L = min(max(p.context_lens[b], 0), p.MBS * BS);
    const int32_t* bt_row = p.block_tables + (int64_t)b * p.MBS;
    const int64_t head_off = (int64_t)g * D * EB + c * S::VEC * EB;

    // ---- q of the G heads, pre-scaled into the exp2 domain ---------------
    float qf[G][8];
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
      const uint4 qv = *reinterpret_cast<const uint4*>(
          qp + ((int64_t)b * p.Hq + g * G + jj) * D + c * 8);
      unpack8(qv, qf[jj]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[jj][e] *= p.scale_log2;
    }

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
      m[jj] = -FLT_MAX;
      l[jj] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[jj][e] = 0.0f;
    }

    // ---- stream the pages j0 .. j1-1 -------------------------------------
    for (int jc = j0; jc < j1; jc += kWave) {
      // this chunk's block ids, one per lane (clamped into the pool)
      const int nchunk = min(kWave, j1 - jc);
      int phys_l = 0;
      if (lane < nchunk) {
        const int v = bt_row[jc + lane];
        phys_l = ((unsigned)v < (unsigned)p.NB) ? v : 0;
      }
      Vec kb[2][LPP], vb[2][LPP];
      float ksc[2], vsc[2];
      auto issue = [&](int k, int buf) {
        const int phys = __builtin_amdgcn_readlane(phys_l, k);
        const uint8_t* kpage = kc + (int64_t)phys * BS * row_bytes + head_off;
        const uint8_t* vpage = vc + (int64_t)phys * BS * row_bytes + head_off;
#pragma unroll
        for (int sl = 0; sl < LPP; ++sl) {
          const int64_t o = (int64_t)(sl * TPW + r) * row_bytes;
          kb[buf][sl] = load_row<S>(kpage + o);
          vb[buf][sl] = load_row<S>(vpage + o);
        }
        if constexpr (S::FP8) {
          ksc[buf] = p.k_scale[(int64_t)phys * Hkv + g];
          vsc[buf] = p.v_scale[(int64_t)phys * Hkv + g];
        }
      };
      auto consume = [&](int k, int buf) {
        const int tok0 = (jc + k) * BS;        // first position of this page
        const bool tail = tok0 + BS > L;       // only the sequence's last page
        float s[LPP][G];
#pragma unroll
        for (int sl = 0; sl < LPP; ++sl) {
          float kf[8];
          unpack8(kb[buf][sl], kf);
#pragma unroll
          for (int jj = 0; jj < G; ++jj) {
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d = fmaf(qf[jj][e], kf[e], d);
            s[sl][jj] = group_sum<LPT>(d);
          }
        }
        if constexpr (S::FP8) {
#pragma unroll
          for (int sl = 0; sl < LPP; ++sl)
#pragma unroll
            for (int jj = 0; jj < G; ++jj) s[sl][jj] *= ksc[buf];
        }
        if (tail) {
#pragma unroll
          for (int sl = 0; sl < LPP; ++sl)
            if (tok0 + sl * TPW + r >= L)
#pragma unroll
              for (int jj = 0; jj < G; ++jj) s[sl][jj] = -INFINITY;
        }
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
          float mx = m[jj];
#pragma unroll
          for (int sl = 0; sl < LPP; ++sl) mx = fmaxf(mx, s[sl][jj]);
          const float alpha = fast_exp2(m[jj] - mx);
          m[jj] = mx;
          l[jj] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[jj][e] *= alpha;
        }
#pragma unroll
        for (int sl = 0; sl < LPP; ++sl) {
          float vf[8];
          unpack8(vb[buf][sl], vf);
          if (tail && tok0 + sl * TPW + r >= L) {
#pragma unroll
            for (int e = 0; e < 8; ++e) vf[e] = 0.0f;
          }
#pragma unroll
          for (int jj = 0; jj < G; ++jj) {
            const float pr = fast_exp2(s[sl][jj] - m[jj]);
            l[jj] += pr;
            const float pv = S::FP8 ? pr * vsc[buf] : pr;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[jj][e] = fmaf(pv, vf[e], acc[jj][e]);
          }
        }
      };
      // two-deep software pipeline: the next page's loads are in flight
      // while the current one is consumed
      issue(0, 0);
      int k = 0;
      for (; k + 1 < nchunk; k += 2) {
        issue(k + 1, 1);
        consume(k, 0);
        if (k + 2 < nchunk) issue(k + 2, 0);
        consume(k + 1, 1);
      }
      if (k < nchunk) consume(k, 0);
    }

    // ---- merge the TPW token rows of the wave -----------------------------
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
      for (int jj = 0; jj < G; ++jj) {
        const float mo = __shfl_xor(m[jj], off);
        const float lo = __shfl_xor(l[jj], off);
        const float mn = fmaxf(m[jj], mo);
        const float f1 = fast_exp2(m[jj] - mn);
        const float f2 = fast_exp2(mo - mn);
        l[jj] = l[jj] * f1 + lo * f2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ao = __shfl_xor(acc[jj][e], off);
          acc[jj][e] = acc[jj][e] * f1 + ao * f2;
        }
        m[jj] = mn;
      }
    }

    // ---- write: final bf16 output, or this wave's share -------------------
    if (lane < LPT) {
      const int seg = b * Hkv + g;
      if (j0 == 0 && j1 == n_b) {
        uint16_t* op = static_cast<uint16_t*>(p.out);
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
          const float inv = 1.0f / l[jj];
          uint4 o;
          o.x = pack_bf16x2(acc[jj][0] * inv, acc[jj][1] * inv);
          o.y = pack_bf16x2(acc[jj][2] * inv, acc[jj][3] * inv);
          o.z = pack_bf16x2(acc[jj][4] * inv, acc[jj][5] * inv);
          o.w = pack_bf16x2(acc[jj][6] * inv, acc[jj][7] * inv);
          *reinterpret_cast<uint4*>(op + ((int64_t)b * p.Hq + g * G + jj) * D + c * 8) = o;
        }
      } else {
        const int64_t row = (int64_t)wave + seg;
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
          float4* dst = reinterpret_cast<float4*>(p.ws_o + (row * G + jj) * D + c * 8);
          dst[0] = make_float4(acc[jj][0], acc[jj][1], acc[jj][2], acc[jj][3]);
          dst[1] = make_float4(acc[jj][4], acc[jj][5], acc[jj][6], acc[jj][7]);
          if (c == 0)
            *reinterpret_cast<float2*>(p.ws_ml + (row * G + jj) * 2) = make_float2(m[jj], l[jj]);
        }
      }
    }
    x = run_start + j1;
  }
}

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

template <class S>
void* partition_fn() {
  return reinterpret_cast<void*>(&partition_kernel<S>);
}

// Dispatch over the supported (D, BS, G, fp8) set.
template <class F>
bool dispatch(int D, int BS, int G, bool fp8, F&& f) {
#define PKV_CASE(d, bs, gg, f8)                                    \
  if (D == d && BS == bs && G == gg && fp8 == f8) {                \
    f(Shape<d, bs, gg, f8>{});                                     \
    return true;                                                   \
  }
#define PKV_G(d, bs, f8) PKV_CASE(d, bs, 1, f8) PKV_CASE(d, bs, 2, f8) PKV_CASE(d, bs, 4, f8) PKV_CASE(d, bs, 8, f8)
#define PKV_BS(d, f8) PKV_G(d, 16, f8) PKV_G(d, 32, f8)
  PKV_BS(64, false) PKV_BS(128, false) PKV_BS(64, true) PKV_BS(128, true)
#undef PKV_BS
#undef PKV_G
#undef PKV_CASE
  return false;
}

}  // namespace

size_t partition_lds_bytes(int B) {
  return sizeof(int32_t) * ((size_t)B + 1 + kAttnBlockThreads);
}

int partition_blocks_per_cu(int D, int BS, int G, bool fp8, size_t lds_bytes) {
  int blocks = 0;
  const bool ok = dispatch(D, BS, G, fp8, [&](auto s) {
    using S = decltype(s);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, partition_kernel<S>,
                                                     kAttnBlockThreads, lds_bytes) != hipSuccess)
      blocks = 0;
  });
  return ok ? blocks : 0;
}

hipError_t launch_partition(const AttnParams& p, int D, int BS, int G, bool fp8, int blocks,
                            hipStream_t stream) {
  const size_t lds = partition_lds_bytes(p.B);
  const bool ok = dispatch(D, BS, G, fp8, [&](auto s) {
    using S = decltype(s);
    hipLaunchKernelGGL(partition_kernel<S>, dim3(blocks), dim3(kAttnBlockThreads), lds, stream, p);
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

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
