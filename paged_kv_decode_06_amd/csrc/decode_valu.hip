// Partition kernel, VALU variant.
//
// Inside a wave, lanes are laid out as TPW token rows of LPT lanes; a lane
// holds 8 consecutive head-dim elements of one token (one 16-byte load for
// bf16, 8 bytes for fp8 / int8).  q for the G heads of the group sits in registers
// as fp32, so each K/V byte is loaded once for the whole GQA group.  Per
// page: partial dot products, a DPP reduction over the LPT lanes of a row,
// online softmax per row in the exp2 domain, PV accumulation with fp32 FMAs.
// The TPW rows are merged with cross-lane shuffles at the end of a piece.
// The work split over waves is described in decode_common.hpp.

#include <float.h>

#include <type_traits>

#include "decode_common.hpp"

namespace pkv {
namespace {

template <int D_, int BS_, int G_, int KIND_>
struct ValuShape {
  static constexpr int D = D_;
  static constexpr int BS = BS_;
  static constexpr int G = G_;
  static constexpr bool Q8 = KIND_ != kKvBf16;    // one-byte codes with per-block scales
  static constexpr bool INT8 = KIND_ == kKvInt8;
  static constexpr int VEC = 8;            // head-dim elements per lane per load
  static constexpr int LPT = D / VEC;      // lanes per token row
  static constexpr int TPW = kWave / LPT;  // token rows per wave-wide load
  static constexpr int LPP = BS / TPW;     // wave-wide loads per page
  static constexpr int EB = Q8 ? 1 : 2;    // bytes per cache element
  using Vec = typename std::conditional<Q8, uint2, uint4>::type;
  static_assert(LPP >= 1 && BS % TPW == 0, "page must hold whole token rows");
};

// Streaming loads: every KV byte is read once, so they are non-temporal.
template <class S>
__device__ __forceinline__ typename S::Vec load_row(const uint8_t* __restrict__ base) {
  const uint32_t* a = reinterpret_cast<const uint32_t*>(base);
  typename S::Vec v;
  v.x = __builtin_nontemporal_load(a + 0);
  v.y = __builtin_nontemporal_load(a + 1);
  if constexpr (!S::Q8) {
    v.z = __builtin_nontemporal_load(a + 2);
    v.w = __builtin_nontemporal_load(a + 3);
  }
  return v;
}

template <class S>
__global__ __launch_bounds__(kAttnBlockThreads) void valu_partition_kernel(const AttnParams p) {
  constexpr int D = S::D, BS = S::BS, G = S::G, LPT = S::LPT, TPW = S::TPW, LPP = S::LPP;
  constexpr int EB = S::EB;
  using Vec = typename S::Vec;

  extern __shared__ int32_t s_pre[];           // [B + 1] then [blockDim] scratch
  int32_t* s_tmp = s_pre + p.B + 1;
  build_prefix(p, BS, s_pre, s_tmp, false);

  const int Hkv = p.Hkv;
  const int total = Hkv * s_pre[p.B];          // pages over all (b, g)
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= p.B; i += blockDim.x) p.ws_pre[i] = s_pre[i];
  if (total == 0) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = blockIdx.x * (kAttnBlockThreads / kWave) + (threadIdx.x >> 6);
  const WorkSplit split = make_split(total, p.total_waves);
  const int r = lane / LPT;                    // token row within a wave-wide load
  const int c = lane % LPT;                    // 8-element chunk of the head dim
  const int64_t row_bytes = (int64_t)Hkv * D * EB;   // one token, all kv heads
  const uint8_t* __restrict__ kc = static_cast<const uint8_t*>(p.k_cache);
  const uint8_t* __restrict__ vc = static_cast<const uint8_t*>(p.v_cache);
  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(p.q);

  run_split(split, wave, [&](int x, const int x_end, const int piece) {
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
        if constexpr (S::Q8) {
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
          if constexpr (S::INT8)
            unpack8_i8(kb[buf][sl], kf);
          else
            unpack8(kb[buf][sl], kf);
#pragma unroll
          for (int jj = 0; jj < G; ++jj) {
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d = fmaf(qf[jj][e], kf[e], d);
            s[sl][jj] = group_sum<LPT>(d);
          }
        }
        if constexpr (S::Q8) {
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
          if constexpr (S::INT8)
            unpack8_i8(vb[buf][sl], vf);
          else
            unpack8(vb[buf][sl], vf);
          if (tail && tok0 + sl * TPW + r >= L) {
#pragma unroll
            for (int e = 0; e < 8; ++e) vf[e] = 0.0f;
          }
#pragma unroll
          for (int jj = 0; jj < G; ++jj) {
            const float pr = fast_exp2(s[sl][jj] - m[jj]);
            l[jj] += pr;
            const float pv = S::Q8 ? pr * vsc[buf] : pr;
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
        const int64_t row = (int64_t)piece + seg;
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
  });
}

}  // namespace

int valu_blocks_per_cu(int D, int BS, int G, int kind, int B) {
  int blocks = 0;
  const size_t lds_bytes = prefix_lds_bytes(B);
  const bool ok = dispatch_shapes<ValuShape>(D, BS, G, kind, [&](auto s) {
    using S = decltype(s);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, valu_partition_kernel<S>,
                                                     kAttnBlockThreads, lds_bytes) != hipSuccess)
      blocks = 0;
  });
  return ok ? blocks : 0;
}

hipError_t launch_partition_valu(const AttnParams& p, int D, int BS, int G, int kind, int blocks,
                                 hipStream_t stream) {
  const size_t lds = prefix_lds_bytes(p.B);
  const bool ok = dispatch_shapes<ValuShape>(D, BS, G, kind, [&](auto s) {
    using S = decltype(s);
    hipLaunchKernelGGL(valu_partition_kernel<S>, dim3(blocks), dim3(kAttnBlockThreads), lds, stream, p);
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
