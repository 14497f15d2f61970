// Partition kernel, MFMA variant.
//
// The GQA group is the N dimension of both matrix products, so one wave
// serves all G <= 16 query heads of a kv head with the matrix cores and
// each K/V byte is read once per group:
//
//   scores  S^T[t][h] = sum_d K[t][d] q[h][d]       16x16x32 bf16 MFMA:
//           A = 16 tokens x 32 dims of K (straight from the page, one
//           16-byte load per lane), B = the group's q (heads past G are 0)
//   output  O[h][d] += sum_t P[h][t] V[t][d]          16x16x16 bf16 MFMA:
//           A = P in exactly the register layout S^T came out in,
//           B = V read back transposed from an LDS copy of the tile
//
// Lane l (n = l % 16, r = l / 16) ends a score step holding S^T for
// tokens 4r..4r+3 of the 16-token block and head n; that is the A-operand
// layout of the 16x16x16 product, so P never leaves its registers.  V is
// the only operand that needs a transpose (it is contiguous along the head
// dim, the product contracts over tokens), so each 16-token V tile is
// staged in LDS (rows padded to avoid bank conflicts) and read back four
// tokens at a time.
//
// fp8: K and V codes are widened to bf16 exactly (every e4m3fn value is a
// bf16 value) before the products; the per-(block, kv head) K scale
// multiplies the scores and the V scale is folded into P.
//
// Online softmax: one running max per head (kept by the lanes of column
// n), raised only when a block brings a larger score; the rescale of O is
// then a wave-uniform branch.  The work split over waves is described in
// decode_common.hpp.

#include <float.h>

#include "decode_common.hpp"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

template <int D_, int BS_, int G_, bool FP8_>
struct MfmaShape {
  static constexpr int D = D_;
  static constexpr int BS = BS_;
  static constexpr int G = G_;
  static constexpr bool FP8 = FP8_;
  static constexpr int EB = FP8 ? 1 : 2;      // bytes per cache element
  static constexpr int NKK = D / 32;          // score k-steps (16x16x32)
  static constexpr int NBN = D / 16;          // output n-blocks (16x16x16)
  static constexpr int SUB = BS / 16;         // 16-token blocks per page
  static constexpr int CH = D * EB / 64;      // 16-byte loads per lane per 16-token block
  static constexpr int STRIDE = 2 * D + 16;   // LDS pitch (bytes) of a bf16 V tile row
  static_assert(G >= 1 && G <= 16, "the group is the 16-wide N dimension");
  static_assert(CH >= 1 && BS % 16 == 0, "shape");
};

__device__ __forceinline__ short bf16_bits(float x) {
  return __builtin_bit_cast(short, (__bf16)x);
}

// 16 e4m3fn codes -> 16 bf16 (exact).
__device__ __forceinline__ void fp8x16_to_bf16(const uint4 c, bf16x8_t& lo, bf16x8_t& hi) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
    bf16x8_t& dst = k < 2 ? lo : hi;
    const int o = (k & 1) * 4;
    dst[o + 0] = (__bf16)a[0];
    dst[o + 1] = (__bf16)a[1];
    dst[o + 2] = (__bf16)b[0];
    dst[o + 3] = (__bf16)b[1];
  }
}

template <class S>
__global__ __launch_bounds__(kAttnBlockThreads) void mfma_partition_kernel(const AttnParams p) {
  constexpr int D = S::D, BS = S::BS, G = S::G, EB = S::EB;
  constexpr int NKK = S::NKK, NBN = S::NBN, SUB = S::SUB, CH = S::CH, STRIDE = S::STRIDE;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int32_t* s_pre = reinterpret_cast<int32_t*>(smem);       // [B + 1]
  int32_t* s_tmp = s_pre + p.B + 1;                          // [blockDim]
  build_prefix(p.context_lens, p.B, BS, p.MBS, s_pre, s_tmp);

  const int Hkv = p.Hkv;
  const int total = Hkv * s_pre[p.B];
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= p.B; i += blockDim.x) p.ws_pre[i] = s_pre[i];
  if (total == 0) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave_in_block = threadIdx.x >> 6;
  const int wave = blockIdx.x * kAttnWavesPerBlock + wave_in_block;
  const size_t pre_bytes = (sizeof(int32_t) * ((size_t)p.B + 1 + kAttnBlockThreads) + 15) & ~size_t(15);
  unsigned char* vtile = smem + pre_bytes + (size_t)wave_in_block * (16 * STRIDE);

  const int n = lane & 15;        // head column of S^T / O, token row of K and V loads
  const int r = lane >> 4;        // 4-token group of S^T / O rows; 16-byte chunk of a row
  const int W = p.total_waves;
  const int Q = (total + W - 1) / W;
  int x = wave * Q;
  const int x_end = min(total, x + Q);
  const int64_t row_bytes = (int64_t)Hkv * D * EB;
  const unsigned char* __restrict__ kc = static_cast<const unsigned char*>(p.k_cache);
  const unsigned char* __restrict__ vc = static_cast<const unsigned char*>(p.v_cache);
  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(p.q);

  while (x < x_end) {
    const Piece pc = locate_piece(s_pre, p.B, Hkv, x, x_end);
    const int b = pc.b, g = pc.g;
    const int L = min(max(p.context_lens[b], 0), p.MBS * BS);
    const int32_t* bt_row = p.block_tables + (int64_t)b * p.MBS;
    // byte offset of this lane's first chunk inside a token row
    const int64_t lane_off = (int64_t)g * D * EB + 16 * r;

    // ---- q of the group as the B operand of the score product -------------
    // element i of k-step kk holds dim d(kk, r, i):
    //   bf16: 32 kk + 8 r + i        fp8: 64 (kk/2) + 16 r + 8 (kk%2) + i
    // (any fixed permutation of the head dim works as long as K uses it too)
    bf16x8_t qB[NKK];
    {
      const uint16_t* qrow = qp + ((int64_t)b * p.Hq + g * G + n) * D;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int d0 = S::FP8 ? 64 * (kk / 2) + 16 * r + 8 * (kk % 2) : 32 * kk + 8 * r;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n < G) v = *reinterpret_cast<const uint4*>(qrow + d0);
        qB[kk] = __builtin_bit_cast(bf16x8_t, v);
      }
    }

    float4_t O[NBN];
#pragma unroll
    for (int nb = 0; nb < NBN; ++nb) O[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -FLT_MAX;   // running max of head n (exp2 domain)
    float l_run = 0.0f;       // this lane's share of head n's sum

    for (int jc = pc.j0; jc < pc.j1; jc += kWave) {
      const int nchunk = min(kWave, pc.j1 - jc);
      int phys_l = 0;
      if (lane < nchunk) {
        const int v = bt_row[jc + lane];
        phys_l = ((unsigned)v < (unsigned)p.NB) ? v : 0;
      }
      uint4 kb[2][CH], vb[2][CH];
      float ksc[2], vsc[2];
      // one unit = 16 tokens: block k of the chunk, sub-block sb
      auto issue = [&](int u, int buf) {
        const int k = u / SUB, sb = u % SUB;
        const int phys = __builtin_amdgcn_readlane(phys_l, k);
        const int64_t base = ((int64_t)phys * BS + sb * 16 + n) * row_bytes + lane_off;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          kb[buf][j] = *reinterpret_cast<const uint4*>(kc + base + 64 * j);
          vb[buf][j] = *reinterpret_cast<const uint4*>(vc + base + 64 * j);
        }
        if constexpr (S::FP8) {
          ksc[buf] = p.k_scale[(int64_t)phys * Hkv + g];
          vsc[buf] = p.v_scale[(int64_t)phys * Hkv + g];
        }
      };
      auto consume = [&](int u, int buf) {
        const int k = u / SUB, sb = u % SUB;
        const int tok0 = (jc + k) * BS + sb * 16;   // position of the unit's first token
        const bool tail = tok0 + 16 > L;

        // scores: S^T (16 tokens x 16 heads), lane holds tokens 4r..4r+3 of head n
        float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          if constexpr (S::FP8) {
            bf16x8_t lo, hi;
            fp8x16_to_bf16(kb[buf][j], lo, hi);
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, qB[2 * j], s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, qB[2 * j + 1], s, 0, 0, 0);
          } else {
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, kb[buf][j]), qB[j], s, 0, 0, 0);
          }
        }
        const float c = S::FP8 ? p.scale_log2 * ksc[buf] : p.scale_log2;
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] *= c;
        if (tail) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tok0 + 4 * r + i >= L) s[i] = -INFINITY;
        }

        // V tile -> LDS as bf16 rows (token n of the unit); rows past the
        // history are written as zeros so that P = 0 meets V = 0, not NaN
        {
          const bool dead = tail && tok0 + n >= L;
          unsigned char* dst = vtile + n * STRIDE;
#pragma unroll
          for (int j = 0; j < CH; ++j) {
            uint4 v = vb[buf][j];
            if (dead) v = make_uint4(0, 0, 0, 0);
            if constexpr (S::FP8) {
              bf16x8_t lo, hi;
              fp8x16_to_bf16(v, lo, hi);
              const int d0 = 64 * j + 16 * r;
              *reinterpret_cast<bf16x8_t*>(dst + 2 * d0) = lo;
              *reinterpret_cast<bf16x8_t*>(dst + 2 * d0 + 16) = hi;
            } else {
              *reinterpret_cast<uint4*>(dst + 64 * j + 16 * r) = v;
            }
          }
        }

        // online softmax, one max per head (column n)
        float pm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        pm = fmaxf(pm, __shfl_xor(pm, 16));
        pm = fmaxf(pm, __shfl_xor(pm, 32));
        if (__builtin_amdgcn_ballot_w64(pm > m_run) != 0) {
          const float m_new = fmaxf(m_run, pm);
          const float alpha = fast_exp2(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
          // O rows are heads 4r + i: fetch their factors from columns 4r + i
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a = __shfl(alpha, 4 * r + i);
#pragma unroll
            for (int nb = 0; nb < NBN; ++nb) O[nb][i] *= a;
          }
        }
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[i] = fast_exp2(s[i] - m_run);
          l_run += pr[i];
        }
        const float pv = S::FP8 ? vsc[buf] : 1.0f;
        short4_t pa;
#pragma unroll
        for (int i = 0; i < 4; ++i) pa[i] = bf16_bits(pr[i] * pv);

        // O += P V, B operand = V[4r + i][16 nb + n] read back from LDS
        const unsigned char* src = vtile + (4 * r) * STRIDE + 2 * n;
#pragma unroll
        for (int nb = 0; nb < NBN; ++nb) {
          short4_t vB;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vB[i] = *reinterpret_cast<const short*>(src + i * STRIDE + 32 * nb);
          O[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vB, O[nb], 0, 0, 0);
        }
      };
      const int nunits = nchunk * SUB;
      issue(0, 0);
      int u = 0;
      for (; u + 1 < nunits; u += 2) {
        issue(u + 1, 1);
        consume(u, 0);
        if (u + 2 < nunits) issue(u + 2, 0);
        consume(u + 1, 1);
      }
      if (u < nunits) consume(u, 0);
    }

    // ---- finish the piece ---------------------------------------------------
    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);            // head n's sum, in every row group
    float l_row[4];                             // sums of the O rows 4r + i
#pragma unroll
    for (int i = 0; i < 4; ++i) l_row[i] = __shfl(l_tot, 4 * r + i);
    const int seg = b * Hkv + g;
    if (pc.j0 == 0 && pc.j1 == pc.n_b) {
      uint16_t* op = static_cast<uint16_t*>(p.out);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * r + i;
        if (h < G) {
          const float inv = 1.0f / l_row[i];
          uint16_t* orow = op + ((int64_t)b * p.Hq + g * G + h) * D + n;
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb)
            orow[16 * nb] = (uint16_t)f32_to_bf16_rne(O[nb][i] * inv);
        }
      }
    } else {
      const int64_t row = (int64_t)wave + seg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * r + i;
        if (h < G) {
          float* orow = p.ws_o + (row * G + h) * D + n;
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb) orow[16 * nb] = O[nb][i];
        }
      }
      if (lane < G)
        *reinterpret_cast<float2*>(p.ws_ml + (row * G + lane) * 2) = make_float2(m_run, l_tot);
    }
    x = pc.run_start + pc.j1;
  }
}

}  // namespace

size_t mfma_stage_lds_bytes(int D) {
  return (size_t)kAttnWavesPerBlock * 16 * (2 * D + 16);
}

static size_t mfma_lds_total(int B, int D) {
  return ((prefix_lds_bytes(B) + 15) & ~size_t(15)) + mfma_stage_lds_bytes(D);
}

int mfma_blocks_per_cu(int D, int BS, int G, bool fp8, int B) {
  int blocks = 0;
  const size_t lds = mfma_lds_total(B, D);
  const bool ok = dispatch_shapes<MfmaShape>(D, BS, G, fp8, [&](auto s) {
    using S = decltype(s);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, mfma_partition_kernel<S>,
                                                     kAttnBlockThreads, lds) != hipSuccess)
      blocks = 0;
  });
  return ok ? blocks : 0;
}

hipError_t launch_partition_mfma(const AttnParams& p, int D, int BS, int G, bool fp8, int blocks,
                                 hipStream_t stream) {
  const size_t lds = mfma_lds_total(p.B, D);
  const bool ok = dispatch_shapes<MfmaShape>(D, BS, G, fp8, [&](auto s) {
    using S = decltype(s);
    hipLaunchKernelGGL(mfma_partition_kernel<S>, dim3(blocks), dim3(kAttnBlockThreads), lds,
                       stream, p);
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
