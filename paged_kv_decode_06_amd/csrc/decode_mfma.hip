// Partition kernel, MFMA variant.
//
// The GQA group is the N dimension of both matrix products, so one wave
// serves all G <= 16 query heads of a kv head with the matrix cores and
// each K/V byte is read once per group:
//
//   scores  S^T[t][h] = sum_d K[t][d] q[h][d]       16x16x32 bf16 MFMA,
//           A = a 16-token x 32-dim slice of the K tile, B = the group's q
//           (columns past G are zero)
//   output  O[h][d] += sum_t P[h][t] V[t][d]          16x16x16 bf16 MFMA,
//           A = P in exactly the register layout S^T came out in,
//           B = four tokens of one head dim of the V tile
//
// Lane l (n = l % 16, r = l / 16) ends a score step holding S^T for tokens
// 4r..4r+3 of the tile and head n, which is the A-operand layout of the
// 16x16x16 product, so P never leaves its registers.
//
// Data path per 16-token tile: K and V rows are read from HBM with 16-byte
// non-temporal loads laid out as whole 256-byte runs of consecutive lanes
// (the layout that streams best through the memory system), then staged in
// one LDS buffer per wave as bf16 rows with a padded pitch: K first (read
// back as the A operands, 16 bytes a lane), then V over it (read back with
// the gfx950 transposing LDS read, which hands each lane four tokens of one
// head dim, the B operand of the PV product).  fp8 and int8 codes are widened to
// bf16 exactly on the way into LDS; the per-(block, kv head) K scale then
// multiplies the scores and the V scale is folded into P.
//
// Online softmax: one running max per head (kept by the lanes of column
// n), raised only when a tile brings a larger score; the rescale of O is
// then a wave-uniform branch.  The work split over waves is described in
// decode_common.hpp.
//
// Decode step: with k_new set, the kernel also performs the one-token append
// of each sequence (see park_new_rows), so a step is this kernel plus the merge.

#include <float.h>

#include "decode_common.hpp"

// Build-time tuning knob: waves per SIMD the register budget is cut for.
#ifndef PKV_MFMA_WAVES_PER_EU
#define PKV_MFMA_WAVES_PER_EU 3
#endif

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

template <int D_, int BS_, int G_, int KIND_>
struct MfmaShape {
  static constexpr int D = D_;
  static constexpr int BS = BS_;
  static constexpr int G = G_;
  static constexpr bool Q8 = KIND_ != kKvBf16;    // one-byte codes with per-block scales
  static constexpr bool INT8 = KIND_ == kKvInt8;  // (else fp8 e4m3fn when Q8)
  static constexpr int EB = Q8 ? 1 : 2;         // bytes per cache element
  static constexpr int RB = D * EB;           // bytes of one token's head row in the cache
  static constexpr int LPR = RB / 16;         // lanes per row (16 bytes each)
  static constexpr int RPI = kWave / LPR;     // rows per wave-wide load
  static constexpr int NI = 16 / RPI;         // wave-wide loads per 16-token tile
  static constexpr int NKK = D / 32;          // score k-steps (16x16x32)
  static constexpr int NBN = D / 16;          // output n-blocks (16x16x16)
  static constexpr int SUB = BS / 16;         // 16-token tiles per page
  static constexpr int PITCH = 2 * D + 32;    // LDS row pitch (bytes) of a bf16 tile
  static constexpr bool KV_TOGETHER = 16 * RB <= 2048;   // issue a tile's K and V loads at once
  static_assert(G >= 1 && G <= 16, "the group is the 16-wide N dimension");
  static_assert(NI >= 1 && BS % 16 == 0, "shape");
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

// 16 int8 codes -> 16 bf16 (exact: |code| <= 128 has at most 8 significant bits).
__device__ __forceinline__ void i8x16_to_bf16(const uint4 c, bf16x8_t& lo, bf16x8_t& hi) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    bf16x8_t& dst = k < 2 ? lo : hi;
    const int o = (k & 1) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[o + e] = (__bf16)(float)(int8_t)(w[k] >> (8 * e));
  }
}

template <class S>
__device__ __forceinline__ void q8x16_to_bf16(const uint4 c, bf16x8_t& lo, bf16x8_t& hi) {
  if constexpr (S::INT8)
    i8x16_to_bf16(c, lo, hi);
  else
    fp8x16_to_bf16(c, lo, hi);
}

// Streaming 16-byte load: every KV byte is read once, so it is marked
// non-temporal (probe measurements on this layout: ~10% more bandwidth).
__device__ __forceinline__ uint4 load_nt(const unsigned char* p) {
  const uint32_t* a = reinterpret_cast<const uint32_t*>(p);
  uint4 v;
  v.x = __builtin_nontemporal_load(a + 0);
  v.y = __builtin_nontemporal_load(a + 1);
  v.z = __builtin_nontemporal_load(a + 2);
  v.w = __builtin_nontemporal_load(a + 3);
  return v;
}

typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// Store one 16-token tile (this lane's NI chunks, already in registers) into
// the wave's LDS buffer as bf16 rows of PITCH bytes.  When `zero_dead`, rows
// at or past `live` and rows in [gap_lo, gap_hi) (keys between the sinks and
// the window) are written as zeros (V: P = 0 must meet V = 0, not NaN).
template <class S>
__device__ __forceinline__ void stage_tile(unsigned char* tile, const uint4 (&ch)[S::NI],
                                           int lane, int live, bool zero_dead, int gap_lo = 0,
                                           int gap_hi = 0) {
  const int rr = lane / S::LPR, c = lane % S::LPR;
#pragma unroll
  for (int s = 0; s < S::NI; ++s) {
    const int row = s * S::RPI + rr;
    uint4 v = ch[s];
    if (zero_dead && (row >= live || (row >= gap_lo && row < gap_hi))) v = make_uint4(0, 0, 0, 0);
    unsigned char* dst = tile + row * S::PITCH;
    if constexpr (S::Q8) {
      bf16x8_t lo, hi;
      q8x16_to_bf16<S>(v, lo, hi);
      *reinterpret_cast<bf16x8_t*>(dst + 32 * c) = lo;
      *reinterpret_cast<bf16x8_t*>(dst + 32 * c + 16) = hi;
    } else {
      *reinterpret_cast<uint4*>(dst + 16 * c) = v;
    }
  }
}

// Decode-step append inside the partition kernel.  The tile holding
// position L - 1 of a (sequence, kv head) is read by exactly one wave, the
// one whose piece holds the run's last page.  That wave stores the step's
// new row in the cache and writes the same values over that row of its
// staged tile in LDS (after the tile's own rows: LDS writes of a wave land
// in order), so it attends to what an append before the call would have
// left; no other wave reads the row.  All the work is done early: the new
// rows are loaded beside q at the start of the run, and when the first tile
// of the chunk holding the last page has its loads in flight, the rows are
// encoded (fp8 / int8), stored to the cache and parked in the wave's LDS slot in
// tile format, hidden behind that tile's load latency; the tile holding
// position L - 1 then only copies two rows within LDS.
// fp8 / int8: a token at offset 0 opens its block and sets the block's scale
// to amax / 448 (fp8) or amax / 127 (int8) first; otherwise the block keeps
// its scale (the same arithmetic as the stand-alone append).

// 8 int8 codes -> 8 bf16 (exact).
__device__ __forceinline__ bf16x8_t i8x8_to_bf16(const uint2 c) {
  bf16x8_t r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (__bf16)(float)(int8_t)(c.x >> (8 * e));
    r[4 + e] = (__bf16)(float)(int8_t)(c.y >> (8 * e));
  }
  return r;
}

// 8 e4m3fn codes -> 8 bf16 (exact).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(const uint2 c) {
  bf16x8_t r;
  const uint32_t w[2] = {c.x, c.y};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
    r[4 * k + 0] = (__bf16)a[0];
    r[4 * k + 1] = (__bf16)a[1];
    r[4 * k + 2] = (__bf16)b[0];
    r[4 * k + 3] = (__bf16)b[1];
  }
  return r;
}

// Park the new K and V rows of kv head g in the wave's LDS slot `rows`
// ([K | V], 2 D bytes each, tile format) and store them in the cache rows
// `kdst` / `vdst`.  Lane l < D / 4 holds `part`, the bf16 elements
// 8 l' .. 8 l' + 7 of the K row (l < D / 8, l' = l) or of the V row
// (l' = l - D / 8).  fp8 / int8: `sk` / `sv` come in as the block's scales and
// leave as the scales after the append (set from the rows when `opens`;
// lane 0 then stores them at `skw` / `svw`).
template <class S>
__device__ __forceinline__ void park_new_rows(const uint4 part, int lane, unsigned char* rows,
                                              unsigned char* kdst, unsigned char* vdst,
                                              bool opens, float& sk, float& sv, float* skw,
                                              float* svw) {
  constexpr int D = S::D;
  const bool is_k = lane < D / 8;
  const bool mine = lane < D / 4;
  const int c = is_k ? lane : lane - D / 8;
  if constexpr (S::Q8) {
    float x[8];
    unpack8(part, x);   // lanes past the rows hold zeros
    auto block_scale = [](float amax) {
      return S::INT8 ? int8_block_scale(amax) : fp8_block_scale(amax);
    };
    auto enc = [](float v, float sc) {
      return S::INT8 ? int8_encode_scaled(v, sc) : fp8_encode_scaled(v, sc);
    };
    if (opens) {
      float am = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) am = fmaxf(am, __builtin_fabsf(x[e]));
      const float amk = wave_max(is_k ? am : 0.0f);
      const float amv = wave_max(is_k ? 0.0f : am);
      sk = block_scale(amk);
      sv = block_scale(amv);
      if (lane == 0) {
        *skw = sk;
        *svw = sv;
      }
    }
    const float sc = is_k ? sk : sv;
    uint2 codes;
    codes.x = enc(x[0], sc) | (enc(x[1], sc) << 8) | (enc(x[2], sc) << 16) | (enc(x[3], sc) << 24);
    codes.y = enc(x[4], sc) | (enc(x[5], sc) << 8) | (enc(x[6], sc) << 16) | (enc(x[7], sc) << 24);
    if (mine) {
      *reinterpret_cast<uint2*>((is_k ? kdst : vdst) + 8 * c) = codes;
      *reinterpret_cast<bf16x8_t*>(rows + 16 * lane) =
          S::INT8 ? i8x8_to_bf16(codes) : fp8x8_to_bf16(codes);
    }
  } else {
    if (mine) {
      *reinterpret_cast<uint4*>((is_k ? kdst : vdst) + 16 * c) = part;
      *reinterpret_cast<uint4*>(rows + 16 * lane) = part;
    }
  }
}

// Copy a parked row (2 D bytes in tile format) over row `tr` of the tile.
template <class S>
__device__ __forceinline__ void take_new_row(const unsigned char* row, unsigned char* tile, int tr,
                                             int lane) {
  if (lane < S::D / 8)
    *reinterpret_cast<uint4*>(tile + tr * S::PITCH + 16 * lane) =
        *reinterpret_cast<const uint4*>(row + 16 * lane);
}

// GEN: the generalised call (several queries per sequence, a window); the
// decode instantiations (GEN = false) carry none of its per-lane state.
template <class S, bool GEN>
__global__ __launch_bounds__(kAttnBlockThreads) __attribute__((amdgpu_waves_per_eu(PKV_MFMA_WAVES_PER_EU, PKV_MFMA_WAVES_PER_EU)))
void mfma_partition_kernel(const AttnParams p) {
  constexpr int D = S::D, BS = S::BS, G = S::G, RB = S::RB;
  constexpr int NI = S::NI, RPI = S::RPI, LPR = S::LPR;
  constexpr int NKK = S::NKK, NBN = S::NBN, SUB = S::SUB, PITCH = S::PITCH;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int32_t* s_pre = reinterpret_cast<int32_t*>(smem);       // [B + 1]
  int32_t* s_tmp = s_pre + p.B + 1;                          // [blockDim]
  build_prefix(p, BS, s_pre, s_tmp);

  const int Hkv = p.Hkv;
  const int total = Hkv * s_pre[p.B];
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= p.B; i += blockDim.x) p.ws_pre[i] = s_pre[i];
  if (total == 0) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave_in_block = threadIdx.x >> 6;
  const int wave = blockIdx.x * kAttnWavesPerBlock + wave_in_block;
  const size_t pre_bytes = (sizeof(int32_t) * ((size_t)p.B + 1 + kAttnBlockThreads) + 15) & ~size_t(15);
  constexpr int WAVE_LDS = 16 * PITCH + 4 * D;   // staged tile + the new K and V rows (bf16)
  unsigned char* tile = smem + pre_bytes + (size_t)wave_in_block * WAVE_LDS;
  unsigned char* new_rows = tile + 16 * PITCH;     // [K row | V row], 2 D bytes each

  const int n = lane & 15;        // head column of S^T and O; K row of the A operand
  const int r = lane >> 4;        // 4-token group of S^T rows; 4-head group of O rows
  const WorkSplit split = make_split(total, p.total_waves);
  const int64_t row_bytes = (int64_t)Hkv * RB;
  // this lane's 16-byte chunk of a token row, for the global loads
  const int load_row = lane / LPR;
  const int load_off = 16 * (lane % LPR);
  // tile offsets of the operand reads
  const int k_rd = n * PITCH + 16 * r;                               // + 64 kk
  const int v_rd = (4 * r + (n >> 2)) * PITCH + 8 * (n & 3);         // + 32 nb
  const unsigned char* __restrict__ kc = static_cast<const unsigned char*>(p.k_cache);
  const unsigned char* __restrict__ vc = static_cast<const unsigned char*>(p.v_cache);
  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(p.q);

  run_split(split, wave, [&](int x, const int x_end, const int piece) {
  while (x < x_end) {
    const Piece pc = locate_piece(s_pre, p.B, Hkv, x, x_end);
    const int b = pc.b, g = pc.g;
    const int L_in = p.context_lens[b];
    const int L = min(max(L_in, 0), p.MBS * BS);
    // a length outside [1, MBS * BS] breaks the contract: no append then
    // (the decode step is one query per sequence: never the GEN instantiation)
    const bool append = !GEN && p.k_new != nullptr && L == L_in && L >= 1;
    const int32_t* bt_row = p.block_tables + (int64_t)b * p.MBS;
    const int64_t head_off = (int64_t)g * RB + load_off;
    // query tokens: column n of S^T / row n of O is query n / G, head n % G
    const int ql = GEN ? seq_queries(p, b) : 1;
    const int ncol = G * ql;
    const int r0 = GEN && p.q_start != nullptr ? p.q_start[b] : b;   // first q / out row
    const SeqRange sr = GEN ? seq_range(L, ql, p.sinks, p.window, BS) : SeqRange{0, 0, 0};
    auto table_page = [&](int j) { return !GEN || j < sr.ps ? j : j + sr.gap; };
    // keys column n sees: j <= lim_n (bottom-right causal), and with a window
    // j >= lo_n or j < sinks
    const int lim_n = n < ncol ? L - ql + n / G : -1;
    const int lo_n = lim_n - p.window + 1;
    const bool windowed = GEN && p.window > 0;
    const int gap_end = L - ql - p.window + 1;    // keys in [sinks, gap_end) no query sees

    // q of the group as the B operand: element i of k-step kk is head dim
    // 32 kk + 8 r + i, the same dims the K operand's element i holds
    bf16x8_t qB[NKK];
    {
      const uint16_t* qrow = qp + ((int64_t)(r0 + n / G) * p.Hq + g * G + n % G) * D + 8 * r;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n < ncol) v = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
        qB[kk] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
    // The decode step's new rows when this piece holds the run's last page
    // (loaded beside q; lane l < D / 4 takes 16 bytes of [K row | V row]).
    const bool has_new = append && pc.j1 == pc.n_b;
    uint4 new_part = make_uint4(0, 0, 0, 0);
    if (has_new && lane < D / 4) {
      const int64_t src = ((int64_t)b * Hkv + g) * D;
      new_part = lane < D / 8
                     ? *reinterpret_cast<const uint4*>(p.k_new + src + 8 * lane)
                     : *reinterpret_cast<const uint4*>(p.v_new + src + 8 * (lane - D / 8));
    }
    float new_ksc = 1.0f, new_vsc = 1.0f;   // fp8 / int8: the last block's scales after the append

    float4_t O[NBN];
#pragma unroll
    for (int nb = 0; nb < NBN; ++nb) O[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -FLT_MAX;   // running max of head n (exp2 domain)
    float l_run = 0.0f;       // this lane's share of head n's sum

    for (int jc = pc.j0; jc < pc.j1; jc += kWave) {
      const int nchunk = min(kWave, pc.j1 - jc);
      int phys_l = 0;
      bool valid_l = false;
      if (lane < nchunk) {
        const int v = bt_row[table_page(jc + lane)];
        valid_l = (unsigned)v < (unsigned)p.NB;
        phys_l = valid_l ? v : 0;
      }
      const uint64_t valid = __builtin_amdgcn_ballot_w64(valid_l);   // pages with a real block id
      const int k_last = pc.n_b - 1 - jc;             // the run's last page in this chunk, if < nchunk
      const bool new_here = has_new && k_last < nchunk && ((valid >> k_last) & 1);
      uint4 kb[NI], vb[NI];
      float ksc = 1.0f, vsc = 1.0f;
      // one unit = one 16-token tile: page k of the chunk, tile sb.  Bytes
      // in flight per wave: a 4 KB half tile (bf16, D = 128) is enough on
      // its own, so its V loads are issued only once the K loads have
      // landed (issuing both at once measured ~7% slower); 2 KB halves
      // (fp8 / int8, or D = 64) issue K and V together (~3% faster than in turn).
      // The other waves of the CU overlap their compute with the waits;
      // issuing the next tile early does not pay for the registers it costs.
      auto tile_base = [&](int u) {
        const int k = u / SUB, sb = u % SUB;
        const int phys = __builtin_amdgcn_readlane(phys_l, k);
        return ((int64_t)phys * BS + sb * 16 + load_row) * row_bytes + head_off;
      };
      auto issue = [&](const unsigned char* __restrict__ src, int64_t base, uint4 (&ch)[NI]) {
#pragma unroll
        for (int s = 0; s < NI; ++s) ch[s] = load_nt(src + base + (int64_t)s * RPI * row_bytes);
      };
      const int nunits = nchunk * SUB;
      for (int u = 0; u < nunits; ++u) {
        const int k = u / SUB, sb = u % SUB;
        const int tok0 = table_page(jc + k) * BS + sb * 16;   // position of the tile's first token
        const int live = L - tok0;                  // rows of the tile inside the history
        // the decode step's new token goes to row live - 1 of this tile
        const bool new_tile = new_here && k == k_last && live >= 1 && live <= 16;
        const int64_t base = tile_base(u);
        issue(kc, base, kb);
        if constexpr (S::KV_TOGETHER) issue(vc, base, vb);
        if (new_here && u == 0) {   // park the new rows while this tile's loads fly
          const int blk = __builtin_amdgcn_readlane(phys_l, k_last);
          const int off = (L - 1) % BS;
          const int64_t row = ((int64_t)blk * BS + off) * row_bytes + (int64_t)g * RB;
          const int64_t sslot = (int64_t)blk * Hkv + g;
          if constexpr (S::Q8) {
            if (off != 0) {
              new_ksc = p.k_scale[sslot];
              new_vsc = p.v_scale[sslot];
            }
          }
          park_new_rows<S>(new_part, lane, new_rows, p.k_cache_w + row, p.v_cache_w + row,
                           off == 0, new_ksc, new_vsc, p.k_scale_w + sslot, p.v_scale_w + sslot);
        }
        if constexpr (S::Q8) {
          const int phys = __builtin_amdgcn_readlane(phys_l, k);
          ksc = p.k_scale[(int64_t)phys * Hkv + g];
          vsc = p.v_scale[(int64_t)phys * Hkv + g];
        }

        // K tile -> LDS -> A operands; scores S^T (16 tokens x 16 heads)
        stage_tile<S>(tile, kb, lane, live, false);
        if (new_tile) {
          take_new_row<S>(new_rows, tile, live - 1, lane);
          if constexpr (S::Q8) {
            ksc = new_ksc;
            vsc = new_vsc;
          }
        }
        if constexpr (!S::KV_TOGETHER) {
          __builtin_amdgcn_sched_barrier(0);   // keep the V loads behind the K wait
          issue(vc, base, vb);
        }
        float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(tile + k_rd + 64 * kk);
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qB[kk], s, 0, 0, 0);
        }
        const float c = S::Q8 ? p.scale_log2 * ksc : p.scale_log2;
        // rows past a_rel are in column n's future (decode: past the history)
        const int a_rel = GEN ? lim_n - tok0 : live - 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[i] *= c;
          if (4 * r + i > a_rel) s[i] = -INFINITY;
        }
        if (windowed) {
          const int lo_rel = lo_n - tok0, sk_rel = p.sinks - tok0;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * r + i < lo_rel && 4 * r + i >= sk_rel) s[i] = -INFINITY;
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
        short4_t pa;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pr = fast_exp2(s[i] - m_run);
          l_run += pr;
          pa[i] = bf16_bits(S::Q8 ? pr * vsc : pr);
        }

        // V tile -> the same LDS buffer (its K reads are done, LDS is in
        // order within a wave) -> transposed B operands, O += P V
        if (windowed)
          stage_tile<S>(tile, vb, lane, live, true, p.sinks - tok0, gap_end - tok0);
        else
          stage_tile<S>(tile, vb, lane, live, true);
        if (new_tile) take_new_row<S>(new_rows + 2 * D, tile, live - 1, lane);
#pragma unroll
        for (int nb = 0; nb < NBN; ++nb) {
          // (C-style cast: generic -> LDS address space)
          const short4_t vB =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(tile + v_rd + 32 * nb));
          O[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vB, O[nb], 0, 0, 0);
        }
      }
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
        const int c = 4 * r + i;   // O row: query c / G, head c % G
        if (c < ncol) {
          // (a query that sees no key gets 0)
          const float inv = !GEN || l_row[i] > 0.0f ? 1.0f / l_row[i] : 0.0f;
          uint16_t* orow = op + ((int64_t)(r0 + c / G) * p.Hq + g * G + c % G) * D + n;
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb)
            orow[16 * nb] = (uint16_t)f32_to_bf16_rne(O[nb][i] * inv);
        }
      }
    } else {
      const int64_t row = (int64_t)piece + seg;
      const int C = p.cols;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 4 * r + i;
        if (c < ncol) {
          float* orow = p.ws_o + (row * C + c) * D + n;
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb) orow[16 * nb] = O[nb][i];
        }
      }
      if (lane < ncol)
        *reinterpret_cast<float2*>(p.ws_ml + (row * C + lane) * 2) = make_float2(m_run, l_tot);
    }
    x = pc.run_start + pc.j1;
  }
  });
}

}  // namespace

size_t mfma_stage_lds_bytes(int D) {
  return (size_t)kAttnWavesPerBlock * (16 * (2 * D + 32) + 4 * D);
}

static size_t mfma_lds_total(int B, int D) {
  return ((prefix_lds_bytes(B) + 15) & ~size_t(15)) + mfma_stage_lds_bytes(D);
}

// Occupancy of the decode instantiation; the generalised one is held to the
// same waves per SIMD (amdgpu_waves_per_eu), so one grid size serves both.
int mfma_blocks_per_cu(int D, int BS, int G, int kind, int B) {
  int blocks = 0, blocks_gen = 0;
  const size_t lds = mfma_lds_total(B, D);
  const bool ok = dispatch_shapes<MfmaShape>(D, BS, G, kind, [&](auto s) {
    using S = decltype(s);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, mfma_partition_kernel<S, false>,
                                                     kAttnBlockThreads, lds) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks_gen, mfma_partition_kernel<S, true>,
                                                     kAttnBlockThreads, lds) != hipSuccess)
      blocks = blocks_gen = 0;
  });
  return ok ? (blocks < blocks_gen ? blocks : blocks_gen) : 0;
}

hipError_t launch_partition_mfma(const AttnParams& p, int D, int BS, int G, int kind, int blocks,
                                 hipStream_t stream) {
  const size_t lds = mfma_lds_total(p.B, D);
  const bool gen = p.q_start != nullptr || p.max_q > 1 || p.window > 0;
  const bool ok = dispatch_shapes<MfmaShape>(D, BS, G, kind, [&](auto s) {
    using S = decltype(s);
    if (gen)
      hipLaunchKernelGGL((mfma_partition_kernel<S, true>), dim3(blocks), dim3(kAttnBlockThreads),
                         lds, stream, p);
    else
      hipLaunchKernelGGL((mfma_partition_kernel<S, false>), dim3(blocks), dim3(kAttnBlockThreads),
                         lds, stream, p);
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
