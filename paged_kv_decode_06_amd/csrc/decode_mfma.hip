// Partition kernel, MFMA variant.
//
// The GQA group is the N dimension of both matrix products, so one wave
// serves all G <= 16 query heads of a kv head with the matrix cores and
// each K/V byte is read once per group:
//
//   scores  S^T[t][h] = sum_d K[t][d] q[h][d]       16x16x32 bf16 MFMA,
//           A = a 16-token x 32-dim slice of the K tile, B = the group's q
//           (columns past G are zero)
//   output  O^T[d][h] += sum_t V[t][d] P[h][t]        16x16x16 bf16 MFMA,
//           A = four tokens of one head dim of the V tile, B = P^T in
//           exactly the register layout S^T came out in (P as two bf16
//           terms, high and low part, one product each: P to 2^-16)
//
// Lane l (n = l % 16, r = l / 16) ends a score step holding S^T for tokens
// 4r..4r+3 of the tile and column n, which is the B-operand layout of the
// 16x16x16 product, so P never leaves its registers; O^T comes out with
// column n in the same lanes, so the softmax rescale of O needs no shuffle.
// In the decode instantiations a wave may serve a unit of HG adjacent kv
// heads at once (their HG * G query heads are the columns; see the kernel).
//
// Data path per 16-token tile: K and V rows are read from HBM with 16-byte
// non-temporal loads laid out as whole runs of consecutive lanes per unit
// row (the layout that streams best through the memory system), then staged
// in one LDS buffer per wave as bf16 rows with a padded pitch: K first (read
// back as the A operands, 16 bytes a lane), then V over it (read back with
// the gfx950 transposing LDS read, which hands each lane four tokens of one
// head dim, the A operand of the PV product).  fp8 and int8 codes are widened
// to bf16 exactly on the way into LDS; the per-(block, kv head) K scale then
// multiplies the scores and the V scale is folded into P.
//
// Online softmax: one running max per column, raised only when a tile
// brings a larger score; the rescale of O is then a wave-uniform branch.
// The work split over waves is described in decode_common.hpp.
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
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// HG: kv heads one wave serves together (a unit).  Their rows sit side by
// side in every cache row, so a unit row is one contiguous run of HG * RB
// bytes; the HG * G query heads of the unit fill the 16 MFMA columns.
template <int D_, int BS_, int G_, int KIND_, int HG_ = 1>
struct MfmaShape {
  static constexpr int D = D_;
  static constexpr int BS = BS_;
  static constexpr int G = G_;
  static constexpr int HG = HG_;
  static constexpr int UG = HG * G;           // query heads of a unit (columns used)
  static constexpr bool Q8 = KIND_ != kKvBf16;    // one-byte codes with per-block scales
  static constexpr bool INT8 = KIND_ == kKvInt8;  // (else fp8 e4m3fn when Q8)
  static constexpr int EB = Q8 ? 1 : 2;         // bytes per cache element
  static constexpr int RB = D * EB;           // bytes of one token's head row in the cache
  static constexpr int URB = HG * RB;         // bytes of one token's unit row
  static constexpr int LPR = URB / 16;        // lanes per unit row (16 bytes each)
  static constexpr int RPI = kWave / LPR;     // rows per wave-wide load
  static constexpr int NI = 16 / RPI;         // wave-wide loads per 16-token tile
  static constexpr int NKK = D / 32;          // score k-steps (16x16x32)
  static constexpr int NBN = D / 16;          // output n-blocks (16x16x16)
  static constexpr int SUB = BS / 16;         // 16-token tiles per page
  static constexpr int PITCH = HG * 2 * D + 32;   // LDS row pitch (bytes) of a bf16 tile
  // issue a tile's K and V loads at once: when a half tile is 2 KB or less,
  // and for int8 units of several heads (4 KB halves; measured 2% faster on
  // a B128 BS32 step, while the same order made fp8 2.5% slower)
  static constexpr bool KV_TOGETHER = 16 * URB <= 2048 || (INT8 && HG > 1);
  // waves per SIMD: a unit of several heads keeps several times the bytes
  // of a one-head tile in flight per wave, and two such waves per SIMD
  // measured faster than three (bf16 D = 128, two heads: 107 vs 111 us on
  // a B64 step), although the registers would fit three
  static constexpr int WPE = HG > 1 ? 2 : PKV_MFMA_WAVES_PER_EU;
  static_assert(UG >= 1 && UG <= 16, "the unit's heads are the 16-wide N dimension");
  static_assert(LPR <= kWave && NI >= 1 && BS % 16 == 0, "shape");
};

__device__ __forceinline__ short bf16_bits(float x) {
  return __builtin_bit_cast(short, (__bf16)x);
}

// Two e4m3fn codes (the low or high half of w) -> two bf16, exactly: every
// e4m3fn value is a bf16 value.  Two routes give the same bits (checked on
// all 65536 code pairs of both halves): the gfx950 scaled conversion with
// scale 1, one instruction, or fp8 -> fp32 pairs then fp32 -> bf16.  Which
// is faster depends on the instantiation (fp8 workload: the first 1.5%
// faster with two-head units, 1.5% slower with one head), so the tile
// widening takes it as a parameter.
template <bool SCALED, bool HIGH>
__device__ __forceinline__ bf16x2_t fp8x2_to_bf16(uint32_t w) {
  if constexpr (SCALED) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH);
  } else {
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HIGH);
    return bf16x2_t{(__bf16)f[0], (__bf16)f[1]};
  }
}

// 16 e4m3fn codes -> 16 bf16 (exact).
template <bool SCALED>
__device__ __forceinline__ void fp8x16_to_bf16(const uint4 c, bf16x8_t& lo, bf16x8_t& hi) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x2_t a = fp8x2_to_bf16<SCALED, false>(w[k]);
    const bf16x2_t b = fp8x2_to_bf16<SCALED, true>(w[k]);
    bf16x8_t& dst = k < 2 ? lo : hi;
    const int o = (k & 1) * 4;
    dst[o + 0] = a[0];
    dst[o + 1] = a[1];
    dst[o + 2] = b[0];
    dst[o + 3] = b[1];
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
    fp8x16_to_bf16<(S::HG > 1)>(c, lo, hi);
}

// Tile loads: buffer loads off a descriptor for the tile's first byte
// (wave-uniform), a 32-bit per-lane offset and a per-load scalar offset, so
// a tile costs one vector register of addressing however many loads it
// takes.  Every KV byte is read once, so the loads are non-temporal (probe
// measurements on this layout: ~10% more bandwidth).  Descriptor: stride 0,
// 2^31 - 1 bytes of range (a tile spans 16 cache rows), 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const unsigned char* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* u = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, 0, 0x7fffffff, 0x00020000);
}

constexpr int kCachePolicyNT = 2;   // the non-temporal bit of the buffer instructions

__device__ __forceinline__ uint4 load_tile_chunk(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCachePolicyNT);
  return make_uint4(v[0], v[1], v[2], v[3]);
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
// position L - 1 of a (sequence, unit) run is read by exactly one wave, the
// one whose piece holds the run's last page.  That wave stores the step's
// new rows (the unit's HG kv heads) in the cache and writes the same values
// over that row of its staged tile in LDS (after the tile's own rows: LDS
// writes of a wave land in order), so it attends to what an append before
// the call would have left; no other wave reads the row.  The work is done
// early: the new rows are loaded beside q at the start of the run, and when
// the first tile of the chunk holding the last page has its loads in flight,
// the rows are encoded (fp8 / int8) and parked in the wave's LDS slot in
// tile format, hidden behind that tile's load latency; the tile holding
// position L - 1 then only copies two unit rows within LDS.  The cache
// stores wait until the run's tiles are all read (store_new_rows).
// fp8 / int8: a token at offset 0 opens its block and sets the block's
// per-head scales to amax / 448 (fp8) or amax / 127 (int8) first; otherwise
// the block keeps its scales (the same arithmetic as the stand-alone append).

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
    const bf16x2_t a = fp8x2_to_bf16<true, false>(w[k]);
    const bf16x2_t b = fp8x2_to_bf16<true, true>(w[k]);
    r[4 * k + 0] = a[0];
    r[4 * k + 1] = a[1];
    r[4 * k + 2] = b[0];
    r[4 * k + 3] = b[1];
  }
  return r;
}

// The new rows of a unit as 16-byte bf16 chunks: chunks [0, CH) are the K
// rows of its HG kv heads (D / 8 chunks each, in head order), [CH, 2 CH) the
// V rows; lane l holds chunks l, l + 64, ... (NP of them).
template <class S>
struct NewRows {
  static constexpr int CH = S::HG * S::D / 8;
  static constexpr int NP = (2 * CH + kWave - 1) / kWave;
};

// Park the unit's new K and V rows in the wave's LDS slot `rows` ([K | V],
// 2 CH chunks, tile format).  fp8 / int8: `ks` / `vs` are the block's scales
// of the unit's heads (read when the token lands inside the block); when it
// opens the block the scales are set from the rows.  `codes_out` leave as
// this lane's encoded chunks and `gsc_out` as the unit's K and V scales after
// the append, for store_new_rows; `sk` / `sv` as the scales of head `mem`.
template <class S>
__device__ __forceinline__ void park_new_rows(const uint4 (&part)[NewRows<S>::NP], int lane,
                                              int mem, unsigned char* rows, bool opens, float& sk,
                                              float& sv, const float* ks, const float* vs,
                                              uint2 (&codes_out)[NewRows<S>::NP],
                                              float (&gsc_out)[2 * S::HG]) {
  constexpr int HG = S::HG, CH = NewRows<S>::CH, NP = NewRows<S>::NP;
  constexpr int CPH = S::D / 8;   // chunks per head row
  if constexpr (S::Q8) {
    auto block_scale = [](float amax) {
      return S::INT8 ? int8_block_scale(amax) : fp8_block_scale(amax);
    };
    auto enc = [](float v, float sc) {
      return S::INT8 ? int8_encode_scaled(v, sc) : fp8_encode_scaled(v, sc);
    };
    float x[NP][8];
    int grp[NP];   // scale group of chunk i: K of head j -> j, V of head j -> HG + j; -1: none
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int q = lane + kWave * i;
      unpack8(part[i], x[i]);
      grp[i] = q < CH ? q / CPH : (q < 2 * CH ? HG + (q - CH) / CPH : -1);
    }
    float gsc[2 * HG];   // the groups' scales after the append (wave-uniform)
    if (opens) {
      float amc[NP];     // amax of chunk i
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        amc[i] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amc[i] = fmaxf(amc[i], __builtin_fabsf(x[i][e]));
      }
#pragma unroll
      for (int gi = 0; gi < 2 * HG; ++gi) {
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < NP; ++i) am = fmaxf(am, grp[i] == gi ? amc[i] : 0.0f);
        gsc[gi] = block_scale(wave_max(am));
      }
    } else {
#pragma unroll
      for (int j = 0; j < HG; ++j) {
        gsc[j] = ks[j];
        gsc[HG + j] = vs[j];
      }
    }
#pragma unroll
    for (int gi = 0; gi < 2 * HG; ++gi) gsc_out[gi] = gsc[gi];
    sk = gsc[0];
    sv = gsc[HG];
#pragma unroll
    for (int j = 1; j < HG; ++j) {
      if (mem == j) {
        sk = gsc[j];
        sv = gsc[HG + j];
      }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      float sc = gsc[0];
#pragma unroll
      for (int gi = 1; gi < 2 * HG; ++gi)
        if (grp[i] == gi) sc = gsc[gi];
      codes_out[i] = make_uint2(0, 0);
      if (grp[i] >= 0) {
        const int q = lane + kWave * i;
        uint2 codes;
        codes.x = enc(x[i][0], sc) | (enc(x[i][1], sc) << 8) | (enc(x[i][2], sc) << 16) |
                  (enc(x[i][3], sc) << 24);
        codes.y = enc(x[i][4], sc) | (enc(x[i][5], sc) << 8) | (enc(x[i][6], sc) << 16) |
                  (enc(x[i][7], sc) << 24);
        codes_out[i] = codes;
        *reinterpret_cast<bf16x8_t*>(rows + 16 * q) =
            S::INT8 ? i8x8_to_bf16(codes) : fp8x8_to_bf16(codes);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int q = lane + kWave * i;
      if (q < 2 * CH) *reinterpret_cast<uint4*>(rows + 16 * q) = part[i];
    }
  }
}

// Store the parked rows in the cache unit rows `kdst` / `vdst` (bf16: the
// rows themselves; fp8 / int8: their codes) and, when the token opened the
// block, the unit's scales in `ksw` / `vsw` (lane 0).  Called once the run's
// tiles have all been read: a wave's memory counter covers stores as well as
// loads, so a store issued earlier would hold up the waits for the tiles
// loaded after it.
template <class S>
__device__ __forceinline__ void store_new_rows(const uint4 (&part)[NewRows<S>::NP],
                                               const uint2 (&codes)[NewRows<S>::NP],
                                               const float (&gsc)[2 * S::HG], int lane,
                                               unsigned char* kdst, unsigned char* vdst,
                                               bool opens, float* ksw, float* vsw) {
  constexpr int HG = S::HG, CH = NewRows<S>::CH, NP = NewRows<S>::NP;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int q = lane + kWave * i;
    if (q < 2 * CH) {
      const bool is_k = q < CH;
      const int c = is_k ? q : q - CH;
      if constexpr (S::Q8)
        *reinterpret_cast<uint2*>((is_k ? kdst : vdst) + 8 * c) = codes[i];
      else
        *reinterpret_cast<uint4*>((is_k ? kdst : vdst) + 16 * c) = part[i];
    }
  }
  if constexpr (S::Q8) {
    if (opens && lane == 0) {
#pragma unroll
      for (int j = 0; j < HG; ++j) {
        ksw[j] = gsc[j];
        vsw[j] = gsc[HG + j];
      }
    }
  }
}

// Copy a parked unit row (HG * 2 D bytes in tile format) over row `tr` of
// the tile.
template <class S>
__device__ __forceinline__ void take_new_row(const unsigned char* row, unsigned char* tile, int tr,
                                             int lane) {
  if (lane < NewRows<S>::CH)
    *reinterpret_cast<uint4*>(tile + tr * S::PITCH + 16 * lane) =
        *reinterpret_cast<const uint4*>(row + 16 * lane);
}

// RoPE inside the decode step: rotate the columns' q (the B operands) and,
// when this piece appends, the unit's new K rows, at position `pos`.  Lane
// j < D / 2 computes the cosine and sine of pair j's angle (pos * f_j, one
// rounded fp64 product; rope_sincos) into the wave's tile buffer, which is free until the
// first tile is staged (LDS accesses of a wave run in order); each lane then
// rotates its pairs with the fp64 arithmetic of the RoPE append kernel, so
// the rotated values are bit for bit those of that kernel.  The q lane (n, r)
// holds dims 32 kk + 8 r .. + 7, pairs 16 kk + 4 r + t; a K chunk c of a
// head row holds dims 8 c .. 8 c + 7, pairs 4 c + t.
template <class S>
__device__ __forceinline__ void rope_rotate(const AttnParams& p, int pos, int lane, int r,
                                            unsigned char* scratch, bf16x8_t (&qB)[S::NKK],
                                            uint4 (&new_part)[NewRows<S>::NP], bool has_new) {
  constexpr int HP = S::D / 2, CH = NewRows<S>::CH, CPH = S::D / 8;
  double2* cs = reinterpret_cast<double2*>(scratch);
  if (lane < HP) {
    double sn, c;
    rope_sincos(__dmul_rn((double)pos, p.rope_freq[lane]), &sn, &c);
    cs[lane] = make_double2(c, sn);
  }
#pragma unroll
  for (int kk = 0; kk < S::NKK; ++kk) {
    uint4 w = __builtin_bit_cast(uint4, qB[kk]);
    uint32_t* e = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const double2 a = cs[16 * kk + 4 * r + t];
      e[t] = rotate_pair(e[t], a.x, a.y);
    }
    qB[kk] = __builtin_bit_cast(bf16x8_t, w);
  }
  if (has_new) {
#pragma unroll
    for (int i = 0; i < NewRows<S>::NP; ++i) {
      const int q = lane + kWave * i;
      if (q < CH) {   // a K chunk
        const int c = q % CPH;
        uint32_t* e = reinterpret_cast<uint32_t*>(&new_part[i]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const double2 a = cs[4 * c + t];
          e[t] = rotate_pair(e[t], a.x, a.y);
        }
      }
    }
  }
}

// Workgroup combine.  The waves of a workgroup stream consecutive pieces,
// so a run that crosses the edge between two of them has its shares there:
// the end share of the earlier piece (the run continues past it) and the
// head share of the later one (or its only share, if the piece lies inside
// the run).  Each wave leaves at most two shares in LDS: a head share (the
// piece starts inside a run and finishes it) in its head slot, and an end
// share (the piece ends inside a run) in its tile buffer, each as o
// [W][D], then m and l [W] (W = p.wgc, the slot's column capacity), with a
// descriptor (segment,
// starts at the run's first page, ends at its last).  After the workgroup
// barrier the shares, in axis order, are grouped by run: a group that starts
// at the run's first page and ends at its last is the whole run, finished
// here (bf16 out); any other is merged into one share row of the workgroup,
// row g + segment, for the merge kernel.  Combining is by the log-sum-exp
// rule of the merge kernel, in a fixed order, so results stay deterministic.
__host__ __device__ constexpr int wgc_slot_bytes(int D, int wcols) {
  return wcols * (D + 2) * (int)sizeof(float);
}

// The parking slot: a 16-column share, o as [D / 16][64 lanes] float4 (each
// lane its own values) and then (m, l) of the columns, or a bf16 output of
// up to 32 columns (as [2][D / 16][64 lanes] uint2).  It overlays the append
// rows (unused by the generalised instantiations) and extends past them.
__host__ __device__ constexpr int park_slot_bytes(int D) { return wgc_slot_bytes(D, 16); }

// Park mode 2 (the chain combine with two column tiles): the parking slot
// moves back so that the wave's first park_slot_bytes(D), from its tile
// buffer on, hold a second 16-column share once the piece's tiles are done;
// this is how far it moves past the tile buffer.
__host__ __device__ constexpr int park_share_ext_bytes(int hg, int D) {
  return park_slot_bytes(D) > 16 * (hg * 2 * D + 32) ? park_slot_bytes(D) - 16 * (hg * 2 * D + 32)
                                                     : 0;
}

// Bytes a wave keeps after its staged tile: the append rows (or the parking
// slot over them, in park mode 2 after the extension) and the combine's
// head slot.
__host__ __device__ constexpr int wave_rows_bytes(int hg, int D, int wgc, int park) {
  return (park == 2 ? park_share_ext_bytes(hg, D) : 0) +
         (park && park_slot_bytes(D) > 4 * hg * D ? park_slot_bytes(D) : 4 * hg * D) +
         wgc_slot_bytes(D, wgc);
}

template <class S, bool GEN>
// s_qs: the query-row offsets in LDS (q_start[0..B]) when qs_lds, which the
// generalised runs read there rather than from memory, where the load would
// wait for the wave's last stores too.
__device__ __forceinline__ void wgc_combine(const AttnParams& p, unsigned char* waves_lds,
                                            int wave_lds, const int* s_desc, int U,
                                            const int32_t* s_qs, bool qs_lds) {
  constexpr int D = S::D, UG = S::UG, G = S::G, HG = S::HG;
  constexpr int TPR = D / 4;                    // threads per column (4 dims each)
  // Share slots in axis order: wave w's head share is slot 2w, its end share
  // slot 2w + 1.  Every slot index below is a constant once the loops are
  // unrolled, so the descriptors stay in registers (an array indexed at run
  // time would live in scratch memory, whose loads wait on the wave's
  // outstanding global stores too).
  constexpr int NS = 2 * kAttnWavesPerBlock;
  __syncthreads();
  int sseg[NS], sflg[NS];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    sseg[sl] = s_desc[2 * sl];
    sflg[sl] = s_desc[2 * sl + 1];
  }
  auto share = [&](int sl) {
    return reinterpret_cast<const float*>(
        waves_lds + (sl / 2) * wave_lds + (sl % 2 == 0 ? 16 * S::PITCH + 32 * NewRows<S>::CH : 0));
  };
  const int t = threadIdx.x;
  const int d4 = (t % TPR) * 4;
  const int W = p.wgc;                          // a slot's column capacity
  int prev = -1;                                // run of the last share seen
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int seg = sseg[i];
    if (seg < 0 || seg == prev) continue;       // no share, or not its run's first
    prev = seg;
    const int b = seg / U, u = seg % U;
    int ql = 1, r0 = b;   // query count, first q / out row
    if constexpr (GEN) {
      if (qs_lds) {
        r0 = s_qs[b];
        ql = min(max(s_qs[b + 1] - r0, 0), p.max_q);
      } else {
        ql = seq_queries(p, b);
        r0 = p.q_start != nullptr ? p.q_start[b] : b;
      }
    }
    // the run's shares are slots i .. last (consecutive: shares are in axis order)
    int last = i;
#pragma unroll
    for (int k = i + 1; k < NS; ++k)
      if (sseg[k] == seg) last = k;
    int lflg = sflg[i];
#pragma unroll
    for (int k = i + 1; k < NS; ++k)
      if (k == last) lflg = sflg[k];
    const bool whole = (sflg[i] & 1) && (lflg & 2);   // the whole run: out
    // (kAttnBlockThreads / TPR columns a pass: 8 at D = 128, 16 at D = 64)
    for (int c = t / TPR; c < UG * ql; c += kAttnBlockThreads / TPR) {
      float M = -FLT_MAX;
#pragma unroll
      for (int k = i; k < NS; ++k)
        if (sseg[k] == seg) M = fmaxf(M, share(k)[W * D + c]);
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      float den = 0.0f;
#pragma unroll
      for (int k = i; k < NS; ++k)
        if (sseg[k] == seg) {
          const float* sh = share(k);
          const float w = fast_exp2(sh[W * D + c] - M);
          const float4 o = *reinterpret_cast<const float4*>(sh + c * D + d4);
          den = fmaf(w, sh[W * D + W + c], den);
          acc.x = fmaf(w, o.x, acc.x);
          acc.y = fmaf(w, o.y, acc.y);
          acc.z = fmaf(w, o.z, acc.z);
          acc.w = fmaf(w, o.w, acc.w);
        }
      if (whole) {
        const float inv = den > 0.0f ? 1.0f / den : 0.0f;   // (0: the query sees no key)
        uint16_t* orow = static_cast<uint16_t*>(p.out) +
                         ((int64_t)(r0 + c / UG) * p.Hq + u * HG * G + c % UG) * D + d4;
        *reinterpret_cast<uint2*>(orow) =
            make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
      } else {                                 // the workgroup's share row of the run
        const int64_t row = (int64_t)blockIdx.x + seg;
        const int C = p.cols;
        *reinterpret_cast<float4*>(p.ws_o + (row * C + c) * D + d4) = acc;
        if (d4 == 0) *reinterpret_cast<float2*>(p.ws_ml + (row * C + c) * 2) = make_float2(M, den);
      }
    }
  }
}

// GEN: the generalised call (several queries per sequence, a window); the
// decode instantiations (GEN = false) carry none of its per-lane state.
// Both may serve several kv heads per wave (S::HG; the generalised call when
// HG * G * max_q <= 16).  ROPE: the decode step with RoPE (instantiated
// apart, so that the other kernels do not carry its registers).
//
// Units of HG > 1 kv heads: the unit's HG * G query heads (times the
// queries per sequence) are the columns, column n reading kv head
// `mem` = (n % UG) / G of the unit.  The scores
// run one MFMA chain per kv head of the unit (K of that head times every
// column's q) and each column keeps its own head's chain; the output runs
// O^T += V_j^T P_j^T per head j with P_j = P restricted to head j's columns,
// so every column sums only its own head's values.
//
// NCT: 16-column tiles a wave serves.  The generalised call with one kv head
// per wave takes up to 32 columns (G * max_q <= 32) as two tiles: column
// c = 16 ct + n of tile ct.  Both tiles' score and output products take the
// same K and V operands, read from LDS once, so the cache is still streamed
// once; each tile keeps its own q operands, O^T accumulators and softmax
// state.
template <class S, bool GEN, bool ROPE = false, int NCT = 1>
__global__ __launch_bounds__(kAttnBlockThreads)
__attribute__((amdgpu_waves_per_eu(NCT > 1 ? 2 : S::WPE, NCT > 1 ? 2 : S::WPE)))
void mfma_partition_kernel(const AttnParams p) {
  constexpr int D = S::D, BS = S::BS, G = S::G, RB = S::RB, HG = S::HG, UG = S::UG;
  constexpr int NI = S::NI, RPI = S::RPI, LPR = S::LPR;
  constexpr int NKK = S::NKK, NBN = S::NBN, SUB = S::SUB, PITCH = S::PITCH;
  constexpr int NP = NewRows<S>::NP, CH = NewRows<S>::CH;
  static_assert(!(GEN && ROPE), "RoPE is fused into the decode step only");
  static_assert(NCT == 1 || (NCT == 2 && GEN && HG == 1), "two column tiles: generalised, one head");
  // P enters the PV product as two bf16 parts (see below).  When the columns
  // fit in 8 of the 16, column n + 8 repeats column n's query and carries
  // the low part, so one product covers both and the halves are added once
  // per piece; otherwise each part has a product of its own.  The choice
  // goes by G (at most 4: a unit of either size fits in 8 columns), so one-
  // and two-head units of a group sum alike; the generalised instantiation
  // takes it when the call's columns fit too (one query per sequence).
  constexpr bool DUP_OK = NCT == 1 && G <= 4;
  constexpr bool ALWAYS_DUP = DUP_OK && !GEN;
  const bool dup = ALWAYS_DUP || (DUP_OK && p.cols <= 8);   // (wave-uniform)

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int32_t* s_pre = reinterpret_cast<int32_t*>(smem);       // [B + 1]
  int32_t* s_tmp = s_pre + p.B + 1;                          // [blockDim]
  // The lengths' LDS copy is addressed through s_tmp whether or not it is
  // kept, so every access to it stays an LDS access (a pointer that is LDS
  // or NULL would be a generic one, read with a flat load whose wait also
  // covers the wave's outstanding global stores).
  const bool len_lds = len_lds_entries(p.B) != 0;
  const bool qs_lds = len_lds && qs_lds_entries(p.B) != 0;
  int32_t* s_len = s_tmp + kAttnBlockThreads;   // [B] if len_lds, then [B + 1] if qs_lds
  build_prefix(p, BS, s_pre, s_tmp, len_lds);

  const int Hkv = p.Hkv;
  const int U = Hkv / HG;                  // units per sequence
  const int total = U * s_pre[p.B];
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= p.B; i += blockDim.x) p.ws_pre[i] = s_pre[i];
  if (total == 0) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave_in_block = threadIdx.x >> 6;
  const int wave = blockIdx.x * kAttnWavesPerBlock + wave_in_block;
  const size_t pre_bytes = (sizeof(int32_t) * prefix_lds_words(p.B) + 15) & ~size_t(15);
  // per wave: staged tile, the new K and V unit rows (bf16) and, with the
  // workgroup combine, a slot for the share of the run the piece starts in
  static_assert(32 * CH == 4 * HG * D, "append rows: a K and a V unit row of bf16");
  const int wave_lds = 16 * PITCH + wave_rows_bytes(HG, D, p.wgc, p.park);
  unsigned char* tile = smem + pre_bytes + (size_t)wave_in_block * wave_lds;
  unsigned char* new_rows = tile + 16 * PITCH;     // [K unit row | V unit row], 16 CH bytes each
  float* head_slot = reinterpret_cast<float*>(new_rows + 32 * CH);
  // workgroup combine: (segment, flags) of each wave's head and end shares;
  // with p.chain, entries 0 and 1 describe the share in the parking slot
  int* s_desc = reinterpret_cast<int*>(smem + pre_bytes + (size_t)kAttnWavesPerBlock * wave_lds);
  if ((p.wgc || p.chain) && lane < 4) s_desc[4 * wave_in_block + lane] = -1;

  const int n = lane & 15;        // column of S^T and O^T (a query head); K row of the A operand
  const int r = lane >> 4;        // 4-token group of S^T rows; 4-dim group of O^T rows
  // kv head of the unit that column n reads: column n is query n / UG, head
  // n % UG of the unit (columns past the used ones also land on a head of
  // the unit, so their loads stay in it)
  const int mem = HG > 1 ? (n % UG) / G : 0;
  const WorkSplit split = make_split(total, p.total_waves);
  const int64_t row_bytes = (int64_t)Hkv * RB;
  // this lane's 16-byte chunk of a unit row, for the global loads: a 32-bit
  // offset from the tile's (wave-uniform) first byte, so the loads take the
  // scalar-base + vector-offset form
  const uint32_t lane_off = (uint32_t)((lane / LPR) * row_bytes + 16 * (lane % LPR));
  // tile offsets of the operand reads (+ 2 D bytes per kv head of the unit)
  const int k_rd = n * PITCH + 16 * r;                               // + 64 kk
  const int v_rd = (4 * r + (n >> 2)) * PITCH + 8 * (n & 3);         // + 32 nb
  const unsigned char* __restrict__ kc = static_cast<const unsigned char*>(p.k_cache);
  const unsigned char* __restrict__ vc = static_cast<const unsigned char*>(p.v_cache);
  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(p.q);

  // O^T, the running max and this lane's share of the sum of the current
  // run (kept after the piece for the chain combine below)
  float4_t O[NCT][NBN];   // O^T: lane (n, r) holds dims 16 nb + 4 r + i of column n
  float m_run[NCT];       // running max of column n (exp2 domain)
  float l_run[NCT];       // this lane's share of column n's sum
  // parking slot offsets: output [ct][nb][lane] uint2; share (last tile)
  // [nb][lane] float4, then (m, l) of its 16 columns
  auto park_out_at = [&](int ct, int nb) { return 8 * (kWave * (NBN * ct + nb) + lane); };
  auto park_o_at = [&](int nb) { return 16 * (kWave * nb + lane); };
  const int park_ml_at = 16 * kWave * NBN;
  // Chain combine (p.chain: generalised calls, one kv head per wave).  A
  // wave whose last run goes on past its piece keeps that share in O (the
  // walker: its run started in the piece, or it is the workgroup's first
  // wave); a later wave of the workgroup whose piece starts inside a run
  // puts its share of it in its parking slot instead of memory.  After the
  // workgroup's barrier each walker folds in the slots that follow it in
  // wave order, up to the one ending the run or the workgroup's last wave,
  // and writes the run's bf16 output (it saw the whole run) or one share
  // row, g + segment for workgroup g, as the workgroup combine does.
  // With two column tiles (park mode 2) a follower's share takes both its
  // slot (tile 1) and the share-sized area from its tile buffer on (tile 0,
  // written there once its piece's tiles are done).
  constexpr bool CHAIN = GEN && HG == 1;
  int ch_seg = -1;                 // the walker's run (wave-uniform; -1: none)
  bool ch_first = false;           // its share starts at the run's first page
  int ch_r0 = 0, ch_g0 = 0, ch_ncol = 0;
  float ch_l[NCT];                 // column c's sum over the walker's share
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) ch_l[ct] = 0.0f;
  // with the chain, workgroup g stores its share rows at g + segment
  // (without it, a piece's rows are at piece + segment)
  const int64_t row_owner = p.chain ? (int64_t)blockIdx.x : 0;

  run_split(split, wave, [&](int x, const int x_end, const int piece) {
  // The append's cache stores wait for the end of the piece: a store counts
  // against the same wait counter as the loads that follow it, so stores
  // issued between runs would hold up the next run's first tiles until they
  // complete.  (A piece holding several runs' last pages stores the earlier
  // ones when the next arrives.)
  uint4 pend_part[NP];
  uint2 pend_codes[NP];
  float pend_gsc[2 * HG];
  int64_t pend_row = 0, pend_sslot = 0;
  bool pend_opens = false, pending = false;
  auto flush_pending = [&]() {
    store_new_rows<S>(pend_part, pend_codes, pend_gsc, lane, p.k_cache_w + pend_row,
                      p.v_cache_w + pend_row, pend_opens,
                      S::Q8 ? p.k_scale_w + pend_sslot : nullptr,
                      S::Q8 ? p.v_scale_w + pend_sslot : nullptr);
  };
  // Likewise the bf16 output of a run the piece finishes by itself (kernels
  // with two kv heads per wave and one column tile: the others have no
  // registers to spare); a lane whose column is past the call's leaves
  // out_row NULL.
  constexpr bool DEFER_OUT = NCT == 1 && HG > 1;
  uint2 out_pend[DEFER_OUT ? NBN : 1];
  uint16_t* out_row = nullptr;
  bool out_pending = false;   // (wave-uniform)
  auto flush_out = [&]() {
    if (out_row != nullptr) {
#pragma unroll
      for (int nb = 0; nb < NBN; ++nb)
        *reinterpret_cast<uint2*>(out_row + 16 * nb) = out_pend[DEFER_OUT ? nb : 0];
    }
  };
  // Kernels with one kv head per wave have no registers to keep a whole
  // result in: with p.park, one result that more runs of the piece follow
  // waits in the wave's parking slot instead (its bf16 output, packed; or its
  // share, whose first tile stays in registers when there are two) and goes
  // to memory after the piece's last tile.  Stored at once it would hold up
  // the next run, whose first waits cover the stores and whose store acks
  // take longer than a load round trip (skipping such stores measured 5% of
  // the verify workload, with one of them in a sixth of the pieces, and 15%
  // of its 70B-shaped mix).  Only scalars describe the parked result.
  constexpr bool PARK = GEN && HG == 1;
  constexpr bool PARK_REG = PARK && NCT == 2;   // (the share's tile 0 in registers)
  // (see park_slot_bytes; park mode 2: see park_share_ext_bytes)
  unsigned char* const park_slot =
      new_rows + (PARK_REG && p.park == 2 ? park_share_ext_bytes(HG, D) : 0);
  float4_t park_o0[PARK_REG ? NBN : 1];
  bool h0_regs = false;        // a walker's share waits with its tile 0 in park_o0
  float park_m0 = 0.0f, park_l0 = 0.0f;
  // (wave-uniform) 0: empty, 1: output, 2: share, 3: share for a walker
  int park_kind = 0;
  int64_t park_row = 0;        // share row, or the output's first query row
  int park_g0 = 0, park_ncol = 0;
  auto flush_park = [&]() {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      // (with the repeated columns of a call of at most 8 columns, the used
      // columns are still the lanes' n < 8)
      const int c = 16 * ct + n;
      if (park_kind == 1) {
        if (c < park_ncol) {
          uint16_t* orow = static_cast<uint16_t*>(p.out) +
                           ((park_row + c / UG) * p.Hq + park_g0 * G + c % UG) * D + 4 * r;
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb)
            *reinterpret_cast<uint2*>(orow + 16 * nb) =
                *reinterpret_cast<const uint2*>(park_slot + park_out_at(ct, nb));
        }
      } else {
        const int C = p.cols;
        const bool in_regs = PARK_REG && ct == 0;
        if (c < park_ncol) {
          float* orow = p.ws_o + (park_row * C + c) * D + 4 * r;
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb) {
            float4 v;
            if (in_regs)
              v = make_float4(park_o0[nb][0], park_o0[nb][1], park_o0[nb][2], park_o0[nb][3]);
            else
              v = *reinterpret_cast<const float4*>(park_slot + park_o_at(nb));
            *reinterpret_cast<float4*>(orow + 16 * nb) = v;
          }
        }
        if (lane < 16 && 16 * ct + lane < park_ncol) {
          const float2 ml = in_regs ? make_float2(park_m0, park_l0)
                                    : *reinterpret_cast<const float2*>(park_slot + park_ml_at + 8 * lane);
          *reinterpret_cast<float2*>(p.ws_ml + (park_row * C + 16 * ct + lane) * 2) = ml;
        }
      }
    }
    park_kind = 0;
  };
  while (x < x_end) {
    Piece pc = locate_piece(s_pre, p.B, U, p.run_cost, x, x_end);
    // (wave-uniform: kept in scalar registers)
    pc.b = __builtin_amdgcn_readfirstlane(pc.b);
    pc.u = __builtin_amdgcn_readfirstlane(pc.u);
    pc.n_b = __builtin_amdgcn_readfirstlane(pc.n_b);
    pc.run_start = __builtin_amdgcn_readfirstlane(pc.run_start);
    pc.j0 = __builtin_amdgcn_readfirstlane(pc.j0);
    pc.j1 = __builtin_amdgcn_readfirstlane(pc.j1);
    pc.next = __builtin_amdgcn_readfirstlane(pc.next);
    if (pc.j0 == pc.j1) {   // only the slots ahead of the run's pages
      x = pc.next;
      continue;
    }
    const int b = pc.b, g0 = pc.u * HG;   // the unit's first kv head
    int L_in;
    if (len_lds)
      L_in = s_len[b];
    else   // (a buffer load: a plain load here would be merged with the LDS read above)
      L_in = (int)__builtin_amdgcn_raw_buffer_load_b32(
          tile_rsrc(reinterpret_cast<const unsigned char*>(p.context_lens)), 0, (uint32_t)b * 4, 0);
    const int L = min(max(L_in, 0), p.MBS * BS);
    // a length outside [1, MBS * BS] breaks the contract: no append then
    // (the decode step is one query per sequence: never the GEN instantiation)
    const bool append = !GEN && p.k_new != nullptr && L == L_in && L >= 1;
    const int32_t* bt_row = p.block_tables + (int64_t)b * p.MBS;
    const int64_t head_off = (int64_t)g0 * RB;
    // column n: query token n / UG of the sequence, query head g0 G + n % UG
    // (decode: one query, the unit's UG heads)
    int ql = 1, r0 = b;   // query count, first q / out row
    if constexpr (GEN) {
      if (qs_lds) {
        r0 = s_len[p.B + b];
        ql = min(max(s_len[p.B + b + 1] - r0, 0), p.max_q);
      } else {
        ql = seq_queries(p, b);
        r0 = p.q_start != nullptr ? p.q_start[b] : b;
      }
    }
    const int ncol = UG * ql;
    const SeqRange sr = GEN ? seq_range(L, ql, p.sinks, p.window, BS) : SeqRange{0, 0, 0};
    auto table_page = [&](int j) { return !GEN || j < sr.ps ? j : j + sr.gap; };
    // column c = 16 ct + n of tile ct: query c / UG, query head g0 G + c % UG.
    // Keys it sees: j <= lim (bottom-right causal), and with a window j >= lo
    // or j < sinks.
    int col_q[NCT], col_h[NCT], lim_n[NCT], lo_n[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int c = dup ? (n & 7) : 16 * ct + n;   // (dup: column n + 8 repeats column n)
      col_q[ct] = c / UG;
      col_h[ct] = g0 * G + c % UG;
      lim_n[ct] = c < ncol ? L - ql + col_q[ct] : -1;
      lo_n[ct] = lim_n[ct] - p.window + 1;
    }
    const bool windowed = GEN && p.window > 0;
    const int gap_end = L - ql - p.window + 1;    // keys in [sinks, gap_end) no query sees

    // q of the columns as the B operand: element i of k-step kk is head dim
    // 32 kk + 8 r + i, the same dims the K operand's element i holds
    bf16x8_t qB[NCT][NKK];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const uint16_t* qrow = qp + ((int64_t)(r0 + col_q[ct]) * p.Hq + col_h[ct]) * D + 8 * r;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if ((dup ? (n & 7) : 16 * ct + n) < ncol) v = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
        qB[ct][kk] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
    // The decode step's new rows when this piece holds the run's last page
    // (loaded beside q; see NewRows for the chunks a lane takes).
    const bool has_new = append && pc.j1 == pc.n_b;
    uint4 new_part[NP];
    {
      const int64_t src = ((int64_t)b * Hkv + g0) * D;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int q = lane + kWave * i;
        new_part[i] = make_uint4(0, 0, 0, 0);
        if (has_new && q < 2 * CH)
          new_part[i] = q < CH ? *reinterpret_cast<const uint4*>(p.k_new + src + 8 * q)
                               : *reinterpret_cast<const uint4*>(p.v_new + src + 8 * (q - CH));
      }
    }
    // the page-table entries of the run's first chunk (lane l: page j0 + l),
    // loaded beside q and the new rows
    int bt_first = -1;
    if (lane < min(kWave, pc.j1 - pc.j0)) bt_first = bt_row[table_page(pc.j0 + lane)];
    // (RoPE here, with those loads in flight: inside the chunk or tile loop
    // it raised the loop's registers and measured slower)
    if constexpr (ROPE) rope_rotate<S>(p, L_in - 1, lane, r, tile, qB[0], new_part, has_new);
    float new_ksc = 1.0f, new_vsc = 1.0f;   // fp8 / int8: head mem's last-block scales after the append
    // the append's cache stores, issued after the run's last tile (store_new_rows)
    uint2 new_codes[NP];
    float new_gsc[2 * HG];
    int64_t new_row = 0, new_sslot = 0;
    bool new_opens = false, parked = false;

#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int nb = 0; nb < NBN; ++nb) O[ct][nb] = float4_t{0.f, 0.f, 0.f, 0.f};
      m_run[ct] = -FLT_MAX;
      l_run[ct] = 0.0f;
    }

    for (int jc = pc.j0; jc < pc.j1; jc += kWave) {
      const int nchunk = min(kWave, pc.j1 - jc);
      int v = bt_first;
      if (jc != pc.j0) {
        v = -1;
        if (lane < nchunk) v = bt_row[table_page(jc + lane)];
      }
      const bool valid_l = (unsigned)v < (unsigned)p.NB;   // (-1: past the chunk)
      const int phys_l = valid_l ? v : 0;
      const uint64_t valid = __builtin_amdgcn_ballot_w64(valid_l);   // pages with a real block id

      const int k_last = pc.n_b - 1 - jc;             // the run's last page in this chunk, if < nchunk
      const bool new_here = has_new && k_last < nchunk && ((valid >> k_last) & 1);
      uint4 kb[NI], vb[NI];
      float ksc = 1.0f, vsc = 1.0f;
      // u indexes the chunk's 16-token tiles: page k of the chunk, tile sb.
      // Bytes in flight per wave: a half tile of 4 KB or more (bf16, D =
      // 128) is enough on its own, so its V loads are issued only once the K
      // loads have landed (issuing both at once measured ~7% slower with one
      // head per wave, 2-3% with two); 2 KB halves (one head, fp8 / int8 or
      // D = 64) issue K and V together (~3% faster than in turn), and so do
      // int8 units (see KV_TOGETHER).  The other waves of the CU overlap
      // their compute with the waits; issuing the next tile's K early
      // measured 3-7% slower.
      auto tile_base = [&](int u) {   // (wave-uniform)
        const int k = u / SUB, sb = u % SUB;
        const int phys = __builtin_amdgcn_readlane(phys_l, k);
        return ((int64_t)phys * BS + sb * 16) * row_bytes + head_off;
      };
      auto issue = [&](const unsigned char* __restrict__ src, int64_t base, uint4 (&ch)[NI]) {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(src + base);
#pragma unroll
        for (int s = 0; s < NI; ++s)
          ch[s] = load_tile_chunk(rs, lane_off, (uint32_t)(s * RPI * row_bytes));
      };
      // tiles of the chunk; in the run's last page only those holding a
      // position below L (a tile past the history would add nothing)
      int nunits = nchunk * SUB;
      if (jc + nchunk == pc.n_b) {
        const int last_pos = table_page(pc.n_b - 1) * BS;   // first position of the last page
        nunits -= SUB - (L - last_pos + 15) / 16;
      }
      for (int u = 0; u < nunits; ++u) {
        const int k = u / SUB, sb = u % SUB;
        const int tok0 = table_page(jc + k) * BS + sb * 16;   // position of the tile's first token
        const int live = L - tok0;                  // rows of the tile inside the history
        // the decode step's new token goes to row live - 1 of this tile
        const bool new_tile = new_here && k == k_last && live >= 1 && live <= 16;
        if constexpr (S::Q8) {   // the tile's scales: scalar loads, then column n's head
          const int phys = __builtin_amdgcn_readlane(phys_l, k);
          const float* ks = p.k_scale + (int64_t)phys * Hkv + g0;
          const float* vs = p.v_scale + (int64_t)phys * Hkv + g0;
          ksc = ks[0];
          vsc = vs[0];
#pragma unroll
          for (int j = 1; j < HG; ++j) {
            const float kj = ks[j], vj = vs[j];
            if (mem == j) {
              ksc = kj;
              vsc = vj;
            }
          }
        }
        const int64_t base = tile_base(u);
        issue(kc, base, kb);
        if constexpr (S::KV_TOGETHER) issue(vc, base, vb);
        if (new_here && u == 0) {   // park the new rows while this tile's loads fly
          const int blk = __builtin_amdgcn_readlane(phys_l, k_last);
          const int off = (L - 1) % BS;
          new_row = ((int64_t)blk * BS + off) * row_bytes + (int64_t)g0 * RB;
          new_sslot = (int64_t)blk * Hkv + g0;
          new_opens = off == 0;
          parked = true;
          // (bf16 caches have no scales: null pointers then)
          park_new_rows<S>(new_part, lane, mem, new_rows, new_opens, new_ksc, new_vsc,
                           S::Q8 ? p.k_scale + new_sslot : nullptr,
                           S::Q8 ? p.v_scale + new_sslot : nullptr, new_codes, new_gsc);
        }

        // K tile -> LDS -> A operands; scores S^T (16 tokens x 16 columns)
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
        float4_t s[NCT];
        {
          float4_t sh[NCT][HG];   // one chain per kv head of the unit
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int j = 0; j < HG; ++j) sh[ct][j] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int j = 0; j < HG; ++j) {
              const bf16x8_t a =
                  *reinterpret_cast<const bf16x8_t*>(tile + k_rd + 2 * D * j + 64 * kk);
#pragma unroll
              for (int ct = 0; ct < NCT; ++ct)
                sh[ct][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qB[ct][kk], sh[ct][j], 0, 0, 0);
            }
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            s[ct] = sh[ct][0];
#pragma unroll
            for (int j = 1; j < HG; ++j)
              if (mem == j) s[ct] = sh[ct][j];
          }
        }
        const float c = S::Q8 ? p.scale_log2 * ksc : p.scale_log2;
        short4_t pb[NCT], pl[NCT];   // P^T in two bf16 parts (high, low)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          // rows past a_rel are in column n's future (decode: past the history)
          const int a_rel = GEN ? lim_n[ct] - tok0 : live - 1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s[ct][i] *= c;
            if (4 * r + i > a_rel) s[ct][i] = -INFINITY;
          }
          if (windowed) {
            const int lo_rel = lo_n[ct] - tok0, sk_rel = p.sinks - tok0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * r + i < lo_rel && 4 * r + i >= sk_rel) s[ct][i] = -INFINITY;
          }

          // online softmax, one max per column n
          float pm = fmaxf(fmaxf(s[ct][0], s[ct][1]), fmaxf(s[ct][2], s[ct][3]));
          pm = fmaxf(pm, __shfl_xor(pm, 16));
          pm = fmaxf(pm, __shfl_xor(pm, 32));
          if (__builtin_amdgcn_ballot_w64(pm > m_run[ct]) != 0) {
            const float m_new = fmaxf(m_run[ct], pm);
            const float alpha = fast_exp2(m_run[ct] - m_new);
            m_run[ct] = m_new;
            l_run[ct] *= alpha;
            // O^T columns are this lane's column: its own factor
#pragma unroll
            for (int nb = 0; nb < NBN; ++nb)
#pragma unroll
              for (int i = 0; i < 4; ++i) O[ct][nb][i] *= alpha;
          }
          // P^T as the B operand: lane (n, r) holds column n, tokens 4r..4r+3,
          // the layout S^T came out in.  The weight x goes in as two bf16
          // terms, hi = bf16(x) and lo = bf16(x - hi) (x - hi is exact in
          // fp32), so the product sees x to 2^-16 relative instead of bf16's
          // 2^-8: with few keys of large, cancelling values a single bf16
          // rounding of P could move the output by 2^-8 sum_t p_t |v_t|.
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pr = fast_exp2(s[ct][i] - m_run[ct]);
            l_run[ct] += pr;
            const float x = S::Q8 ? pr * vsc : pr;
            const __bf16 hi = (__bf16)x;
            const short lo = bf16_bits(x - (float)hi);
            // (dup: the lanes of columns 8..15 carry the low part)
            pb[ct][i] = dup && n >= 8 ? lo : __builtin_bit_cast(short, hi);
            if constexpr (!ALWAYS_DUP) pl[ct][i] = lo;
          }
        }

        // V tile -> the same LDS buffer (its K reads are done, LDS is in
        // order within a wave) -> transposed A operands, O^T += V^T P^T
        if (windowed)
          stage_tile<S>(tile, vb, lane, live, true, p.sinks - tok0, gap_end - tok0);
        else
          stage_tile<S>(tile, vb, lane, live, true);
        if (new_tile) take_new_row<S>(new_rows + 16 * CH, tile, live - 1, lane);
#pragma unroll
        for (int j = 0; j < HG; ++j) {
          short4_t pj[NCT], plj[NCT];
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            pj[ct] = pb[ct];
            if constexpr (!ALWAYS_DUP) plj[ct] = pl[ct];
            if (HG > 1 && mem != j) {
              pj[ct] = short4_t{0, 0, 0, 0};
              if constexpr (!ALWAYS_DUP) plj[ct] = short4_t{0, 0, 0, 0};
            }
          }
          // every V operand of this kv head first, then the products (the
          // reads stay pipelined whatever the register pressure elsewhere)
          short4_t vA[NBN];
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb)   // (C-style cast: generic -> LDS address space)
            vA[nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_short4_t*)(tile + v_rd + 2 * D * j + 32 * nb));
          if (ALWAYS_DUP || dup) {
#pragma unroll
            for (int nb = 0; nb < NBN; ++nb)
#pragma unroll
              for (int ct = 0; ct < NCT; ++ct)
                O[ct][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vA[nb], pj[ct], O[ct][nb], 0, 0, 0);
          } else {
#pragma unroll
            for (int nb = 0; nb < NBN; ++nb)
#pragma unroll
              for (int ct = 0; ct < NCT; ++ct)
                O[ct][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                    vA[nb], plj[ct],
                    __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vA[nb], pj[ct], O[ct][nb], 0, 0, 0),
                    0, 0, 0);
          }
        }
      }
    }

    if (parked) {   // (wave-uniform)
      if (pending) flush_pending();
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        pend_part[i] = new_part[i];
        pend_codes[i] = new_codes[i];
      }
#pragma unroll
      for (int i = 0; i < 2 * HG; ++i) pend_gsc[i] = new_gsc[i];
      pend_row = new_row;
      pend_sslot = new_sslot;
      pend_opens = new_opens;
      pending = true;
    }

    // ---- finish the piece ---------------------------------------------------
    if (dup) {   // column n's high-part sum plus column n + 8's low-part sum
#pragma unroll
      for (int nb = 0; nb < NBN; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[0][nb][i] += __shfl_xor(O[0][nb][i], 8);
    }
    const int seg = b * U + pc.u;
    // (PARK: the slot is free and more runs of the piece follow)
    const bool to_park = PARK && p.park && park_kind == 0 && pc.next < x_end;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int c = 16 * ct + n;
      float l_tot = l_run[ct];
      l_tot += __shfl_xor(l_tot, 16);
      l_tot += __shfl_xor(l_tot, 32);            // column n's sum, in every row group
      if (pc.j0 == 0 && pc.j1 == pc.n_b) {
        if constexpr (DEFER_OUT) {
          if (out_pending) flush_out();
          out_pending = true;
          out_row = nullptr;
        }
        if (to_park) {
          // (a query that sees no key gets 0)
          const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb)
            *reinterpret_cast<uint2*>(park_slot + park_out_at(ct, nb)) =
                make_uint2(pack_bf16x2(O[ct][nb][0] * inv, O[ct][nb][1] * inv),
                           pack_bf16x2(O[ct][nb][2] * inv, O[ct][nb][3] * inv));
          park_kind = 1;
          park_row = r0;
          park_g0 = g0;
          park_ncol = ncol;
        } else if (c < ncol) {
          // (a query that sees no key gets 0)
          const float inv = !GEN || l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
          uint16_t* orow = static_cast<uint16_t*>(p.out) +
                           ((int64_t)(r0 + col_q[ct]) * p.Hq + col_h[ct]) * D + 4 * r;
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb) {
            const uint2 v = make_uint2(pack_bf16x2(O[ct][nb][0] * inv, O[ct][nb][1] * inv),
                                       pack_bf16x2(O[ct][nb][2] * inv, O[ct][nb][3] * inv));
            if constexpr (DEFER_OUT)
              out_pend[nb] = v;
            else
              *reinterpret_cast<uint2*>(orow + 16 * nb) = v;
          }
          if constexpr (DEFER_OUT) out_row = orow;
        }
      } else if (NCT == 1 && p.wgc) {
        // the share goes to LDS for the workgroup combine: a piece ending
        // inside the run leaves its end share in its (now free) tile buffer,
        // one starting inside a run that it finishes in its head slot
        const bool is_end = pc.j1 < pc.n_b;
        float* sh = is_end ? reinterpret_cast<float*>(tile) : head_slot;
        if (c < ncol) {
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb)
            *reinterpret_cast<float4*>(sh + c * D + 16 * nb + 4 * r) =
                make_float4(O[ct][nb][0], O[ct][nb][1], O[ct][nb][2], O[ct][nb][3]);
          if (r == 0) {
            sh[p.wgc * D + c] = m_run[ct];
            sh[p.wgc * D + p.wgc + c] = l_tot;
          }
        }
        if (lane == 0) {
          s_desc[4 * wave_in_block + 2 * is_end] = seg;
          s_desc[4 * wave_in_block + 2 * is_end + 1] = (pc.j0 == 0) | (pc.j1 == pc.n_b) << 1;
        }
      } else if (CHAIN && p.chain && pc.j0 > 0 && wave_in_block > 0) {
        // a run an earlier wave of the workgroup carries (the piece's first
        // run, so the slot is free): its share waits in the slot for that
        // wave, and nothing of it is stored here.  With two tiles, tile 0
        // goes to the area from the tile buffer on, which is free only
        // after the piece's last tile: until then it waits in park_o0.
        if (PARK_REG && ct == 0 && pc.next < x_end) {
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb) park_o0[nb] = O[ct][nb];
          park_m0 = m_run[ct];
          park_l0 = l_tot;
          h0_regs = true;
        } else {
          unsigned char* const dst = PARK_REG && ct == 0 ? tile : park_slot;
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb)
            *reinterpret_cast<float4*>(dst + park_o_at(nb)) =
                make_float4(O[ct][nb][0], O[ct][nb][1], O[ct][nb][2], O[ct][nb][3]);
          if (lane < 16)
            *reinterpret_cast<float2*>(dst + park_ml_at + 8 * lane) = make_float2(m_run[ct], l_tot);
        }
        park_kind = 3;
        if (lane == 0) {
          s_desc[4 * wave_in_block] = seg;
          s_desc[4 * wave_in_block + 1] = (pc.j1 == pc.n_b) << 1;
        }
      } else if (CHAIN && p.chain && pc.next == x_end && pc.j1 < pc.n_b) {
        // the run goes on past the piece: this wave walks it (O and m_run
        // are left as they are; the piece has no more runs)
        ch_seg = seg;
        ch_first = pc.j0 == 0;
        ch_l[ct] = l_tot;
        ch_r0 = r0;
        ch_g0 = g0;
        ch_ncol = ncol;
      } else if (to_park) {
        if (PARK_REG && ct == 0) {
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb) park_o0[nb] = O[ct][nb];
          park_m0 = m_run[ct];
          park_l0 = l_tot;
        } else {
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb)
            *reinterpret_cast<float4*>(park_slot + park_o_at(nb)) =
                make_float4(O[ct][nb][0], O[ct][nb][1], O[ct][nb][2], O[ct][nb][3]);
          // (lanes 0..15: column 16 ct + lane's max and sum)
          if (lane < 16)
            *reinterpret_cast<float2*>(park_slot + park_ml_at + 8 * lane) =
                make_float2(m_run[ct], l_tot);
        }
        park_kind = 2;
        park_row = (p.chain ? row_owner : (int64_t)piece) + seg;
        park_ncol = ncol;
      } else {
        const int64_t row = (p.chain ? row_owner : (int64_t)piece) + seg;
        const int C = p.cols;
        if (c < ncol) {
          float* orow = p.ws_o + (row * C + c) * D + 4 * r;
#pragma unroll
          for (int nb = 0; nb < NBN; ++nb)
            *reinterpret_cast<float4*>(orow + 16 * nb) =
                make_float4(O[ct][nb][0], O[ct][nb][1], O[ct][nb][2], O[ct][nb][3]);
        }
        // (lanes 0..15: the tile's columns, once each; one tile: ncol <= 16)
        if (NCT == 1 ? lane < ncol : lane < 16 && 16 * ct + lane < ncol)
          *reinterpret_cast<float2*>(p.ws_ml + (row * C + 16 * ct + lane) * 2) =
              make_float2(m_run[ct], l_tot);
      }
    }
    x = pc.next;
  }
  if (pending) flush_pending();
  if constexpr (DEFER_OUT)
    if (out_pending) flush_out();
  if constexpr (PARK)
    if (park_kind == 1 || park_kind == 2) flush_park();   // (3: a walker's)
  if constexpr (PARK_REG) {
    if (h0_regs) {   // (wave-uniform; the tile buffer is free now)
#pragma unroll
      for (int nb = 0; nb < NBN; ++nb)
        *reinterpret_cast<float4*>(tile + park_o_at(nb)) =
            make_float4(park_o0[nb][0], park_o0[nb][1], park_o0[nb][2], park_o0[nb][3]);
      if (lane < 16)
        *reinterpret_cast<float2*>(tile + park_ml_at + 8 * lane) = make_float2(park_m0, park_l0);
    }
  }
  });
  if constexpr (NCT == 1)
    if (p.wgc) wgc_combine<S, GEN>(p, smem + pre_bytes, wave_lds, s_desc, U, s_len + p.B, qs_lds);
  if constexpr (CHAIN) {
    if (p.chain) {
      __syncthreads();   // every wave's slot share and descriptor are in place
      if (ch_seg >= 0) {
        // fold in the later waves' shares of the run, in wave order, by the
        // log-sum-exp rule (column c's max and sum are the same in every
        // row group of lanes)
        float M[NCT], Ls[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          M[ct] = m_run[ct];
          Ls[ct] = ch_l[ct];
        }
        bool ends = false;
        for (int j = wave_in_block + 1; j < kAttnWavesPerBlock; ++j) {
          if (__builtin_amdgcn_readfirstlane(s_desc[4 * j]) != ch_seg) break;
          const int flg = __builtin_amdgcn_readfirstlane(s_desc[4 * j + 1]);
          const unsigned char* wb = smem + pre_bytes + (size_t)j * wave_lds;   // wave j's tile buffer
          const unsigned char* slot_j =
              wb + 16 * PITCH + (NCT == 2 && p.park == 2 ? park_share_ext_bytes(HG, D) : 0);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            const unsigned char* sl = NCT == 2 && ct == 0 ? wb : slot_j;   // (tile 0: see h0_regs)
            const float2 ml = *reinterpret_cast<const float2*>(sl + park_ml_at + 8 * n);
            const float Mn = fmaxf(M[ct], ml.x);
            const float a = fast_exp2(M[ct] - Mn), w = fast_exp2(ml.x - Mn);
            Ls[ct] = fmaf(ml.y, w, Ls[ct] * a);
#pragma unroll
            for (int nb = 0; nb < NBN; ++nb) {
              const float4 o = *reinterpret_cast<const float4*>(sl + park_o_at(nb));
              O[ct][nb][0] = fmaf(o.x, w, O[ct][nb][0] * a);
              O[ct][nb][1] = fmaf(o.y, w, O[ct][nb][1] * a);
              O[ct][nb][2] = fmaf(o.z, w, O[ct][nb][2] * a);
              O[ct][nb][3] = fmaf(o.w, w, O[ct][nb][3] * a);
            }
            M[ct] = Mn;
          }
          if (flg & 2) {
            ends = true;
            break;
          }
        }
        const bool whole = ch_first && ends;   // (else the workgroup's share row)
        const int64_t row = row_owner + ch_seg;
        const int C = p.cols;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const int c = 16 * ct + n;
          if (whole) {
            if (c < ch_ncol) {
              const float inv = Ls[ct] > 0.0f ? 1.0f / Ls[ct] : 0.0f;   // (0: the query sees no key)
              uint16_t* orow = static_cast<uint16_t*>(p.out) +
                               ((int64_t)(ch_r0 + c / UG) * p.Hq + ch_g0 * G + c % UG) * D + 4 * r;
#pragma unroll
              for (int nb = 0; nb < NBN; ++nb)
                *reinterpret_cast<uint2*>(orow + 16 * nb) =
                    make_uint2(pack_bf16x2(O[ct][nb][0] * inv, O[ct][nb][1] * inv),
                               pack_bf16x2(O[ct][nb][2] * inv, O[ct][nb][3] * inv));
            }
          } else {
            if (c < ch_ncol) {
              float* orow = p.ws_o + (row * C + c) * D + 4 * r;
#pragma unroll
              for (int nb = 0; nb < NBN; ++nb)
                *reinterpret_cast<float4*>(orow + 16 * nb) =
                    make_float4(O[ct][nb][0], O[ct][nb][1], O[ct][nb][2], O[ct][nb][3]);
            }
            // (lanes 0..15: column 16 ct + lane, row group 0)
            if (lane < 16 && c < ch_ncol)
              *reinterpret_cast<float2*>(p.ws_ml + (row * C + c) * 2) = make_float2(M[ct], Ls[ct]);
          }
        }
      }
    }
  }
}

// Calls f(MfmaShape<D, BS, G, kind, hg>{}) for the combination given at run
// time: hg = 1, or hg = kUnitHeads(G).
// Two heads per wave measured best on every decode workload (B64 / B4 /
// B256 / B128 bf16, fp8 and int8 shapes): 2-4% faster steps than one head
// (fp8: 6%), while four heads lost on bf16 D = 128 G = 4 (3% slower steps:
// the wider partial rows and the 2-waves-per-SIMD grid cost more than the
// 1 KB runs gain).
constexpr int kUnitHeads(int G) { return G <= 8 ? 2 : 1; }

template <int D_, int BS_, int G_, int K_>
struct ShapeKey {
  static constexpr int D = D_, BS = BS_, G = G_, K = K_;
};

template <class F>
bool dispatch_mfma(int D, int BS, int G, int kind, int hg, F&& f) {
  bool ok = false;
  auto one = [&](auto key) {
    using Kt = decltype(key);
    constexpr int H = kUnitHeads(Kt::G);
    if (hg == 1) {
      f(MfmaShape<Kt::D, Kt::BS, Kt::G, Kt::K, 1>{});
      ok = true;
    } else if (hg == H) {
      f(MfmaShape<Kt::D, Kt::BS, Kt::G, Kt::K, H>{});
      ok = true;
    }
  };
  if (G == 16) {   // groups of 16 (this kernel only): one kv head's queries fill the columns
#define PKV_G16(d, bs, k) \
  if (D == d && BS == bs && kind == k) one(ShapeKey<d, bs, 16, k>{});
#define PKV_G16_K(d, bs) PKV_G16(d, bs, kKvBf16) PKV_G16(d, bs, kKvFp8) PKV_G16(d, bs, kKvInt8)
    PKV_G16_K(64, 16) PKV_G16_K(64, 32) PKV_G16_K(128, 16) PKV_G16_K(128, 32)
#undef PKV_G16_K
#undef PKV_G16
    return ok;
  }
  dispatch_shapes<ShapeKey>(D, BS, G, kind, one);
  return ok;
}

}  // namespace

int mfma_unit_heads(int G) { return kUnitHeads(G); }

bool mfma_tile_holds_share(int D, int hg, int wgc) {
  return wgc_slot_bytes(D, wgc) <= 16 * (hg * 2 * D + 32);   // (MfmaShape::PITCH rows)
}

size_t mfma_stage_lds_bytes(int D, int hg, int wgc, int park) {
  return (size_t)kAttnWavesPerBlock * (16 * (hg * 2 * D + 32) + wave_rows_bytes(hg, D, wgc, park)) +
         (wgc || park ? 4 * kAttnWavesPerBlock * sizeof(int) : 0);
}

int mfma_park_slot_bytes(int D) { return park_slot_bytes(D); }

// Units of several kv heads run at two workgroups (8 waves) per CU: each
// workgroup reserves at least this much LDS, so a third one never fits
// (three waves per SIMD measured slower for them: see MfmaShape::WPE).
constexpr size_t kUnitLdsFloor = 56 * 1024;

static size_t mfma_lds_total(int B, int D, int hg, int wgc, int park = 0) {
  const size_t t =
      ((prefix_lds_bytes(B) + 15) & ~size_t(15)) + mfma_stage_lds_bytes(D, hg, wgc, park);
  return hg > 1 && t < kUnitLdsFloor ? kUnitLdsFloor : t;
}

// Workgroups per CU at `wpe` waves per SIMD (4 SIMDs a CU).
constexpr int blocks_at(int wpe) { return wpe * 4 / kAttnWavesPerBlock; }

// The decode and the generalised instantiations of one unit size are held to
// the same waves per SIMD (amdgpu_waves_per_eu), so one grid size serves
// both (the smaller of their occupancies, should registers ever differ).
// The occupancy query goes by the registers a kernel ended up with, which
// may allow more waves than it was compiled for (a one-head kernel at 128
// VGPRs would run 4 per SIMD, measured 13-15% slower than 3), so the grid
// is capped at the waves per SIMD of the instantiation.
// col_tiles = 2: the generalised instantiation with two column tiles alone.
int mfma_blocks_per_cu(int D, int BS, int G, int kind, int B, int hg, int col_tiles, int wgc,
                       int park) {
  int blocks = 0, blocks_gen = 0, cap = 0;
  const size_t lds = mfma_lds_total(B, D, hg, col_tiles == 1 ? wgc : 0, park);
  if (col_tiles == 2) {
    const bool ok = hg == 1 && dispatch_mfma(D, BS, G, kind, 1, [&](auto s) {
      using S = decltype(s);
      if constexpr (S::HG == 1) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &blocks, mfma_partition_kernel<S, true, false, 2>, kAttnBlockThreads, lds) != hipSuccess)
          blocks = 0;
        cap = blocks_at(2);
      }
    });
    return ok ? (blocks < cap ? blocks : cap) : 0;
  }
  if (col_tiles != 1) return 0;
  const bool ok = dispatch_mfma(D, BS, G, kind, hg, [&](auto s) {
    using S = decltype(s);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, mfma_partition_kernel<S, false>,
                                                     kAttnBlockThreads, lds) != hipSuccess)
      blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks_gen, mfma_partition_kernel<S, true>,
                                                     kAttnBlockThreads, lds) != hipSuccess)
      blocks_gen = 0;
    cap = blocks_at(S::WPE);
  });
  if (!ok) return 0;
  const int b = blocks < blocks_gen ? blocks : blocks_gen;
  return b < cap ? b : cap;
}

hipError_t launch_partition_mfma(const AttnParams& p, int D, int BS, int G, int kind, int blocks,
                                 hipStream_t stream) {
  const size_t lds = mfma_lds_total(p.B, D, p.hg, p.wgc, p.park);
  const bool gen = p.q_start != nullptr || p.max_q > 1 || p.window > 0;
  if (gen && p.rope) return hipErrorInvalidValue;
  const int cols = p.hg * G * p.max_q;
  // two column tiles: the generalised call with one kv head per wave only
  if (p.hg < 1 || p.Hkv % p.hg != 0 || cols != p.cols || cols > 32 ||
      (cols > 16 && (!gen || p.hg != 1)) ||
      (p.wgc && (cols > p.wgc || (p.wgc != 8 && p.wgc != 16) || kPiecesPerWave != 1 ||
                 !mfma_tile_holds_share(D, p.hg, p.wgc))) ||
      (p.park && (!gen || p.hg != 1 || p.wgc)) ||
      (p.park == 2 && (cols <= 16 || !p.chain)) || p.park < 0 || p.park > 2 ||
      (p.chain && (!p.park || cols <= 8 || (cols > 16) != (p.park == 2) || kPiecesPerWave != 1)))
    return hipErrorInvalidValue;
  const bool ok = dispatch_mfma(D, BS, G, kind, p.hg, [&](auto s) {
    using S = decltype(s);
    if (gen) {
      if constexpr (S::HG == 1) {
        if (cols > 16) {
          hipLaunchKernelGGL((mfma_partition_kernel<S, true, false, 2>), dim3(blocks),
                             dim3(kAttnBlockThreads), lds, stream, p);
          return;
        }
      }
      hipLaunchKernelGGL((mfma_partition_kernel<S, true>), dim3(blocks),
                         dim3(kAttnBlockThreads), lds, stream, p);
      return;
    }
    if (p.rope)
      hipLaunchKernelGGL((mfma_partition_kernel<S, false, true>), dim3(blocks),
                         dim3(kAttnBlockThreads), lds, stream, p);
    else
      hipLaunchKernelGGL((mfma_partition_kernel<S, false>), dim3(blocks),
                         dim3(kAttnBlockThreads), lds, stream, p);
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
