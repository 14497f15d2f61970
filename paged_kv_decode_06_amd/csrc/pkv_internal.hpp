// Host-side interface between the C ABI (pkv_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace pkv {

// Cache element kinds (the PKV_KV_* values of the C ABI).  fp8 and int8
// caches hold one-byte codes with an fp32 scale per (block, kv head).
enum KvKind : int { kKvBf16 = 0, kKvFp8 = 1, kKvInt8 = 2 };

// Arguments of the attention kernels.  Pointers are device pointers.
struct AttnParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float scale_log2;     // softmax scale * log2(e): scores live in the exp2 domain
  int B, Hq, Hkv, NB, MBS;
  // Query tokens (bottom-right causal, see decode_common.hpp): sequence b
  // owns q/out rows q_start[b] .. q_start[b+1]-1 (q_start NULL: row b only);
  // at most max_q of them, G * max_q <= 32.  cols = hg * G * max_q columns
  // per share row.  window > 0 hides keys more than window - 1 positions behind a
  // query except the first `sinks` positions.
  const int32_t* q_start;
  int max_q, cols;
  int sinks, window;
  // kv heads one partition wave serves together (a unit of adjacent kv
  // heads): the work axis runs over (sequence, unit, page), U = Hkv / hg
  // units per sequence, and cols = hg * G * max_q <= 16 (up to 32 with
  // hg = 1 in the generalised call: two 16-column tiles).  The VALU kernel
  // always takes 1.
  int hg;
  int total_waves;      // persistent waves of the partition grid
  // wgc: the waves of a workgroup (consecutive pieces) combine their shares
  // of a run in LDS at the end; a run inside the workgroup's range is
  // finished there, and one crossing its edge leaves one share row per
  // workgroup (row g + segment, g the workgroup) instead of one per piece.
  // Its value is the column capacity of a wave's share slots (8 or 16;
  // 0: no combine).
  int wgc;
  // park (generalised calls with one kv head per wave, no combine): a run's
  // result that more runs of the piece follow waits in an LDS slot of the
  // wave until the piece's end (mfma_park_slot_bytes).  2: the same, with
  // the slot moved back so that a second share fits from the tile buffer on
  // (the chain combine with two column tiles).
  int park;
  // chain (with park, more than 8 columns): the shares of a run that crosses
  // the edge between consecutive waves of a workgroup are combined by the
  // first of them after the workgroup's barrier (the later ones leave theirs
  // in their parking slots), so that, as with wgc, a run leaves at most one
  // share row per workgroup (row g + segment) and one finished inside the
  // workgroup's range is written as bf16 output there.
  int chain;
  // run_cost: slots of no pages the work split puts ahead of each non-empty
  // (sequence, unit) run, so that pieces holding several runs get fewer
  // pages (0 for the VALU kernel); the prefix sums in ws_pre count slots.
  int run_cost;
  // workspace (see workspace_layout)
  int32_t* ws_pre;      // [B + 1] slots-per-sequence prefix sums (see run_cost)
  float* ws_ml;         // [rows, cols, 2] running max (log2 domain) and sum
  float* ws_o;          // [rows, cols, D] unnormalised partial outputs
  // Fused append (the decode step): when k_new is non-NULL, the new token of
  // sequence b ([B, Hkv, D] bf16) is stored at position context_lens[b] - 1
  // by the wave that reads that position, which also attends to it.  The
  // writable views alias k_cache / v_cache / k_scale / v_scale.
  const uint16_t* k_new;
  const uint16_t* v_new;
  unsigned char* k_cache_w;
  unsigned char* v_cache_w;
  float* k_scale_w;
  float* v_scale_w;
  // RoPE inside the decode step (MFMA kernel, one query per sequence): when
  // rope is set, q and the new keys arrive unrotated and each wave rotates
  // them at position context_lens[b] - 1 with the D / 2 frequencies
  // rope_freq (see RopeParams), as the RoPE append kernel does.
  int rope;
  double rope_freq[64];
};

struct WorkspaceLayout {
  size_t pre_off, ml_off, o_off, total;
  int rows;
};

// Pieces per wave on the work axis (the split is described in
// decode_common.hpp); a piece k that shares a (sequence, kv head) segment
// with other pieces writes row k + segment.
#ifndef PKV_PIECES_PER_WAVE
#define PKV_PIECES_PER_WAVE 1
#endif
constexpr int kPiecesPerWave = PKV_PIECES_PER_WAVE;

constexpr int kAttnBlockThreads = 256;   // 4 independent waves per workgroup
constexpr int kAttnWavesPerBlock = kAttnBlockThreads / 64;

// Shares are combined within workgroups (AttnParams::wgc) when a share row
// has at most this many columns (more than 8 only with two kv heads per
// wave, whose tile buffer holds a 16-column share) and the batch at most
// kWgcMaxBatch sequences, and the LDS for it fits beside the rest at the
// same occupancy.
constexpr int kWgcMaxCols = 16;
constexpr int kWgcMaxBatch = 1024;

// `U` = units per sequence (Hkv / hg), `cols` = hg * G * (query tokens per
// sequence, at most).  With wgc the share rows are per workgroup.
inline WorkspaceLayout workspace_layout(int B, int U, int cols, int D, int total_waves,
                                        int wgc = 0) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  WorkspaceLayout w;
  w.rows = (wgc ? total_waves / kAttnWavesPerBlock : kPiecesPerWave * total_waves) + B * U;
  w.pre_off = 0;
  w.ml_off = w.pre_off + up(sizeof(int32_t) * (size_t)(B + 1));
  w.o_off = w.ml_off + up(sizeof(float) * 2 * (size_t)w.rows * cols);
  w.total = w.o_off + up(sizeof(float) * (size_t)w.rows * cols * D);
  return w;
}

constexpr int kMaxBatch = 8192;          // sequence prefix sums live in LDS

// Batches up to this size keep their context lengths in LDS beside the
// prefix sums (the partition kernels then read a run's length there instead
// of from memory); larger ones would cost occupancy.
constexpr int kLenLdsMax = 2048;
__host__ __device__ inline int len_lds_entries(int B) { return B <= kLenLdsMax ? B : 0; }

// Batches up to this size also keep the query-row offsets (q_start, B + 1
// entries; b for a call without them) there, so that a generalised run's
// query count and first row come from LDS too: loaded from memory, they
// put a second round trip before its q and page-table loads.  (Bounded so
// that the extra LDS moves no occupancy threshold.)
constexpr int kQsLdsMax = 512;
__host__ __device__ inline int qs_lds_entries(int B) { return B <= kQsLdsMax ? B + 1 : 0; }

// 32-bit words of LDS the sequence prefix sums take: s_pre [B + 1], the
// scan's scratch [kAttnBlockThreads], the lengths [len_lds_entries(B)] and
// the query-row offsets [qs_lds_entries(B)].
__host__ __device__ inline size_t prefix_lds_words(int B) {
  return (size_t)B + 1 + kAttnBlockThreads + len_lds_entries(B) + qs_lds_entries(B);
}

// LDS of the sequence prefix sums (plus the scan scratch, the cached
// lengths and query-row offsets) for B sequences.
inline size_t prefix_lds_bytes(int B) { return sizeof(int32_t) * prefix_lds_words(B); }

// The two partition-kernel variants.  Launchers return hipErrorInvalidValue
// for an unsupported (D, BS, G, kind) combination; *_blocks_per_cu give the
// workgroups that fit on one compute unit (0 if unsupported).
enum class AttnPath { kValu = 0, kMfma = 1 };
hipError_t launch_partition_valu(const AttnParams& p, int D, int BS, int G, int kind, int blocks,
                                 hipStream_t stream);
int valu_blocks_per_cu(int D, int BS, int G, int kind, int B);
// (the VALU variant handles one query per sequence and no window only)
// (the MFMA launch takes the unit size from p.hg)
hipError_t launch_partition_mfma(const AttnParams& p, int D, int BS, int G, int kind, int blocks,
                                 hipStream_t stream);
// The occupancy both instantiations (decode and generalised) with hg kv
// heads per wave reach (0 if there is none: mfma_unit_heads(G) is the one hg
// above 1 that exists); with col_tiles = 2, that of the generalised
// instantiation with two 16-column tiles (hg = 1 only).
// wgc: with the LDS of the workgroup combine for shares of wgc columns;
// park: with the parking slot (AttnParams::park: 0, 1 or 2).
int mfma_blocks_per_cu(int D, int BS, int G, int kind, int B, int hg, int col_tiles = 1,
                       int wgc = 0, int park = 0);
int mfma_unit_heads(int G);
// LDS a workgroup of the MFMA variant needs on top of the prefix sums.
size_t mfma_stage_lds_bytes(int D, int hg, int wgc = 0, int park = 0);
int mfma_park_slot_bytes(int D);
// Whether a wave's tile buffer holds a share of wgc columns (the combine
// keeps a wave's end share there).
bool mfma_tile_holds_share(int D, int hg, int wgc);

// Variant used by the attention calls: MFMA unless PKV_ATTN_KERNEL=valu is
// set when the library loads, or pkv_select_partition_kernel changes it.
AttnPath attn_path();
std::atomic<int>& path_flag();

hipError_t launch_merge(const AttnParams& p, int D, int G, hipStream_t stream);

// Rotary embedding parameters (the Llama 3 scaled frequencies; factor 1:
// plain RoPE) and the D / 2 frequencies they give (rope_freqs, host side).
struct RopeParams {
  double theta, factor, low_freq_factor, high_freq_factor, original_max;
  double freq[64];
};
void rope_freqs(int D, RopeParams& rp);

// RoPE of q (into q_out) and of the new keys, then the append of the rotated
// keys and the values into `slots` (see rope_append.hip).  Hkv <= 8.  With
// positions and slots both NULL, token i is sequence i's new token: position
// context_lens[i] - 1, slot from block_tables ([N, MBS]), as the decode step
// places it.
hipError_t launch_rope_append(const void* q, void* q_out, const void* k_new, const void* v_new,
                              const int32_t* positions, const int32_t* slots, void* k_cache,
                              void* v_cache, float* k_scale, float* v_scale, int N, int Hq,
                              int Hkv, int D, int BS, int NB, int kind, const RopeParams& rp,
                              hipStream_t stream, const int32_t* context_lens = nullptr,
                              const int32_t* block_tables = nullptr, int MBS = 0);

// The check of pkv_validate_inputs (validate.hip): the first violation of
// the device-resident contract, as b << 32 | kind << 28 | page, or ~0 for
// none, is left in *first (a word of device memory).
hipError_t launch_validate(const int32_t* block_tables, const int32_t* context_lens,
                           const float* k_scale, const float* v_scale, int B, int Hkv, int BS,
                           int NB, int MBS, unsigned long long* first, hipStream_t stream);

// Streaming read probe (read_probe.hip): the waves of its persistent grid on
// a device with cu_count compute units, and the launch reading the whole
// 1 KB units of buf into sink[waves].
int read_probe_waves(int cu_count);
hipError_t launch_read_probe(const void* buf, size_t bytes, unsigned* sink, int waves,
                             hipStream_t stream);

// One-token append.  With `slots` NULL the slot of token i is derived from
// the block table instead: position context_lens[i] - 1 of sequence i
// (block_tables is [N, MBS]); a length outside [1, MBS * BS] skips the token.
hipError_t launch_kv_append(const void* k_new, const void* v_new, const int32_t* slots,
                            const int32_t* block_tables, const int32_t* context_lens, int MBS,
                            void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                            int N, int Hkv, int D, int BS, int NB, int kind, hipStream_t stream);

}  // namespace pkv
