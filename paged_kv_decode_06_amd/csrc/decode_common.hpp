// Pieces shared by the partition kernels (VALU and MFMA variants).
//
// Semantics ("Decode Phase Attention Forward Pass", sections 2-5): one query
// token per sequence attends, with no causal mask, over positions
// t < context_lens[b] of its history; position t lives at
// (block_tables[b][t / BS], t % BS); query head h reads kv head h / G.
// Generalised ("Prefill Forward Prefix Caching Explained", the bottom-right
// causal mask; the "Decode Phase" glossary's sliding-window and attention-sink
// bullets): sequence b has q_len query tokens, the last q_len of its L
// positions; query i sees key j iff j <= lim = L - q_len + i and, with a
// window W > 0, also j > lim - W or j < sinks.  Only pages holding a key
// some query sees are on the work axis: the sink pages and the window pages.
// The pages' route gathers the history into a zero-padded dense tensor and
// calls a dense kernel; here nothing is gathered: each wave reads the pages
// in place through the block table, and positions past the context length
// are selected away (never weighted by zero, so stale or NaN bytes in a
// block's tail cannot leak in).
//
// Work split (flash-decoding style split of the context).  The work axis is
// every (sequence b, unit u, page j) triple in that order: position
// U*pre[b] + u*n_b + j, where n_b = ceil(L_b / BS) and pre is the prefix
// sum of n_b.  A unit is the set of kv heads one wave serves together: one
// kv head (U = Hkv units per sequence) or, in the MFMA kernel's decode
// instantiations, HG adjacent kv heads (U = Hkv / HG).  The axis is cut into consecutive pieces of equal page count
// for a persistent grid of W waves, so every wave streams the same number of
// KV bytes (to one page) whatever the length mix.  kPiecesPerWave pieces per wave are
// taken from far apart on the axis; the default is one (measured: a second
// or third piece costs more in per-piece setup than it recovers in balance).
//
// A (b, u) run that one piece covers completely is finished in place (out
// written as bf16); otherwise each piece that touches it leaves (m, l, o)
// for its share in workspace row k + segment (segment = b*U + u).  Both k
// and the segment grow along the axis, so the row is unique, and the rows
// of one segment are consecutive for the merge kernel.  m is kept in the
// exp2 domain (scores times scale*log2(e)).
#pragma once

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

// Query tokens of sequence b (1 without q_start), clamped to [0, max_q].
__device__ __forceinline__ int seq_queries(const AttnParams& p, int b) {
  if (p.q_start == nullptr) return 1;
  return min(max(p.q_start[b + 1] - p.q_start[b], 0), p.max_q);
}

// Context length of sequence b, clamped to [0, MBS * BS].
__device__ __forceinline__ int seq_length(const AttnParams& p, int b, int BS) {
  return min(max(p.context_lens[b], 0), p.MBS * BS);
}

// The pages of a sequence on the work axis: axis page j' < ps is table page
// j'; axis page j' >= ps is table page j' + gap.  Without a window (or when
// the sink pages reach the window) that is every page up to ceil(L / BS);
// otherwise the sink pages [0, ceil(sinks / BS)) and the window pages from
// the one holding L - q_len - W + 1 (the oldest key query 0 sees).
struct SeqRange {
  int n, ps, gap;
};

__device__ __forceinline__ SeqRange seq_range(int L, int ql, int sinks, int window, int BS) {
  const int pe = (L + BS - 1) / BS;
  if (window <= 0) return {pe, pe, 0};
  const int lo = max(L - ql - window + 1, 0);
  const int pw = lo / BS;
  const int ps = min((sinks + BS - 1) / BS, pe);
  if (pw <= ps) return {pe, pe, 0};
  return {ps + (pe - pw), ps, pw - ps};
}

__device__ __forceinline__ int seq_pages(const AttnParams& p, int b, int BS) {
  return seq_range(seq_length(p, b, BS), seq_queries(p, b), p.sinks, p.window, BS).n;
}

// Slots a (sequence, unit) run of sequence b takes on the work axis: its
// pages plus p.run_cost slots of no pages ahead of them (none for an empty
// run), so that the split charges each run the fixed cost of starting it.
__device__ __forceinline__ int seq_slots(const AttnParams& p, int b, int BS) {
  const int n = seq_pages(p, b, BS);
  return n > 0 ? n + p.run_cost : 0;
}

// Sequence slot counts (seq_slots) -> exclusive prefix sums in LDS
// (s_pre[0..B]); with
// keep_len also each sequence's context length as given, in
// s_tmp[kAttnBlockThreads + b] for b < B, and, where qs_lds_entries(B) is
// not 0, its first query row (q_start[b], or b without q_start) in
// s_tmp[kAttnBlockThreads + B + b] for b <= B.
// Called by every thread of the workgroup.  Each thread sums the pages of a
// slice of sequences; the slices' sums are scanned within each wave by lane
// shifts, and the waves' totals are added through LDS (one barrier).
__device__ inline void build_prefix(const AttnParams& p, int BS, int32_t* s_pre, int32_t* s_tmp,
                                    bool keep_len) {
  int32_t* s_len = s_tmp + kAttnBlockThreads;
  const int B = p.B;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int lane = tid & (kWave - 1);
  const int per = (B + nt - 1) / nt;
  const int b0 = tid * per;
  const int b1 = min(B, b0 + per);
  int sum = 0;
  const bool keep_qs = keep_len && qs_lds_entries(B) != 0;
  for (int b = b0; b < b1; ++b) {
    if (keep_len) s_len[b] = p.context_lens[b];
    if (keep_qs) s_len[B + b] = p.q_start != nullptr ? p.q_start[b] : b;
    sum += seq_slots(p, b, BS);
  }
  if (keep_qs && tid == nt - 1) s_len[2 * B] = p.q_start != nullptr ? p.q_start[B] : B;
  int incl = sum;   // inclusive scan of the slice sums within the wave
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == kWave - 1) s_tmp[tid / kWave] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int w = 0; w < tid / kWave; ++w) run += s_tmp[w];
  for (int b = b0; b < b1; ++b) {
    s_pre[b] = run;
    run += seq_slots(p, b, BS);
  }
  if (tid == nt - 1) s_pre[B] = run;
  __syncthreads();
}

// Last b in [0, B) with U * pre[b] <= x (x < U * pre[B]).
__device__ __forceinline__ int find_sequence(const int32_t* s_pre, int B, int U, int x) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (U * s_pre[mid] <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// The axis is cut into N = kPiecesPerWave * W consecutive pieces.  By
// default every piece has Qp = ceil(total / N) pages (the last ones fewer or
// none).  When that leaves more than N / 16 pieces empty although there are
// at least N pages (small workloads: a fifth of the grid for the B4 window
// workload), piece k covers [floor(k total / N), floor((k + 1) total / N))
// instead, floor(total / N) or ceil(total / N) >= 1 pages each, so every wave
// has work (3.3% faster there; level on the configurations that leave few
// pieces empty, except 2.5% slower on the 70B-shaped mix, so those keep the
// rounded-up length).  Either way the empty pieces, if any, come after the
// last page: the merge kernel takes every piece between a run's first and
// last page as one that wrote a share of it.  Wave w streams pieces w,
// w + W, w + 2W, ...
struct WorkSplit {
  int total;      // pages on the axis
  int W;          // waves
  int N;          // pieces
  int Qp;         // piece length of the rounded-up split
  bool balanced;  // the floor(k total / N) split
};

__device__ __forceinline__ WorkSplit make_split(int total, int W) {
  WorkSplit s;
  s.total = total;
  s.W = W;
  s.N = kPiecesPerWave * W;
  s.Qp = total > 0 ? (total + s.N - 1) / s.N : 1;
  const int used = (total + s.Qp - 1) / s.Qp;   // pieces the rounded-up split fills
  s.balanced = total >= s.N && 16 * (s.N - used) > s.N;
  return s;
}

// First axis position of piece k (k <= N).
__device__ __forceinline__ int piece_start(const WorkSplit& s, int k) {
  if (s.balanced) return (int)(((int64_t)k * s.total) / s.N);
  return (int)min((int64_t)k * s.Qp, (int64_t)s.total);
}

// Piece containing axis position x < total: the largest k with start(k) <= x.
__device__ __forceinline__ int piece_of(const WorkSplit& s, int x) {
  if (s.balanced) return (int)((((int64_t)x + 1) * s.N - 1) / s.total);
  return x / s.Qp;
}

// Drives one wave through its pieces; body(x, x_end, k) streams axis pages
// [x, x_end) of piece k (empty pieces are skipped).
template <class Body>
__device__ __forceinline__ void run_split(const WorkSplit& s, int wave, Body&& body) {
  for (int i = 0; i < kPiecesPerWave; ++i) {
    const int k = i * s.W + wave;
    const int x = piece_start(s, k);
    const int x_end = piece_start(s, k + 1);
    if (x < x_end) body(x, x_end, k);
  }
}

// One wave's share of a (sequence, unit) run: pages [j0, j1) of run (b, u)
// of n_b pages (none when j0 == j1: the piece holds only slots ahead of the
// pages); `next` is the axis position after the piece's part of the run.
// The run's slots start at run_start, its pages run_cost slots later.
struct Piece {
  int b, u, n_b, run_start, j0, j1, next;
};

__device__ __forceinline__ Piece locate_piece(const int32_t* s_pre, int B, int U, int run_cost,
                                              int x, int x_end) {
  Piece pc;
  pc.b = find_sequence(s_pre, B, U, x);
  const int m = s_pre[pc.b + 1] - s_pre[pc.b];   // slots of each of the sequence's runs
  const int seg_start = U * s_pre[pc.b];
  pc.u = (x - seg_start) / m;
  pc.run_start = seg_start + pc.u * m;
  pc.n_b = m - run_cost;
  pc.next = pc.run_start + min(m, x_end - pc.run_start);
  pc.j0 = max(x - pc.run_start - run_cost, 0);
  pc.j1 = max(pc.next - pc.run_start - run_cost, 0);
  return pc;
}

// Calls f(Sh<D, BS, G, kind>{}) for the supported combination given at run
// time; false if it is not supported.
template <template <int, int, int, int> class Sh, class F>
bool dispatch_shapes(int D, int BS, int G, int kind, F&& f) {
#define PKV_CASE(d, bs, gg, k)                     \
  if (D == d && BS == bs && G == gg && kind == k) { \
    f(Sh<d, bs, gg, k>{});                         \
    return true;                                   \
  }
#define PKV_G(d, bs, k) \
  PKV_CASE(d, bs, 1, k) PKV_CASE(d, bs, 2, k) PKV_CASE(d, bs, 4, k) PKV_CASE(d, bs, 8, k)
#define PKV_BS(d, k) PKV_G(d, 16, k) PKV_G(d, 32, k)
  PKV_BS(64, kKvBf16) PKV_BS(128, kKvBf16) PKV_BS(64, kKvFp8) PKV_BS(128, kKvFp8)
  PKV_BS(64, kKvInt8) PKV_BS(128, kKvInt8)
#undef PKV_BS
#undef PKV_G
#undef PKV_CASE
  return false;
}

}  // namespace pkv
