// C ABI of libpkv.so (declared in include/pkv.h): argument checks, grid
// sizing and dispatch.  No call allocates device memory or synchronises.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <unordered_map>

#include "../../include/pkv.h"
#include "pkv_internal.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device facts, queried once per (device, kernel variant, LDS size).
struct DeviceCache {
  std::mutex mu;
  std::unordered_map<int, int> cu_count;                 // device -> CUs
  std::unordered_map<unsigned long long, int> blocks;    // key -> blocks per CU
};
DeviceCache& cache() {
  static DeviceCache c;
  return c;
}

int current_device(int* dev) { return hipGetDevice(dev) == hipSuccess ? 0 : -1; }

int cu_count(int dev) {
  auto& c = cache();
  std::lock_guard<std::mutex> lk(c.mu);
  auto it = c.cu_count.find(dev);
  if (it != c.cu_count.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
  c.cu_count[dev] = n;
  return n;
}

// LDS of the partition kernel grows with B; occupancy is looked up for B
// rounded up to a multiple of 64 (at most 128 entries per shape; the calls
// and the workspace queries share the lookup, so they agree on the grid).
// hg: kv heads per wave, col_tiles: 16-column tiles per wave (MFMA only).
int blocks_per_cu(int dev, pkv::AttnPath path, int D, int BS, int G, int kind, int B, int hg,
                  int col_tiles = 1, int wgc = 0, int park = 0) {
  const int Bq = ((B + 63) / 64) * 64;
  const unsigned long long key = ((unsigned long long)park << 58) |
                                 ((unsigned long long)(wgc / 8) << 56) |
                                 ((unsigned long long)col_tiles << 52) |
                                 ((unsigned long long)dev << 44) | ((unsigned long long)hg << 40) |
                                 ((unsigned long long)path << 36) |
                                 ((unsigned long long)D << 28) | ((unsigned long long)BS << 20) |
                                 ((unsigned long long)G << 16) | ((unsigned long long)kind << 12) |
                                 (unsigned long long)(Bq / 64);
  auto& c = cache();
  {
    std::lock_guard<std::mutex> lk(c.mu);
    auto it = c.blocks.find(key);
    if (it != c.blocks.end()) return it->second;
  }
  const int n = path == pkv::AttnPath::kMfma
                    ? pkv::mfma_blocks_per_cu(D, BS, G, kind, Bq, hg, col_tiles, wgc, park)
                    : pkv::valu_blocks_per_cu(D, BS, G, kind, Bq);
  std::lock_guard<std::mutex> lk(c.mu);
  c.blocks[key] = n;
  return n;
}

// (G = 16, one kv head's queries filling the 16 MFMA columns, runs on the
// MFMA kernel only: see path_for)
bool supported(int D, int BS, int G, int kv_dtype) {
  return (D == 64 || D == 128) && (BS == 16 || BS == 32) &&
         (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) &&
         (kv_dtype == PKV_KV_BF16 || kv_dtype == PKV_KV_FP8_E4M3FN || kv_dtype == PKV_KV_INT8);
}

// Persistent grid: every workgroup that fits at once on every CU.
int attention_blocks(pkv::AttnPath path, int D, int BS, int G, int kv_dtype, int B, int hg,
                     int col_tiles = 1, int wgc = 0) {
  int dev;
  if (current_device(&dev) != 0) return 0;
  const int ncu = cu_count(dev);
  const int per_cu = blocks_per_cu(dev, path, D, BS, G, kv_dtype, B, hg, col_tiles, wgc);
  return ncu * per_cu;
}

// Largest unit (kv heads per partition wave) the decode-shaped calls may
// use: 0 = the kernel's own (pkv::mfma_unit_heads), 1 = one kv head.
std::atomic<int>& unit_heads_flag() {
  static std::atomic<int> flag([] {
    const char* e = std::getenv("PKV_UNIT_HEADS");
    return (e && std::string(e) == "1") ? 1 : 0;
  }());
  return flag;
}

// Workgroup combine of the partition kernel's shares (pkv::AttnParams::wgc,
// and the chain of parked shares, pkv::AttnParams::chain): on unless
// PKV_SHARE_COMBINE=0 is set when the library loads or
// pkv_select_share_combine(0) switched it off; see combine_cols and
// share_chain.
std::atomic<int>& share_combine_flag() {
  static std::atomic<int> flag([] {
    const char* e = std::getenv("PKV_SHARE_COMBINE");
    return (e && std::string(e) == "0") ? 0 : 1;
  }());
  return flag;
}

// The column capacity of the combine's share slots for an MFMA call whose
// share rows have `cols` columns (0: no combine): 8 for up to 8 columns, 16
// for up to 16 when a wave's tile buffer holds such a share (two kv heads
// per wave) and the larger slots leave the workgroups per CU as they are.
// Batches above kWgcMaxBatch take none.
int combine_cols(pkv::AttnPath path, int D, int BS, int G, int kind, int B, int hg, int cols) {
  if (path != pkv::AttnPath::kMfma || !share_combine_flag().load(std::memory_order_relaxed) ||
      cols > pkv::kWgcMaxCols || B > pkv::kWgcMaxBatch || pkv::kPiecesPerWave != 1)
    return 0;
  const int w = cols <= 8 ? 8 : 16;
  if (!pkv::mfma_tile_holds_share(D, hg, w)) return 0;
  if (w > 8) {
    int dev;
    if (current_device(&dev) != 0 ||
        blocks_per_cu(dev, path, D, BS, G, kind, B, hg, 1, w) <
            blocks_per_cu(dev, path, D, BS, G, kind, B, hg, 1, 0))
      return 0;
  }
  return w;
}

// Slots of no pages ahead of each run on the MFMA kernel's work axis
// (pkv::AttnParams::run_cost): PKV_RUN_COST when the library loads, else
// kDefaultRunCost; pkv_select_run_cost changes it.
constexpr int kDefaultRunCost = 2;
constexpr int kMaxRunCost = 8;
std::atomic<int>& run_cost_flag() {
  static std::atomic<int> flag([] {
    const char* e = std::getenv("PKV_RUN_COST");
    if (e && *e) {   // (a value that is not a whole number in range keeps the default)
      char* end = nullptr;
      const long v = std::strtol(e, &end, 10);
      if (end && *end == '\0' && v >= 0 && v <= kMaxRunCost) return (int)v;
    }
    return kDefaultRunCost;
  }());
  return flag;
}

// Parking of mid-piece results (pkv::AttnParams::park): on unless
// PKV_RESULT_PARKING=0 is set when the library loads or
// pkv_select_result_parking(0) switched it off; see parking.
std::atomic<int>& parking_flag() {
  static std::atomic<int> flag([] {
    const char* e = std::getenv("PKV_RESULT_PARKING");
    return (e && std::string(e) == "0") ? 0 : 1;
  }());
  return flag;
}


// Columns (kv heads per wave * G * max_q) one partition wave serves: the 16
// MFMA columns, or two tiles of them in the generalised call with one kv
// head per wave.
constexpr int kTileCols = 16;
constexpr int kMaxCols = 2 * kTileCols;

// 16-column tiles of a wave serving `cols` columns.
int col_tiles(int cols) { return (cols + kTileCols - 1) / kTileCols; }

// Whether a generalised MFMA call parks its mid-piece results: one kv head
// per wave, no combine, and the slot leaves the workgroups per CU (hence the
// grid and the workspace) as they are.
int parking(pkv::AttnPath path, int D, int BS, int G, int kind, int B, int hg, int cols, int wgc,
            bool gen) {
  if (!gen || path != pkv::AttnPath::kMfma || hg != 1 || wgc != 0 || cols > kMaxCols ||
      !parking_flag().load(std::memory_order_relaxed))
    return 0;
  int dev;
  if (current_device(&dev) != 0) return 0;
  const int t = col_tiles(cols);
  const int with = blocks_per_cu(dev, path, D, BS, G, kind, B, 1, t, 0, 1);
  return with > 0 && with == blocks_per_cu(dev, path, D, BS, G, kind, B, 1, t, 0, 0) ? 1 : 0;
}

// Whether a parking call combines a run's shares across the edges between
// the waves of a workgroup (pkv::AttnParams::chain): with more than 8
// columns (8 or fewer take the workgroup combine, whose slots hold both of
// a wave's shares), under the share-combine switch.  Two column tiles need
// park mode 2 (room for a second share from the tile buffer on), taken only
// when it leaves the workgroups per CU unchanged; `park` is raised to 2
// then.  It keeps the grid and needs fewer share rows than the workspace
// holds.
int share_chain(int& park, pkv::AttnPath path, int D, int BS, int G, int kind, int B, int cols) {
  if (!park || cols <= 8 || cols > kMaxCols || pkv::kPiecesPerWave != 1 ||
      !share_combine_flag().load(std::memory_order_relaxed))
    return 0;
  if (cols <= kTileCols) return 1;
  int dev;
  if (current_device(&dev) != 0) return 0;
  const int with = blocks_per_cu(dev, path, D, BS, G, kind, B, 1, 2, 0, 2);
  if (with <= 0 || with != blocks_per_cu(dev, path, D, BS, G, kind, B, 1, 2, 0, 0)) return 0;
  park = 2;
  return 1;
}

// Windowed calls whose work is this small (at most this many pages per
// wave with one kv head per wave, bounded by the window on the host) run one
// head per wave: the 1.5x grid starts more streams at once, and on the B4
// 131072-token call with an 8192-token window (about 5 pages per wave) the
// partition kernel measured 2.4% faster (27.7-28.0 vs 28.4-28.7 us).
constexpr int kSmallWindowPagesPerWave = 8;

// Pages a sequence can have on the work axis of a windowed call (sink pages,
// window pages and the partial pages at either end), at most MBS.
long long window_pages_bound(int BS, int MBS, int max_q, int sinks, int window) {
  const long long w = (window + max_q - 1 + BS - 1) / BS + 1 + (sinks + BS - 1) / BS;
  return w < MBS ? w : MBS;
}

// A wave of the MFMA kernel serves hg adjacent kv heads when hg divides
// Hkv, the unit's columns (hg * G per query, max_q queries per sequence)
// fit the 16 of the MFMA, and the wider instantiation still fits two
// workgroups on a CU; otherwise one.  A windowed call (window > 0) whose
// bounded work would give one-head waves at most kSmallWindowPagesPerWave
// pages each takes one head.
int unit_heads(pkv::AttnPath path, int D, int BS, int G, int Hkv, int kv_dtype, int B, bool gen,
               int max_q = 1, int MBS = 0, int sinks = 0, int window = 0) {
  if (path != pkv::AttnPath::kMfma || unit_heads_flag().load(std::memory_order_relaxed) == 1)
    return 1;
  const int hg = pkv::mfma_unit_heads(G);
  if (hg <= 1 || Hkv % hg != 0 || hg * G * max_q > kTileCols) return 1;
  int dev;
  if (current_device(&dev) != 0) return 1;
  if (gen && window > 0 && MBS > 0) {
    const int cols1 = G * max_q;
    const long long waves1 =
        (long long)cu_count(dev) * pkv::kAttnWavesPerBlock *
        blocks_per_cu(dev, path, D, BS, G, kv_dtype, B, 1, col_tiles(cols1),
                      combine_cols(path, D, BS, G, kv_dtype, B, 1, cols1));
    const long long pages1 = (long long)B * Hkv * window_pages_bound(BS, MBS, max_q, sinks, window);
    if (waves1 > 0 && pages1 <= kSmallWindowPagesPerWave * waves1) return 1;
  }
  return blocks_per_cu(dev, path, D, BS, G, kv_dtype, B, hg, 1,
                       combine_cols(path, D, BS, G, kv_dtype, B, hg, hg * G * max_q)) >= 2
             ? hg
             : 1;
}

struct AttnCall {
  pkv::AttnParams p;
  pkv::AttnPath path;
  int D, BS, G, blocks;
  int kind;          // pkv::KvKind (= kv_dtype)
  size_t ws_used = 0;   // workspace bytes the call's layout takes (a multiple of 256)
};

// Room for a rotated copy of q ([B, Hq, D] bf16) at the end of a decode step
// with RoPE's workspace.
size_t rope_q_room(int B, int Hq, int D) {
  return ((size_t)B * Hq * D * 2 + 255) & ~size_t(255);
}

// Options beyond one query per sequence; the defaults are the decode call.
struct QueryOpts {
  const int32_t* q_start = nullptr;
  int max_q = 1;
  int sinks = 0;
  int window = 0;
  bool general = false;   // the generalised call: always the MFMA kernel
};

int check_query_opts(const QueryOpts& o, int G) {
  if (o.max_q < 1) return fail(PKV_ERR_SHAPE, "max_q_len=%d must be at least 1", o.max_q);
  if (o.q_start == nullptr && o.max_q != 1)
    return fail(PKV_ERR_SHAPE, "max_q_len=%d needs q_start (NULL means one query each)", o.max_q);
  if ((long long)G * o.max_q > kMaxCols)
    return fail(PKV_ERR_UNSUPPORTED, "G * max_q_len = %d * %d exceeds %d", G, o.max_q, kMaxCols);
  if (o.sinks < 0 || o.window < 0)
    return fail(PKV_ERR_SHAPE, "sink_tokens=%d and window_tokens=%d must be >= 0", o.sinks, o.window);
  return PKV_OK;
}

// The partition kernel a call runs: the selected one, except that the
// generalised call and groups of 16 always run the MFMA kernel.
pkv::AttnPath path_for(const QueryOpts& o, int G) {
  return o.general || G > 8 ? pkv::AttnPath::kMfma : pkv::attn_path();
}

int prepare_attention(const void* q, const void* k_cache, const void* v_cache,
                      const float* k_scale, const float* v_scale, const int32_t* block_tables,
                      const int32_t* context_lens, float scale, void* out, int B, int Hq, int Hkv,
                      int D, int BS, int NB, int MBS, int kv_dtype, void* workspace,
                      size_t workspace_bytes, AttnCall* call, bool step = false,
                      const void* k_new = nullptr, const void* v_new = nullptr,
                      const QueryOpts& opts = QueryOpts()) {
  g_last_error.clear();
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0 || NB <= 0 || MBS <= 0)
    return fail(PKV_ERR_SHAPE, "sizes must be positive (B may be 0): B=%d Hq=%d Hkv=%d D=%d BS=%d NB=%d MBS=%d",
                B, Hq, Hkv, D, BS, NB, MBS);
  if (Hq % Hkv != 0) return fail(PKV_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  const int G = Hq / Hkv;
  if (!supported(D, BS, G, kv_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "unsupported D=%d BS=%d G=%d kv_dtype=%d", D, BS, G, kv_dtype);
  if (int st = check_query_opts(opts, G)) return st;
  if (B > pkv::kMaxBatch) return fail(PKV_ERR_UNSUPPORTED, "B=%d exceeds %d", B, pkv::kMaxBatch);
  if ((long long)MBS * BS > (1LL << 30))
    return fail(PKV_ERR_SHAPE, "MBS*BS=%lld is too large", (long long)MBS * BS);
  if (B == 0) return PKV_OK;   // nothing to do; pointers may be NULL
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return fail(PKV_ERR_NULL, "a required tensor pointer is NULL");
  if (step && (!k_new || !v_new)) return fail(PKV_ERR_NULL, "k_new and v_new are required");
  if ((((uintptr_t)opts.q_start) & 3u) != 0)
    return fail(PKV_ERR_ALIGN, "q_start must be 4-byte aligned");
  const bool q8 = kv_dtype != PKV_KV_BF16;
  if (q8 && (!k_scale || !v_scale)) return fail(PKV_ERR_NULL, "fp8 / int8 cache needs k_scale and v_scale");
  if (!q8 && (k_scale || v_scale)) return fail(PKV_ERR_SHAPE, "bf16 cache takes no scales");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(PKV_ERR_ALIGN, "q, caches and out must be 16-byte aligned");
  if (step && (!aligned16(k_new) || !aligned16(v_new)))
    return fail(PKV_ERR_ALIGN, "k_new and v_new must be 16-byte aligned");
  if (q8 && ((((uintptr_t)k_scale) | ((uintptr_t)v_scale)) & 3u))
    return fail(PKV_ERR_ALIGN, "scales must be 4-byte aligned");
  const pkv::AttnPath path = path_for(opts, G);
  const bool gen = opts.q_start != nullptr || opts.max_q > 1 || opts.window > 0;
  const int hg = unit_heads(path, D, BS, G, Hkv, kv_dtype, B, gen, opts.max_q, MBS, opts.sinks,
                            opts.window);
  const int cols = hg * G * opts.max_q;
  const int wgc = combine_cols(path, D, BS, G, kv_dtype, B, hg, cols);
  // (parking keeps the grid: the workspace queries need not know of it)
  int park = parking(path, D, BS, G, kv_dtype, B, hg, cols, wgc, gen);
  const int chain = share_chain(park, path, D, BS, G, kv_dtype, B, cols);
  const int blocks = attention_blocks(path, D, BS, G, kv_dtype, B, hg, col_tiles(cols), wgc);
  if (blocks <= 0) return fail(PKV_ERR_HIP, "could not size the grid on the current device");
  const int waves = blocks * pkv::kAttnWavesPerBlock;
  const pkv::WorkspaceLayout lay = pkv::workspace_layout(B, Hkv / hg, cols, D, waves, wgc);
  call->ws_used = lay.total;
  if (!workspace || workspace_bytes < lay.total)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                workspace_bytes, lay.total);
  if (!aligned16(workspace)) return fail(PKV_ERR_ALIGN, "workspace must be 16-byte aligned");

  pkv::AttnParams& p = call->p;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.NB = NB;
  p.MBS = MBS;
  p.q_start = opts.q_start;
  p.max_q = opts.max_q;
  p.cols = cols;
  p.sinks = opts.sinks;
  p.window = opts.window;
  p.hg = hg;
  p.total_waves = waves;
  p.wgc = wgc;
  p.park = park;
  p.chain = chain;
  p.run_cost = path == pkv::AttnPath::kMfma ? run_cost_flag().load(std::memory_order_relaxed) : 0;
  char* ws = static_cast<char*>(workspace);
  p.ws_pre = reinterpret_cast<int32_t*>(ws + lay.pre_off);
  p.ws_ml = reinterpret_cast<float*>(ws + lay.ml_off);
  p.ws_o = reinterpret_cast<float*>(ws + lay.o_off);
  p.k_new = nullptr;
  p.v_new = nullptr;
  p.k_cache_w = nullptr;
  p.v_cache_w = nullptr;
  p.k_scale_w = nullptr;
  p.v_scale_w = nullptr;
  p.rope = 0;
  call->path = path;
  call->D = D;
  call->BS = BS;
  call->G = G;
  call->kind = kv_dtype;
  call->blocks = blocks;
  call->ws_used = lay.total;
  return PKV_OK;
}

hipError_t launch_partition(const AttnCall& c, hipStream_t s) {
  return c.path == pkv::AttnPath::kMfma
             ? pkv::launch_partition_mfma(c.p, c.D, c.BS, c.G, c.kind, c.blocks, s)
             : pkv::launch_partition_valu(c.p, c.D, c.BS, c.G, c.kind, c.blocks, s);
}

}  // namespace

namespace pkv {
std::atomic<int>& path_flag() {
  static std::atomic<int> flag([] {
    const char* e = std::getenv("PKV_ATTN_KERNEL");
    return (e && std::string(e) == "valu") ? (int)AttnPath::kValu : (int)AttnPath::kMfma;
  }());
  return flag;
}
AttnPath attn_path() { return static_cast<AttnPath>(path_flag().load(std::memory_order_relaxed)); }
}  // namespace pkv

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "null pointer";
    case PKV_ERR_SHAPE: return "bad shape";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_WORKSPACE: return "workspace too small";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_ALIGN: return "misaligned pointer";
    case PKV_ERR_INPUT: return "device-resident input breaks the contract";
    default: return "unknown status";
  }
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

int pkv_select_partition_kernel(int variant) {
  if (variant != PKV_PARTITION_VALU && variant != PKV_PARTITION_MFMA)
    return fail(PKV_ERR_UNSUPPORTED, "unknown partition kernel variant %d", variant);
  pkv::path_flag().store(variant, std::memory_order_relaxed);
  return PKV_OK;
}

int pkv_partition_kernel(void) { return (int)pkv::attn_path(); }

int pkv_attention_waves(int B, int Hq, int Hkv, int D, int BS, int kv_dtype) {
  if (B < 1 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || B > pkv::kMaxBatch) return 0;
  const int G = Hq / Hkv;
  if (!supported(D, BS, G, kv_dtype)) return 0;
  const pkv::AttnPath path = path_for(QueryOpts{}, G);
  const int hg = unit_heads(path, D, BS, G, Hkv, kv_dtype, B, false);
  return attention_blocks(path, D, BS, G, kv_dtype, B, hg, 1,
                          combine_cols(path, D, BS, G, kv_dtype, B, hg, hg * G)) *
         pkv::kAttnWavesPerBlock;
}

int pkv_decode_unit_heads(int B, int Hq, int Hkv, int D, int BS, int kv_dtype) {
  if (B < 1 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || B > pkv::kMaxBatch) return 0;
  const int G = Hq / Hkv;
  if (!supported(D, BS, G, kv_dtype)) return 0;
  return unit_heads(path_for(QueryOpts{}, G), D, BS, G, Hkv, kv_dtype, B, false);
}

int pkv_read_probe_waves(void) {
  int dev;
  if (current_device(&dev) != 0) return 0;
  return pkv::read_probe_waves(cu_count(dev));
}

int pkv_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                   void* stream) {
  g_last_error.clear();
  if (bytes == 0) return PKV_OK;
  if (!buf || !sink) return fail(PKV_ERR_NULL, "buf and sink are required");
  if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u))
    return fail(PKV_ERR_ALIGN, "buf must be 16-byte and sink 4-byte aligned");
  const int waves = pkv_read_probe_waves();
  if (waves <= 0) return fail(PKV_ERR_HIP, "could not size the probe's grid on the current device");
  if (sink_words < (size_t)waves)
    return fail(PKV_ERR_WORKSPACE, "sink of %zu words is smaller than the %d waves", sink_words,
                waves);
  hipError_t e = pkv::launch_read_probe(buf, bytes, sink, waves, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_fail(e, "read probe launch");
}

int pkv_select_share_combine(int mode) {
  if (mode != 0 && mode != 1)
    return fail(PKV_ERR_UNSUPPORTED, "share-combine mode %d is not 0 or 1", mode);
  share_combine_flag().store(mode, std::memory_order_relaxed);
  return PKV_OK;
}

int pkv_select_run_cost(int slots) {
  if (slots < 0 || slots > kMaxRunCost)
    return fail(PKV_ERR_UNSUPPORTED, "run cost %d is not in 0..%d", slots, kMaxRunCost);
  run_cost_flag().store(slots, std::memory_order_relaxed);
  return PKV_OK;
}

int pkv_select_result_parking(int mode) {
  if (mode != 0 && mode != 1)
    return fail(PKV_ERR_UNSUPPORTED, "result-parking mode %d is not 0 or 1", mode);
  parking_flag().store(mode, std::memory_order_relaxed);
  return PKV_OK;
}

int pkv_select_unit_heads(int mode) {
  if (mode != 0 && mode != 1) return fail(PKV_ERR_UNSUPPORTED, "unit-heads mode %d is not 0 or 1", mode);
  unit_heads_flag().store(mode, std::memory_order_relaxed);
  return PKV_OK;
}

}  // extern "C"

namespace {
size_t workspace_bytes_for(int B, int Hq, int Hkv, int D, int BS, int MBS, int kv_dtype,
                           int max_q, bool general) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || MBS <= 0 || Hq % Hkv != 0 || max_q < 1) return 0;
  const int G = Hq / Hkv;
  if (!supported(D, BS, G, kv_dtype) || B > pkv::kMaxBatch || G * max_q > kMaxCols) return 0;
  QueryOpts o;
  o.general = general;
  const pkv::AttnPath path = path_for(o, G);
  // the general call is decode-shaped or not depending on q_start and the
  // window, and a small windowed one takes one kv head per wave: size for
  // every unit choice
  size_t need = 0;
  for (int gen = general ? 2 : 0; gen >= 0; --gen) {
    if (gen == 0 && max_q > 1) continue;
    const int hg = gen == 2 ? 1 : unit_heads(path, D, BS, G, Hkv, kv_dtype, B, gen != 0, max_q);
    const int cols = hg * G * max_q;
    const int wgc = combine_cols(path, D, BS, G, kv_dtype, B, hg, cols);
    const int blocks = attention_blocks(path, D, BS, G, kv_dtype, B, hg, col_tiles(cols), wgc);
    if (blocks <= 0) return 0;
    const int waves = blocks * pkv::kAttnWavesPerBlock;
    const size_t t = pkv::workspace_layout(B, Hkv / hg, cols, D, waves, wgc).total;
    if (t > need) need = t;
  }
  return need;
}
}  // namespace

extern "C" {

size_t pkv_paged_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int BS, int MBS,
                                        int kv_dtype) {
  return workspace_bytes_for(B, Hq, Hkv, D, BS, MBS, kv_dtype, 1, false);
}

size_t pkv_paged_attention_workspace_bytes(int B, int Hq, int Hkv, int D, int BS, int MBS,
                                           int kv_dtype, int max_q_len) {
  return workspace_bytes_for(B, Hq, Hkv, D, BS, MBS, kv_dtype, max_q_len, true);
}

size_t pkv_decode_step_rope_workspace_bytes(int B, int Hq, int Hkv, int D, int BS, int MBS,
                                            int kv_dtype) {
  const size_t n = workspace_bytes_for(B, Hq, Hkv, D, BS, MBS, kv_dtype, 1, true);
  return n == 0 ? 0 : n + rope_q_room(B, Hq, D);
}

int pkv_paged_attention(const void* q, const int32_t* q_start, int max_q_len,
                        const void* k_cache, const void* v_cache, const float* k_scale,
                        const float* v_scale, const int32_t* block_tables,
                        const int32_t* context_lens, float scale, int sink_tokens,
                        int window_tokens, void* out, int B, int Hq, int Hkv, int D, int BS,
                        int NB, int MBS, int kv_dtype, void* workspace, size_t workspace_bytes,
                        void* stream) {
  QueryOpts o;
  o.q_start = q_start;
  o.max_q = max_q_len;
  o.sinks = sink_tokens;
  o.window = window_tokens;
  o.general = true;
  AttnCall call;
  int st = prepare_attention(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                             scale, out, B, Hq, Hkv, D, BS, NB, MBS, kv_dtype, workspace,
                             workspace_bytes, &call, false, nullptr, nullptr, o);
  if (st != PKV_OK) return st;
  if (B == 0) return PKV_OK;
  if (q_start == nullptr && max_q_len != 1)
    return fail(PKV_ERR_SHAPE, "max_q_len > 1 needs q_start");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_partition(call, s);
  if (e != hipSuccess) return hip_fail(e, "partition kernel launch");
  e = pkv::launch_merge(call.p, call.D, call.G, s);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "merge kernel launch");
}

int pkv_paged_decode_partition(const void* q, const void* k_cache, const void* v_cache,
                               const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, const int32_t* context_lens,
                               float scale, void* out, int B, int Hq, int Hkv, int D, int BS,
                               int NB, int MBS, int kv_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  AttnCall call;
  int st = prepare_attention(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                             scale, out, B, Hq, Hkv, D, BS, NB, MBS, kv_dtype, workspace,
                             workspace_bytes, &call);
  if (st != PKV_OK) return st;
  if (B == 0) return PKV_OK;
  hipError_t e = launch_partition(call, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_fail(e, "partition kernel launch");
}

int pkv_paged_decode_merge(const void* q, const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_tables, const int32_t* context_lens, float scale,
                           void* out, int B, int Hq, int Hkv, int D, int BS, int NB, int MBS,
                           int kv_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  AttnCall call;
  int st = prepare_attention(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                             scale, out, B, Hq, Hkv, D, BS, NB, MBS, kv_dtype, workspace,
                             workspace_bytes, &call);
  if (st != PKV_OK) return st;
  if (B == 0) return PKV_OK;
  hipError_t e = pkv::launch_merge(call.p, call.D, call.G, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_fail(e, "merge kernel launch");
}

int pkv_paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                               const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, const int32_t* context_lens,
                               float scale, void* out, int B, int Hq, int Hkv, int D, int BS,
                               int NB, int MBS, int kv_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  AttnCall call;
  int st = prepare_attention(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                             scale, out, B, Hq, Hkv, D, BS, NB, MBS, kv_dtype, workspace,
                             workspace_bytes, &call);
  if (st != PKV_OK) return st;
  if (B == 0) return PKV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_partition(call, s);
  if (e != hipSuccess) return hip_fail(e, "partition kernel launch");
  e = pkv::launch_merge(call.p, call.D, call.G, s);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "merge kernel launch");
}

}  // extern "C"

namespace {

// The workspace of pkv_paged_decode_attention_noalloc, for callers that cannot
// allocate: a static device array, one copy per GPU (the loader places it when
// the library's code object is loaded on a device; it stays until the
// process ends).  Host code never passes `scratch` itself to a kernel (on the
// host that name is a stand-in, not a device address): it looks up each
// device's address once, with that device current, and uses that.
constexpr size_t kStaticScratchBytes = PKV_STATIC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

struct ScratchTable {
  std::mutex mu;
  std::unordered_map<int, void*> ptr;   // device -> address of its `scratch`
};
ScratchTable& scratch_table() {
  static ScratchTable t;
  return t;
}

// The current device's address of `scratch` (looked up on the first call on
// that device), or NULL with *err set.
void* static_scratch(hipError_t* err) {
  int dev;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  auto& t = scratch_table();
  std::lock_guard<std::mutex> lk(t.mu);
  auto it = t.ptr.find(dev);
  if (it != t.ptr.end()) return it->second;
  void* p = nullptr;
  *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (*err != hipSuccess || p == nullptr) {
    if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
    return nullptr;
  }
  t.ptr[dev] = p;
  return p;
}

// A placeholder workspace address for the host-side checks (16-byte aligned,
// never dereferenced: the checks launch nothing).
void* const kCheckOnly = reinterpret_cast<void*>(uintptr_t(256));

}  // namespace

extern "C" {

int pkv_paged_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       float scale, void* out, int B, int Hq, int Hkv, int D,
                                       int BS, int NB, int MBS, int kv_dtype, void* stream) {
  AttnCall call;
  // host-side checks and the call's layout first, against the scratch's size
  int st = prepare_attention(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                             scale, out, B, Hq, Hkv, D, BS, NB, MBS, kv_dtype, kCheckOnly,
                             kStaticScratchBytes, &call);
  if (st == PKV_ERR_WORKSPACE)
    return fail(PKV_ERR_WORKSPACE, "these sizes need %zu bytes of workspace, more than the %zu "
                "bytes of the static scratch; use pkv_paged_decode_attention with a workspace",
                call.ws_used, kStaticScratchBytes);
  if (st != PKV_OK) return st;
  if (B == 0) return PKV_OK;
  hipError_t e;
  void* ws = static_scratch(&e);
  if (ws == nullptr) return hip_fail(e, "address of the static scratch");
  st = prepare_attention(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, scale,
                         out, B, Hq, Hkv, D, BS, NB, MBS, kv_dtype, ws, kStaticScratchBytes, &call);
  if (st != PKV_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  e = launch_partition(call, s);
  if (e != hipSuccess) return hip_fail(e, "partition kernel launch");
  e = pkv::launch_merge(call.p, call.D, call.G, s);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "merge kernel launch");
}

int pkv_validate_inputs(const void* q, const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale, const int32_t* block_tables,
                        const int32_t* context_lens, float scale, void* out, int B, int Hq,
                        int Hkv, int D, int BS, int NB, int MBS, int kv_dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  AttnCall call;
  int st = prepare_attention(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                             scale, out, B, Hq, Hkv, D, BS, NB, MBS, kv_dtype, workspace,
                             workspace_bytes, &call);
  if (st != PKV_OK) return st;
  if (B == 0) return PKV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // (the workspace's first word; the attention call rewrites it)
  auto* first = static_cast<unsigned long long*>(workspace);
  const bool q8 = kv_dtype != PKV_KV_BF16;
  hipError_t e = pkv::launch_validate(block_tables, context_lens, q8 ? k_scale : nullptr,
                                      q8 ? v_scale : nullptr, B, Hkv, BS, NB, MBS, first, s);
  if (e != hipSuccess) return hip_fail(e, "validation kernel launch");
  unsigned long long key = 0;
  e = hipMemcpyAsync(&key, first, sizeof(key), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "validation readback");
  if (key == ~0ull) return PKV_OK;
  const int b = (int)(key >> 32), kind = (int)((key >> 28) & 0xf), j = (int)(key & 0xfffffff);
  int32_t val = 0;
  const int32_t* src = kind == 0 ? context_lens + b : block_tables + (long long)b * MBS + j;
  e = hipMemcpy(&val, src, sizeof(val), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "validation readback");
  switch (kind) {
    case 0:
      return fail(PKV_ERR_INPUT, "sequence %d: context length %d outside [1, MBS*BS = %lld]", b,
                  val, (long long)MBS * BS);
    case 1:
      return fail(PKV_ERR_INPUT, "sequence %d, page %d: block id %d outside [0, NB = %d)", b, j,
                  val, NB);
    default:
      return fail(PKV_ERR_INPUT, "sequence %d, page %d (block %d): a %s scale of the block is "
                  "not a positive finite number", b, j, val, kind == 2 ? "K" : "V");
  }
}

}  // extern "C"

namespace {

// The decode step's launches: the first half (append + partition) and, when
// `merge`, the log-sum-exp merge.
// rope != NULL: the decode step with RoPE of q and the new keys inside the
// partition kernel (always the MFMA kernel).
int decode_step_impl(const void* q, const void* k_new, const void* v_new, void* k_cache,
                     void* v_cache, float* k_scale, float* v_scale, const int32_t* block_tables,
                     const int32_t* context_lens, float scale, void* out, int B, int Hq, int Hkv,
                     int D, int BS, int NB, int MBS, int kv_dtype, void* workspace,
                     size_t workspace_bytes, void* stream, bool merge,
                     const pkv::RopeParams* rope = nullptr) {
  AttnCall call;
  QueryOpts opts;
  opts.general = rope != nullptr;
  int st = prepare_attention(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                             scale, out, B, Hq, Hkv, D, BS, NB, MBS, kv_dtype, workspace,
                             workspace_bytes, &call, true, k_new, v_new, opts);
  if (st != PKV_OK) return st;
  if (B == 0) return PKV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  // RoPE with one kv head per wave (odd Hkv, say): the fused kernel's
  // one-head instantiation is slower than the two calls the step is defined
  // to equal (129.9 vs 112.5 us on a B64 Hq32 Hkv8 step), so when the
  // workspace has room for the rotated q, those two calls are what runs:
  // the RoPE append at each sequence's last position, then the attention.
  if (rope && call.path == pkv::AttnPath::kMfma && call.p.hg == 1 && Hkv <= 8) {
    const size_t room = rope_q_room(B, Hq, D);
    if (workspace_bytes >= call.ws_used + room) {
      void* q_rot = static_cast<char*>(workspace) + ((workspace_bytes - room) & ~size_t(255));
      e = pkv::launch_rope_append(q, q_rot, k_new, v_new, nullptr, nullptr, k_cache, v_cache,
                                  k_scale, v_scale, B, Hq, Hkv, D, BS, NB, call.kind, *rope, s,
                                  context_lens, block_tables, MBS);
      if (e != hipSuccess) return hip_fail(e, "rope_kv_append kernel launch");
      call.p.q = q_rot;
      e = launch_partition(call, s);
      if (e != hipSuccess) return hip_fail(e, "partition kernel launch");
      if (!merge) return PKV_OK;
      e = pkv::launch_merge(call.p, call.D, call.G, s);
      return e == hipSuccess ? PKV_OK : hip_fail(e, "merge kernel launch");
    }
  }
  if (call.path == pkv::AttnPath::kMfma) {
    pkv::AttnParams& p = call.p;
    if (rope) {
      p.rope = 1;
      for (int i = 0; i < 64; ++i) p.rope_freq[i] = rope->freq[i];
    }
    p.k_new = static_cast<const uint16_t*>(k_new);
    p.v_new = static_cast<const uint16_t*>(v_new);
    p.k_cache_w = static_cast<unsigned char*>(k_cache);
    p.v_cache_w = static_cast<unsigned char*>(v_cache);
    p.k_scale_w = k_scale;
    p.v_scale_w = v_scale;
    e = launch_partition(call, s);
    if (e != hipSuccess) return hip_fail(e, "partition kernel launch");
  } else {
    e = pkv::launch_kv_append(k_new, v_new, nullptr, block_tables, context_lens, MBS, k_cache,
                              v_cache, k_scale, v_scale, B, Hkv, D, BS, NB, call.kind, s);
    if (e != hipSuccess) return hip_fail(e, "kv_append kernel launch");
    e = launch_partition(call, s);
    if (e != hipSuccess) return hip_fail(e, "partition kernel launch");
  }
  if (!merge) return PKV_OK;
  e = pkv::launch_merge(call.p, call.D, call.G, s);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "merge kernel launch");
}

}  // namespace

extern "C" {

int pkv_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                    void* v_cache, float* k_scale, float* v_scale, const int32_t* block_tables,
                    const int32_t* context_lens, float scale, void* out, int B, int Hq, int Hkv,
                    int D, int BS, int NB, int MBS, int kv_dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return decode_step_impl(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables,
                          context_lens, scale, out, B, Hq, Hkv, D, BS, NB, MBS, kv_dtype,
                          workspace, workspace_bytes, stream, true);
}

int pkv_decode_step_partition(const void* q, const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* block_tables, const int32_t* context_lens,
                              float scale, void* out, int B, int Hq, int Hkv, int D, int BS,
                              int NB, int MBS, int kv_dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return decode_step_impl(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables,
                          context_lens, scale, out, B, Hq, Hkv, D, BS, NB, MBS, kv_dtype,
                          workspace, workspace_bytes, stream, false);
}

int pkv_decode_step_rope(const void* q, const void* k_new, const void* v_new, void* k_cache,
                         void* v_cache, float* k_scale, float* v_scale,
                         const int32_t* block_tables, const int32_t* context_lens, float scale,
                         double rope_theta, double rope_factor, double low_freq_factor,
                         double high_freq_factor, double original_max_len, void* out, int B,
                         int Hq, int Hkv, int D, int BS, int NB, int MBS, int kv_dtype,
                         void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!(rope_theta > 1.0) || !(rope_factor > 0.0) || !(low_freq_factor > 0.0) ||
      !(high_freq_factor > low_freq_factor) || !(original_max_len > 0.0))
    return fail(PKV_ERR_SHAPE, "rope parameters: theta > 1, factor > 0, 0 < low_freq_factor < "
                "high_freq_factor and original_max_len > 0 are required");
  if (D != 64 && D != 128) return fail(PKV_ERR_UNSUPPORTED, "unsupported D=%d", D);
  pkv::RopeParams rp{rope_theta, rope_factor, low_freq_factor, high_freq_factor,
                     original_max_len, {}};
  pkv::rope_freqs(D, rp);
  return decode_step_impl(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables,
                          context_lens, scale, out, B, Hq, Hkv, D, BS, NB, MBS, kv_dtype,
                          workspace, workspace_bytes, stream, true, &rp);
}

int pkv_rope_kv_append(const void* q, void* q_out, const void* k_new, const void* v_new,
                       const int32_t* positions, const int32_t* slot_mapping, void* k_cache,
                       void* v_cache, float* k_scale, float* v_scale, int N, int Hq, int Hkv,
                       int D, int BS, int NB, int kv_dtype, double rope_theta,
                       double rope_factor, double low_freq_factor, double high_freq_factor,
                       double original_max_len, void* stream) {
  g_last_error.clear();
  if (N < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0 || NB <= 0)
    return fail(PKV_ERR_SHAPE, "sizes must be positive (N may be 0): N=%d Hq=%d Hkv=%d D=%d BS=%d NB=%d",
                N, Hq, Hkv, D, BS, NB);
  if ((D != 64 && D != 128) || (BS != 16 && BS != 32) || Hkv > 8 ||
      (kv_dtype != PKV_KV_BF16 && kv_dtype != PKV_KV_FP8_E4M3FN && kv_dtype != PKV_KV_INT8))
    return fail(PKV_ERR_UNSUPPORTED, "unsupported D=%d BS=%d Hkv=%d kv_dtype=%d", D, BS, Hkv, kv_dtype);
  if (!(rope_theta > 1.0) || !(rope_factor > 0.0) || !(low_freq_factor > 0.0) ||
      !(high_freq_factor > low_freq_factor) || !(original_max_len > 0.0))
    return fail(PKV_ERR_SHAPE, "rope parameters: theta > 1, factor > 0, 0 < low_freq_factor < "
                "high_freq_factor and original_max_len > 0 are required");
  if (N == 0) return PKV_OK;   // nothing to do; pointers may be NULL
  if (!q || !q_out || !k_new || !v_new || !positions || !slot_mapping || !k_cache || !v_cache)
    return fail(PKV_ERR_NULL, "a required tensor pointer is NULL");
  const bool q8 = kv_dtype != PKV_KV_BF16;
  if (q8 && (!k_scale || !v_scale)) return fail(PKV_ERR_NULL, "fp8 / int8 cache needs k_scale and v_scale");
  if (!q8 && (k_scale || v_scale)) return fail(PKV_ERR_SHAPE, "bf16 cache takes no scales");
  if ((((uintptr_t)q) | ((uintptr_t)q_out) | ((uintptr_t)k_new) | ((uintptr_t)v_new) |
       ((uintptr_t)k_cache) | ((uintptr_t)v_cache)) & 3u)
    return fail(PKV_ERR_ALIGN, "q, q_out, k_new, v_new and the caches must be 4-byte aligned");
  pkv::RopeParams rp{rope_theta, rope_factor, low_freq_factor, high_freq_factor,
                     original_max_len, {}};
  pkv::rope_freqs(D, rp);
  hipError_t e = pkv::launch_rope_append(q, q_out, k_new, v_new, positions, slot_mapping,
                                         k_cache, v_cache, k_scale, v_scale, N, Hq, Hkv, D, BS,
                                         NB, kv_dtype, rp, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_fail(e, "rope_kv_append kernel launch");
}

int pkv_kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                  void* k_cache, void* v_cache, float* k_scale, float* v_scale, int N, int Hkv,
                  int D, int BS, int NB, int kv_dtype, void* stream) {
  g_last_error.clear();
  if (N < 0 || Hkv <= 0 || D <= 0 || BS <= 0 || NB <= 0)
    return fail(PKV_ERR_SHAPE, "sizes must be positive (N may be 0): N=%d Hkv=%d D=%d BS=%d NB=%d",
                N, Hkv, D, BS, NB);
  if ((D != 64 && D != 128) || (BS != 16 && BS != 32) ||
      (kv_dtype != PKV_KV_BF16 && kv_dtype != PKV_KV_FP8_E4M3FN && kv_dtype != PKV_KV_INT8))
    return fail(PKV_ERR_UNSUPPORTED, "unsupported D=%d BS=%d kv_dtype=%d", D, BS, kv_dtype);
  if (N == 0) return PKV_OK;   // nothing to do; pointers may be NULL
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache)
    return fail(PKV_ERR_NULL, "a required tensor pointer is NULL");
  const bool q8 = kv_dtype != PKV_KV_BF16;
  if (q8 && (!k_scale || !v_scale)) return fail(PKV_ERR_NULL, "fp8 / int8 cache needs k_scale and v_scale");
  if (!q8 && (k_scale || v_scale)) return fail(PKV_ERR_SHAPE, "bf16 cache takes no scales");
  if (!q8 && (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache)))
    return fail(PKV_ERR_ALIGN, "k_new, v_new and the caches must be 16-byte aligned");
  if (N == 0) return PKV_OK;
  hipError_t e = pkv::launch_kv_append(k_new, v_new, slot_mapping, nullptr, nullptr, 0, k_cache,
                                       v_cache, k_scale, v_scale, N, Hkv, D, BS, NB, kv_dtype,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_fail(e, "kv_append kernel launch");
}

}  // extern "C"
