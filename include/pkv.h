/*
 * pkv.h -- C ABI of libpkv.so: decode-phase paged attention and the one-token
 * KV append, hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * What the calls compute is defined by these pages:
 *   - "Decode Phase Attention Forward Pass" (sections 2-5 and the closing
 *     padding caveat): one query token per sequence, q of shape
 *     (batch, heads, dim), attends with no causal mask over the whole history
 *     of its sequence, which is found by walking the sequence's list of
 *     physical blocks; context_lens counts the history including the token
 *     stored this step; query head h reads KV head h / (Hq / Hkv); positions
 *     past the context length take no part in the softmax.
 *   - "tiny-vllm part 5", section on scattering a new token's K/V into
 *     16-token blocks: the new token's rows are written at
 *     (slot / block_size, slot % block_size) before attention runs.
 *   - the "Decode Phase" glossary (memory-bound decode; KV-cache quantisation
 *     to FP8 or INT8, with dequantisation inside the attention kernel): the
 *     fp8 variant stores OCP e4m3fn codes and the int8 variant symmetric
 *     int8 codes, each with an fp32 scale per (block, kv head).
 *
 * Conventions for every call:
 *   - Tensors are caller-owned, contiguous, row-major device memory.  The
 *     library keeps no pointer after a call returns and allocates nothing.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream).
 *     No call synchronises the host with the device, except the debug check
 *     pkv_validate_inputs, so every other call can be captured in a HIP
 *     graph.
 *   - bf16 means IEEE binary32 truncated to its upper 16 bits (stored as
 *     uint16); e4m3fn is the OCP 8-bit format (bias 7, no infinities, max 448).
 *   - Arguments the host can check (null pointers, unsupported shapes or
 *     dtypes, misaligned pointers, a too-small workspace) are checked before
 *     any launch; the call then returns a negative status and enqueues
 *     nothing.  Device-resident data is the caller's contract and is not read
 *     by the host: block ids must lie in [0, NB), 1 <= context_lens[b] <=
 *     MBS * BS, slots must be unique.  The kernels clamp out-of-range ids and
 *     lengths so that a broken contract gives wrong numbers, never an
 *     out-of-bounds access.
 *   - Supported: D in {64, 128}; BS in {16, 32}; Hq / Hkv in {1, 2, 4, 8,
 *     16} (16: the MFMA partition kernel only, which such a call runs
 *     whatever pkv_select_partition_kernel chose).
 *
 * Layouts:
 *   q, out            [B, Hq, D]           bf16
 *   k_cache, v_cache  [NB, BS, Hkv, D]     bf16, e4m3fn or int8 (one token's heads
 *                                          form one contiguous row, blocks
 *                                          are token-major, as in the pages)
 *   k_scale, v_scale  [NB, Hkv]            fp32 (fp8 and int8, else NULL)
 *   block_tables      [B, MBS]             int32; entries past the history
 *                                          are never read
 *   context_lens      [B]                  int32
 *   k_new, v_new      [N, Hkv, D]          bf16
 *   slot_mapping      [N]                  int32; slot = block * BS + offset,
 *                                          negative = no token
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define PKV_OK 0
#define PKV_ERR_NULL (-1)        /* a required pointer is NULL */
#define PKV_ERR_SHAPE (-2)       /* inconsistent or out-of-range sizes */
#define PKV_ERR_UNSUPPORTED (-3) /* D, BS, G or dtype outside the supported set */
#define PKV_ERR_WORKSPACE (-4)   /* workspace NULL or smaller than required */
#define PKV_ERR_HIP (-5)         /* a HIP runtime call failed; see pkv_last_error() */
#define PKV_ERR_ALIGN (-6)       /* a tensor pointer is not 16-byte aligned */
#define PKV_ERR_INPUT (-7)       /* device-resident input breaks the contract (pkv_validate_inputs) */

/* KV cache element types */
#define PKV_KV_BF16 0
#define PKV_KV_FP8_E4M3FN 1
#define PKV_KV_INT8 2

/* Store the step's new token of each of N sequences into the paged cache
 * ("tiny-vllm part 5", scattering into blocks; the first page's note that
 * the K/V of the token generated this step is already in the cache when
 * attention runs).
 *
 * For i < N with s = slot_mapping[i] >= 0: block = s / BS, off = s % BS, and
 * k_cache[block, off, :, :] = k_new[i] (same for V).
 *   bf16: an exact copy of the bits.
 *   fp8:  for each kv head g, if off == 0 the token opens the block and sets
 *         k_scale[block, g] = amax_d |k_new[i, g, d]| / 448 in fp32 (1.0 if
 *         the amax is 0); otherwise the block's existing scale is kept.  Each
 *         element is stored as e4m3fn(x / scale), x / scale a correctly
 *         rounded fp32 division, rounded to nearest even and saturated to
 *         +-448.  Same for V with v_scale.
 *   int8: as fp8 with scale = amax / 127 (1.0 if the amax is 0) and each
 *         element stored as clamp(rint(x / scale), -127, 127), rint rounding
 *         halves to even; the value of a code is code * scale.  (The pages
 *         fix no int8 format; this is the plain symmetric one.)
 * Slots outside [0, NB * BS) are skipped.  k_scale and v_scale must be NULL
 * for bf16 and non-NULL for fp8 and int8.  Two tokens of one call must not
 * share a block when one of them opens it (append them in position order,
 * one call each).  N == 0 is a no-op (pointers may then be NULL). */
int pkv_kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                  void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                  int N, int Hkv, int D, int BS, int NB, int kv_dtype, void* stream);

/* RoPE fused with the append ("tiny-vllm part 5", the RoPE section: each
 * head's pairs (x[2i], x[2i+1]) rotate by pos * f_i, f_i = theta^(-2i/D),
 * with the Llama 3 frequency scaling of the page's table path.  With
 * r = original_max_len * f_i / (2 pi), the turns pair i makes over the
 * original context, and s = clamp((r - low_freq_factor) / (high_freq_factor
 * - low_freq_factor), 0, 1), the frequency used is f_i (s + (1 - s) /
 * rope_factor): slowed by rope_factor for pairs with few turns, kept for
 * pairs with many, fading linearly in r between.  rope_factor = 1 is plain
 * RoPE.  The page's Llama 3 setting is theta 500000, factor 32, 1, 4, 8192.)
 * For each token i < N at position positions[i]:
 *   q_out[i]  = RoPE(q[i])     [N, Hq, D] bf16 (q_out may be q itself)
 *   k_rot     = RoPE(k_new[i]) [Hkv, D]
 *   then exactly pkv_kv_append of (k_rot, v_new[i]) into slot_mapping[i]
 *   (bf16 copy or fp8 / int8 codes, the same scale rule; a slot outside the
 *   pool skips the append, q is rotated all the same).
 * The angle, cos / sin and the rotation are fp64; each rotated element is
 * rounded once to bf16 (nearest even).  Hkv <= 8; D in {64, 128}; pointers
 * 4-byte aligned.  N == 0 is a no-op (pointers may then be NULL). */
int pkv_rope_kv_append(const void* q, void* q_out, const void* k_new, const void* v_new,
                       const int32_t* positions, const int32_t* slot_mapping, void* k_cache,
                       void* v_cache, float* k_scale, float* v_scale, int N, int Hq, int Hkv,
                       int D, int BS, int NB, int kv_dtype, double rope_theta,
                       double rope_factor, double low_freq_factor, double high_freq_factor,
                       double original_max_len, void* stream);

/* Bytes of device workspace pkv_paged_decode_attention needs for these
 * sizes on the current device (it depends on the device's compute-unit
 * count).  Returns 0 for sizes the library does not support. */
size_t pkv_paged_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int BS, int MBS,
                                        int kv_dtype);

/* Decode-phase paged attention ("Decode Phase Attention Forward Pass",
 * sections 2-5):
 *   out[b, h, :] = sum_{t < L_b} softmax_t(scale * <q[b, h], K_t>) * V_t,
 *   L_b = context_lens[b], K_t = k_cache[block_tables[b][t / BS], t % BS,
 *   h / (Hq / Hkv), :] (times k_scale of that block and head for fp8 and int8),
 *   likewise V_t.  No causal mask; nothing past L_b is read.  A sequence with
 *   L_b <= 0 gets out = 0.  B == 0 is a no-op (pointers may then be NULL).
 * Accumulation is fp32; out is rounded to bf16 (round to nearest even).
 * The context is split across the whole GPU (a partition kernel writes
 * fp32 partial results into `workspace`, a merge kernel combines them by
 * log-sum-exp); the workspace contents are scratch and need no clearing.
 * Calls that share a workspace must not overlap in time. */
int pkv_paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                               const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, const int32_t* context_lens,
                               float scale, void* out, int B, int Hq, int Hkv, int D, int BS,
                               int NB, int MBS, int kv_dtype, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Bytes of the static scratch of pkv_paged_decode_attention_noalloc (32 MiB
 * per GPU). */
#define PKV_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/* pkv_paged_decode_attention for callers that cannot allocate device memory
 * (code being captured into a HIP graph, serving loops that must not
 * allocate, harnesses that forbid it): the same arguments without the
 * workspace, the same kernels and the same result, bit for bit.  The
 * partial results go to a static device array of PKV_STATIC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends;
 * the call allocates nothing.  Sizes whose workspace
 * (pkv_paged_decode_workspace_bytes) exceeds it return PKV_ERR_WORKSPACE
 * before any launch.  The scratch needs no clearing, but every call on one
 * GPU shares it: calls that overlap in time on the same GPU (two streams,
 * two host threads) race and give wrong results; serialise them. */
int pkv_paged_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       float scale, void* out, int B, int Hq, int Hkv, int D,
                                       int BS, int NB, int MBS, int kv_dtype, void* stream);

/* The two halves of pkv_paged_decode_attention, with the same arguments:
 * calling partition then merge on one stream is exactly the full call.
 * Exposed so that each kernel can be timed on its own. */
int pkv_paged_decode_partition(const void* q, const void* k_cache, const void* v_cache,
                               const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, const int32_t* context_lens,
                               float scale, void* out, int B, int Hq, int Hkv, int D, int BS,
                               int NB, int MBS, int kv_dtype, void* workspace,
                               size_t workspace_bytes, void* stream);
int pkv_paged_decode_merge(const void* q, const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_tables, const int32_t* context_lens,
                           float scale, void* out, int B, int Hq, int Hkv, int D, int BS,
                           int NB, int MBS, int kv_dtype, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Generalised paged attention: several query tokens per sequence with the
 * bottom-right aligned causal mask ("Prefill Forward Prefix Caching
 * Explained", the section on how the causal mask handles the prefix: query i
 * of q_len new tokens sees key j iff j <= i + kv_len - q_len), and optionally
 * a sliding window with attention sinks (the "Decode Phase" glossary's
 * long-context bullets: only the most recent tokens, plus the first few
 * kept to stabilise attention).
 *   Sequence b has L_b = context_lens[b] keys (its new tokens included, as
 *   stored by pkv_kv_append beforehand) and q_len_b = q_start[b+1] -
 *   q_start[b] queries, the q/out rows q_start[b] .. q_start[b+1]-1 (with
 *   q_start NULL: one query, row b, and max_q_len must be 1).  Query i sees
 *   key j iff j <= lim = L_b - q_len_b + i and, when window_tokens > 0, also
 *   j > lim - window_tokens or j < sink_tokens.  out[row, h, :] is the
 *   softmax(scale <q, K_j>) weighted sum of V_j over the keys it sees, as in
 *   pkv_paged_decode_attention; a query that sees no key gets 0.
 *   q, out  [total_q, Hq, D] bf16; q_start [B + 1] int32 (device), with
 *   q_len_b <= max_q_len (larger ones are clamped; negative ones count as
 *   0).  q_start is device-resident and, like block ids, the caller's
 *   contract: 0 <= q_start[b] <= q_start[b + 1] and q_start[B] <= total_q
 *   (the rows of q and out); the kernels read and write rows q_start[b] ..
 *   q_start[b] + q_len_b - 1 as given, so entries past total_q read and
 *   write out of bounds.  G * max_q_len <= 32
 *   (one wave serves all of a sequence's queries of its kv heads, as the
 *   16-column tiles of its matrix products: two adjacent kv heads in one
 *   tile when 2 * G * max_q_len <= 16, else one kv head in one tile, or in
 *   two when G * max_q_len > 16; larger counts return PKV_ERR_UNSUPPORTED
 *   and a workspace query of 0).  Other
 *   arguments as for pkv_paged_decode_attention; the workspace comes from
 *   pkv_paged_attention_workspace_bytes with the same max_q_len.
 * Always runs the MFMA partition kernel (the VALU variant serves one query
 * per sequence without a window).  With q_start NULL, max_q_len 1 and
 * window_tokens 0 the result is bit-identical to
 * pkv_paged_decode_attention. */
int pkv_paged_attention(const void* q, const int32_t* q_start, int max_q_len,
                        const void* k_cache, const void* v_cache, const float* k_scale,
                        const float* v_scale, const int32_t* block_tables,
                        const int32_t* context_lens, float scale, int sink_tokens,
                        int window_tokens, void* out, int B, int Hq, int Hkv, int D, int BS,
                        int NB, int MBS, int kv_dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Workspace bytes for pkv_paged_attention with at most max_q_len queries per
 * sequence (0 for sizes the library does not support). */
size_t pkv_paged_attention_workspace_bytes(int B, int Hq, int Hkv, int D, int BS, int MBS,
                                           int kv_dtype, int max_q_len);

/* One decode step: the append of each sequence's new token followed by
 * attention, in one call ("tiny-vllm part 5": the new token's K/V is written
 * into its block before attention reads the history; "Decode Phase Attention
 * Forward Pass", sections 2-5, for the attention).  Exactly equivalent to
 *   pkv_kv_append(k_new, v_new, slot, ...);  pkv_paged_decode_attention(...);
 * with slot[b] = block_tables[b][(L_b - 1) / BS] * BS + (L_b - 1) % BS, the
 * position L_b - 1 that context_lens already counts; sequences with L_b
 * outside [1, MBS * BS] or a block id outside [0, NB) there get no append.
 * Caches, scales and out are bit-identical to the two calls.
 *   k_new, v_new  [B, Hkv, D] bf16, 16-byte aligned; other arguments, the
 *   workspace and its size as for pkv_paged_decode_attention.
 * With the MFMA partition kernel the append runs inside it: the one wave
 * that reads position L_b - 1 of (b, kv head g) stores the row and uses it,
 * so the step takes two launches instead of three.  The block receiving a
 * token must not appear in another sequence's table at or past that offset
 * (as for any append before attention).  B == 0 is a no-op. */
int pkv_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                    void* v_cache, float* k_scale, float* v_scale, const int32_t* block_tables,
                    const int32_t* context_lens, float scale, void* out, int B, int Hq, int Hkv,
                    int D, int BS, int NB, int MBS, int kv_dtype, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Workspace bytes for pkv_decode_step_rope: those of
 * pkv_paged_attention_workspace_bytes(..., max_q_len = 1) plus room for a
 * rotated copy of q (B * Hq * D bf16, rounded up to 256 bytes).  0 for an
 * unsupported shape. */
size_t pkv_decode_step_rope_workspace_bytes(int B, int Hq, int Hkv, int D, int BS, int MBS,
                                            int kv_dtype);

/* The decode step with RoPE ("tiny-vllm part 5", the RoPE section, with the
 * frequencies and parameters of pkv_rope_kv_append): q and k_new arrive
 * unrotated; exactly equivalent to
 *   pkv_rope_kv_append(q, q_rot, k_new, v_new, pos, slot, ...);
 *   pkv_paged_decode_attention(q_rot, ...);
 * with pos[b] = context_lens[b] - 1 and slot[b] as for pkv_decode_step:
 * caches, scales and out bit-identical to those two calls (q itself is not
 * changed).  Always runs the MFMA partition kernel, which rotates q in
 * registers and the new key rows before it stores them, so the step is two
 * launches.  Size the workspace with pkv_decode_step_rope_workspace_bytes.
 * When the call serves one kv head per partition wave (odd Hkv, or
 * pkv_select_unit_heads(1)) and Hkv <= 8, the step runs as exactly those
 * two calls instead (three launches; the rotated q goes to the end of the
 * workspace), which is faster there; a workspace of only
 * pkv_paged_attention_workspace_bytes(max_q_len = 1) bytes leaves no room
 * for it and keeps the fused kernel.  The bits are the same either way.
 * D in {64, 128}; other arguments as for pkv_decode_step.  Bad rope
 * parameters give PKV_ERR_SHAPE.  B == 0 is a no-op. */
int pkv_decode_step_rope(const void* q, const void* k_new, const void* v_new, void* k_cache,
                         void* v_cache, float* k_scale, float* v_scale,
                         const int32_t* block_tables, const int32_t* context_lens, float scale,
                         double rope_theta, double rope_factor, double low_freq_factor,
                         double high_freq_factor, double original_max_len, void* out, int B,
                         int Hq, int Hkv, int D, int BS, int NB, int MBS, int kv_dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/* The first half of pkv_decode_step (the append and the partition kernel),
 * same arguments; following it with pkv_paged_decode_merge on the same
 * stream and workspace is exactly pkv_decode_step.  Exposed so that the
 * step's partition launch can be timed on its own. */
int pkv_decode_step_partition(const void* q, const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* block_tables, const int32_t* context_lens,
                              float scale, void* out, int B, int Hq, int Hkv, int D, int BS,
                              int NB, int MBS, int kv_dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Debug check of the device-resident inputs of pkv_paged_decode_attention
 * (same arguments; the attention calls trust them): every context length in
 * [1, MBS * BS], the block ids of the pages each history uses
 * (j < ceil(L_b / BS), "Decode Phase Attention Forward Pass", sections 2-3)
 * in [0, NB), and for fp8 / int8 caches the K and V scales of those blocks
 * positive and finite.  Runs the host checks of the attention call, one
 * check kernel on `stream` (using the workspace's first 8 bytes), then
 * SYNCHRONISES the stream.  Returns PKV_OK, or PKV_ERR_INPUT with the first
 * violation (lowest sequence, then kind, then page) in pkv_last_error(). */
int pkv_validate_inputs(const void* q, const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale, const int32_t* block_tables,
                        const int32_t* context_lens, float scale, void* out, int B, int Hq,
                        int Hkv, int D, int BS, int NB, int MBS, int kv_dtype, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* pkv_status_string(int status);

/* Detail of the last failing call on this host thread ("" if none). */
const char* pkv_last_error(void);

/* Number of persistent waves the grid of a decode call (one query per
 * sequence, no window) with these sizes uses on the current device, under
 * the current selections (0 if unsupported or the device cannot be
 * queried).  Informational. */
int pkv_attention_waves(int B, int Hq, int Hkv, int D, int BS, int kv_dtype);

/* Kv heads one wave of the MFMA partition kernel serves together in such a
 * call (a unit of adjacent kv heads whose rows lie side by side in every
 * cache row, so a wave streams one contiguous run of unit * D * elem bytes
 * per token): 2 when Hkv is even and the wider kernel fits two workgroups
 * on a compute unit, else 1; always 1 for the VALU kernel.  (The
 * generalised call, pkv_paged_attention, takes the same unit when its
 * 2 * G * max_q_len columns fit the 16 of the MFMA, else 1.)  The result
 * does not depend on it beyond floating-point summation order.  0 if
 * unsupported.  Informational. */
int pkv_decode_unit_heads(int B, int Hq, int Hkv, int D, int BS, int kv_dtype);

/* Streaming-read probe: the read bandwidth the device reaches with nothing
 * but 16-byte non-temporal loads, the ceiling the attention kernels' KV
 * reads are measured against (the "Decode Phase" glossary bounds a decode
 * step by the KV cache bytes over the memory bandwidth).  Reads every whole
 * 1 KB unit of `buf` (device memory, 16-byte aligned; a tail under 1 KB is
 * not read) with a persistent grid, and stores one XOR fold per wave in
 * sink (device memory, at least pkv_read_probe_waves() uint32 words;
 * PKV_ERR_WORKSPACE if smaller).  bytes == 0 is a no-op.  Asynchronous on
 * `stream`. */
int pkv_read_probe_waves(void);
int pkv_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                   void* stream);

/* mode 0 (default): units as above; mode 1: one kv head per wave always.
 * Process-wide, read at the start of every attention call and workspace
 * query, like pkv_select_partition_kernel (switch only between calls, size
 * the workspace after switching).  PKV_UNIT_HEADS=1 in the environment
 * selects mode 1 when the library loads.  PKV_ERR_UNSUPPORTED for another
 * value. */
int pkv_select_unit_heads(int mode);

/* mode 1 (default): the waves of a partition workgroup, which stream
 * consecutive pieces of the work, combine their partial results for the
 * runs they share in LDS, so a run inside a workgroup's range is finished
 * there and one crossing its edge leaves one partial row per workgroup
 * instead of one per wave (taken by MFMA calls with B <= 1024 whose
 * partial rows have at most 8 columns, i.e. kv heads per wave x G x queries
 * per sequence <= 8, or at most 16 with two kv heads per wave where the
 * larger LDS keeps the grid's size).  Generalised calls with one kv head
 * per wave and 9 to 32 columns, which park mid-piece results (see
 * pkv_select_result_parking; with more than 16 columns only where room for
 * a second share per wave leaves the grid's size), combine instead the
 * shares of a run that crosses the edge between consecutive waves of a
 * workgroup, in the first of those waves after the workgroup's barrier,
 * with the same one row per workgroup.  Mode 0: one partial row per wave always.  The result
 * differs only in floating-point summation order.  Process-wide, read at
 * the start of every attention call and workspace query, like
 * pkv_select_unit_heads.  PKV_SHARE_COMBINE=0 in the environment selects
 * mode 0 when the library loads.  PKV_ERR_UNSUPPORTED for another value. */
int pkv_select_share_combine(int mode);

/* mode 1 (default): in a generalised call (pkv_paged_attention with
 * q_start, several queries or a window) whose partition waves serve one kv
 * head and one 16-column tile without the combine above, a wave keeps the
 * result of a run that it finishes before its last one in LDS and writes it
 * out after its last tile, where a store issued at once would hold up the
 * next run's loads (taken when the LDS slot leaves the workgroups per CU as
 * they are, so the grid and the workspace do not change).  mode 0 stores
 * every result when its run ends.  The two give the same bits.
 * Process-wide, read at the start of every attention call, like
 * pkv_select_unit_heads.  PKV_RESULT_PARKING=0 in the environment selects
 * mode 0 when the library loads.  PKV_ERR_UNSUPPORTED for another value. */
int pkv_select_result_parking(int mode);

/* The MFMA partition kernel cuts its work (every (sequence, kv-head unit)
 * run's pages, in order) into equal pieces, one per wave; a wave pays a fixed
 * cost for each run it starts (the run's q, page-table and first tile
 * round trips).  The split therefore counts `slots` extra positions ahead
 * of each non-empty run, so a piece holding several runs gets fewer pages.
 * 0..8 (default 2; PKV_RUN_COST in the environment sets it when the library
 * loads); the split, not the result, changes (floating-point summation
 * order aside).  Process-wide, read at the start of every attention call.
 * PKV_ERR_UNSUPPORTED for another value. */
int pkv_select_run_cost(int slots);

/* Partition-kernel variants.  Both compute the same attention; MFMA (the
 * default) puts the GQA group on the matrix cores, VALU uses fp32 vector
 * FMAs.  The choice is process-wide and is read at the start of every
 * attention call, workspace query included, so switch only between calls
 * (never while another thread is inside one) and size the workspace after
 * switching.  The environment variable PKV_ATTN_KERNEL=valu selects VALU
 * when the library loads.  Returns PKV_ERR_UNSUPPORTED for another value. */
#define PKV_PARTITION_VALU 0
#define PKV_PARTITION_MFMA 1
int pkv_select_partition_kernel(int variant);
int pkv_partition_kernel(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
