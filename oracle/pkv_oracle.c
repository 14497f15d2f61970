/*
 * pkv_oracle.c -- plain, slow, fp64 CPU oracle for decode-phase paged
 * attention and the one-token KV append.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this library.  The product path
 * (the HIP library and its Python binding) never includes, links or calls
 * anything here, and nothing here includes a header of the product path.
 *
 * What it computes, and where the pages say so:
 *
 *  - Attention ("Decode Phase Attention Forward Pass", sections 2-5): one
 *    query token per sequence, q of shape (batch, heads, dim), attends with no
 *    causal mask over the sequence's whole history.  The history is reached by
 *    walking the sequence's list of physical blocks: position t lives at
 *    (block_tables[b][t / block_size], t % block_size).  context_lens[b]
 *    counts the tokens including the one appended this step.  Query head h
 *    reads KV head h / G, G = Hq / Hkv (the repeat_interleave grouping of
 *    section 3).  Scores are scale * <q, k>; softmax; weighted sum of V.
 *    Positions t >= context_lens[b] do not exist: they are never read, so
 *    no padding takes part in the softmax (the closing caveat of that page
 *    explains why a zero-padded gather would be wrong).
 *    The softmax is the plain two-pass definition (max, then exp and sum),
 *    in fp64, with no blocking or online rescaling.
 *
 *  - KV append ("tiny-vllm part 5", section "Gathering K/V into a batched
 *    buffer and scattering into blocks"): the new token's K and V rows go to
 *    (block, offset) = (slot / block_size, slot % block_size).  A slot below
 *    zero means "no token" and is skipped.
 *
 *  - fp8 KV ("Decode Phase" glossary, the KV-cache quantisation bullet): the
 *    cache stores OCP e4m3fn codes with one fp32 scale per (block, kv head).
 *    A token that opens a block (offset 0) sets that block's scale to
 *    amax|x| / 448 (1.0 if amax is 0); every token is stored as
 *    e4m3fn(round-to-nearest-even, saturating)(x / scale), x / scale taken in
 *    fp32.  A token landing in an already-open block keeps the block's
 *    scale and saturates.
 *
 * Layouts (all row-major, contiguous):
 *   q, out            [B, Hq, D]         q is bf16 bits, out is fp64
 *   k_cache, v_cache  [NB, BS, Hkv, D]   bf16 bits or e4m3fn bytes
 *   k_scale, v_scale  [NB, Hkv]          fp32 (fp8 only)
 *   block_tables      [B, MBS]           int32
 *   context_lens      [B]                int32
 *   k_new, v_new      [N, Hkv, D]        bf16 bits
 *   slot_mapping      [N]                int32
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define PKVO_KV_BF16 0
#define PKVO_KV_FP8 1

#define PKVO_OK 0
#define PKVO_ERR_NULL (-1)
#define PKVO_ERR_SHAPE (-2)
#define PKVO_ERR_NOMEM (-3)

/* ---- scalar formats ------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
double pkvo_bf16_to_f64(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static float bf16_to_f32(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* OCP 8-bit floating point, E4M3 ("fn": no infinities, one NaN pattern per
 * sign).  Bias 7.  Exponent field 0 is subnormal: m/8 * 2^-6.  Otherwise
 * (1 + m/8) * 2^(e-7).  S.1111.111 is NaN, so the largest finite magnitude is
 * 1.75 * 2^8 = 448. */
double pkvo_e4m3fn_to_f64(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Encode a binary32 value to e4m3fn, round to nearest, ties to even,
 * saturating at +-448.  Done by exhaustive search over the 127 non-negative
 * finite codes so that it can be checked by eye: the nearest code wins; on a
 * tie the code whose significand is even (lowest code bit clear) wins.  The
 * sign bit is copied from x, so -0.0 and negative values that round to zero
 * give 0x80.  NaN input gives 0x7F (the oracle is never fed NaN). */
uint8_t pkvo_e4m3fn_from_f32(float x) {
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  int best = 0;
  double best_err = a; /* code 0 has value 0 */
  for (int c = 1; c <= 0x7E; ++c) {
    double err = fabs(pkvo_e4m3fn_to_f64((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(sign | best);
}

void pkvo_e4m3fn_decode_array(const uint8_t* codes, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = pkvo_e4m3fn_to_f64(codes[i]);
}

void pkvo_e4m3fn_encode_array(const float* x, uint8_t* codes, int64_t n) {
  for (int64_t i = 0; i < n; ++i) codes[i] = pkvo_e4m3fn_from_f32(x[i]);
}

/* ---- attention ------------------------------------------------------------ */

static double load_kv(const void* cache, const float* scales, int kv_dtype,
                      size_t row, int d, size_t scale_idx) {
  if (kv_dtype == PKVO_KV_BF16)
    return pkvo_bf16_to_f64(((const uint16_t*)cache)[row + (size_t)d]);
  return pkvo_e4m3fn_to_f64(((const uint8_t*)cache)[row + (size_t)d]) *
         (double)scales[scale_idx];
}

/* out[b, h, :] for every sequence b and query head h.  If `weights` is not
 * NULL it receives the softmax weight of every position, [B, Hq, MBS*BS]
 * (positions >= context_lens[b] are left at 0).  A sequence with
 * context_lens[b] <= 0 has no history; its output is 0.  Returns a status. */
int pkvo_paged_decode_attention(const uint16_t* q, const void* k_cache,
                                const void* v_cache, const float* k_scale,
                                const float* v_scale, const int32_t* block_tables,
                                const int32_t* context_lens, float scale,
                                double* out, double* weights, int B, int Hq,
                                int Hkv, int D, int BS, int NB, int MBS,
                                int kv_dtype, int nthreads) {
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PKVO_ERR_NULL;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0 || NB <= 0 || MBS <= 0 ||
      Hq % Hkv != 0)
    return PKVO_ERR_SHAPE;
  if (kv_dtype != PKVO_KV_BF16 && kv_dtype != PKVO_KV_FP8) return PKVO_ERR_SHAPE;
  if (kv_dtype == PKVO_KV_FP8 && (!k_scale || !v_scale)) return PKVO_ERR_NULL;
  for (int b = 0; b < B; ++b) {
    int L = context_lens[b];
    if (L > MBS * BS) return PKVO_ERR_SHAPE;
    for (int t = 0; t < L; t += BS) {
      int p = block_tables[(size_t)b * MBS + t / BS];
      if (p < 0 || p >= NB) return PKVO_ERR_SHAPE;
    }
  }
  const int G = Hq / Hkv;
  const int n_units = B * Hkv;
  int status = PKVO_OK;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int u = 0; u < n_units; ++u) {
    const int b = u / Hkv;
    const int g = u % Hkv;
    const int L = context_lens[b];
    double* s = L > 0 ? (double*)malloc(sizeof(double) * (size_t)L) : NULL;
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if ((L > 0 && !s) || !acc) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      status = PKVO_ERR_NOMEM;
      free(s);
      free(acc);
      continue;
    }
    for (int j = 0; j < G; ++j) {
      const int h = g * G + j;
      const uint16_t* qh = q + ((size_t)b * Hq + h) * D;
      double* oh = out + ((size_t)b * Hq + h) * D;
      if (L <= 0) {
        for (int d = 0; d < D; ++d) oh[d] = 0.0;
        continue;
      }
      /* pass 1: scores over the logical history, walking the block table */
      for (int t = 0; t < L; ++t) {
        const int p = block_tables[(size_t)b * MBS + t / BS];
        const int o = t % BS;
        const size_t row = (((size_t)p * BS + o) * Hkv + g) * D;
        const size_t si = (size_t)p * Hkv + g;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
          dot += pkvo_bf16_to_f64(qh[d]) * load_kv(k_cache, k_scale, kv_dtype, row, d, si);
        s[t] = (double)scale * dot;
      }
      /* pass 2: softmax (max, exponentials, normaliser) */
      double m = s[0];
      for (int t = 1; t < L; ++t)
        if (s[t] > m) m = s[t];
      double Z = 0.0;
      for (int t = 0; t < L; ++t) {
        s[t] = exp(s[t] - m);
        Z += s[t];
      }
      /* pass 3: weighted sum of V */
      for (int d = 0; d < D; ++d) acc[d] = 0.0;
      for (int t = 0; t < L; ++t) {
        const int p = block_tables[(size_t)b * MBS + t / BS];
        const int o = t % BS;
        const size_t row = (((size_t)p * BS + o) * Hkv + g) * D;
        const size_t si = (size_t)p * Hkv + g;
        const double w = s[t] / Z;
        if (weights) weights[((size_t)b * Hq + h) * ((size_t)MBS * BS) + t] = w;
        for (int d = 0; d < D; ++d) acc[d] += w * load_kv(v_cache, v_scale, kv_dtype, row, d, si);
      }
      for (int d = 0; d < D; ++d) oh[d] = acc[d];
    }
    free(s);
    free(acc);
  }
  return status;
}

/* ---- KV append ------------------------------------------------------------ */

static void append_fp8_row(const uint16_t* x, uint8_t* dst, float* scale_slot,
                           int opens_block, int D) {
  float sc;
  if (opens_block) {
    float amax = 0.0f;
    for (int d = 0; d < D; ++d) {
      float a = fabsf(bf16_to_f32(x[d]));
      if (a > amax) amax = a;
    }
    sc = amax / 448.0f;
    if (amax == 0.0f) sc = 1.0f;
    *scale_slot = sc;
  } else {
    sc = *scale_slot;
  }
  for (int d = 0; d < D; ++d) {
    const float y = bf16_to_f32(x[d]) / sc; /* binary32, correctly rounded */
    dst[d] = pkvo_e4m3fn_from_f32(y);
  }
}

/* In-place append of N tokens into host copies of the caches. */
int pkvo_kv_append(const uint16_t* k_new, const uint16_t* v_new,
                   const int32_t* slot_mapping, void* k_cache, void* v_cache,
                   float* k_scale, float* v_scale, int N, int Hkv, int D, int BS,
                   int NB, int kv_dtype) {
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKVO_ERR_NULL;
  if (N < 0 || Hkv <= 0 || D <= 0 || BS <= 0 || NB <= 0) return PKVO_ERR_SHAPE;
  if (kv_dtype != PKVO_KV_BF16 && kv_dtype != PKVO_KV_FP8) return PKVO_ERR_SHAPE;
  if (kv_dtype == PKVO_KV_FP8 && (!k_scale || !v_scale)) return PKVO_ERR_NULL;
  const size_t row_elems = (size_t)Hkv * D;
  for (int i = 0; i < N; ++i) {
    const int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    if (slot >= (int64_t)NB * BS) return PKVO_ERR_SHAPE;
    const int64_t blk = slot / BS;
    const int off = (int)(slot % BS);
    const uint16_t* kr = k_new + (size_t)i * row_elems;
    const uint16_t* vr = v_new + (size_t)i * row_elems;
    const size_t dst = ((size_t)blk * BS + off) * row_elems;
    if (kv_dtype == PKVO_KV_BF16) {
      memcpy((uint16_t*)k_cache + dst, kr, row_elems * 2);
      memcpy((uint16_t*)v_cache + dst, vr, row_elems * 2);
    } else {
      for (int g = 0; g < Hkv; ++g) {
        append_fp8_row(kr + (size_t)g * D, (uint8_t*)k_cache + dst + (size_t)g * D,
                       &k_scale[blk * Hkv + g], off == 0, D);
        append_fp8_row(vr + (size_t)g * D, (uint8_t*)v_cache + dst + (size_t)g * D,
                       &v_scale[blk * Hkv + g], off == 0, D);
      }
    }
  }
  return PKVO_OK;
}
