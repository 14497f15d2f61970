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
 *  - INT8 KV (the same glossary: the KV cache may be quantised to INT8, with
 *    dequantisation in the attention kernel; the pages fix no format, so the
 *    plainest symmetric one is taken): one fp32 scale per (block, kv head);
 *    a token that opens a block sets it to amax|x| / 127 (1.0 if amax is 0);
 *    every element is stored as the int8 code clamp(rint(x / scale), -127,
 *    127), x / scale in fp32 and rint rounding halves to even; the value is
 *    code * scale.
 *
 *  - Generalised attention ("Prefill Forward Prefix Caching Explained",
 *    section on the bottom-right causal mask; the "Decode Phase" glossary's
 *    sliding-window and attention-sink bullets): sequence b has q_len_b
 *    query tokens, the last q_len_b of its L_b = context_lens[b] positions.
 *    Query i (0 <= i < q_len_b) sees key j iff j <= lim = L_b - q_len_b + i
 *    and, when a window W > 0 is given, also j > lim - W or j < S (the first
 *    S "sink" tokens stay visible).  q_len_b = 1 with no window is the
 *    decode attention above.
 *
 *  - RoPE ("tiny-vllm part 5", section "RoPE: one current position,
 *    recomputed on every call"): the pair (x[2i], x[2i+1]) of every head is
 *    rotated by the angle pos * f_i, with f_i = theta^(-2i/D) scaled as the
 *    Llama 3 table path scales it (frequencies whose wavelength exceeds
 *    original_max / low_freq_factor are divided by `factor`; between that and
 *    original_max / high_freq_factor they are blended linearly in
 *    original_max / wavelength).  Everything in fp64; the rotated vector is
 *    rounded to bf16 (nearest even), as the model's K and Q would be stored.
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
#define PKVO_KV_INT8 2

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

/* INT8: the code of a binary32 quotient y: nearest integer, halves to even
 * (the C library's rint in the default rounding mode), clamped to
 * [-127, 127]; NaN gives 0 (the oracle is never fed NaN). */
int8_t pkvo_int8_from_f32(float y) {
  if (isnan(y)) return 0;
  double r = rint((double)y); /* y is exact in double, so this rounds y itself */
  if (r > 127.0) r = 127.0;
  if (r < -127.0) r = -127.0;
  return (int8_t)r;
}

/* ---- attention ------------------------------------------------------------ */

static double load_kv(const void* cache, const float* scales, int kv_dtype,
                      size_t row, int d, size_t scale_idx) {
  if (kv_dtype == PKVO_KV_BF16)
    return pkvo_bf16_to_f64(((const uint16_t*)cache)[row + (size_t)d]);
  if (kv_dtype == PKVO_KV_INT8)
    return (double)((const int8_t*)cache)[row + (size_t)d] * (double)scales[scale_idx];
  return pkvo_e4m3fn_to_f64(((const uint8_t*)cache)[row + (size_t)d]) *
         (double)scales[scale_idx];
}

static int valid_dtype(int kv_dtype) {
  return kv_dtype == PKVO_KV_BF16 || kv_dtype == PKVO_KV_FP8 || kv_dtype == PKVO_KV_INT8;
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
  if (!valid_dtype(kv_dtype)) return PKVO_ERR_SHAPE;
  if (kv_dtype != PKVO_KV_BF16 && (!k_scale || !v_scale)) return PKVO_ERR_NULL;
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

/* Generalised attention: out[r, h, :] for every query row r and head h.
 * q_start == NULL: one query per sequence, row b (q_len_b = 1).  Otherwise
 * sequence b owns rows q_start[b] .. q_start[b+1]-1.  Query i of sequence b
 * sees key j iff j <= lim = L - q_len + i and (window <= 0 || j > lim - window
 * || j < sinks).  A query that sees no key gets out = 0.  `weights`, if not
 * NULL, is [total_q, Hq, MBS*BS] and receives the weight of every position.
 * The softmax is the plain two-pass definition over the visible keys. */
int pkvo_paged_attention(const uint16_t* q, const int32_t* q_start, const void* k_cache,
                         const void* v_cache, const float* k_scale, const float* v_scale,
                         const int32_t* block_tables, const int32_t* context_lens, float scale,
                         int sinks, int window, double* out, double* weights, int B, int Hq,
                         int Hkv, int D, int BS, int NB, int MBS, int kv_dtype, int nthreads) {
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PKVO_ERR_NULL;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0 || NB <= 0 || MBS <= 0 ||
      Hq % Hkv != 0 || sinks < 0)
    return PKVO_ERR_SHAPE;
  if (!valid_dtype(kv_dtype)) return PKVO_ERR_SHAPE;
  if (kv_dtype != PKVO_KV_BF16 && (!k_scale || !v_scale)) return PKVO_ERR_NULL;
  for (int b = 0; b < B; ++b) {
    const int L = context_lens[b];
    const int ql = q_start ? q_start[b + 1] - q_start[b] : 1;
    if (L > MBS * BS || ql < 0) return PKVO_ERR_SHAPE;
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
    const int L = context_lens[b] > 0 ? context_lens[b] : 0;
    const int r0 = q_start ? q_start[b] : b;
    const int ql = q_start ? q_start[b + 1] - q_start[b] : 1;
    double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    char* vis = (char*)malloc((size_t)(L > 0 ? L : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if (!s || !vis || !acc) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      status = PKVO_ERR_NOMEM;
      free(s);
      free(vis);
      free(acc);
      continue;
    }
    for (int i = 0; i < ql; ++i) {
      const int lim = L - ql + i; /* bottom-right aligned causal limit */
      int any = 0;
      for (int t = 0; t < L; ++t) {
        int v = t <= lim;
        if (v && window > 0) v = (t > lim - window) || (t < sinks);
        vis[t] = (char)v;
        any |= v;
      }
      for (int j = 0; j < G; ++j) {
        const int h = g * G + j;
        const size_t rh = (size_t)(r0 + i) * Hq + h;
        const uint16_t* qh = q + rh * D;
        double* oh = out + rh * D;
        if (!any) {
          for (int d = 0; d < D; ++d) oh[d] = 0.0;
          continue;
        }
        double m = -INFINITY;
        for (int t = 0; t < L; ++t) {
          if (!vis[t]) continue;
          const int p = block_tables[(size_t)b * MBS + t / BS];
          const size_t row = (((size_t)p * BS + t % BS) * Hkv + g) * D;
          const size_t si = (size_t)p * Hkv + g;
          double dot = 0.0;
          for (int d = 0; d < D; ++d)
            dot += pkvo_bf16_to_f64(qh[d]) * load_kv(k_cache, k_scale, kv_dtype, row, d, si);
          s[t] = (double)scale * dot;
          if (s[t] > m) m = s[t];
        }
        double Z = 0.0;
        for (int t = 0; t < L; ++t) {
          if (!vis[t]) continue;
          s[t] = exp(s[t] - m);
          Z += s[t];
        }
        for (int d = 0; d < D; ++d) acc[d] = 0.0;
        for (int t = 0; t < L; ++t) {
          if (!vis[t]) continue;
          const int p = block_tables[(size_t)b * MBS + t / BS];
          const size_t row = (((size_t)p * BS + t % BS) * Hkv + g) * D;
          const size_t si = (size_t)p * Hkv + g;
          const double w = s[t] / Z;
          if (weights) weights[rh * ((size_t)MBS * BS) + t] = w;
          for (int d = 0; d < D; ++d) acc[d] += w * load_kv(v_cache, v_scale, kv_dtype, row, d, si);
        }
        for (int d = 0; d < D; ++d) oh[d] = acc[d];
      }
    }
    free(s);
    free(vis);
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

static void append_int8_row(const uint16_t* x, int8_t* dst, float* scale_slot,
                            int opens_block, int D) {
  float sc;
  if (opens_block) {
    float amax = 0.0f;
    for (int d = 0; d < D; ++d) {
      float a = fabsf(bf16_to_f32(x[d]));
      if (a > amax) amax = a;
    }
    sc = amax / 127.0f;
    if (amax == 0.0f) sc = 1.0f;
    *scale_slot = sc;
  } else {
    sc = *scale_slot;
  }
  for (int d = 0; d < D; ++d) {
    const float y = bf16_to_f32(x[d]) / sc; /* binary32, correctly rounded */
    dst[d] = pkvo_int8_from_f32(y);
  }
}

/* In-place append of N tokens into host copies of the caches. */
int pkvo_kv_append(const uint16_t* k_new, const uint16_t* v_new,
                   const int32_t* slot_mapping, void* k_cache, void* v_cache,
                   float* k_scale, float* v_scale, int N, int Hkv, int D, int BS,
                   int NB, int kv_dtype) {
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKVO_ERR_NULL;
  if (N < 0 || Hkv <= 0 || D <= 0 || BS <= 0 || NB <= 0) return PKVO_ERR_SHAPE;
  if (!valid_dtype(kv_dtype)) return PKVO_ERR_SHAPE;
  if (kv_dtype != PKVO_KV_BF16 && (!k_scale || !v_scale)) return PKVO_ERR_NULL;
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
    } else if (kv_dtype == PKVO_KV_INT8) {
      for (int g = 0; g < Hkv; ++g) {
        append_int8_row(kr + (size_t)g * D, (int8_t*)k_cache + dst + (size_t)g * D,
                        &k_scale[blk * Hkv + g], off == 0, D);
        append_int8_row(vr + (size_t)g * D, (int8_t*)v_cache + dst + (size_t)g * D,
                        &v_scale[blk * Hkv + g], off == 0, D);
      }
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

/* ---- RoPE ----------------------------------------------------------------- */

/* Frequencies f_i, i < D/2, of the rotary embedding ("tiny-vllm part 5",
 * RoPE section): pair i turns by f_i = theta^(-2i/D) radians per position,
 * then the Llama 3 scaling of the page's table path.  That scaling is stated
 * here by what it does to a pair: count the turns the pair makes over the
 * original training context, r = original_max * f_i / (2 pi).  A pair making
 * at most low_freq_factor turns there is slowed down by `factor`, one making
 * at least high_freq_factor turns is kept, and in between the slowdown
 * fades linearly in r:
 *   s = clamp((r - low_freq_factor) / (high_freq_factor - low_freq_factor), 0, 1)
 *   f_i' = f_i * (s + (1 - s) / factor).
 * (r <= low is a wavelength 2 pi / f_i >= original_max / low_freq_factor.)
 * factor = 1 leaves every frequency unscaled. */
void pkvo_rope_freqs(int D, double theta, double factor, double low_freq_factor,
                     double high_freq_factor, double original_max, double* f) {
  const double two_pi = 2.0 * 3.14159265358979323846;
  for (int i = 0; i < D / 2; ++i) {
    const double fi = pow(theta, -(2.0 * i) / (double)D);
    const double turns = original_max * fi / two_pi;
    double s = (turns - low_freq_factor) / (high_freq_factor - low_freq_factor);
    if (s < 0.0) s = 0.0;
    if (s > 1.0) s = 1.0;
    f[i] = fi * (s + (1.0 - s) / factor);
  }
}

/* Nearest-even rounding of a double straight to bf16 bits (8 significant
 * bits).  Not via binary32: a double just above a bf16 midpoint could round
 * to the midpoint in binary32 and then to even, below.  |x| = m 2^e with
 * m in [0.5, 1); the 8-bit significand is m 2^8 rounded to an integer, ties
 * to even; the result is exact in binary32, whose top 16 bits are the bf16.
 * (Normal range only; the oracle's values are O(1).) */
static uint16_t f64_to_bf16_bits(double x) {
  if (isnan(x)) return 0x7fc0;
  if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
  int e;
  const double m = frexp(fabs(x), &e);
  double q = m * 256.0; /* exact: a power-of-two scaling */
  double lo = floor(q);
  const double frac = q - lo; /* exact */
  if (frac > 0.5 || (frac == 0.5 && fmod(lo, 2.0) != 0.0)) lo += 1.0;
  float f = (float)ldexp(lo, e - 8); /* exact: at most 9 significant bits */
  if (x < 0) f = -f;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* Rotate x [N, H, D] (bf16 bits) at positions pos[N]; y gets bf16 bits (may
 * alias x).  If y_f64 is not NULL it receives the unrounded rotation. */
void pkvo_rope_apply(const uint16_t* x, const int32_t* pos, int N, int H, int D, const double* f,
                     uint16_t* y, double* y_f64) {
  for (int n = 0; n < N; ++n) {
    for (int h = 0; h < H; ++h) {
      const size_t base = ((size_t)n * H + h) * D;
      for (int i = 0; i < D / 2; ++i) {
        const double a = (double)pos[n] * f[i];
        const double c = cos(a), sn = sin(a);
        const double x0 = pkvo_bf16_to_f64(x[base + 2 * i]);
        const double x1 = pkvo_bf16_to_f64(x[base + 2 * i + 1]);
        const double r0 = x0 * c - x1 * sn;
        const double r1 = x0 * sn + x1 * c;
        if (y_f64) {
          y_f64[base + 2 * i] = r0;
          y_f64[base + 2 * i + 1] = r1;
        }
        y[base + 2 * i] = f64_to_bf16_bits(r0);
        y[base + 2 * i + 1] = f64_to_bf16_bits(r1);
      }
    }
  }
}
