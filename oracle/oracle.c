/*
 * CPU oracle for the DSA sparse-attention layer: lightning-indexer scores -> exact top-k ->
 * exact MLA attention over the selected latents.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code with the GPU path (no headers, helpers, tables or
 * constants) and the GPU path never calls it.
 *
 * Sources (page titles and sections; the pages are the specification):
 *   [K31] "vLLM Delivers Day-0 Support for Kimi K3.1 Pro" (wpnews.pro), sections
 *         "Sparse Attention in K3.1 Pro", "KV cache footprint", "A KV cache for three kinds of
 *         state", "AMD / Quantization: Native MXFP4 indexer".
 *   [K31] also, section "Low-latency decode: a fused DSA decode path", for the step before the
 *         path: the indexer query quantised after the head weights are multiplied into it, and the
 *         appended token's index key and latent written into the cache (the quantisers at the end of
 *         this file).
 *   The pages defer the indexer's scoring rule to DeepSeek-V3.2's lightning indexer; the rule
 *   used here is that indexer's: score = sum_h w[h] * ReLU(scale_s * q[h] . k[s]).
 *   Number formats follow their published definitions: OCP 8-bit Floating Point (E4M3),
 *   OCP Microscaling Formats v1.0 (E2M1 elements, E8M0 scales), NVFP4 (E2M1 elements with
 *   E4M3 scales per 16 elements and one fp32 tensor scale), bfloat16.
 *
 * Everything is computed in double precision with plain loops, in the order the definitions
 * state.  The indexer score is also computed once in fp32 in a fixed order (d ascending, then
 * h ascending) so callers can assert that the inputs are on a grid where fp32 is exact.
 *
 * Parity pins (tests under tests/): codecs against torch's float8 casts and the OCP value
 * tables; scores against hand-worked fixtures, one-hot closed forms, q = 0, scale pull-out and
 * head-permutation invariance; top-k against its defining order property and brute force on
 * tiny inputs; attention against float64 scaled-dot-product attention from torch when the
 * selected set is every visible token, and, when it is a strict subset (k below the visible
 * count), against the same attention over latents decoded independently (torch's E4M3 cast, the
 * OCP E2M1 table) at the selected indices with their own scales; FP8 latent dequantisation
 * against a hand-worked fixture with a distinct scale per token; attention against single-token
 * / identical-latent / q = 0 closed forms, and against permutation and causality invariants;
 * quantisers against an arithmetic
 * round-half-even formulation on each format's grid, midpoints, saturation, exact round trips of
 * representable tokens, the scale rules and error bounds of each format, and the query-scale fold
 * through the scoring rule.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ format decoders */

/* OCP FP8 E4M3 (the "fn" variant): 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent
 * field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN; there is no infinity. */
double orc_e4m3(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
  double v;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* OCP MX E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent field 0 encodes the
 * subnormal m * 0.5.  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double orc_e2m1(uint8_t nib) {
  int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* OCP MX E8M0 scale: 2^(E-127); E = 255 is NaN. */
double orc_e8m0(uint8_t c) { return c == 255 ? NAN : ldexp(1.0, (int)c - 127); }

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double orc_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Index-key element d of one token.  FP8 keys: e4m3 code.  MXFP4 keys: e2m1 element times the
 * E8M0 scale of its 32-element block; element 2j is the low nibble of byte j. */
static double ikey_elem(int fmt, int D, const uint8_t* key, const uint8_t* mx_scale, int d) {
  if (fmt == 0) return orc_e4m3(key[d]);
  uint8_t byte = key[d / 2];
  uint8_t nib = (d & 1) ? (byte >> 4) : (byte & 0xF);
  (void)D;
  return orc_e2m1(nib) * orc_e8m0(mx_scale[d / 32]);
}

/* ------------------------------------------------------------------ indexer */

/*
 * Lightning-indexer scores of one query row against tokens [0, n) ([K31] "Sparse Attention in
 * K3.1 Pro": every earlier token is scored by 32 light heads over FP8 keys; "Native MXFP4
 * indexer": the same scores from MXFP4 keys).
 *
 *   score[s] = sum_{h<H} w[h] * max(0, scale_s * sum_{d<D} q[h,d] * k[s,d])
 *
 * q: [H*D] E4M3 codes; w: [H] fp32 (any query quantisation scale is folded into w).
 * key_fmt 0 (FP8): key [n*D] E4M3 codes, key_scale float[n] (scale_s).
 * key_fmt 1 (MXFP4): key [n*D/2] packed E2M1, key_scale uint8[n*D/32] E8M0; scale_s = 1.
 * Writes score64[n] (double) and, if score32 != NULL, the same sum evaluated in fp32 with
 * d ascending then h ascending.  Returns the number of tokens where the two differ.
 */
int64_t orc_indexer_scores(int H, int D, int key_fmt, const uint8_t* q, const float* w, int64_t n,
                           const uint8_t* key, const void* key_scale, double* score64,
                           float* score32) {
  int64_t mismatches = 0;
  const int key_bytes = key_fmt == 0 ? D : D / 2;
  double* qd = (double*)malloc(sizeof(double) * (size_t)H * D);
  for (int i = 0; i < H * D; ++i) qd[i] = orc_e4m3(q[i]);
#pragma omp parallel reduction(+ : mismatches)
  {
    double* kd = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(static)
    for (int64_t s = 0; s < n; ++s) {
      const uint8_t* ks = key + s * key_bytes;
      const uint8_t* mxs = key_fmt == 1 ? (const uint8_t*)key_scale + s * (D / 32) : NULL;
      double scale = key_fmt == 0 ? (double)((const float*)key_scale)[s] : 1.0;
      for (int d = 0; d < D; ++d) kd[d] = ikey_elem(key_fmt, D, ks, mxs, d);
      double acc = 0.0;
      float acc32 = 0.0f;
      for (int h = 0; h < H; ++h) {
        double dot = 0.0;
        float dot32 = 0.0f;
        for (int d = 0; d < D; ++d) {
          dot += qd[h * D + d] * kd[d];
          dot32 += (float)qd[h * D + d] * (float)kd[d];
        }
        double t = scale * dot;
        acc += (double)w[h] * (t > 0.0 ? t : 0.0);
        float t32 = (float)scale * dot32;
        acc32 += w[h] * (t32 > 0.0f ? t32 : 0.0f);
      }
      score64[s] = acc;
      if (score32) score32[s] = acc32;
      if ((double)acc32 != acc) mismatches++;
    }
    free(kd);
  }
  free(qd);
  return mismatches;
}

/* ------------------------------------------------------------------ top-k */

typedef struct {
  double score;
  int64_t idx;
} scored_t;

static int by_score_desc_idx_asc(const void* a, const void* b) {
  const scored_t* x = (const scored_t*)a;
  const scored_t* y = (const scored_t*)b;
  if (x->score > y->score) return -1; /* -0.0 and +0.0 compare equal here */
  if (x->score < y->score) return 1;
  return (x->idx > y->idx) - (x->idx < y->idx);
}

static int by_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/*
 * Exact top-k of one row ([K31] "Sparse Attention in K3.1 Pro": keep the 2,048 highest-scoring
 * tokens).  Order: score descending, then token index ascending (lower index wins a tie; -0 and
 * +0 are equal).  The selected min(k, n) indices are returned sorted ascending; idx[count..k)
 * is set to -1.
 */
void orc_topk(int64_t n, const double* score, int k, int32_t* idx, int32_t* count) {
  scored_t* all = (scored_t*)malloc(sizeof(scored_t) * (size_t)(n > 0 ? n : 1));
  for (int64_t s = 0; s < n; ++s) {
    all[s].score = score[s];
    all[s].idx = s;
  }
  qsort(all, (size_t)n, sizeof(scored_t), by_score_desc_idx_asc);
  int64_t c = n < k ? n : k;
  for (int64_t i = 0; i < c; ++i) idx[i] = (int32_t)all[i].idx;
  qsort(idx, (size_t)c, sizeof(int32_t), by_i32);
  for (int64_t i = c; i < k; ++i) idx[i] = -1;
  *count = (int32_t)c;
  free(all);
}

/* ------------------------------------------------------------------ latents */

/* FP8 latent ([K31] "Sparse Attention in K3.1 Pro": 576-byte FP8 latent per token): element d
 * is the E4M3 code times the token's fp32 scale. */
void orc_dequant_latent_fp8(int D, const uint8_t* codes, float scale, double* out) {
  for (int d = 0; d < D; ++d) out[d] = orc_e4m3(codes[d]) * (double)scale;
}

/* NVFP4 latent ([K31] "A KV cache for three kinds of state": the latent may be NVFP4): element d
 * is E2M1(element) * E4M3(scale of block d/16) * fp32 tensor scale; element 2j is the low
 * nibble of byte j. */
void orc_dequant_latent_nvfp4(int D, const uint8_t* packed, const uint8_t* bscale,
                              float tensor_scale, double* out) {
  for (int d = 0; d < D; ++d) {
    uint8_t byte = packed[d / 2];
    uint8_t nib = (d & 1) ? (byte >> 4) : (byte & 0xF);
    out[d] = orc_e2m1(nib) * orc_e4m3(bscale[d / 16]) * (double)tensor_scale;
  }
}

/* ------------------------------------------------------------------ attention */

/*
 * Exact MLA attention of one query row over the selected latents ([K31] "Sparse Attention in
 * K3.1 Pro": attention is exact, restricted to the chosen tokens, for all heads alike; the latent is
 * shared by all heads).  For each head h:
 *   logit_j = softmax_scale * sum_{d<Dqk} q[h,d] * c[j,d]
 *   p_j     = exp(logit_j - max) / sum_j exp(logit_j - max)
 *   out[h]  = sum_j p_j * c[j, 0:Dv]          (the value is the first Dv latent dims)
 *   lse[h]  = max + ln sum_j exp(logit_j - max)
 * q: [H*Dqk] bf16 bits; c: [nsel*Dqk] dequantised latents.  nsel = 0 gives out = 0 and
 * lse = -inf.
 */
void orc_sparse_mla(int H, int Dqk, int Dv, const uint16_t* q, int64_t nsel, const double* c,
                    double softmax_scale, double* out, double* lse) {
#pragma omp parallel
  {
    double* logit = (double*)malloc(sizeof(double) * (size_t)(nsel > 0 ? nsel : 1));
    double* qh = (double*)malloc(sizeof(double) * (size_t)Dqk);
#pragma omp for schedule(static)
    for (int h = 0; h < H; ++h) {
      for (int d = 0; d < Dqk; ++d) qh[d] = orc_bf16(q[(int64_t)h * Dqk + d]);
      double mx = -INFINITY;
      for (int64_t j = 0; j < nsel; ++j) {
        double dot = 0.0;
        for (int d = 0; d < Dqk; ++d) dot += qh[d] * c[j * Dqk + d];
        logit[j] = softmax_scale * dot;
        if (logit[j] > mx) mx = logit[j];
      }
      double denom = 0.0;
      for (int64_t j = 0; j < nsel; ++j) {
        logit[j] = exp(logit[j] - mx);
        denom += logit[j];
      }
      for (int d = 0; d < Dv; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j < nsel; ++j) acc += logit[j] * c[j * Dqk + d];
        out[(int64_t)h * Dv + d] = nsel > 0 ? acc / denom : 0.0;
      }
      lse[h] = nsel > 0 ? mx + log(denom) : -INFINITY;
    }
    free(logit);
    free(qh);
  }
}

/* ------------------------------------------------------------------ one DSA layer */

/*
 * The whole layer for the query rows of one sequence ([K31] "Sparse Attention in K3.1 Pro":
 * score every earlier token, keep the top k, attend exactly over them).  Row r sits at absolute
 * position row_pos[r] and sees tokens [0, row_pos[r]] (the new token's key and latent are in the
 * cache before it is scored).  Logical (unpaged) inputs of the sequence, ntok tokens:
 *   key_fmt 0: keys [ntok*128] E4M3 + key_scale float[ntok]; 1: keys [ntok*64] + E8M0 [ntok*4]
 *   lat_fmt 0: lat [ntok*576] E4M3 + lat_scale float[ntok];  1: lat [ntok*288] + E4M3 [ntok*36]
 * Per row: qidx [32*128] E4M3, w [32] fp32, qmla [96*576] bf16.
 * Outputs: idx [nrows*k] (ascending, -1 padded), count [nrows], out [nrows*96*512],
 * lse [nrows*96]; scores [nrows*ntok] if not NULL (positions past row_pos are set to -inf).
 * Returns the number of visible scores where fp32 and fp64 evaluation differ.
 */
int64_t orc_dsa_rows(int key_fmt, int lat_fmt, int nrows, const int64_t* row_pos,
                     const uint8_t* qidx, const float* w, const uint16_t* qmla, int64_t ntok,
                     const uint8_t* keys, const void* key_scale, const uint8_t* lat,
                     const void* lat_scale, float lat_tensor_scale, int k, double softmax_scale,
                     int32_t* idx, int32_t* count, double* out, double* lse, double* scores) {
  const int IH = 32, ID = 128, H = 96, DQK = 576, DV = 512;
  int64_t mism = 0;
  double* sc = (double*)malloc(sizeof(double) * (size_t)(ntok > 0 ? ntok : 1));
  float* sc32 = (float*)malloc(sizeof(float) * (size_t)(ntok > 0 ? ntok : 1));
  double* c = (double*)malloc(sizeof(double) * (size_t)k * DQK);
  for (int r = 0; r < nrows; ++r) {
    int64_t nvis = row_pos[r] + 1;
    if (nvis > ntok) nvis = ntok;
    mism += orc_indexer_scores(IH, ID, key_fmt, qidx + (int64_t)r * IH * ID, w + (int64_t)r * IH,
                               nvis, keys, key_scale, sc, sc32);
    if (scores) {
      for (int64_t s = 0; s < ntok; ++s) scores[(int64_t)r * ntok + s] = s < nvis ? sc[s] : -INFINITY;
    }
    int32_t* ri = idx + (int64_t)r * k;
    orc_topk(nvis, sc, k, ri, &count[r]);
    for (int j = 0; j < count[r]; ++j) {
      int64_t s = ri[j];
      if (lat_fmt == 0)
        orc_dequant_latent_fp8(DQK, lat + s * DQK, ((const float*)lat_scale)[s], c + (int64_t)j * DQK);
      else
        orc_dequant_latent_nvfp4(DQK, lat + s * (DQK / 2), (const uint8_t*)lat_scale + s * (DQK / 16),
                                 lat_tensor_scale, c + (int64_t)j * DQK);
    }
    orc_sparse_mla(H, DQK, DV, qmla + (int64_t)r * H * DQK, count[r], c, softmax_scale,
                   out + (int64_t)r * H * DV, lse + (int64_t)r * H);
  }
  free(sc);
  free(sc32);
  free(c);
  return mism;
}

/* ------------------------------------------------------------------ quantisers (the step
 * before the path: the appended token's index key and latent written into its paged row, and the
 * indexer query quantised with its scale folded into the head weight; [K31] "A KV cache for three
 * kinds of state" for the formats, "Low-latency decode: a fused DSA decode path" for the step).
 *
 * Rounding is round-to-nearest, ties to the even code (mantissa LSB 0), found by exhaustive
 * search over the finite codes of the format; a magnitude beyond the largest finite value takes
 * the largest (saturation).  The sign bit is that of x (so -0 and negative values rounding to 0
 * give the negative zero code).  Arithmetic on the way (amax, the division by the scale) is in
 * fp32, as a kernel does it. */

static uint8_t nearest_mag(double a, int ncodes, double (*dec)(uint8_t)) {
  uint8_t best = 0;
  double bestd = INFINITY;
  for (int c = 0; c < ncodes; ++c) {
    const double d = fabs(dec((uint8_t)c) - a);
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = (uint8_t)c;
      bestd = d;
    }
  }
  return best;
}

/* e4m3 code of x: magnitudes 0x00..0x7E (0x7F is NaN). */
uint8_t orc_quant_e4m3(float x) {
  return (uint8_t)((signbit(x) ? 0x80 : 0) | nearest_mag(fabs((double)x), 0x7F, orc_e4m3));
}

/* e2m1 nibble of x: magnitudes 0..7. */
uint8_t orc_quant_e2m1(float x) {
  return (uint8_t)((signbit(x) ? 0x8 : 0) | nearest_mag(fabs((double)x), 8, orc_e2m1));
}

static float bf16f(uint16_t b) { return (float)orc_bf16(b); }

static float amax_bf16(int n, const uint16_t* x) {
  float m = 0.f;
  for (int i = 0; i < n; ++i) m = fmaxf(m, fabsf(bf16f(x[i])));
  return m;
}

/* One token of D bf16 values as FP8 with a per-token scale: s = amax / 448 (1 when amax is 0),
 * code_d = e4m3(x_d / s).  (FP8 index keys and FP8 latents.) */
void orc_quant_fp8_token(int D, const uint16_t* x, uint8_t* codes, float* scale) {
  const float amax = amax_bf16(D, x);
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  for (int d = 0; d < D; ++d) codes[d] = orc_quant_e4m3(bf16f(x[d]) / s);
  *scale = s;
}

/* One MXFP4 index key (OCP MX): per block of 32 elements the E8M0 scale X = 2^(floor(log2
 * amax) - 2) (E2M1's largest exponent is 2; X = 1 when amax is 0), elements e2m1(x / X),
 * element 2j in the low nibble of byte j. */
void orc_quant_mxfp4_key(int D, const uint16_t* x, uint8_t* packed, uint8_t* e8m0) {
  memset(packed, 0, (size_t)D / 2);
  for (int b = 0; b < D / 32; ++b) {
    const float amax = amax_bf16(32, x + 32 * b);
    int E = 127;
    if (amax > 0.f) {
      int e;
      frexpf(amax, &e);  /* amax = m 2^e, m in [0.5, 1): floor(log2 amax) = e - 1 */
      E = (e - 1) - 2 + 127;
      if (E < 0) E = 0;
      if (E > 254) E = 254;
    }
    e8m0[b] = (uint8_t)E;
    const float X = ldexpf(1.0f, E - 127);
    for (int i = 0; i < 32; ++i) {
      const int d = 32 * b + i;
      const uint8_t nib = orc_quant_e2m1(bf16f(x[d]) / X);
      packed[d / 2] |= (uint8_t)((d & 1) ? nib << 4 : nib);
    }
  }
}

/* One NVFP4 latent: per block of 16 elements the E4M3 block scale bs = e4m3((amax / 6) / ts)
 * with ts the fp32 tensor scale; elements e2m1(x / (bs * ts)) (0 when bs * ts is 0); element
 * 2j in the low nibble of byte j. */
void orc_quant_nvfp4_latent(int D, const uint16_t* x, float ts, uint8_t* packed, uint8_t* bscale) {
  memset(packed, 0, (size_t)D / 2);
  for (int b = 0; b < D / 16; ++b) {
    const float amax = amax_bf16(16, x + 16 * b);
    const uint8_t bs = orc_quant_e4m3((amax / 6.0f) / ts);
    bscale[b] = bs;
    const float sd = (float)orc_e4m3(bs) * ts;
    for (int i = 0; i < 16; ++i) {
      const int d = 16 * b + i;
      const uint8_t nib = sd > 0.f ? orc_quant_e2m1(bf16f(x[d]) / sd) : 0;
      packed[d / 2] |= (uint8_t)((d & 1) ? nib << 4 : nib);
    }
  }
}

/* Indexer query of one row: per head h a scale s_h = amax_h / 448 (1 when amax_h is 0), codes
 * e4m3(q / s_h), and the head weight w'_h = w_h * s_h (fp32), so that
 * w'_h ReLU(q'_h . k) = w_h ReLU(s_h q'_h . k) ~ w_h ReLU(q_h . k). */
void orc_quantize_query(int H, int D, const uint16_t* q, const float* w, uint8_t* codes,
                        float* wout) {
  for (int h = 0; h < H; ++h) {
    float s;
    orc_quant_fp8_token(D, q + (size_t)h * D, codes + (size_t)h * D, &s);
    wout[h] = w[h] * s;
  }
}
