/* Host driver of the oracle (oracle/oracle.c) and the input generator (synth/synth.c) for the
 * AddressSanitizer / UndefinedBehaviorSanitizer build that tests/test_host_sanitizers.py makes:
 * every exported routine runs once on small inputs, including the edge cases (all codes of each
 * format, fewer visible tokens than k, tied scores, strided shard pools).  Exit status 0 and no
 * sanitizer report is the pass. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_e4m3(uint8_t c);
double orc_e2m1(uint8_t nib);
double orc_e8m0(uint8_t c);
double orc_bf16(uint16_t b);
int64_t orc_indexer_scores(int H, int D, int key_fmt, const uint8_t* q, const float* w, int64_t n,
                           const uint8_t* key, const void* key_scale, double* score64,
                           float* score32);
void orc_topk(int64_t n, const double* score, int k, int32_t* idx, int32_t* count);
void orc_sparse_mla(int H, int Dqk, int Dv, const uint16_t* q, int64_t nsel, const double* c,
                    double softmax_scale, double* out, double* lse);
int64_t orc_dsa_rows(int key_fmt, int lat_fmt, int nrows, const int64_t* row_pos,
                     const uint8_t* qidx, const float* w, const uint16_t* qmla, int64_t ntok,
                     const uint8_t* keys, const void* key_scale, const uint8_t* lat,
                     const void* lat_scale, float lat_tensor_scale, int k, double softmax_scale,
                     int32_t* idx, int32_t* count, double* out, double* lse, double* scores);
void orc_quant_fp8_token(int D, const uint16_t* x, uint8_t* codes, float* scale);
void orc_quant_mxfp4_key(int D, const uint16_t* x, uint8_t* packed, uint8_t* e8m0);
void orc_quant_nvfp4_latent(int D, const uint16_t* x, float ts, uint8_t* packed, uint8_t* bscale);
void orc_quantize_query(int H, int D, const uint16_t* q, const float* w, uint8_t* codes,
                        float* wout);
uint16_t synth_enc_bf16(float x);
void synth_ikey_fp8(uint64_t seed, int64_t seq, int64_t tok0, int64_t ntok, uint8_t* codes,
                    float* scale);
void synth_ikey_mxfp4(uint64_t seed, int64_t seq, int64_t tok0, int64_t ntok, uint8_t* packed,
                      uint8_t* e8m0);
void synth_latent_fp8(uint64_t seed, int64_t seq, int64_t tok0, int64_t ntok, uint8_t* codes,
                      float* scale);
void synth_latent_nvfp4(uint64_t seed, int64_t seq, int64_t tok0, int64_t ntok, uint8_t* packed,
                        uint8_t* bscale);
void synth_qidx(uint64_t seed, int64_t row0, int64_t nrows, int wq, uint8_t* q, float* w);
void synth_qmla(uint64_t seed, int64_t row0, int64_t nrows, uint16_t* q);
void synth_fill_pool(uint64_t seed, int ikey_fmt, int lat_fmt, int block_size, int64_t row_bytes,
                     int64_t lat_off, int64_t lat_scale_off, int64_t ikey_off,
                     int64_t ikey_scale_off, int64_t num_blocks, uint8_t* pool, int num_seqs,
                     const int32_t* block_table, int64_t ld_bt, const int64_t* seq_len,
                     const int64_t* seq_id, int64_t tok_stride, int64_t tok_offset);

enum { NT = 300, IH = 32, ID = 128, H = 96, DQK = 576, DV = 512, K = 64, R = 3 };

int main(void) {
  double acc = 0;
  for (int c = 0; c < 256; ++c) {
    const double v = orc_e4m3((uint8_t)c), e = orc_e8m0((uint8_t)c);
    if (!isnan(v)) acc += v;
    if (!isnan(e) && !isinf(e)) acc += e * 1e-30;
    acc += orc_bf16((uint16_t)(c << 8)) * 1e-40;
  }
  for (int c = 0; c < 16; ++c) acc += orc_e2m1((uint8_t)c);

  /* quantisers on bf16 data with zeros, negative zeros and large values */
  uint16_t x[DQK];
  for (int i = 0; i < DQK; ++i) x[i] = synth_enc_bf16((float)(sin(0.37 * i) * (i % 7 == 0 ? 1e3 : 1.0)));
  x[3] = 0x8000;
  uint8_t codes[DQK], packed[DQK / 2], e8[DQK / 32], bs[DQK / 16];
  float s;
  orc_quant_fp8_token(DQK, x, codes, &s);
  orc_quant_mxfp4_key(ID, x, packed, e8);
  orc_quant_nvfp4_latent(DQK, x, 0.25f, packed, bs);
  uint16_t qb[IH * ID];
  float wq[IH], wq2[IH];
  for (int i = 0; i < IH * ID; ++i) qb[i] = x[i % DQK];
  for (int h = 0; h < IH; ++h) wq[h] = 0.1f * (float)(h - 16);
  uint8_t qcodes[IH * ID];
  orc_quantize_query(IH, ID, qb, wq, qcodes, wq2);
  acc += s + wq2[5];

  /* generated keys, latents, queries of one sequence; scores, select, attention */
  const uint64_t seed = 99;
  uint8_t* keys = (uint8_t*)malloc(NT * ID);
  float* kscale = (float*)malloc(NT * sizeof(float));
  uint8_t* mkeys = (uint8_t*)malloc(NT * ID / 2);
  uint8_t* mscale = (uint8_t*)malloc(NT * 4);
  uint8_t* lat = (uint8_t*)malloc(NT * DQK);
  float* lscale = (float*)malloc(NT * sizeof(float));
  uint8_t* nlat = (uint8_t*)malloc(NT * DQK / 2);
  uint8_t* nscale = (uint8_t*)malloc(NT * 36);
  synth_ikey_fp8(seed, 0, 0, NT, keys, kscale);
  synth_ikey_mxfp4(seed, 0, 0, NT, mkeys, mscale);
  synth_latent_fp8(seed, 0, 0, NT, lat, lscale);
  synth_latent_nvfp4(seed, 0, 0, NT, nlat, nscale);
  uint8_t* qi = (uint8_t*)malloc(R * IH * ID);
  float* w = (float*)malloc(R * IH * sizeof(float));
  uint16_t* qm = (uint16_t*)malloc(R * H * DQK * sizeof(uint16_t));
  synth_qidx(seed, 0, R, 8, qi, w);
  synth_qmla(seed, 0, R, qm);
  double* s64 = (double*)malloc(NT * sizeof(double));
  float* s32 = (float*)malloc(NT * sizeof(float));
  acc += (double)orc_indexer_scores(IH, ID, 0, qi, w, NT, keys, kscale, s64, s32);
  acc += (double)orc_indexer_scores(IH, ID, 1, qi, w, NT, mkeys, mscale, s64, s32);
  int32_t idx[K], cnt;
  orc_topk(NT, s64, K, idx, &cnt);
  orc_topk(20, s64, K, idx, &cnt); /* fewer than k */
  for (int i = 0; i < NT; ++i) s64[i] = (double)(i % 3); /* ties */
  orc_topk(NT, s64, K, idx, &cnt);
  double* c = (double*)malloc((size_t)10 * DQK * sizeof(double));
  for (int i = 0; i < 10 * DQK; ++i) c[i] = sin(0.1 * i);
  double* out = (double*)malloc((size_t)R * H * DV * sizeof(double));
  double* lse = (double*)malloc((size_t)R * H * sizeof(double));
  orc_sparse_mla(H, DQK, DV, qm, 10, c, 0.07, out, lse);
  orc_sparse_mla(H, DQK, DV, qm, 0, c, 0.07, out, lse); /* nothing selected */
  const int64_t rp[R] = {NT - 1, 40, 0};
  int32_t ridx[R * K], rcnt[R];
  double* sc = (double*)malloc((size_t)R * NT * sizeof(double));
  acc += (double)orc_dsa_rows(0, 0, R, rp, qi, w, qm, NT, keys, kscale, lat, lscale, 1.0f, K,
                              0.07, ridx, rcnt, out, lse, sc);
  acc += (double)orc_dsa_rows(1, 1, R, rp, qi, w, qm, NT, mkeys, mscale, nlat, nscale, 0.5f, K,
                              0.07, ridx, rcnt, out, lse, NULL);

  /* a small pool of two sequences, and a strided shard of it */
  const int bsz = 64;
  const int64_t row_bytes = 45568, lat_off = 0, lat_scale_off = 36864, ikey_off = 37120,
                ikey_scale_off = 45312;
  const int64_t lens[2] = {150, 70};
  const int32_t bt[2 * 3] = {4, 0, 2, 1, 3, -1};
  uint8_t* pool = (uint8_t*)malloc((size_t)6 * row_bytes);
  synth_fill_pool(seed, 0, 0, bsz, row_bytes, lat_off, lat_scale_off, ikey_off, ikey_scale_off, 6,
                  pool, 2, bt, 3, lens, NULL, 1, 0);
  /* MXFP4 keys (64 + 4 B per token) and NVFP4 latents (288 + 36 B) in the same row size */
  synth_fill_pool(seed, 1, 1, bsz, row_bytes, 0, 18432, 20736, 24832, 6, pool, 2, bt, 3, lens,
                  NULL, 3, 2);
  acc += pool[ikey_off + 5];

  printf("sanitize driver ok %g\n", acc);
  free(keys); free(kscale); free(mkeys); free(mscale); free(lat); free(lscale); free(nlat);
  free(nscale); free(qi); free(w); free(qm); free(s64); free(s32); free(c); free(out); free(lse);
  free(sc); free(pool);
  return 0;
}
