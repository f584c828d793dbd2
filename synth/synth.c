/*
 * Seeded synthetic inputs for the DSA sparse-attention layer (indexer -> top-k -> sparse MLA).
 *
 * This file is shared by the GPU path (which reads the paged pool it writes) and by the CPU
 * oracle (which reads the logical arrays it writes).  It holds no part of the method: no scoring,
 * selection, attention or format decoding.  It only draws counter-based random numbers and
 * encodes them into the storage formats the layer consumes (OCP FP8 E4M3, OCP MX FP4 E2M1 with
 * E8M0 block scales, NVFP4 = E2M1 with E4M3 block-16 scales, bfloat16).
 *
 * Every value is a pure function of (seed, stream, index), so any slice of any tensor can be
 * regenerated on its own: the oracle regenerates the sequences it checks without the pool, and
 * the pool writer fills blocks in any order.
 *
 * "Exact-grid" values (index keys, indexer queries, head weights, key scales) are restricted so
 * that every partial sum of the indexer score is an exactly representable fp32 number: queries
 * and FP8 keys take values k/4 with |k| <= 16, head weights k/4 with |k| <= wq, FP8 key scales
 * 2^-e with e in 0..6, and MXFP4 key block scales 2^-2..2^0.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_STREAM_IKEY 1u
#define SYNTH_STREAM_IKEY_SCALE 2u
#define SYNTH_STREAM_LATENT 3u
#define SYNTH_STREAM_LATENT_SCALE 4u
#define SYNTH_STREAM_QIDX 5u
#define SYNTH_STREAM_W 6u
#define SYNTH_STREAM_QMLA 7u
#define SYNTH_STREAM_IKEY_MX 8u
#define SYNTH_STREAM_IKEY_MX_SCALE 9u
#define SYNTH_STREAM_LATENT_NV 10u

#define IDX_DIM 128
#define IDX_HEADS 32
#define MLA_HEADS 96
#define MLA_DQK 576

/* ---------------------------------------------------------------- counter-based RNG */

/* SplitMix64 finaliser (Steele, Lea, Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014). */
static inline uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint32_t tensor, uint64_t sub) {
  return mix64(mix64(seed ^ ((uint64_t)tensor << 56)) ^ mix64(sub + 0x632BE59BD9B4E019ull));
}

uint64_t synth_hash(uint64_t seed, uint32_t tensor, uint64_t sub, uint64_t index) {
  return mix64(stream_key(seed, tensor, sub) ^ (index * 0xD1B54A32D192ED03ull));
}

static inline double u01(uint64_t h) { /* (0,1), 53 bits */
  return ((double)(h >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* Two standard normals for element pair `pair` (elements 2*pair and 2*pair+1): Box-Muller on two
 * 32-bit uniforms taken from one hash, in single precision. */
static inline void normal_pair(uint64_t key, uint64_t pair, double* n0, double* n1) {
  uint64_t h = mix64(key ^ (pair * 0xD1B54A32D192ED03ull));
  float u1 = ((float)(uint32_t)(h >> 40) + 0.5f) * (1.0f / 16777216.0f);          /* (0,1) */
  float u2 = (float)(uint32_t)(h & 0xFFFFFFu) * (1.0f / 16777216.0f);              /* [0,1) */
  float r = sqrtf(-2.0f * logf(u1));
  float sn, cs;
  sincosf(6.2831853f * u2, &sn, &cs);
  *n0 = (double)(r * cs);
  *n1 = (double)(r * sn);
}

/* One standard normal per index (the matching half of its pair). */
static inline double normal_at(uint64_t key, uint64_t index) {
  double a, b;
  normal_pair(key, index >> 1, &a, &b);
  return (index & 1) ? b : a;
}

/* ---------------------------------------------------------------- encoders (inputs only) */

/* float -> OCP FP8 E4M3 code, round to nearest even, saturating to +-448 (bit manipulation on
 * the binary32 encoding: keep 3 mantissa bits with ties to even; below 2^-6 the step is 2^-9). */
static inline uint8_t enc_e4m3_f(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  uint8_t s = (u >> 31) ? 0x80 : 0;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7F;  /* NaN (never generated) */
  if (a >= 0x43E80000u) return s | 0x7E; /* |x| >= 464: saturate */
  if (a < 0x3C800000u) {               /* |x| < 2^-6: subnormal grid m * 2^-9 */
    float f;
    memcpy(&f, &a, 4);
    return s | (uint8_t)nearbyintf(f * 512.0f);  /* 8 rounds up to the smallest normal */
  }
  int e = (int)(a >> 23) - 127;
  uint32_t m = a & 0x7FFFFFu;
  uint32_t r = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20; /* 3 bits, ties to even */
  if (r == 8) { r = 0; ++e; }
  uint32_t code = ((uint32_t)(e + 7) << 3) | r;
  return s | (uint8_t)(code > 0x7E ? 0x7E : code);
}

uint8_t synth_enc_e4m3(double x) { return enc_e4m3_f((float)x); }

/* float -> OCP E2M1 nibble, round to nearest even, saturating to +-6. */
uint8_t synth_enc_e2m1(double x) {
  uint8_t s = (x < 0) ? 0x8 : 0;
  double a = fabs(x);
  if (a > 5.0) return s | 0x7; /* above the 4..6 midpoint: 6 (and saturate); 5 ties to 4 */
  int e;
  frexp(a, &e);
  int ue = e - 1;
  if (a == 0) return s;
  if (ue < 0) ue = 0;
  double ulp = ldexp(1.0, ue - 1);
  double r = nearbyint(a / ulp);
  if (ue == 0 && r < 2) return s | (uint8_t)r; /* 0 or 0.5 (subnormal) */
  if (r >= 4) { r = 2; ue += 1; }
  if (ue > 2) return s | 0x7;
  return s | (uint8_t)(((ue + 1) << 1) | ((int)r - 2));
}

/* Quantise to the E4M3 grid and return the grid value (for choosing NVFP4 block scales). */
static double round_to_e4m3_value(double a) { /* a >= 0 */
  if (a == 0) return 0;
  if (a >= 464.0) return 448.0;
  int e;
  frexp(a, &e);
  int ue = e - 1;
  if (ue < -6) ue = -6;
  double ulp = ldexp(1.0, ue - 3);
  double v = nearbyint(a / ulp) * ulp;
  return v > 448.0 ? 448.0 : v;
}

/* float -> bfloat16 bits, round to nearest even (finite inputs). */
uint16_t synth_enc_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

static inline double grid_quarter(double n, int kmax) { /* N(0,1) -> k/4, |k| <= kmax */
  double k = nearbyint(4.0 * n);
  if (k > kmax) k = kmax;
  if (k < -kmax) k = -kmax;
  return k / 4.0;
}

/* ---------------------------------------------------------------- logical tensors */

/* FP8 index keys of sequence `seq`, tokens [tok0, tok0+ntok): codes [ntok,128], scale [ntok]. */
void synth_ikey_fp8(uint64_t seed, int64_t seq, int64_t tok0, int64_t ntok, uint8_t* codes,
                    float* scale) {
  uint64_t kk = stream_key(seed, SYNTH_STREAM_IKEY, (uint64_t)seq);
  uint64_t ks = stream_key(seed, SYNTH_STREAM_IKEY_SCALE, (uint64_t)seq);
#pragma omp parallel for schedule(static) if (ntok > 256)
  for (int64_t t = 0; t < ntok; ++t) {
    uint64_t s = (uint64_t)(tok0 + t);
    for (int d = 0; d < IDX_DIM; d += 2) {
      double n0, n1;
      normal_pair(kk, (s * IDX_DIM + d) >> 1, &n0, &n1);
      codes[t * IDX_DIM + d] = synth_enc_e4m3(grid_quarter(n0, 16));
      codes[t * IDX_DIM + d + 1] = synth_enc_e4m3(grid_quarter(n1, 16));
    }
    int e = (int)(mix64(ks ^ (s * 0xD1B54A32D192ED03ull)) % 7u);
    scale[t] = (float)ldexp(1.0, -e);
  }
}

/* MXFP4 index keys: packed e2m1 [ntok,64] (element 2j in the low nibble of byte j) and E8M0
 * block-32 scales [ntok,4] drawn from {125,126,127} (2^-2 .. 2^0). */
void synth_ikey_mxfp4(uint64_t seed, int64_t seq, int64_t tok0, int64_t ntok, uint8_t* packed,
                      uint8_t* e8m0) {
  uint64_t kk = stream_key(seed, SYNTH_STREAM_IKEY_MX, (uint64_t)seq);
  uint64_t ks = stream_key(seed, SYNTH_STREAM_IKEY_MX_SCALE, (uint64_t)seq);
#pragma omp parallel for schedule(static) if (ntok > 256)
  for (int64_t t = 0; t < ntok; ++t) {
    uint64_t s = (uint64_t)(tok0 + t);
    for (int j = 0; j < IDX_DIM / 2; ++j) {
      double n0, n1;
      normal_pair(kk, (s * IDX_DIM + 2 * j) >> 1, &n0, &n1);
      uint8_t lo = synth_enc_e2m1(2.0 * n0);
      uint8_t hi = synth_enc_e2m1(2.0 * n1);
      packed[t * 64 + j] = (uint8_t)(lo | (hi << 4));
    }
    for (int b = 0; b < 4; ++b)
      e8m0[t * 4 + b] = (uint8_t)(125 + mix64(ks ^ ((s * 4 + b) * 0xD1B54A32D192ED03ull)) % 3u);
  }
}

/* FP8 latents: codes [ntok,576] = E4M3(N(0,1)), per-token fp32 scale U[0.5,2). */
void synth_latent_fp8(uint64_t seed, int64_t seq, int64_t tok0, int64_t ntok, uint8_t* codes,
                      float* scale) {
  uint64_t kk = stream_key(seed, SYNTH_STREAM_LATENT, (uint64_t)seq);
  uint64_t ks = stream_key(seed, SYNTH_STREAM_LATENT_SCALE, (uint64_t)seq);
#pragma omp parallel for schedule(static) if (ntok > 256)
  for (int64_t t = 0; t < ntok; ++t) {
    uint64_t s = (uint64_t)(tok0 + t);
    for (int d = 0; d < MLA_DQK; d += 2) {
      double n0, n1;
      normal_pair(kk, (s * MLA_DQK + d) >> 1, &n0, &n1);
      codes[t * MLA_DQK + d] = synth_enc_e4m3(n0);
      codes[t * MLA_DQK + d + 1] = synth_enc_e4m3(n1);
    }
    scale[t] = (float)(0.5 + 1.5 * u01(mix64(ks ^ (s * 0xD1B54A32D192ED03ull))));
  }
}

/* NVFP4 latents: packed e2m1 [ntok,288] (element 2j low nibble of byte j) and E4M3 block-16
 * scales [ntok,36].  Block scale = E4M3(amax/6); codes = E2M1(x / block scale).  The fp32 tensor
 * scale is not part of the stored page. */
void synth_latent_nvfp4(uint64_t seed, int64_t seq, int64_t tok0, int64_t ntok, uint8_t* packed,
                        uint8_t* bscale) {
  uint64_t kk = stream_key(seed, SYNTH_STREAM_LATENT_NV, (uint64_t)seq);
#pragma omp parallel for schedule(static) if (ntok > 256)
  for (int64_t t = 0; t < ntok; ++t) {
    uint64_t s = (uint64_t)(tok0 + t);
    double x[16];
    for (int b = 0; b < MLA_DQK / 16; ++b) {
      double amax = 0;
      for (int i = 0; i < 16; i += 2) normal_pair(kk, (s * MLA_DQK + b * 16 + i) >> 1, &x[i], &x[i + 1]);
      for (int i = 0; i < 16; ++i)
        if (fabs(x[i]) > amax) amax = fabs(x[i]);
      double sv = round_to_e4m3_value(amax / 6.0);
      bscale[t * 36 + b] = synth_enc_e4m3(sv);
      for (int i = 0; i < 16; i += 2) {
        uint8_t lo = sv > 0 ? synth_enc_e2m1(x[i] / sv) : 0;
        uint8_t hi = sv > 0 ? synth_enc_e2m1(x[i + 1] / sv) : 0;
        packed[t * 288 + b * 8 + i / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

/* Indexer query of rows [row0, row0+nrows): q codes [n,32,128] on the k/4 (|k|<=16) grid and head
 * weights w [n,32] on the k/4 (|k|<=wq) grid. */
void synth_qidx(uint64_t seed, int64_t row0, int64_t nrows, int wq, uint8_t* q, float* w) {
  uint64_t kq = stream_key(seed, SYNTH_STREAM_QIDX, 0);
  uint64_t kw = stream_key(seed, SYNTH_STREAM_W, 0);
  for (int64_t r = 0; r < nrows; ++r) {
    uint64_t row = (uint64_t)(row0 + r);
    for (int i = 0; i < IDX_HEADS * IDX_DIM; ++i)
      q[r * IDX_HEADS * IDX_DIM + i] =
          synth_enc_e4m3(grid_quarter(normal_at(kq, row * IDX_HEADS * IDX_DIM + i), 16));
    for (int h = 0; h < IDX_HEADS; ++h)
      w[r * IDX_HEADS + h] = (float)grid_quarter(normal_at(kw, row * IDX_HEADS + h), wq);
  }
}

/* MLA query of rows [row0, row0+nrows): bf16 [n,96,576] of N(0,1). */
void synth_qmla(uint64_t seed, int64_t row0, int64_t nrows, uint16_t* q) {
  uint64_t kq = stream_key(seed, SYNTH_STREAM_QMLA, 0);
  const int64_t per = (int64_t)MLA_HEADS * MLA_DQK;
  for (int64_t r = 0; r < nrows; ++r) {
    uint64_t row = (uint64_t)(row0 + r);
#pragma omp parallel for schedule(static) if (per > 4096)
    for (int64_t i = 0; i < per; ++i)
      q[r * per + i] = synth_enc_bf16((float)normal_at(kq, row * (uint64_t)per + (uint64_t)i));
  }
}

/* ---------------------------------------------------------------- pool writer */

/* FP8 index keys of tokens [0, ntok) of a block into its key page, in the page's load order:
 * byte b of slot t sits at 2048 (t / 16) + 1024 (b / 64) + 256 ((b / 16) % 4) + 16 (t % 16) + b % 16,
 * so that the 16-byte pieces one 64-lane load takes (one per lane) form a contiguous 1 KB run. */
static void put_fp8_keys(uint8_t* page, const uint8_t* key, int64_t ntok) {
  for (int64_t t = 0; t < ntok; ++t)
    for (int q = 0; q < IDX_DIM / 16; ++q)
      memcpy(page + 2048 * (t / 16) + 1024 * (q / 4) + 256 * (q % 4) + 16 * (t % 16),
             key + t * IDX_DIM + 16 * q, 16);
}

/*
 * Fill a block-packed pool.  Each pool row holds `block_size` tokens; the byte offsets inside a
 * row are given by the caller (they come from the library's layout descriptor):
 *   lat_off       latent page  [bs][576] e4m3   | NVFP4: [bs][288] packed e2m1
 *   lat_scale_off latent scale [bs] f32         | NVFP4: [bs][36] e4m3 block scales
 *   ikey_off      index keys   [bs][128] e4m3 in load order (put_fp8_keys) | MXFP4: [bs][64] packed e2m1
 *   ikey_scale_off key scale   [bs] f32         | MXFP4: [bs][4] e8m0
 * Token s of sequence b lives in pool row block_table[b*ld_bt + s/bs], slot s%bs.  Slots past a
 * sequence's length and rows no sequence uses are filled with 0xFF bytes (NaN in E4M3, E8M0 and
 * fp32), so a stray read shows up as a NaN.
 */
void synth_fill_pool(uint64_t seed, int ikey_fmt, int lat_fmt, int block_size, int64_t row_bytes,
                     int64_t lat_off, int64_t lat_scale_off, int64_t ikey_off,
                     int64_t ikey_scale_off, int64_t num_blocks, uint8_t* pool, int num_seqs,
                     const int32_t* block_table, int64_t ld_bt, const int64_t* seq_len,
                     const int64_t* seq_id, int64_t tok_stride, int64_t tok_offset) {
  const int bs = block_size;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < num_blocks; ++b) memset(pool + b * row_bytes, 0xFF, (size_t)row_bytes);

  int64_t total_blocks = 0;
  for (int q = 0; q < num_seqs; ++q) total_blocks += (seq_len[q] + bs - 1) / bs;
#pragma omp parallel
  {
    uint8_t lat[64 * MLA_DQK];
    uint8_t lat_nv_scale[64 * 36];
    float lat_scale[64];
    uint8_t key[64 * IDX_DIM];
    float key_scale[64];
    uint8_t key_mx_scale[64 * 4];
#pragma omp for schedule(dynamic, 16)
    for (int64_t gb = 0; gb < total_blocks; ++gb) {
      int q = 0;
      int64_t acc = 0;
      for (; q < num_seqs; ++q) {
        int64_t nb = (seq_len[q] + bs - 1) / bs;
        if (gb < acc + nb) break;
        acc += nb;
      }
      int64_t blk = gb - acc;
      int64_t tok0 = blk * bs;
      int64_t ntok = seq_len[q] - tok0;
      if (ntok > bs) ntok = bs;
      int64_t phys = block_table[q * ld_bt + blk];
      uint8_t* row = pool + phys * row_bytes;
      int64_t sid = seq_id ? seq_id[q] : q;
      if (tok_stride != 1 || tok_offset != 0) {
        /* a token-interleaved shard: pool token t is generator token t * stride + offset */
        for (int64_t i = 0; i < ntok; ++i) {
          const int64_t g = (tok0 + i) * tok_stride + tok_offset;
          if (lat_fmt == 0)
            synth_latent_fp8(seed, sid, g, 1, lat + i * MLA_DQK, lat_scale + i);
          else
            synth_latent_nvfp4(seed, sid, g, 1, lat + i * 288, lat_nv_scale + i * 36);
          if (ikey_fmt == 0)
            synth_ikey_fp8(seed, sid, g, 1, key + i * IDX_DIM, key_scale + i);
          else
            synth_ikey_mxfp4(seed, sid, g, 1, key + i * 64, key_mx_scale + i * 4);
        }
        if (lat_fmt == 0) {
          memcpy(row + lat_off, lat, (size_t)(ntok * MLA_DQK));
          memcpy(row + lat_scale_off, lat_scale, (size_t)(ntok * 4));
        } else {
          memcpy(row + lat_off, lat, (size_t)(ntok * 288));
          memcpy(row + lat_scale_off, lat_nv_scale, (size_t)(ntok * 36));
        }
        if (ikey_fmt == 0) {
          put_fp8_keys(row + ikey_off, key, ntok);
          memcpy(row + ikey_scale_off, key_scale, (size_t)(ntok * 4));
        } else {
          memcpy(row + ikey_off, key, (size_t)(ntok * 64));
          memcpy(row + ikey_scale_off, key_mx_scale, (size_t)(ntok * 4));
        }
        continue;
      }
      if (lat_fmt == 0) {
        synth_latent_fp8(seed, sid, tok0, ntok, lat, lat_scale);
        memcpy(row + lat_off, lat, (size_t)(ntok * MLA_DQK));
        memcpy(row + lat_scale_off, lat_scale, (size_t)(ntok * 4));
      } else {
        synth_latent_nvfp4(seed, sid, tok0, ntok, lat, lat_nv_scale);
        memcpy(row + lat_off, lat, (size_t)(ntok * 288));
        memcpy(row + lat_scale_off, lat_nv_scale, (size_t)(ntok * 36));
      }
      if (ikey_fmt == 0) {
        synth_ikey_fp8(seed, sid, tok0, ntok, key, key_scale);
        put_fp8_keys(row + ikey_off, key, ntok);
        memcpy(row + ikey_scale_off, key_scale, (size_t)(ntok * 4));
      } else {
        synth_ikey_mxfp4(seed, sid, tok0, ntok, key, key_mx_scale);
        memcpy(row + ikey_off, key, (size_t)(ntok * 64));
        memcpy(row + ikey_scale_off, key_mx_scale, (size_t)(ntok * 4));
      }
    }
  }
}
