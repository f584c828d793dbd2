// The step before the DSA path ("vLLM Delivers Day-0 Support for Kimi K3.1 Pro", §Low-latency
// decode: a fused DSA decode path): the indexer query is quantised to FP8 with each head's scale
// folded into its head weight, and each new token's index key and latent are quantised into their
// row of the paged pool (§A KV cache for three kinds of state gives the formats).
//
// Both kernels are HBM-light (a few hundred bytes per token or head) and run one wave per token or
// per head.  Every quantiser is round-to-nearest, ties to the even code, saturating at the
// format's largest finite value, with the same fp32 operations (amax, one correctly rounded
// division by the scale) a CPU writes down from the format definitions, so the codes are exact
// functions of the bf16 inputs.  Inputs are finite (NaN and infinity are outside the domain).
#include "dsa_kernels.h"

namespace dsa {
namespace {

// |x| -> E4M3 code, sign from x.  Normals: round the fp32 mantissa to 3 bits (half to even) and
// rebias the exponent 127 -> 7; below 2^-6 the grid is m * 2^-9 (m = 8 is the smallest normal).
__device__ __forceinline__ uint32_t enc_e4m3(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7FFFFFFFu;
  uint32_t mag;
  if (a >= 0x43E00000u) {            // |x| >= 448: the largest finite code
    mag = 0x7Eu;
  } else if (a < 0x3C800000u) {      // |x| < 2^-6
    mag = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    mag = (r >> 20) - (120u << 3);
  }
  return sign | mag;
}

__device__ __forceinline__ float dec_e4m3(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float v = e ? __builtin_amdgcn_ldexpf(1.0f + 0.125f * (float)m, (int)e - 7)
                    : (float)m * 0.001953125f;
  return (c & 0x80u) ? -v : v;
}

// |x| -> E2M1 nibble {0, .5, 1, 1.5, 2, 3, 4, 6}, sign from x.  Each binade is a uniform grid, so
// rint (half to even) on the scaled value lands on the even code at every midpoint.
__device__ __forceinline__ uint32_t enc_e2m1(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 8u;
  const float a = fabsf(x);
  uint32_t m;
  if (a < 2.0f)
    m = (uint32_t)__builtin_rintf(a * 2.0f);     // codes 0..4 (4 is 2.0)
  else if (a < 4.0f)
    m = (uint32_t)__builtin_rintf(a) + 2u;       // 2, 3, 4 -> codes 4, 5, 6
  else
    m = a > 5.0f ? 7u : 6u;                      // 5 ties to 4 (code 6); above 6 saturates
  return sign | m;
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

template <int W>  // max over groups of W consecutive lanes
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float fp8_token_scale(float amax) {
  return amax > 0.0f ? amax / 448.0f : 1.0f;
}

struct CacheWriteArgs {
  uint8_t* base;
  int64_t row_bytes, lat_off, lat_scale_off, ikey_off, ikey_scale_off;
  int64_t tokens;          // num_blocks * 64
  const int64_t* slot;     // [n] physical rows
  const uint16_t* ikey;    // [n][128] bf16 or null
  const uint16_t* latent;  // [n][576] bf16 or null
  float tensor_scale;      // NVFP4 latent tensor scale
  int32_t n;
};

// Token t's index key into its row (one wave; lane l holds elements 2l, 2l+1).
template <int IKFMT>
__device__ __forceinline__ void write_index_key(const CacheWriteArgs& a, int t, int lane,
                                                uint8_t* row, int64_t s) {
  const uint32_t p = reinterpret_cast<const uint32_t*>(a.ikey + (size_t)t * DSA_INDEX_DIM)[lane];
  const float x0 = bf16_lo(p), x1 = bf16_hi(p);
  if (IKFMT == DSA_IKEY_FP8) {
    const float sc = fp8_token_scale(group_max<64>(fmaxf(fabsf(x0), fabsf(x1))));
    const uint32_t c = enc_e4m3(x0 / sc) | (enc_e4m3(x1 / sc) << 8);
    // the page's load order: byte b of slot s at 2048 (s / 16) + 1024 (b / 64) + 256 ((b / 16) % 4)
    // + 16 (s % 16) + b % 16; this lane's bytes are b = 2 lane, 2 lane + 1
    const int64_t at = 2048 * (s >> 4) + 1024 * (lane >> 5) + 256 * ((lane >> 3) & 3) +
                       16 * (s & 15) + 2 * (lane & 7);
    *reinterpret_cast<uint16_t*>(row + a.ikey_off + at) = (uint16_t)c;
    if (lane == 0) reinterpret_cast<float*>(row + a.ikey_scale_off)[s] = sc;
  } else {
    // OCP MX block of 32 = 16 lanes: E8M0 exponent floor(log2 amax) - 2 (E2M1's top exponent)
    const float amax = group_max<16>(fmaxf(fabsf(x0), fabsf(x1)));
    int e = 127;
    if (amax > 0.0f) e = min(max(__builtin_amdgcn_frexp_expf(amax) - 1 - 2 + 127, 0), 254);
    const float X = __builtin_amdgcn_ldexpf(1.0f, e - 127);
    const uint32_t c = enc_e2m1(x0 / X) | (enc_e2m1(x1 / X) << 4);
    (row + a.ikey_off + s * (DSA_INDEX_DIM / 2))[lane] = (uint8_t)c;
    if ((lane & 15) == 0) (row + a.ikey_scale_off + s * 4)[lane >> 4] = (uint8_t)e;
  }
}

// One wave per token.  Index key: lane l holds elements 2l, 2l+1.  Latent: 144 chunks of four
// elements; lane l holds chunks l, l + 64 and (lanes 0..15) l + 128, so an NVFP4 block of 16 is
// four consecutive lanes.
template <int IKFMT, int LFMT>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.n) return;
  const int64_t slot = a.slot[t];
  if (slot < 0 || slot >= a.tokens) return;  // padding or outside the pool: nothing written
  uint8_t* row = a.base + (slot >> 6) * a.row_bytes;
  const int64_t s = slot & 63;

  if (a.ikey) write_index_key<IKFMT>(a, t, lane, row, s);

  if (a.latent) {
    const uint2* src = reinterpret_cast<const uint2*>(a.latent + (size_t)t * DSA_MLA_DQK);
    uint2 v[3];
    float m[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int c = lane + 64 * j;
      v[j] = (c < 144) ? src[c] : make_uint2(0u, 0u);
      m[j] = fmaxf(fmaxf(fabsf(bf16_lo(v[j].x)), fabsf(bf16_hi(v[j].x))),
                   fmaxf(fabsf(bf16_lo(v[j].y)), fabsf(bf16_hi(v[j].y))));
    }
    if (LFMT == DSA_LATENT_FP8) {
      const float sc = fp8_token_scale(group_max<64>(fmaxf(fmaxf(m[0], m[1]), m[2])));
      uint32_t* dst = reinterpret_cast<uint32_t*>(row + a.lat_off + s * DSA_MLA_DQK);
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int c = lane + 64 * j;
        if (c < 144)
          dst[c] = enc_e4m3(bf16_lo(v[j].x) / sc) | (enc_e4m3(bf16_hi(v[j].x) / sc) << 8) |
                   (enc_e4m3(bf16_lo(v[j].y) / sc) << 16) | (enc_e4m3(bf16_hi(v[j].y) / sc) << 24);
      }
      if (lane == 0) reinterpret_cast<float*>(row + a.lat_scale_off)[s] = sc;
    } else {
      // NVFP4 block of 16 = 4 lanes: E4M3 block scale of (amax / 6) / tensor scale
      uint16_t* dst = reinterpret_cast<uint16_t*>(row + a.lat_off + s * (DSA_MLA_DQK / 2));
      uint8_t* bsd = row + a.lat_scale_off + s * (DSA_MLA_DQK / 16);
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int c = lane + 64 * j;
        const float amax = group_max<4>(m[j]);
        const uint32_t bs = enc_e4m3((amax / 6.0f) / a.tensor_scale);
        const float sd = dec_e4m3(bs) * a.tensor_scale;
        uint32_t code = 0;
        if (sd > 0.0f)
          code = enc_e2m1(bf16_lo(v[j].x) / sd) | (enc_e2m1(bf16_hi(v[j].x) / sd) << 4) |
                 (enc_e2m1(bf16_lo(v[j].y) / sd) << 8) | (enc_e2m1(bf16_hi(v[j].y) / sd) << 12);
        if (c < 144) {
          dst[c] = (uint16_t)code;
          if ((c & 3) == 0) bsd[c >> 2] = (uint8_t)bs;
        }
      }
    }
  }
}

// Query head h (one wave): 128 elements, two per lane.
__device__ __forceinline__ void quantize_query_head(const uint16_t* __restrict__ q, const float* w,
                                                    uint8_t* __restrict__ qo, float* wo, int h,
                                                    int lane) {
  const uint32_t p = reinterpret_cast<const uint32_t*>(q + (size_t)h * DSA_INDEX_DIM)[lane];
  const float x0 = bf16_lo(p), x1 = bf16_hi(p);
  const float sc = fp8_token_scale(group_max<64>(fmaxf(fabsf(x0), fabsf(x1))));
  reinterpret_cast<uint16_t*>(qo + (size_t)h * DSA_INDEX_DIM)[lane] =
      (uint16_t)(enc_e4m3(x0 / sc) | (enc_e4m3(x1 / sc) << 8));
  const float wh = w[h];
  if (lane == 0) wo[h] = wh * sc;
}

__global__ __launch_bounds__(256) void quantize_query_kernel(const uint16_t* __restrict__ q,
                                                             const float* w, uint8_t* __restrict__ qo,
                                                             float* wo, int32_t heads_total) {
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (h >= heads_total) return;
  quantize_query_head(q, w, qo, wo, h, threadIdx.x & 63);
}

// The indexer front in one launch: workgroups [0, key_blocks) write the new tokens' index keys
// (four tokens each), the rest quantise the query heads (four heads each).  The two halves touch
// disjoint memory, so the split is only a partition of the grid.
template <int IKFMT>
__global__ __launch_bounds__(256) void indexer_front_kernel(CacheWriteArgs a, int32_t key_blocks,
                                                            const uint16_t* __restrict__ q,
                                                            const float* w, uint8_t* __restrict__ qo,
                                                            float* wo, int32_t heads_total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if ((int)blockIdx.x < key_blocks) {
    const int t = blockIdx.x * 4 + wave;
    if (t >= a.n) return;
    const int64_t slot = a.slot[t];
    if (slot < 0 || slot >= a.tokens) return;
    write_index_key<IKFMT>(a, t, lane, a.base + (slot >> 6) * a.row_bytes, slot & 63);
  } else {
    const int h = (blockIdx.x - key_blocks) * 4 + wave;
    if (h >= heads_total) return;
    quantize_query_head(q, w, qo, wo, h, lane);
  }
}

}  // namespace

hipError_t launch_cache_write(const PoolView& pool, uint8_t* base, int ikey_fmt, int lat_fmt,
                              float tensor_scale, int32_t n, const int64_t* slot,
                              const uint16_t* ikey, const uint16_t* latent, hipStream_t st) {
  CacheWriteArgs a;
  a.base = base;
  a.row_bytes = pool.row_bytes;
  a.lat_off = pool.lat_off;
  a.lat_scale_off = pool.lat_scale_off;
  a.ikey_off = pool.ikey_off;
  a.ikey_scale_off = pool.ikey_scale_off;
  a.tokens = pool.tokens;
  a.slot = slot;
  a.ikey = ikey;
  a.latent = latent;
  a.tensor_scale = tensor_scale;
  a.n = n;
  const dim3 grid((n + 3) / 4), block(256);
  if (ikey_fmt == DSA_IKEY_FP8 && lat_fmt == DSA_LATENT_FP8)
    cache_write_kernel<DSA_IKEY_FP8, DSA_LATENT_FP8><<<grid, block, 0, st>>>(a);
  else if (ikey_fmt == DSA_IKEY_FP8)
    cache_write_kernel<DSA_IKEY_FP8, DSA_LATENT_NVFP4><<<grid, block, 0, st>>>(a);
  else if (lat_fmt == DSA_LATENT_FP8)
    cache_write_kernel<DSA_IKEY_MXFP4, DSA_LATENT_FP8><<<grid, block, 0, st>>>(a);
  else
    cache_write_kernel<DSA_IKEY_MXFP4, DSA_LATENT_NVFP4><<<grid, block, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_quantize_query(int32_t num_rows, const uint16_t* q, const float* w, uint8_t* qo,
                                 float* wo, hipStream_t st) {
  const int32_t heads = num_rows * DSA_INDEX_HEADS;
  quantize_query_kernel<<<dim3((heads + 3) / 4), dim3(256), 0, st>>>(q, w, qo, wo, heads);
  return hipGetLastError();
}

hipError_t launch_indexer_front(const PoolView& pool, uint8_t* base, int ikey_fmt, int32_t n,
                                const int64_t* slot, const uint16_t* ikey, int32_t num_rows,
                                const uint16_t* q, const float* w, uint8_t* qo, float* wo,
                                hipStream_t st) {
  CacheWriteArgs a{};
  a.base = base;
  a.row_bytes = pool.row_bytes;
  a.ikey_off = pool.ikey_off;
  a.ikey_scale_off = pool.ikey_scale_off;
  a.tokens = pool.tokens;
  a.slot = slot;
  a.ikey = ikey;
  a.n = n;
  const int32_t key_blocks = (n + 3) / 4;
  const int32_t heads = num_rows * DSA_INDEX_HEADS;
  const dim3 grid(key_blocks + (heads + 3) / 4), block(256);
  if (ikey_fmt == DSA_IKEY_FP8)
    indexer_front_kernel<DSA_IKEY_FP8><<<grid, block, 0, st>>>(a, key_blocks, q, w, qo, wo, heads);
  else
    indexer_front_kernel<DSA_IKEY_MXFP4><<<grid, block, 0, st>>>(a, key_blocks, q, w, qo, wo,
                                                                  heads);
  return hipGetLastError();
}

}  // namespace dsa
