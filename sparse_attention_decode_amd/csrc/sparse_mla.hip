// Exact MLA attention over the selected latents (decode with split-K, and prefill).
//
// Source: "vLLM Delivers Day-0 Support for Kimi K3.1 Pro" — §Sparse Attention in K3.1 Pro (MLA
// runs exactly over only the selected tokens; every query head attends over those tokens'
// latents); §Prefill: shard the attention by token (the latent is shared by all heads, so one
// workgroup serves all 96 heads of a row and reads each latent once); §AMD / Prefill (one
// workgroup per query row across the heads, reading the selected tokens straight from the FP8
// cache); §A KV cache for three kinds of state (FP8 or NVFP4 latents).
//
// For row r, head h and selected tokens j (idx >= 0):
//   c_j = latent (FP8 code * token scale, or E2M1 * E4M3 block scale * tensor scale)
//   logit_j = softmax_scale * q[r,h] . c_j      (576 dims; no positional encoding)
//   out[r,h] = sum_j softmax(logit)_j * c_j[0:512]
//
// Design (gfx950): a workgroup of 6 waves takes one row (or one split of its selected set), wave w
// owning heads [16w, 16w+16).  Tiles of 32 selected tokens are gathered from the paged pool, the
// codes converted exactly and staged twice in LDS: token-major bf16 (A operand of S^T = C Q^T,
// against the bf16 query) and dim-major fp16 (A operand of O^T = V^T P^T; the probabilities go
// in as fp16, whose 11-bit significand keeps their rounding well inside the output tolerance).  Per-token scales stay out of the MFMA
// operands: they multiply the logits and the probabilities.  With S^T and O^T the softmax
// statistics of a head live in the same lane as that head's output column, and the probabilities
// of S^T are already in B-operand position for PV (the K order of the PV contraction is permuted
// to match), so no register shuffles or LDS round trips are needed between the two products.
// Softmax is online (running max and sum per head, in base 2).
#include "dsa_kernels.h"

namespace dsa {

namespace {

constexpr int kWavesM = DSA_MLA_HEADS / 16;  // 6
constexpr int kThreadsM = kWavesM * kWave;    // 384
constexpr int kTile = 32;                     // selected tokens per tile
constexpr int kKSteps = DSA_MLA_DQK / 32;     // 18
constexpr int kCtStride = DSA_MLA_DQK + 8;    // bf16 elements per token row (padded)
constexpr int kVtStride = kTile + 4;          // bf16 elements per dim row (padded)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct MlaShared {
  uint16_t ct[kTile * kCtStride];          // [token][dim] bf16
  uint16_t vt[DSA_MLA_DV * kVtStride];     // [dim][token] fp16
  float tscale[kTile];                     // per-token scale (0 = no token)
  int32_t valid[kTile];
};

// Store 16 latent values (exact fp32) of token t, dims d0..d0+15: bf16 into the token-major tile
// (QK^T operand) and, for value dims, fp16 into the dim-major tile (PV operand).  Every FP8 and
// NVFP4 latent value is exactly representable in both formats.
__device__ __forceinline__ void store_dims(MlaShared& sh, int t, int d0, const float* v) {
  uint32_t* crow = reinterpret_cast<uint32_t*>(&sh.ct[t * kCtStride + d0]);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    crow[i] = (__float_as_uint(v[2 * i]) >> 16) | (__float_as_uint(v[2 * i + 1]) & 0xFFFF0000u);
  if (d0 < DSA_MLA_DV) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sh.vt[(d0 + i) * kVtStride + t] = (uint16_t)f16_bits(v[i]);
  }
}

// Gather one tile of selected latents into LDS.  FP8: 36 pieces of 16 dims per token.  NVFP4:
// 36 pieces of 16 dims (8 packed bytes + one E4M3 block scale) per token.
template <int LFMT>
__device__ void stage_tile(MlaShared& sh, const MlaArgs& a, const int32_t* bt, const int32_t* idx,
                           int j, int jend, int nvis) {
  const int tid = threadIdx.x;
  constexpr int kPieces = kTile * (DSA_MLA_DQK / 16);  // 1152
  for (int q = tid; q < kPieces; q += kThreadsM) {
    const int t = q / (DSA_MLA_DQK / 16), p = q % (DSA_MLA_DQK / 16);
    const int jj = j + t;
    const int s = jj < jend ? idx[jj] : -1;
    float vals[16];
    if (s >= 0 && s < nvis) {
      const uint8_t* row = a.pool.base + (int64_t)bt[s / kBlock] * a.pool.row_bytes;
      const int slot = s % kBlock;
      if (LFMT == DSA_LATENT_FP8) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + a.pool.lat_off +
                                                        slot * DSA_MLA_DQK + 16 * p);
        fp8x4_to_f32x4(v.x, vals);
        fp8x4_to_f32x4(v.y, vals + 4);
        fp8x4_to_f32x4(v.z, vals + 8);
        fp8x4_to_f32x4(v.w, vals + 12);
        if (p == 0) {
          sh.tscale[t] = *reinterpret_cast<const float*>(row + a.pool.lat_scale_off + slot * 4);
          sh.valid[t] = 1;
        }
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(row + a.pool.lat_off +
                                                        slot * (DSA_MLA_DQK / 2) + 8 * p);
        const float bs = fp8_to_f32(row[a.pool.lat_scale_off + slot * (DSA_MLA_DQK / 16) + p]);
        fp4x8_scaled_to_f32x8(v.x, bs, vals);
        fp4x8_scaled_to_f32x8(v.y, bs, vals + 8);
        if (p == 0) {
          sh.tscale[t] = a.tensor_scale;
          sh.valid[t] = 1;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) vals[i] = 0.f;
      if (p == 0) {
        sh.tscale[t] = 0.f;
        sh.valid[t] = 0;
      }
    }
    store_dims(sh, t, 16 * p, vals);
  }
}

template <int LFMT>
__global__ __launch_bounds__(kThreadsM) void sparse_mla_kernel(MlaArgs a) {
  __shared__ MlaShared sh;
  const int row = blockIdx.x, split = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int head = 16 * wave + c;  // this lane's head in S^T / O^T columns

  // sequence of the row
  int seq;
  {
    int lo = 0, hi = a.batch.num_seqs - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (a.batch.seq_row_start[mid] <= row) lo = mid; else hi = mid - 1;
    }
    seq = lo;
  }
  const int32_t* bt = a.batch.block_table + (int64_t)seq * a.batch.ld_bt;
  const int32_t* idx = a.idx + (int64_t)row * a.k;
  const int nvis = a.batch.row_pos[row] + 1;  // selected indices outside [0, nvis) are ignored
  const int j0 = split * a.tokens_per_split;
  const int j1 = min(a.k, j0 + a.tokens_per_split);

  // Q^T fragments (B operand): lane holds head 16w+c, dims 32ks + 8g .. + 8
  v8bf qf[kKSteps];
  {
    const uint16_t* qr = a.q + ((int64_t)row * DSA_MLA_HEADS + head) * DSA_MLA_DQK;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const uint4 v = *reinterpret_cast<const uint4*>(qr + 32 * ks + 8 * g);
      qf[ks] = __builtin_bit_cast(v8bf, v);
    }
  }
  v4f o[DSA_MLA_DV / 16];
#pragma unroll
  for (int mt = 0; mt < DSA_MLA_DV / 16; ++mt) o[mt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float qk_scale = a.softmax_scale * kLog2e;

  for (int j = j0; j < j1; j += kTile) {
    __syncthreads();
    stage_tile<LFMT>(sh, a, bt, idx, j, j1, nvis);
    __syncthreads();

    // S^T (tokens x heads) for the two 16-token halves of the tile
    v4f st[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* arow = &sh.ct[(16 * h2 + c) * kCtStride + 8 * g];
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const uint4 v = *reinterpret_cast<const uint4*>(arow + 32 * ks);
        acc = mfma_bf16(__builtin_bit_cast(v8bf, v), qf[ks], acc);
      }
      st[h2] = acc;
    }
    // logits in base 2; lane holds tokens 16*h2 + 4g + i for its head
    float x[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * h2 + 4 * g + i;
        const float v = sh.valid[t] ? st[h2][i] * sh.tscale[t] * qk_scale : -INFINITY;
        x[h2][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
    uint32_t pb[4];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * h2 + 4 * g + i;
        const float p = (x[h2][i] == -INFINITY) ? 0.f : exp2f(x[h2][i] - m_new);
        psum += p;
        pv[i] = p * sh.tscale[t];  // the token scale of c_j multiplies its value row
      }
      // fp16 pairs (round to nearest even): K slots 8g + 4*h2 + i  <->  token 16*h2 + 4g + i
#pragma unroll
      for (int i = 0; i < 2; ++i) pb[2 * h2 + i] = f16_bits(pv[2 * i]) | (f16_bits(pv[2 * i + 1]) << 16);
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const v8h pfrag = __builtin_bit_cast(v8h, uint4{pb[0], pb[1], pb[2], pb[3]});

    // O^T (dims x heads) += V^T P^T; A operand lane: dim 16mt + c, tokens {4g..4g+3, 16+4g..}
#pragma unroll
    for (int mt = 0; mt < DSA_MLA_DV / 16; ++mt) {
      o[mt] *= alpha;
      const uint16_t* vrow = &sh.vt[(16 * mt + c) * kVtStride];
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 4 * g);
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * g);
      const v8h af = __builtin_bit_cast(v8h, uint4{lo.x, lo.y, hi.x, hi.y});
      o[mt] = mfma_f16(af, pfrag, o[mt]);
    }
  }

  // lane holds O^T[16mt + 4g + i][head]
  if (a.nsplit == 1) {
    const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
    uint16_t* orow = a.out + ((int64_t)row * DSA_MLA_HEADS + head) * DSA_MLA_DV;
#pragma unroll
    for (int mt = 0; mt < DSA_MLA_DV / 16; ++mt) {
      uint32_t b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t u = __float_as_uint(o[mt][i] * inv);
        b[i] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
      }
      *reinterpret_cast<uint2*>(orow + 16 * mt + 4 * g) = uint2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
    }
    if (a.lse && g == 0)
      a.lse[(int64_t)row * DSA_MLA_HEADS + head] =
          (l_run > 0.f) ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const int64_t slot = ((int64_t)row * a.nsplit + split) * DSA_MLA_HEADS + head;
    float* po = a.part_o + slot * DSA_MLA_DV;
#pragma unroll
    for (int mt = 0; mt < DSA_MLA_DV / 16; ++mt)
      *reinterpret_cast<float4*>(po + 16 * mt + 4 * g) =
          float4{o[mt][0], o[mt][1], o[mt][2], o[mt][3]};
    if (g == 0) {
      a.part_ml[2 * slot] = m_run;
      a.part_ml[2 * slot + 1] = l_run;
    }
  }
}

// Merge the splits of each row by log-sum-exp.  grid (rows, 96 heads / 2); 256 threads: two heads,
// 128 threads x 4 dims each.
__global__ __launch_bounds__(256) void mla_combine_kernel(MlaArgs a) {
  const int row = blockIdx.x;
  const int head = 2 * blockIdx.y + (threadIdx.x >> 7);
  const int d = 4 * (threadIdx.x & 127);
  const int64_t base = (int64_t)row * a.nsplit * DSA_MLA_HEADS + head;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_ml[2 * (base + (int64_t)s * DSA_MLA_HEADS)]);
  float L = 0.f;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    for (int s = 0; s < a.nsplit; ++s) {
      const int64_t slot = base + (int64_t)s * DSA_MLA_HEADS;
      const float m = a.part_ml[2 * slot], l = a.part_ml[2 * slot + 1];
      if (m == -INFINITY) continue;
      const float wgt = exp2f(m - M);
      L += wgt * l;
      const float4 v = *reinterpret_cast<const float4*>(a.part_o + slot * DSA_MLA_DV + d);
      acc.x += wgt * v.x;
      acc.y += wgt * v.y;
      acc.z += wgt * v.z;
      acc.w += wgt * v.w;
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  const float f[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  uint32_t b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t u = __float_as_uint(f[i]);
    b[i] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  }
  *reinterpret_cast<uint2*>(a.out + ((int64_t)row * DSA_MLA_HEADS + head) * DSA_MLA_DV + d) =
      uint2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
  if (a.lse && d == 0)
    a.lse[(int64_t)row * DSA_MLA_HEADS + head] = (L > 0.f) ? (M + log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

int mla_num_splits(int32_t num_rows, int32_t k) {
  const int tiles = (k + kTile - 1) / kTile;
  int want = (256 + num_rows - 1) / (num_rows > 0 ? num_rows : 1);
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  return want;
}

size_t mla_workspace_bytes(int32_t num_rows, int32_t k) {
  const int ns = mla_num_splits(num_rows, k);
  if (ns <= 1) return 0;
  return (size_t)num_rows * ns * DSA_MLA_HEADS * (DSA_MLA_DV + 2) * sizeof(float);
}

hipError_t launch_sparse_mla(const MlaArgs& a0, int lat_fmt, hipStream_t s) {
  MlaArgs a = a0;
  if (a.batch.num_rows <= 0) return hipSuccess;
  dim3 grid((unsigned)a.batch.num_rows, (unsigned)a.nsplit);
  if (lat_fmt == DSA_LATENT_FP8)
    hipLaunchKernelGGL(sparse_mla_kernel<DSA_LATENT_FP8>, grid, dim3(kThreadsM), 0, s, a);
  else
    hipLaunchKernelGGL(sparse_mla_kernel<DSA_LATENT_NVFP4>, grid, dim3(kThreadsM), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)a.batch.num_rows, DSA_MLA_HEADS / 2),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
