// Exact MLA attention over the selected latents (decode with split-K, and prefill).
//
// Source: "vLLM Delivers Day-0 Support for Kimi K3.1 Pro" — §Sparse Attention in K3.1 Pro (MLA
// is computed exactly, but only over the chosen tokens, and all heads use the same chosen
// tokens' latents); §Prefill: shard the attention by token (the latent is shared by all heads, so one
// workgroup serves all 96 heads of a row and reads each latent once); §AMD / Prefill (one
// workgroup per query row across the heads, reading the selected tokens straight from the FP8
// cache); §A KV cache for three kinds of state (FP8 or NVFP4 latents).
//
// For row r, head h and selected tokens j (idx >= 0):
//   c_j = latent (FP8 code * token scale, or E2M1 * E4M3 block scale * tensor scale)
//   logit_j = softmax_scale * q[r,h] . c_j      (576 dims; no positional encoding)
//   out[r,h] = sum_j softmax(logit)_j * c_j[0:512]
//
// Design (gfx950).  A workgroup of 12 waves takes one row (or one split of its selected set).
// Waves 2h and 2h+1 own heads [16h, 16h+16); wave 2h+d computes the half d of the QK contraction
// (288 of the 576 dims) and the half d of the output dims (256 of 512), so a wave holds 36 query
// registers and 64 accumulator registers, and three waves share each SIMD.  Tiles of 32 selected
// tokens are gathered from the paged pool straight into LDS with direct global->LDS loads (no
// registers held in flight), kStages - 1 tiles ahead of the tile being processed.  Each stage is
// its own LDS variable and barriers wait on LDS traffic only, so reading a tile never waits for
// the gathers of later tiles.  The pool rows to gather are handed over in a lane-distributed
// register (one batch of 21 tiles per register), read with readlane: no memory round trip sits
// between a tile and its gathers.
//   QK^T: S^T[tokens x heads] = C Q^T on bf16 MFMA.  The query stays in registers (B operand);
//         the latent tile is the A operand.  FP8 latents are read raw from LDS and converted to
//         bf16 in registers (exact); NVFP4 latents are decoded once per tile into a bf16 tile.
//         The two partial S^T of a wave pair are added through LDS (both waves then hold the
//         same bits, so their softmax statistics agree exactly).
//   PV:   O^T[dims x heads] = V^T P^T on fp16 MFMA.  V^T comes from a dim-major fp16 copy of the
//         value dims, converted once per tile for all head groups; P^T is S^T's softmax, already
//         in B-operand position: the K order of this contraction is permuted so that lane group g
//         holds tokens {4g..4g+3, 16+4g..16+4g+3}, and the dim-major tile stores tokens in that
//         order.
// Per-token scales stay out of the MFMA operands (they multiply the logits and the
// probabilities), so every operand is an exact conversion of the stored codes.  fp16 for P keeps
// its rounding well inside the output tolerance.  Softmax is online, in base 2.  With S^T and
// O^T a head's softmax statistics live in the same lane as that head's output column.
// LDS rows are padded so that the MFMA operand reads are bank-conflict free.
#include "dsa_kernels.h"

namespace dsa {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWavesM = 2 * DSA_MLA_HEADS / 16;  // 12: 6 head groups x 2 halves
constexpr int kThreadsM = kWavesM * kWave;        // 768
constexpr int kTile = 32;                         // selected tokens per tile
constexpr int kSteps = DSA_MLA_DQK / 32 / 2;      // 9 K steps of 32 dims per wave (half of 576)
constexpr int kDvHalf = DSA_MLA_DV / 2;           // 256 output dims per wave
#ifndef DSA_MLA_STAGES
#define DSA_MLA_STAGES 3
#endif
// Gather pipeline: while tile j is processed, tiles j+1 .. j+kAhead are in flight.
constexpr int kStages = DSA_MLA_STAGES;
constexpr int kAhead = kStages - 1;
static_assert(kStages >= 3 && kStages <= 6, "stage variables raw0..raw5");
constexpr int kRowsPerWave = (kTile + kWavesM - 1) / kWavesM;  // 3 (rows >= 32 are dummies)
constexpr int kSlots = kRowsPerWave * kWavesM;                  // 36 LDS rows per stage
// Pool rows of a wave's gathers, one register per batch of tiles: lane 3T + r holds the row of
// tile T's row r of the batch (kBatchTiles tiles per register).
constexpr int kBatchTiles = kWave / kRowsPerWave;  // 21
// Every wave issues exactly this many gathers per tile (data + scale per row, dummies included),
// so waiting for a tile is "all but the newest tile's gathers are done".
constexpr int kGathersPerWave = 2 * kRowsPerWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 4.f;  // base-2 headroom of the running max (probabilities <= 16)

// FP8 latents
constexpr int kRaw8 = 592;   // raw row bytes: 576 codes + pad (148 dwords: b128 reads conflict-free)
// NVFP4 latents
constexpr int kRaw4 = 336;   // raw row bytes: 288 packed + 36 block scales + pad
constexpr int kCt4 = 1168;   // bf16 token-major row bytes: 1152 + pad (292 dwords)
constexpr int kVt4 = 80;     // fp16 dim-major row bytes (both formats): 64 + pad (20 dwords)

template <int LFMT>
struct Geo {
  static constexpr bool kFp8 = LFMT == DSA_LATENT_FP8;
  static constexpr int kRaw = kFp8 ? kRaw8 : kRaw4;
  static constexpr int kVt = kVt4;
  static constexpr int kCtBytes = kFp8 ? 16 : kTile * kCt4;  // decoded tile (NVFP4 only)
};

// One pipeline stage: where a gathered tile lands.  Each stage's buffers are separate
// __shared__ variables, so the compiler can tell the reads of one stage from the gathers still
// landing in the others (one shared array would make it wait for every gather before any read).
struct Stage {
  uint8_t* raw;    // [kSlots][kRaw] latent rows as stored (rows >= kTile: dummy gathers)
  float* tsc;      // [kSlots] FP8 token scales
  int32_t* valid;  // [kTile] slot holds a selected, visible token
};

// The value of x, opaque to the optimiser: lane-dependent addresses derived from it inside the tile
// loop are recomputed each tile (a few VALU) instead of being hoisted out of the loop, where they
// would hold registers for the whole loop and push the kernel into spills.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Direct global->LDS copies.  Lane l copies `bytes` bytes from src + voff (src wave-uniform) to LDS
// address lds + bytes * l.  Issued through inline assembly, so the compiler does not track them:
// the tile loop waits for them explicitly (s_waitcnt vmcnt by count, then an LDS barrier).  Left
// to the compiler, its LDS-DMA tracking made some LDS writes wait for every copy in flight, which
// undid the gather pipeline.  Untracked copies only ever make the compiler's own waits stricter.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}
// The gathers are non-temporal: each selected latent is read once per step.
// m0 carries the LDS address of each copy.  The compiler does not otherwise use m0 in these
// kernels (their ISA has no m0 access but these writes), so setting it here disturbs nothing; it
// is listed as clobbered, which the compiler notes it cannot promise to honour for m0.
#define DSA_GATHER_POLICY " nt"
__device__ __forceinline__ void lds_copy16(const uint8_t* src, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" DSA_GATHER_POLICY
               :: "v"(voff), "s"(src), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(const uint8_t* src, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" DSA_GATHER_POLICY
               :: "v"(voff), "s"(src), "s"(lds) : "memory", "m0");
}

// Position of tile token t (quad q = t / 4, u = t % 4) in a dim-major row: the K slot that holds
// it in the PV contraction.
__device__ __forceinline__ int vt_pos(int t) {
  const int q = t >> 2, u = t & 3;
  return 8 * (q & 3) + 4 * (q >> 2) + u;
}

// Issue the direct global->LDS gathers of tile j (selected slots [j, min(j+32, jend))) into stage
// st.  Wave w gathers tile rows w, w+12, w+24, whose pool rows are lanes lb, lb+1, lb+2 of `pv`.
// Rows past the tile (slots 32..35 of the stage) and slots without a token gather a dummy row,
// so that every wave issues kGathersPerWave loads per tile: the wave's first real row of the
// tile again if it has one, else `ph_spread`, a pool row that depends on the workgroup and wave
// (never one row for everybody: thousands of requests to one address would queue on one memory
// channel).  Every gather lands in the stage's own LDS variable, and its pool row is
// wave-uniform (scalar base address, 32-bit lane offset).
template <int LFMT>
__device__ __forceinline__ void issue_tile(const Stage& st, int pv, int lb, int ph_spread,
                                           const MlaArgs& a, int j, int jend, int lane) {
  using G = Geo<LFMT>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ph_first = (j + wave < jend) ? __builtin_amdgcn_readlane(pv, lb) : -1;
  const int ph_dummy = ph_first >= 0 ? ph_first : ph_spread;
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int t = wave + kWavesM * r;  // < kSlots
    const int jj = j + t;
    const int ph = (t < kTile && jj < jend) ? __builtin_amdgcn_readlane(pv, lb + r) : -1;
    if (t < kTile && lane == 0) st.valid[t] = ph >= 0;
    const int src = __builtin_amdgcn_readfirstlane(ph >= 0 ? ph : ph_dummy);  // >= 0
    const uint8_t* row = a.pool.base + (int64_t)(src >> 6) * a.pool.row_bytes;
    const int slot = src & (kBlock - 1);
    uint8_t* dst = st.raw + t * G::kRaw;
    if constexpr (G::kFp8) {
      const uint8_t* lat = row + a.pool.lat_off + slot * DSA_MLA_DQK;
      const uint8_t* scl = row + a.pool.lat_scale_off + slot * 4;
      if (lane < DSA_MLA_DQK / 16) lds_copy16(lat, 16 * lane, lds_addr(dst));
      if (lane == 0) lds_copy4(scl, 0, lds_addr(st.tsc + t));
    } else {
      const uint8_t* lat = row + a.pool.lat_off + slot * (DSA_MLA_DQK / 2);
      const uint8_t* scl = row + a.pool.lat_scale_off + slot * (DSA_MLA_DQK / 16);
      if (lane < DSA_MLA_DQK / 32) lds_copy16(lat, 16 * lane, lds_addr(dst));
      if (lane < DSA_MLA_DQK / 64) lds_copy4(scl, 4 * lane, lds_addr(dst + DSA_MLA_DQK / 2));
    }
  }
}

// FP8: dim-major fp16 copy of the value dims of a stage, converted once per tile for all head
// groups (fp8 -> fp16 is exact).  A thread takes a block of 4 dims x 4 tokens: two conversions
// per token give its four values as two half-word pairs, and half-word permutes transpose them
// into four dim rows of 4 tokens.  Tokens that are not selected get zeros, so their (zero)
// probabilities never meet stale data.
__device__ __forceinline__ void build_fp8(const Stage& st, uint8_t* vt, int tid) {
  for (int blk = tid; blk < (DSA_MLA_DV / 4) * (kTile / 4); blk += kThreadsM) {
    const int tq = blk & 7, db = blk >> 3;  // token quad, 4-dim block
    // the four tokens' flags in one read; every row read unconditionally, then selected
    const int4 ok = *reinterpret_cast<const int4*>(st.valid + 4 * tq);
    const int okv[4] = {ok.x, ok.y, ok.z, ok.w};
    uint32_t lo[4], hi[4];  // token u: fp16 of dims (4db, 4db+1) and of (4db+2, 4db+3)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t r = *reinterpret_cast<const uint32_t*>(st.raw + (4 * tq + u) * kRaw8 + 4 * db);
      r = okv[u] ? r : 0u;
      lo[u] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r, 1.0f, false));
      hi[u] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r, 1.0f, true));
    }
    // dim row 4db+i: tokens 0..3 of the quad, K slots vt_pos(4 tq) .. +3
    uint8_t* row = vt + 4 * db * kVt4 + 2 * vt_pos(4 * tq);
    *reinterpret_cast<uint2*>(row) = uint2{__builtin_amdgcn_perm(lo[1], lo[0], 0x05040100u),
                                           __builtin_amdgcn_perm(lo[3], lo[2], 0x05040100u)};
    *reinterpret_cast<uint2*>(row + kVt4) = uint2{__builtin_amdgcn_perm(lo[1], lo[0], 0x07060302u),
                                                  __builtin_amdgcn_perm(lo[3], lo[2], 0x07060302u)};
    *reinterpret_cast<uint2*>(row + 2 * kVt4) = uint2{__builtin_amdgcn_perm(hi[1], hi[0], 0x05040100u),
                                                      __builtin_amdgcn_perm(hi[3], hi[2], 0x05040100u)};
    *reinterpret_cast<uint2*>(row + 3 * kVt4) = uint2{__builtin_amdgcn_perm(hi[1], hi[0], 0x07060302u),
                                                      __builtin_amdgcn_perm(hi[3], hi[2], 0x07060302u)};
  }
}

// NVFP4: decode a stage once into the bf16 token-major tile and the fp16 dim-major tile (E2M1 x
// E4M3 products are exact in both).
__device__ __forceinline__ void build_nvfp4(const Stage& st, uint8_t* ct, uint8_t* vt, int tid) {
  for (int it = tid; it < (DSA_MLA_DQK / 16) * kTile; it += kThreadsM) {
    const int t = it & 31, blk = it >> 5;  // token, 16-dim block
    float v[16];
    if (st.valid[t]) {
      const uint2 p = *reinterpret_cast<const uint2*>(st.raw + t * kRaw4 + 8 * blk);
      const float s = fp8_to_f32(st.raw[t * kRaw4 + DSA_MLA_DQK / 2 + blk]);
      fp4x8_scaled_to_f32x8(p.x, s, v);
      fp4x8_scaled_to_f32x8(p.y, s, v + 8);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.f;
    }
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = (__float_as_uint(v[2 * i]) >> 16) | (__float_as_uint(v[2 * i + 1]) & 0xFFFF0000u);
    uint4* crow = reinterpret_cast<uint4*>(ct + t * kCt4 + 32 * blk);
    crow[0] = uint4{w[0], w[1], w[2], w[3]};
    crow[1] = uint4{w[4], w[5], w[6], w[7]};
    if (16 * blk < DSA_MLA_DV) {
      const int pos = vt_pos(t);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        *reinterpret_cast<uint16_t*>(vt + (16 * blk + i) * kVt4 + 2 * pos) = (uint16_t)f16_bits(v[i]);
    }
  }
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v8bf fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const uint4 r = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
  return __builtin_bit_cast(v8bf, r);
}

// K step i of contraction half dh: lane group g holds dims [288dh + 32i + 8g, +8).  The nine steps
// of a half cover its 288 dims once; A and B operands use the same dims.
constexpr int kHalfDims = DSA_MLA_DQK / 2;

// Latent tile as the A operand of QK^T: token t, dims [d, d+8) (d = 288dh + 32i + 8g).
template <int LFMT>
__device__ __forceinline__ v8bf qk_operand(const Stage& st, const uint8_t* ct, int t, int d) {
  if constexpr (LFMT == DSA_LATENT_FP8) {
    const uint2 v = *reinterpret_cast<const uint2*>(st.raw + t * kRaw8 + d);
    return fp8x8_to_bf16(v.x, v.y);
  } else {
    return __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(ct + t * kCt4 + 2 * d));
  }
}

// Dim-major fp16 value tile as the A operand of PV: dim row d, lane group g (8 K slots).
__device__ __forceinline__ v8h pv_operand(const uint8_t* vt, int d, int g) {
  return __builtin_bit_cast(v8h, *reinterpret_cast<const uint4*>(vt + d * kVt4 + 16 * g));
}

// PHYS: the select's physical pool rows are given (else selected indices + block table).
template <int LFMT, bool PHYS>
__global__ __launch_bounds__(kThreadsM) void sparse_mla_kernel(MlaArgs a) {
  using G = Geo<LFMT>;
  constexpr int kRawBytes = kSlots * G::kRaw;
  __shared__ __attribute__((aligned(16))) uint8_t raw0[kRawBytes], raw1[kRawBytes], raw2[kRawBytes];
  __shared__ __attribute__((aligned(16))) uint8_t raw3[kStages > 3 ? kRawBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t raw4[kStages > 4 ? kRawBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t raw5[kStages > 5 ? kRawBytes : 16];
  __shared__ __attribute__((aligned(16))) float tsc0[kSlots], tsc1[kSlots], tsc2[kSlots],
      tsc3[kSlots], tsc4[kSlots], tsc5[kSlots];
  __shared__ __attribute__((aligned(16))) int32_t valid0[kTile], valid1[kTile], valid2[kTile],
      valid3[kTile], valid4[kTile],
      valid5[kTile];
  __shared__ __attribute__((aligned(16))) uint8_t vt[DSA_MLA_DV * G::kVt];
  __shared__ __attribute__((aligned(16))) uint8_t ct[G::kCtBytes];
  __shared__ __attribute__((aligned(16))) v4f sx[kWavesM][2][kWave];  // partial S^T exchange
  __shared__ float amx[kWavesM][16];
  const Stage stages[6] = {{raw0, tsc0, valid0}, {raw1, tsc1, valid1}, {raw2, tsc2, valid2},
                           {raw3, tsc3, valid3}, {raw4, tsc4, valid4}, {raw5, tsc5, valid5}};

  const int row = blockIdx.x, split = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps wave math scalar
  const int g = lane >> 4, c = lane & 15;
  const int dh = wave & 1;                // half of the QK dims and of the output dims
  const int head = 16 * (wave >> 1) + c;  // this lane's head in S^T / O^T columns

  const int32_t* idx = a.idx + (int64_t)row * a.k;
  const int32_t* prow = a.phys + (int64_t)row * a.k;
  const int nvis = a.batch.row_pos[row] + 1;  // selected indices outside [0, nvis) are ignored
  // The split's slots of the selection: fixed ranges of tokens_per_split, or, when the row's
  // count of selected entries is given, that many entries spread evenly over the splits.
  int nsel = a.k, per = a.tokens_per_split;
  if (a.count) {
    nsel = min(a.k, max(0, a.count[row]));
    per = max(kTile, ((nsel + a.nsplit - 1) / a.nsplit + kTile - 1) / kTile * kTile);
  }
  const int j0 = split * per;
  const int j1 = max(j0, min(nsel, j0 + per));
  const int32_t* bt = nullptr;
  if (!PHYS) {  // sequence of the row, by one ballot per 64 sequences
    int seq = 0;
    for (int b0 = 0; b0 < a.batch.num_seqs; b0 += kWave) {
      const int b = b0 + lane;
      const bool ended = b < a.batch.num_seqs && a.batch.seq_row_start[b + 1] <= row;
      seq += __popcll(__ballot(ended));
    }
    bt = a.batch.block_table + (int64_t)seq * a.batch.ld_bt;
  }

  // Pool rows of this wave's gathers for tiles [tb, tb + kBatchTiles) of the split (lane 3T + r:
  // tile tb + T, row wave + 12r), or -1 where there is no visible selected token.
  const int ntiles = (j1 - j0 + kTile - 1) / kTile;
  // dummy gather row of this wave when a tile has no real row for it (see issue_tile)
  const int ph_spread = __builtin_amdgcn_readfirstlane(
      (int)(((int64_t)blockIdx.x * 7919 + (int64_t)blockIdx.y * 131 + wave * 17) % a.pool.tokens));
  auto load_batch = [&](int tb) {
    const int T = lane / kRowsPerWave, r = lane % kRowsPerWave;
    const int t = wave + kWavesM * r;
    const int jj = j0 + kTile * (tb + T) + t;
    const bool in = T < kBatchTiles && t < kTile && jj < j1;
    int ph = -1;
    if (PHYS) {
      // unconditional (entry 0 stands in for lanes without a slot), so that the query loads
      // behind it are in flight at the same time
      const int jc = in ? jj : 0;
      const int v = *reinterpret_cast<const int32_t*>(reinterpret_cast<const uint8_t*>(prow) +
                                                      (uint32_t)(4 * jc));  // scalar base
      ph = (in && v < a.pool.tokens) ? v : -1;
      if (in && v >= a.pool.tokens && a.status) atomicOr(a.status, DSA_DEVERR_POOL_ROW);
    } else if (in) {
      const int s = idx[jj];
      if (s >= 0 && s < nvis) {
        const int b = bt[s / kBlock];
        const bool ok = b >= 0 && (int64_t)b * kBlock < a.pool.tokens;
        ph = ok ? b * kBlock + (s % kBlock) : -1;
        if (!ok && a.status) atomicOr(a.status, DSA_DEVERR_BLOCK_ID);
      }
    }
    return ph;
  };

  // Prologue: the query loads go first (unconditional), the pool rows of the first batches right
  // behind them, so both round trips overlap.
  // Q^T fragments (B operand) of this wave's half of the contraction
  const int kd = kHalfDims * dh;  // first dim of the half (wave-uniform)
  v8bf qf[kSteps];
  {
    const uint16_t* qr = a.q + ((int64_t)row * DSA_MLA_HEADS + head) * DSA_MLA_DQK + kd + 8 * g;
#pragma unroll
    for (int i = 0; i < kSteps; ++i)
      qf[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(qr + 32 * i));
  }
  asm volatile("" ::: "memory");  // keep the query loads ahead of the pool-row loads
  int tb = 0;
  int pv = load_batch(0);
  int pv_next = ntiles > kBatchTiles ? load_batch(kBatchTiles) : -1;
  // The pool rows and the query arrive together (one wait, before the first gather is issued:
  // the gathers are invisible to the compiler, and a wait of its own behind them would be a full
  // drain of the pipeline).
#pragma unroll
  for (int i = 0; i < kSteps; ++i) asm volatile("" ::"v"(qf[i]), "v"(pv), "v"(pv_next));
#pragma unroll
  for (int T = 0; T < kAhead; ++T)
    if (T < ntiles)
      issue_tile<LFMT>(stages[T], pv, kRowsPerWave * T, ph_spread, a, j0 + T * kTile, j1, lane);

  v4f o[kDvHalf / 16];
#pragma unroll
  for (int mt = 0; mt < kDvHalf / 16; ++mt) o[mt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float qk_scale = a.softmax_scale * kLog2e;

  for (int jb = j0; jb < j1; jb += kStages * kTile) {
#pragma unroll
    for (int s = 0; s < kStages; ++s) {  // unrolled: stage s is a compile-time choice
      const int j = jb + s * kTile;
      if (j >= j1) break;
      const Stage& cur = stages[s];
      // All but the gathers of the tiles issued after tile j are done: tile j has landed (this
      // wave's part).  Tiles past the split's end are never issued, so near the end fewer are.
      {
        const int newer = min(kAhead - 1, ntiles - 1 - (j - j0) / kTile);
        static_assert(kAhead - 1 <= 4, "wait counts below");
        if (newer >= 4) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * kGathersPerWave) : "memory");
        else if (newer == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * kGathersPerWave) : "memory");
        else if (newer == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kGathersPerWave) : "memory");
        else if (newer == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kGathersPerWave) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      lds_barrier();  // everyone's part landed; the previous tile's readers are done
      const int tl = opaque((int)threadIdx.x);
      const int ln = tl & 63, gl = ln >> 4, cl = ln & 15;
      if constexpr (G::kFp8)
        build_fp8(cur, vt, tl);
      else
        build_nvfp4(cur, ct, vt, tl);
      if constexpr (!G::kFp8) lds_barrier();  // the QK operands come from the decoded tile

      // this wave's half of S^T (tokens x heads) for the two 16-token halves of the tile
      v4f sfr[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kSteps; ++i)
          acc = mfma_bf16(qk_operand<LFMT>(cur, ct, 16 * h2 + cl, kd + 32 * i + 8 * gl), qf[i], acc);
        sfr[h2] = acc;
        sx[wave][h2][ln] = acc;
      }
      lds_barrier();  // partial S^T of both halves, and the value tile, are in LDS
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) sfr[h2] += sx[wave ^ 1][h2][ln];

      // logits in base 2; lane holds tokens 16*h2 + 4g + i for its head.  The four tokens'
      // flags and scales are read at once, unconditionally; stale LDS bits of slots without a
      // token are selected away, never used.
      float x[2][4], ts[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int t0 = 16 * h2 + 4 * gl;
        const int4 ok4 = *reinterpret_cast<const int4*>(cur.valid + t0);
        const int okv[4] = {ok4.x, ok4.y, ok4.z, ok4.w};
        float scv[4] = {a.tensor_scale, a.tensor_scale, a.tensor_scale, a.tensor_scale};
        if constexpr (G::kFp8) {
          const float4 s4 = *reinterpret_cast<const float4*>(cur.tsc + t0);
          scv[0] = s4.x; scv[1] = s4.y; scv[2] = s4.z; scv[3] = s4.w;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = okv[i] != 0;
          const float scl = ok ? scv[i] : 0.f;
          ts[h2][i] = scl;
          const float v = ok ? sfr[h2][i] * scl * qk_scale : -INFINITY;
          x[h2][i] = v;
          tmax = fmaxf(tmax, v);
        }
      }
      tmax = xor32_max(xor16_max(tmax));
      // Lazy rescaling: the running max only moves when a logit exceeds it by more than 2^4, so
      // probabilities stay <= 16 and O is rarely rescaled.  The fp16 probability times the token
      // scale must stay finite: token (or tensor) scales below 4096.
      const float m_old = m_run;
      const float m_new = (tmax > m_run + kLazyMax) ? tmax : m_run;
      // v_exp_f32 directly (exp2(-inf) = 0; results below the fp32 normal range flush to zero,
      // negligible next to the token that set the running max, whose probability is 1)
      const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      const float mref = (m_new == -INFINITY) ? 0.f : m_new;  // all logits -inf: p = 0, not NaN
      float psum = 0.f;
      uint32_t pb[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(x[h2][i] - mref);
          psum += p;
          pv[i] = p * ts[h2][i];  // the token scale of c_j multiplies its value row
        }
        // K slots 8g + 4*h2 + i  <->  token 16*h2 + 4g + i
#pragma unroll
        for (int i = 0; i < 2; ++i)
          pb[2 * h2 + i] = f16_bits(pv[2 * i]) | (f16_bits(pv[2 * i + 1]) << 16);
      }
      psum = xor32_sum(xor16_sum(psum));
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const v8h pfrag = __builtin_bit_cast(v8h, uint4{pb[0], pb[1], pb[2], pb[3]});
      // wave-uniform, rarely taken; never while the running max is still -inf (O is all zeros)
      if (__builtin_amdgcn_readfirstlane(__any(alpha != 1.f && m_old != -INFINITY))) {
#pragma unroll
        for (int mt = 0; mt < kDvHalf / 16; ++mt) o[mt] *= alpha;
      }

      // O^T (dims x heads) += V^T P^T; A operand lane: dim 256dh + 16mt + c, K slots 8g .. 8g+7
#pragma unroll
      for (int mt = 0; mt < kDvHalf / 16; ++mt)
        o[mt] = mfma_f16(pv_operand(vt, kDvHalf * dh + 16 * mt + cl, gl), pfrag, o[mt]);

      // Gathers of tile j + kAhead into the stage tile j - 1 used (every wave passed this tile's
      // first barrier, so no one reads it any more).  Issued last: a wave that finds the gather
      // queue full stalls here, where it would otherwise wait at the next barrier.
      {
        const int T = (j - j0) / kTile + kAhead;
        if (T - tb == kBatchTiles) {  // next batch of pool rows (loaded one batch ahead)
          tb += kBatchTiles;
          pv = pv_next;
          if (tb + kBatchTiles < ntiles) pv_next = load_batch(tb + kBatchTiles);
        }
        if (T < ntiles)
          issue_tile<LFMT>(stages[(s + kAhead) % kStages], pv, kRowsPerWave * (T - tb), ph_spread, a,
                           j + kAhead * kTile, j1, ln);
      }
    }
  }

  // the gathers issued ahead of the last tiles (dummies) land before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // lane holds O^T[256dh + 16mt + 4g + i][head]
  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
  if (a.out_direct) {
    uint16_t* orow = a.out + ((int64_t)row * DSA_MLA_HEADS + head) * DSA_MLA_DV + kDvHalf * dh;
#pragma unroll
    for (int mt = 0; mt < kDvHalf / 16; ++mt) {
      uint32_t b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t u = __float_as_uint(o[mt][i] * inv);
        b[i] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
      }
      *reinterpret_cast<uint2*>(orow + 16 * mt + 4 * g) = uint2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
    }
    if (a.lse && g == 0 && dh == 0)
      a.lse[(int64_t)row * DSA_MLA_HEADS + head] =
          (l_run > 0.f) ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    // Split partial: this split's normalised output as fp16 scaled by a power of two chosen from
    // the head's largest value in the split (11 significant bits relative to that value, for any
    // latent scale), the scale's exponent, and the split's base-2 log-sum-exp.  The fp16 values
    // keep the accumulator layout (wave, mt, lane, 4 values), so every store is 512 contiguous
    // bytes.
    const int64_t slot = ((int64_t)row * a.split_slots + a.split_base + split) * DSA_MLA_HEADS + head;
    float amax = 0.f;
#pragma unroll
    for (int mt = 0; mt < kDvHalf / 16; ++mt)
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(o[mt][0]), fabsf(o[mt][1])),
                               fmaxf(fabsf(o[mt][2]), fabsf(o[mt][3]))));
    amax *= inv;
    amax = xor32_max(xor16_max(amax));
    if (g == 0) amx[wave][c] = amax;
    lds_barrier();
    amax = fmaxf(amax, amx[wave ^ 1][c]);  // over all 512 dims of the head
    // 2^e * amax lies in [2^14, 2^15): well inside fp16's range and above its subnormals
    const int e = (amax > 0.f) ? 14 - ilogbf(amax) : 0;
    const float sc = inv * ldexpf(1.f, e);
    uint2* po = reinterpret_cast<uint2*>(a.part_o) +
                (((int64_t)row * a.split_slots + a.split_base + split) * kWavesM + wave) *
                    (kDvHalf / 16) * kWave + lane;
#pragma unroll
    for (int mt = 0; mt < kDvHalf / 16; ++mt) {
      // Large partial sets are streamed out (non-temporal): read once by the combine, they
      // should not sit dirty in the memory-side cache and be written back while the next step's
      // scorer streams keys.  Small ones stay cached for the combine.
      const v2u w = {f16_bits(o[mt][0] * sc) | (f16_bits(o[mt][1] * sc) << 16),
                     f16_bits(o[mt][2] * sc) | (f16_bits(o[mt][3] * sc) << 16)};
      if (a.nt_partials)
        __builtin_nontemporal_store(w, reinterpret_cast<v2u*>(po + mt * kWave));
      else
        *reinterpret_cast<v2u*>(po + mt * kWave) = w;
    }
    if (g == 0 && dh == 0) {
      a.part_lse[slot] = (l_run > 0.f) ? m_run + log2f(l_run) : -INFINITY;
      a.part_exp[slot] = e;
    }
  }
}

// Merge the splits of each row by log-sum-exp: out = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M)
// with o_s the split's normalised output.  grid (rows, 12 waves x 2 halves); 512 threads: thread
// (mt8, lane) takes accumulator block mt = 8 * blockIdx.y % 2 + mt8 of the attention wave
// blockIdx.y / 2, i.e. head 16 * (wave / 2) + lane % 16, dims 256 * (wave % 2) + 16 mt + 4 (lane / 16)
// + 0..3.  Partial loads are 8 contiguous bytes per thread (4 KB per workgroup and split).
// G: splits per group (4, 8 or 16), the smallest that covers nsplit when it can.
template <int G>
__global__ __launch_bounds__(512) void mla_combine_kernel(MlaArgs a) {
  const int row = blockIdx.x;
  const int wave = blockIdx.y >> 1;
  const int mt = 8 * (blockIdx.y & 1) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int head = 16 * (wave >> 1) + (lane & 15);
  const int d = kDvHalf * (wave & 1) + 16 * mt + 4 * (lane >> 4);
  const int64_t hbase = (int64_t)row * a.split_slots * DSA_MLA_HEADS + head;
  const uint2* pbase = reinterpret_cast<const uint2*>(a.part_o) +
                       ((int64_t)row * a.split_slots * kWavesM + wave) * (kDvHalf / 16) * kWave +
                       mt * kWave + lane;
  const int64_t pstride = (int64_t)kWavesM * (kDvHalf / 16) * kWave;  // one split
  // One pass over groups of G splits: every load of a group (log-sum-exp, exponent and partial)
  // is in flight before any is used, and a running maximum rescales what earlier groups added,
  // so up to G splits take one memory round trip.
  float M = -INFINITY, L = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < a.split_slots; s0 += G) {
    float ls[G];
    int ex[G];
    uint2 v[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int sp = min(s0 + u, a.split_slots - 1);  // past the end: a repeat, weighted 0 below
      ls[u] = a.part_lse[hbase + (int64_t)sp * DSA_MLA_HEADS];
      ex[u] = a.part_exp[hbase + (int64_t)sp * DSA_MLA_HEADS];
      v[u] = pbase[(int64_t)sp * pstride];
    }
    float gm = -INFINITY;
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (s0 + u < a.split_slots) gm = fmaxf(gm, ls[u]);
    const float m_new = fmaxf(M, gm);
    if (m_new == -INFINITY) continue;  // nothing attended so far
    const float r = exp2f(M - m_new);  // M = -inf: 0 (L and acc are 0 then)
    L *= r;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= r;
    M = m_new;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const float wgt = (s0 + u < a.split_slots && ls[u] != -INFINITY) ? exp2f(ls[u] - M) : 0.f;
      L += wgt;
      const float w2 = ldexpf(wgt, -ex[u]);
      acc[0] += w2 * (float)__builtin_bit_cast(_Float16, (uint16_t)(v[u].x & 0xFFFFu));
      acc[1] += w2 * (float)__builtin_bit_cast(_Float16, (uint16_t)(v[u].x >> 16));
      acc[2] += w2 * (float)__builtin_bit_cast(_Float16, (uint16_t)(v[u].y & 0xFFFFu));
      acc[3] += w2 * (float)__builtin_bit_cast(_Float16, (uint16_t)(v[u].y >> 16));
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  uint32_t b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t u = __float_as_uint(acc[i] * inv);
    b[i] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  }
  *reinterpret_cast<uint2*>(a.out + ((int64_t)row * DSA_MLA_HEADS + head) * DSA_MLA_DV + d) =
      uint2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
  if (a.lse && mt == 0 && (wave & 1) == 0 && lane < 16)
    a.lse[(int64_t)row * DSA_MLA_HEADS + head] = (L > 0.f) ? (M + log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

#ifndef DSA_MLA_MAX_SPLITS
#define DSA_MLA_MAX_SPLITS 32
#endif
#ifndef DSA_MLA_TARGET_WGS
#define DSA_MLA_TARGET_WGS 256
#endif
// Splits of each row's selected set: enough workgroups to fill the chip (about 256), or, for a
// batch-invariant call, fixed 128-token parts (a function of k alone).
int mla_num_splits(int32_t num_rows, int32_t k, bool invariant) {
  if (invariant) return (k + 4 * kTile - 1) / (4 * kTile);
  const int tiles = (k + kTile - 1) / kTile;
  const int64_t rows = num_rows > 0 ? num_rows : 1;
  // at most 32 splits (64 tokens each at k = 2,048): below that size a split is one tile, and the
  // combine's extra round over the slots costs more than the parallelism gains (one row: 1.4 us)
  const int cap = tiles < DSA_MLA_MAX_SPLITS ? tiles : DSA_MLA_MAX_SPLITS;
  // One workgroup fits a CU (its LDS), so a launch of rows x ns workgroups runs in
  // ceil(rows ns / 256) waves of workgroups, each lasting about kFixedTiles + (tiles per split)
  // tile-times (the fixed part: query and pool-row loads, the first gathers' round trip, the
  // partial stores).  The split count with the least of that wins, the fewest splits on a tie
  // (less for the combine): 96 speculative rows take 5 splits (two waves of 13 tiles) rather than
  // 3 (two waves of 22), 16 decode rows 16, one row 32.
  constexpr int64_t kFixedTiles = 3;
  int best = 1;
  int64_t best_cost = -1;
  for (int ns = 1; ns <= cap; ++ns) {
    const int64_t per = (tiles + ns - 1) / ns;
    const int64_t waves = (rows * ns + DSA_MLA_TARGET_WGS - 1) / DSA_MLA_TARGET_WGS;
    const int64_t cost = waves * (kFixedTiles + per);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = ns;
    }
  }
  return best;
}

size_t mla_workspace_bytes(int32_t num_rows, int32_t k, bool invariant) {
  const int ns = mla_num_splits(num_rows, k, invariant);
  if (ns <= 1) return 0;
  return (size_t)num_rows * ns * DSA_MLA_HEADS * (DSA_MLA_DV * sizeof(uint16_t) + 2 * sizeof(float));
}

hipError_t launch_mla_combine(const MlaArgs& a, hipStream_t s) {
  if (a.batch.num_rows <= 0) return hipSuccess;
  const dim3 cgrid((unsigned)a.batch.num_rows, 2 * kWavesM);
  if (a.split_slots <= 4)
    hipLaunchKernelGGL(mla_combine_kernel<4>, cgrid, dim3(512), 0, s, a);
  else if (a.split_slots <= 8)
    hipLaunchKernelGGL(mla_combine_kernel<8>, cgrid, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(mla_combine_kernel<16>, cgrid, dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_mla(const MlaArgs& a, int lat_fmt, bool combine, hipStream_t s) {
  if (a.batch.num_rows <= 0) return hipSuccess;
  dim3 grid((unsigned)a.batch.num_rows, (unsigned)a.nsplit);
  if (lat_fmt == DSA_LATENT_FP8)
    if (a.phys)
      hipLaunchKernelGGL((sparse_mla_kernel<DSA_LATENT_FP8, true>), grid, dim3(kThreadsM), 0, s, a);
    else
      hipLaunchKernelGGL((sparse_mla_kernel<DSA_LATENT_FP8, false>), grid, dim3(kThreadsM), 0, s, a);
  else if (a.phys)
    hipLaunchKernelGGL((sparse_mla_kernel<DSA_LATENT_NVFP4, true>), grid, dim3(kThreadsM), 0, s, a);
  else
    hipLaunchKernelGGL((sparse_mla_kernel<DSA_LATENT_NVFP4, false>), grid, dim3(kThreadsM), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.out_direct || !combine) return e;
  return launch_mla_combine(a, s);
}

}  // namespace dsa
