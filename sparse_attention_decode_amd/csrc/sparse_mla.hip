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
// Wave 4g + q belongs to head group g (heads [32g, 32g + 32)) and is its quarter q: it computes
// the quarter q of the QK contraction (144 of the 576 dims) for the group's 32 heads and all 32
// tokens of a tile, and the quarter q of the output dims (128 of 512), so it holds 36 query
// registers and 64 accumulator registers, and three waves share each SIMD.  Both products use
// the 32x32x16 MFMA shapes, which on this GPU issue at twice the rate per flop of the 16x16x32
// ones, and every A operand read from LDS serves 32 heads.  Tiles of 32 selected tokens are
// gathered from the paged pool straight into LDS with direct global->LDS loads (no registers
// held in flight), kStages - 1 tiles ahead of the tile being processed.  Each stage is its own
// LDS variable and barriers wait on LDS traffic only, so reading a tile never waits for the
// gathers of later tiles.  The split's pool rows are resolved once into an LDS list, and a tile
// is gathered as 16-byte chunks at consecutive LDS addresses, full 64-lane gathers with a 64-bit
// address per lane (FP8: two per wave from 10 waves; NVFP4: one per wave from 11), with no per-row
// scalar work and no exec masking.
//   QK^T: S^T[tokens x heads] = C Q^T on bf16 MFMA.  The query stays in registers (B operand);
//         the latent tile is the A operand.  FP8 latents are read raw from LDS and converted to
//         bf16 in registers (exact); NVFP4 latents are decoded once per tile into a bf16 tile.
//         The four quarter partials of S^T are exchanged through LDS so that quarter q ends up
//         with the whole sum for tokens [8q, 8q + 8) (added in quarter order).
//   softmax: quarter q turns its 8 tokens' logits into probabilities relative to its own
//         largest logit and leaves them (fp16, times the token scale), that maximum and their
//         sum in LDS; every wave of the group then reads all four, takes the tile maximum, and
//         rescales each quarter's probabilities to the row's running maximum as it loads them.
//   PV:   O^T[dims x heads] = V^T P^T on fp16 MFMA.  The rows of V^T are read from token-major
//         tiles with the LDS transpose reads (8 tokens of one dim per lane): FP8 from the
//         gathered stage itself, converted to fp16 in registers (exact), NVFP4 from the fp16
//         value tile its decode writes beside the bf16 one.
// Per-token scales stay out of the MFMA operands (they multiply the logits and the
// probabilities), so every operand is an exact conversion of the stored codes.  fp16 for P keeps
// its rounding well inside the output tolerance.  Softmax is online, in base 2.  With S^T and
// O^T a head's softmax statistics live in the same lane as that head's output column.
// LDS rows are padded so that the MFMA operand reads are bank-conflict free.
#include "dsa_kernels.h"

namespace dsa {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef int lds_v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) lds_v2i_t lds_v2i;
typedef short lds_v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) lds_v4s_t lds_v4s;

constexpr int kHeadGroups = DSA_MLA_HEADS / 32;   // 3 groups of 32 heads
constexpr int kQuarters = 4;                       // waves per head group
constexpr int kWavesM = kHeadGroups * kQuarters;   // 12
constexpr int kThreadsM = kWavesM * kWave;         // 768
constexpr int kTile = 32;                          // selected tokens per tile
constexpr int kQkSteps = DSA_MLA_DQK / kQuarters / 16;  // 9 K steps of 16 dims per wave
constexpr int kDvTiles = DSA_MLA_DV / kQuarters / 32;   // 4 tiles of 32 output dims per wave
constexpr int kPsRow = 80;                         // fp16 probability row: 32 tokens + pad
#ifndef DSA_MLA_STAGES
#define DSA_MLA_STAGES 3
#endif
// Gather pipeline: while tile j is processed, tiles j+1 .. j+kAhead are in flight.
constexpr int kStages = DSA_MLA_STAGES;
constexpr int kAhead = kStages - 1;
static_assert(kStages >= 3 && kStages <= 6, "stage variables raw0..raw5");
constexpr int kRowsPerWave = (kTile + kWavesM - 1) / kWavesM;  // 3 (rows >= 32 are spare)
constexpr int kSlots = kRowsPerWave * kWavesM;                  // 36 LDS rows per stage
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 4.f;  // base-2 headroom of the running max (probabilities <= 16)

// FP8 latents
constexpr int kRaw8 = 592;   // raw row bytes: 576 codes + pad (148 dwords: b128 reads conflict-free)
// NVFP4 latents
constexpr int kRaw4 = 336;   // raw row bytes: 288 packed codes + 48 (the 36 block scales and 12 past)
constexpr int kCt4 = 1168;   // bf16 token-major row bytes: 1152 + pad (292 dwords; rows 16-byte aligned)
constexpr int kHt4 = 1056;   // fp16 token-major row bytes of the value dims: 1024 + pad (264
                              // dwords: the four rows one transpose read meets sit in distinct banks)

// A tile is copied into its stage as 16-byte chunks at consecutive LDS addresses: chunk c is part
// c % kChunks of row c / kChunks, parts [0, kLatChunks) the token's latent bytes and the rest the
// 16-byte pieces from its scales on (FP8: one, the 4 scale bytes and 12 past them, into the row's
// pad; NVFP4: three, the 36 block-scale bytes and 12 past them; the pool layout keeps 12 bytes of
// the row behind the scale page).  Gathering waves 0 .. kGatherWaves - 1 each issue kGathers full
// 64-lane copies per tile, chunks [kWaveChunks w, +kWaveChunks); lanes past the tile re-read its
// last chunk into the stage's spare rows.  Every gathering wave issues the same number of copies
// per tile, so waiting for a tile is "all but the newest tiles' copies are done".
template <int LFMT>
struct Geo {
  static constexpr bool kFp8 = LFMT == DSA_LATENT_FP8;
  static constexpr int kRaw = kFp8 ? kRaw8 : kRaw4;
  static constexpr int kLatBytes = kFp8 ? DSA_MLA_DQK : DSA_MLA_DQK / 2;  // latent bytes per token
  static constexpr int kSclBytes = kFp8 ? 4 : DSA_MLA_DQK / 16;           // scale bytes per token
  static constexpr int kLatChunks = kLatBytes / 16;                       // 36 / 18
  static constexpr int kChunks = kRaw / 16;                               // 37 / 21 per row
  static constexpr int kTileChunks = kTile * kChunks;                     // 1184 / 672 per tile
  static constexpr int kGathers = kFp8 ? 2 : 1;       // copies per gathering wave and tile
  static constexpr int kWaveChunks = kGathers * kWave;                    // 128 / 64
  static constexpr int kGatherWaves = (kTileChunks + kWaveChunks - 1) / kWaveChunks;  // 10 / 11
  static constexpr int kHtBytes = kFp8 ? 16 : kTile * kHt4;  // fp16 value tile (NVFP4 only)
  static constexpr int kCtBytes = kFp8 ? 16 : kTile * kCt4;  // decoded tile (NVFP4 only)
  static_assert(kChunks * 16 == kRaw && kLatChunks * 16 == kLatBytes, "whole chunks");
  static_assert((kChunks - kLatChunks) * 16 >= kSclBytes &&
                (kChunks - kLatChunks) * 16 - kSclBytes <= 12, "scale pieces read at most 12 bytes past");
  static_assert(kGatherWaves <= kWavesM, "gathering waves");
  static_assert(kGatherWaves * kWaveChunks * 16 <= kSlots * kRaw, "copies stay in the stage");
};

// One pipeline stage: where a gathered tile lands.  Each stage's buffers are separate
// __shared__ variables, so the compiler can tell the reads of one stage from the gathers still
// landing in the others (one shared array would make it wait for every gather before any read).
struct Stage {
  uint8_t* raw;    // [kSlots][kRaw] latent rows as stored (rows >= kTile: spare)
  float* tsc;      // [kSlots] FP8 token scales
};

// The value of x, opaque to the optimiser: lane-dependent addresses derived from it inside the tile
// loop are recomputed each tile (a few VALU) instead of being hoisted out of the loop, where they
// would hold registers for the whole loop and push the kernel into spills.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Direct global->LDS copies.  Lane l copies 16 bytes from its own 64-bit address to LDS address
// lds + 16 l.  Issued through inline assembly, so the compiler does not track them:
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
__device__ __forceinline__ void lds_copy16_va(uint64_t addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" DSA_GATHER_POLICY
               :: "v"(addr), "s"(lds) : "memory", "m0");
}

// The chunk gathers of one tile into stage st.  rows: the tile's 32 pool rows (-1: no token; such
// a row gathers pool row `spare` instead, whose data is never used).  Each lane finds its chunk's
// row in LDS and forms the address itself, so a gathering wave issues kGathers instructions and no
// per-row scalar work.
template <int LFMT>
__device__ __forceinline__ void issue_tile(const Stage& st, const int32_t* rows, const MlaArgs& a,
                                           int wave, int lane, int spare) {
  using G = Geo<LFMT>;
  if (wave >= G::kGatherWaves) return;
#pragma unroll
  for (int i = 0; i < G::kGathers; ++i) {
    const int c = min(G::kWaveChunks * wave + kWave * i + lane, G::kTileChunks - 1);
    const int t = c / G::kChunks, part = c - G::kChunks * t;
    const int ph = rows[t];
    const uint32_t src = (uint32_t)(ph >= 0 ? ph : spare);
    const uint32_t slot = src & (kBlock - 1);
    // offsets inside a pool row fit 32 bits; the latent or the scale offset picked by a mask,
    // not a branch
    const uint32_t lat = (uint32_t)a.pool.lat_off + slot * G::kLatBytes + 16u * part;
    uint32_t scl = (uint32_t)a.pool.lat_scale_off + slot * G::kSclBytes;
    if constexpr (G::kChunks - G::kLatChunks > 1) scl += 16u * (uint32_t)(part - G::kLatChunks);
    const uint32_t within = scl ^ ((lat ^ scl) & (0u - (uint32_t)(part < G::kLatChunks)));
    const uint64_t addr = reinterpret_cast<uint64_t>(a.pool.base) +
                          (uint64_t)(src >> 6) * (uint32_t)a.pool.row_bytes + within;
    lds_copy16_va(addr, lds_addr(st.raw + 16 * (G::kWaveChunks * wave + kWave * i)));
  }
}

// FP8: the tokens' scales, gathered into each row's pad, side by side for the softmax; and, in a
// tile with rows that hold no token (rare: the end of a split, or entries with no visible token),
// the value bytes of those rows cleared, so that PV, which reads the stage itself, multiplies
// their zero probabilities by zeros and never by stale codes (an E4M3 NaN would survive a zero
// probability).  `bad`: the wave-uniform ballot of the tile's rows without a token.
__device__ __forceinline__ void prep_fp8(const Stage& st, const int32_t* rows, uint64_t bad, int tid) {
  if (tid < kTile) st.tsc[tid] = *reinterpret_cast<const float*>(st.raw + tid * kRaw8 + DSA_MLA_DQK);
  if (bad == 0) return;
  constexpr int kParts = DSA_MLA_DV / 16;  // 16-byte pieces of a row's value dims
  for (int it = tid; it < kTile * kParts; it += kThreadsM) {
    const int t = it / kParts, part = it % kParts;
    if (rows[t] < 0) *reinterpret_cast<uint4*>(st.raw + t * kRaw8 + 16 * part) = uint4{0u, 0u, 0u, 0u};
  }
}

// NVFP4: decode a stage once into the bf16 tile (all 576 dims) and the fp16 tile (the 512 value
// dims), both token-major, one 16-dim block of one token per item.  The hardware converts each pair of E2M1 codes to fp32
// unscaled (its scaled form does not apply an arbitrary fp32 scale exactly), the block scale
// multiplies in fp32, and the products (E2M1 x E4M3: at most 6 significant bits, magnitudes in
// [2^-10, 2688] or 0) are exact in bf16 and fp16, so truncation and round-toward-zero give them
// exactly.  Tokens that are not selected decode as +0.
__device__ __forceinline__ void build_nvfp4(const Stage& st, const int32_t* rows, uint8_t* ct,
                                            uint8_t* ht, int tid) {
  for (int it = tid; it < (DSA_MLA_DQK / 16) * kTile; it += kThreadsM) {
    const int t = it & 31, blk = it >> 5;  // token, 16-dim block
    const bool ok = rows[t] >= 0;
    uint2 p = *reinterpret_cast<const uint2*>(st.raw + t * kRaw4 + 8 * blk);
    p = ok ? p : uint2{0u, 0u};  // stale bits of an empty slot become +0 codes
    const float sc = ok ? fp8_to_f32(st.raw[t * kRaw4 + DSA_MLA_DQK / 2 + blk]) : 1.f;
    // byte b of each word holds codes 2b (low nibble) and 2b + 1
    const v2f c[8] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p.x, 1.0f, 0),
                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p.x, 1.0f, 1),
                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p.x, 1.0f, 2),
                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p.x, 1.0f, 3),
                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p.y, 1.0f, 0),
                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p.y, 1.0f, 1),
                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p.y, 1.0f, 2),
                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p.y, 1.0f, 3)};
    uint32_t w[8], h[8];  // bf16 and fp16 pairs (dims 2j, 2j + 1)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a = c[j][0] * sc, b = c[j][1] * sc;
      w[j] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
      h[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
    }
    uint4* crow = reinterpret_cast<uint4*>(ct + t * kCt4 + 32 * blk);
    crow[0] = uint4{w[0], w[1], w[2], w[3]};
    crow[1] = uint4{w[4], w[5], w[6], w[7]};
    if (16 * blk < DSA_MLA_DV) {
      uint4* hrow = reinterpret_cast<uint4*>(ht + t * kHt4 + 32 * blk);
      hrow[0] = uint4{h[0], h[1], h[2], h[3]};
      hrow[1] = uint4{h[4], h[5], h[6], h[7]};
    }
  }
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v8bf fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const uint4 r = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
  return __builtin_bit_cast(v8bf, r);
}

// QK K step i of quarter qt: lane (n, hi) holds dims [144 qt + 16 i + 8 hi, +8) of token n (A operand)
// and of head n (B operand).  The nine steps of a quarter cover its 144 dims once.
constexpr int kQuarterDims = DSA_MLA_DQK / kQuarters;  // 144

// Latent tile as the A operand of QK^T: token t, dims [d, d+8).
template <int LFMT>
__device__ __forceinline__ v8bf qk_operand(const Stage& st, const uint8_t* ct, int t, int d) {
  if constexpr (LFMT == DSA_LATENT_FP8) {
    const uint2 v = *reinterpret_cast<const uint2*>(st.raw + t * kRaw8 + d);
    return fp8x8_to_bf16(v.x, v.y);
  } else {
    return __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(ct + t * kCt4 + 2 * d));
  }
}

// NVFP4: the A operand of PV read from the token-major fp16 value tile by two LDS transpose
// reads.  In each group of 16 lanes a read takes 8 bytes (4 dims) from the address of every lane
// and hands lane i half-word i % 4 of the pieces of lanes 4r + i / 4, r = 0..3, as its element r.
// So lane 4r + q of the group points at token t0 + r, dims [d0 + 4q, +4), and lane i receives
// dim d0 + i of tokens t0 .. t0 + 3; the second read (4 rows further) gives tokens t0 + 4 .. + 7.
__device__ __forceinline__ v8h pv_operand_f16(const uint8_t* p) {
  const lds_v4s_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
  const lds_v4s_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 4 * kHt4));
  typedef short v8s __attribute__((ext_vector_type(8)));
  return __builtin_bit_cast(v8h, v8s{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]});
}

// FP8: the A operand of PV read from the token-major stage itself by the LDS transpose read.  In
// each group of 16 lanes the read takes an 8-byte piece from the address of every lane and hands
// lane i byte i % 8 of the pieces of lanes 2r + i / 8, r = 0..7, as its byte r.  So lane 2r + h of
// the group points at token t0 + r, dims [d0 + 8h, +8), and lane i receives dim d0 + i of tokens
// t0 .. t0 + 7: its row of V^T for one K step.  fp8 -> fp16 is exact.
__device__ __forceinline__ v8h pv_operand_fp8(const uint8_t* p) {
  const lds_v2i_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)p);
  const uint4 r = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[0], 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[0], 1.0f, true)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[1], 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[1], 1.0f, true))};
  return __builtin_bit_cast(v8h, r);
}

// 32x32x16 MFMAs (bf16 for QK, fp16 for PV).  A lane l: row l % 32, K [8 (l / 32), +8); B lane l:
// column l % 32, the same K; result register r of lane l: row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32.
__device__ __forceinline__ v16f mfma32_bf16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma32_f16(v8h a, v8h b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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
  constexpr int kTsc = G::kFp8 ? kSlots : 4;  // FP8 token scales (NVFP4 has none)
  __shared__ __attribute__((aligned(16))) float tsc0[kTsc], tsc1[kTsc], tsc2[kTsc],
      tsc3[kTsc], tsc4[kTsc], tsc5[kTsc];
  __shared__ __attribute__((aligned(16))) uint8_t ht[G::kHtBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ct[G::kCtBytes];
  // partial S^T exchange: [head group][token quarter][source quarter, own one skipped][lane]
  __shared__ __attribute__((aligned(16))) v4f sx[kHeadGroups][kQuarters][kQuarters - 1][kWave];
  // probabilities (fp16) of a tile: [head group][head][token], rows padded to 80 bytes
  __shared__ __attribute__((aligned(16))) uint8_t ps[kHeadGroups * 32 * kPsRow];
  // pool rows of the split's selected entries in order (-1: no visible token), padded with -1 to
  // whole tiles (a split never spans more than k <= DSA_MAX_TOPK entries)
  __shared__ __attribute__((aligned(16))) int32_t plist[DSA_MAX_TOPK];
  // per head: each quarter's largest logit and its probability sum (relative to that logit)
  __shared__ __attribute__((aligned(16))) float mqs[kHeadGroups][32][kQuarters];
  __shared__ __attribute__((aligned(16))) float lqs[kHeadGroups][32][kQuarters];
  const Stage stages[6] = {{raw0, tsc0}, {raw1, tsc1}, {raw2, tsc2},
                           {raw3, tsc3}, {raw4, tsc4}, {raw5, tsc5}};

  const int row = blockIdx.x, split = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps wave math scalar
  const int n = lane & 31, hi = lane >> 5;
  const int hg = wave >> 2, qt = wave & 3;  // head group (32 heads), quarter
  const int head = 32 * hg + n;             // this lane's head in S^T / O^T columns

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

  const int ntiles = (j1 - j0 + kTile - 1) / kTile;
  // A row without a token gathers a spare row whose data is never used: a pool row that depends
  // on the workgroup and wave (never one row for everybody: thousands of requests to one address
  // would queue on one memory channel).
  const int ph_spread = __builtin_amdgcn_readfirstlane(
      (int)(((int64_t)blockIdx.x * 7919 + (int64_t)blockIdx.y * 131 + wave * 17) % a.pool.tokens));
  // The pool row of the split's selected entry jj, or -1 where there is none (past the split's
  // end, an empty or invisible entry, or a pool row or block outside the pool: the last two are
  // also reported in the status word).
  auto resolve = [&](int jj) {
    int ph = -1;
    if (jj < j1) {
      if (PHYS) {
        const int v = prow[jj];
        ph = v < a.pool.tokens ? v : -1;
        if (v >= a.pool.tokens && a.status) atomicOr(a.status, DSA_DEVERR_POOL_ROW);
      } else {
        const int sidx = idx[jj];
        if (sidx >= 0 && sidx < nvis) {
          const int b = bt[sidx / kBlock];
          const bool ok = b >= 0 && (int64_t)b * kBlock < a.pool.tokens;
          ph = ok ? b * kBlock + (sidx % kBlock) : -1;
          if (!ok && a.status) atomicOr(a.status, DSA_DEVERR_BLOCK_ID);
        }
      }
    }
    return ph;
  };

  // Prologue: the query loads go first (unconditional), the split's pool rows right behind them,
  // so both round trips overlap.
  // Q^T fragments (B operand) of this wave's quarter of the contraction
  const int kd = kQuarterDims * qt;  // first dim of the quarter (wave-uniform)
  v8bf qf[kQkSteps];
  {
    const uint16_t* qr = a.q + ((int64_t)row * DSA_MLA_HEADS + head) * DSA_MLA_DQK + kd + 8 * hi;
#pragma unroll
    for (int i = 0; i < kQkSteps; ++i)
      qf[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(qr + 16 * i));
  }
  asm volatile("" ::: "memory");  // keep the query loads ahead of the pool-row loads
  {
    // the split's pool rows, resolved once: every load in flight at once, then one LDS barrier
    constexpr int kIters = (DSA_MAX_TOPK + kThreadsM - 1) / kThreadsM;
    int ph[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) ph[it] = resolve(j0 + tid + kThreadsM * it);
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int e = tid + kThreadsM * it;
      if (e < ntiles * kTile) plist[e] = ph[it];
    }
    lds_barrier();
    // The query has arrived too (one wait, before the first gather is issued: the gathers are
    // invisible to the compiler, and a wait of its own behind them would be a full drain of the
    // pipeline).
#pragma unroll
    for (int i = 0; i < kQkSteps; ++i) asm volatile("" ::"v"(qf[i]));
#pragma unroll
    for (int T = 0; T < kAhead; ++T)
      if (T < ntiles) issue_tile<LFMT>(stages[T], plist + kTile * T, a, wave, lane, ph_spread);
  }

  // O^T (dims x heads) of this wave: dims [128 qt + 32 dt, +32) x the group's 32 heads
  v16f o[kDvTiles];
#pragma unroll
  for (int dt = 0; dt < kDvTiles; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
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
        constexpr int kG = G::kGathers;
        if (newer >= 4) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * kG) : "memory");
        else if (newer == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * kG) : "memory");
        else if (newer == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kG) : "memory");
        else if (newer == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kG) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      lds_barrier();  // everyone's part landed; the previous tile's readers are done
      const int tl = opaque((int)threadIdx.x);
      const int ln = tl & 63, nl = ln & 31, hl = ln >> 5;
      const int32_t* rows = plist + (j - j0);  // >= 0: a token
      if constexpr (G::kFp8)
        prep_fp8(cur, rows, __ballot(rows[nl] < 0), tl);
      else
        build_nvfp4(cur, rows, ct, ht, tl);
      if constexpr (!G::kFp8) lds_barrier();  // the QK operands come from the decoded tile

      // this wave's quarter of S^T (32 tokens x the group's 32 heads)
      v16f acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int i = 0; i < kQkSteps; ++i)
        acc = mfma32_bf16(qk_operand<LFMT>(cur, ct, nl, kd + 16 * i + 8 * hl), qf[i], acc);
      // hand the token quarters of the other waves of the group their part of this partial
#pragma unroll
      for (int rho = 0; rho < kQuarters; ++rho)
        if (rho != qt)
          sx[hg][rho][qt < rho ? qt : qt - 1][ln] =
              v4f{acc[4 * rho], acc[4 * rho + 1], acc[4 * rho + 2], acc[4 * rho + 3]};
      lds_barrier();  // partial S^T of every quarter (and FP8's cleared rows) are in LDS

      // S^T of this wave's token quarter: tokens 8 qt + 4 hl + i, head nl; the four partials
      // are added in quarter order
      v4f sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int src = 0; src < kQuarters; ++src) {
        const v4f p = (src == qt) ? v4f{acc[4 * qt], acc[4 * qt + 1], acc[4 * qt + 2], acc[4 * qt + 3]}
                                  : sx[hg][qt][src < qt ? src : src - 1][ln];
        sq = (src == 0) ? p : sq + p;
      }

      // logits in base 2; the four tokens' flags and scales are read at once, unconditionally;
      // stale LDS bits of slots without a token are selected away, never used
      const int t0 = 8 * qt + 4 * hl;
      const int4 ok4 = *reinterpret_cast<const int4*>(rows + t0);
      const int okv[4] = {ok4.x, ok4.y, ok4.z, ok4.w};
      float scv[4] = {a.tensor_scale, a.tensor_scale, a.tensor_scale, a.tensor_scale};
      if constexpr (G::kFp8) {
        const float4 s4 = *reinterpret_cast<const float4*>(cur.tsc + t0);
        scv[0] = s4.x; scv[1] = s4.y; scv[2] = s4.z; scv[3] = s4.w;
      }
      float x[4], ts[4];
      float mq = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = okv[i] >= 0;
        ts[i] = ok ? scv[i] : 0.f;
        x[i] = ok ? sq[i] * ts[i] * qk_scale : -INFINITY;
        mq = fmaxf(mq, x[i]);
      }
      mq = xor32_max(mq);  // the quarter's 8 tokens
      // probabilities relative to the quarter's own largest logit (<= 1); the reader rescales
      // them to the row's running maximum.  A quarter without tokens has p = 0.
      const float mrq = (mq == -INFINITY) ? 0.f : mq;
      float psq = 0.f;
      uint32_t pw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(x[2 * i] - mrq);
        const float p1 = __builtin_amdgcn_exp2f(x[2 * i + 1] - mrq);
        psq += p0 + p1;
        // the token scale of c_j multiplies its value row
        pw[i] = f16_bits(p0 * ts[2 * i]) | (f16_bits(p1 * ts[2 * i + 1]) << 16);
      }
      psq = xor32_sum(psq);
      *reinterpret_cast<uint2*>(ps + (32 * hg + nl) * kPsRow + 2 * t0) = uint2{pw[0], pw[1]};
      if (hl == 0) {
        mqs[hg][nl][qt] = mq;
        lqs[hg][nl][qt] = psq;
      }
      lds_barrier();  // every quarter's probabilities, maxima and sums are in LDS

      // Lazy rescaling: the running max only moves when a logit exceeds it by more than 2^4, so
      // probabilities stay <= 16 and O is rarely rescaled.  The fp16 probability times the token
      // scale must stay finite: token (or tensor) scales below 4096.  Every wave of the group
      // computes the same values from the same LDS words.
      // the probabilities of this lane's PV operands are read with the maxima and sums, so that
      // the three reads take one LDS round trip
      v8h pf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pf[ks] = __builtin_bit_cast(
            v8h, *reinterpret_cast<const uint4*>(ps + (32 * hg + nl) * kPsRow + 2 * (16 * ks + 8 * hl)));
      const float4 m4 = *reinterpret_cast<const float4*>(&mqs[hg][nl][0]);
      const float4 l4 = *reinterpret_cast<const float4*>(&lqs[hg][nl][0]);
      const float mqv[4] = {m4.x, m4.y, m4.z, m4.w};
      const float lqv[4] = {l4.x, l4.y, l4.z, l4.w};
      const float tmax = fmaxf(fmaxf(mqv[0], mqv[1]), fmaxf(mqv[2], mqv[3]));
      const float m_old = m_run;
      const float m_new = (tmax > m_run + kLazyMax) ? tmax : m_run;
      // v_exp_f32 directly (exp2(-inf) = 0; results below the fp32 normal range flush to zero,
      // negligible next to the token that set the running max, whose probability is 1)
      const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      const float mref = (m_new == -INFINITY) ? 0.f : m_new;  // all logits -inf: p = 0, not NaN
      float fq[4], psum = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        fq[q] = (mqv[q] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mqv[q] - mref);
        psum += lqv[q] * fq[q];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      // wave-uniform, rarely taken; never while the running max is still -inf (O is all zeros)
      if (__builtin_amdgcn_readfirstlane(__any(alpha != 1.f && m_old != -INFINITY))) {
#pragma unroll
        for (int dt = 0; dt < kDvTiles; ++dt) o[dt] *= alpha;
      }

      // O^T (dims x heads) += V^T P^T, 16 tokens per step: tokens [16 ks + 8 hl, +8) of head nl
      // come from quarter 2 ks + hl, rescaled to the running maximum
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const _Float16 f = (_Float16)(hl ? fq[2 * ks + 1] : fq[2 * ks]);
        const v8h p = pf[ks] * f;
        if constexpr (G::kFp8) {
          // lane (group g = ln / 16, j = ln % 16): token 16 ks + 8 hl + j / 2, dims
          // 128 qt + 32 dt + 16 (g % 2) + 8 (j % 2)
          const uint8_t* vb = cur.raw + (16 * ks + 8 * hl + ((ln & 15) >> 1)) * kRaw8 + 128 * qt +
                              16 * ((ln >> 4) & 1) + 8 * (ln & 1);
#pragma unroll
          for (int dt = 0; dt < kDvTiles; ++dt)
            o[dt] = mfma32_f16(pv_operand_fp8(vb + 32 * dt), p, o[dt]);
        } else {
          // lane (group g = ln / 16, j = ln % 16): token 16 ks + 8 hl + j / 4 (and 4 rows on),
          // dims 128 qt + 32 dt + 16 (g % 2) + 4 (j % 4)
          const uint8_t* vb = ht + (16 * ks + 8 * hl + ((ln & 15) >> 2)) * kHt4 +
                              2 * (128 * qt + 16 * ((ln >> 4) & 1) + 4 * (ln & 3));
#pragma unroll
          for (int dt = 0; dt < kDvTiles; ++dt)
            o[dt] = mfma32_f16(pv_operand_f16(vb + 64 * dt), p, o[dt]);
        }
      }

      // Gathers of tile j + kAhead into the stage tile j - 1 used (every wave passed this tile's
      // first barrier, so no one reads it any more).  Issued last: a wave that finds the gather
      // queue full stalls here, where it would otherwise wait at the next barrier.
      {
        const int T = (j - j0) / kTile + kAhead;
        if (T < ntiles)
          issue_tile<LFMT>(stages[(s + kAhead) % kStages], plist + kTile * T, a, wave, ln, ph_spread);
      }
    }
  }

  // the gathers issued ahead of the last tiles land before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // lane holds O^T[128 qt + 32 dt + 8 b + 4 hi + i][head] in o[dt][4 b + i]
  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
  if (a.out_direct) {
    uint16_t* orow = a.out + ((int64_t)row * DSA_MLA_HEADS + head) * DSA_MLA_DV + 128 * qt + 4 * hi;
#pragma unroll
    for (int dt = 0; dt < kDvTiles; ++dt)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t u = __float_as_uint(o[dt][4 * b + i] * inv);
          w[i] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
        }
        *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * b) = uint2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
      }
    if (a.lse && qt == 0 && hi == 0)
      a.lse[(int64_t)row * DSA_MLA_HEADS + head] =
          (l_run > 0.f) ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    // Split partial: this split's normalised output as fp16 scaled by a power of two chosen from
    // the head's largest value in the split (11 significant bits relative to that value, for any
    // latent scale), the scale's exponent, and the split's base-2 log-sum-exp.  The fp16 values
    // keep the accumulator layout (wave, register octet, lane, 8 values), so every store is
    // 1,024 contiguous bytes.
    const int64_t slot = ((int64_t)row * a.split_slots + a.split_base + split) * DSA_MLA_HEADS + head;
    float amax = 0.f;
#pragma unroll
    for (int dt = 0; dt < kDvTiles; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(o[dt][r]));
    amax *= inv;
    amax = xor32_max(amax);
    // the partial S^T exchange area is free once every wave has passed the last tile's third
    // barrier, which it has before any wave gets here
    float (*amx)[32][kQuarters] = reinterpret_cast<float (*)[32][kQuarters]>(&sx[0][0][0][0]);
    if (hi == 0) amx[hg][n][qt] = amax;
    lds_barrier();
    {
      const float4 m4 = *reinterpret_cast<const float4*>(&amx[hg][n][0]);
      amax = fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w));  // over all 512 dims of the head
    }
    // 2^e * amax lies in [2^14, 2^15): well inside fp16's range and above its subnormals
    const int e = (amax > 0.f) ? 14 - ilogbf(amax) : 0;
    const float sc = inv * ldexpf(1.f, e);
    uint4* po = reinterpret_cast<uint4*>(a.part_o) +
                (((int64_t)row * a.split_slots + a.split_base + split) * kWavesM + wave) * 8 * kWave +
                lane;
#pragma unroll
    for (int oc = 0; oc < 8; ++oc) {
      // Large partial sets are streamed out (non-temporal): read once by the combine, they
      // should not sit dirty in the memory-side cache and be written back while the next step's
      // scorer streams keys.  Small ones stay cached for the combine.
      const v16f& od = o[oc >> 1];
      const int r0 = 8 * (oc & 1);
      const v4u w = {f16_bits(od[r0] * sc) | (f16_bits(od[r0 + 1] * sc) << 16),
                     f16_bits(od[r0 + 2] * sc) | (f16_bits(od[r0 + 3] * sc) << 16),
                     f16_bits(od[r0 + 4] * sc) | (f16_bits(od[r0 + 5] * sc) << 16),
                     f16_bits(od[r0 + 6] * sc) | (f16_bits(od[r0 + 7] * sc) << 16)};
      if (a.nt_partials)
        __builtin_nontemporal_store(w, reinterpret_cast<v4u*>(po + oc * kWave));
      else
        *reinterpret_cast<v4u*>(po + oc * kWave) = w;
    }
    if (qt == 0 && hi == 0) {
      a.part_lse[slot] = (l_run > 0.f) ? m_run + log2f(l_run) : -INFINITY;
      a.part_exp[slot] = e;
    }
  }
}

// Merge the splits of each row by log-sum-exp: out = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M)
// with o_s the split's normalised output.  grid (rows, 12 attention waves); 512 threads: thread
// (oc, lane) takes register octet oc of the attention wave blockIdx.y, i.e. head
// 32 (wave / 4) + lane % 32 and dims 128 (wave % 4) + 32 (oc / 2) + 16 (oc % 2) + 4 (lane / 32)
// + {0..3, 8..11}.  Partial loads are 16 contiguous bytes per thread (8 KB per workgroup and split).
// G: splits per group (4, 8, 16 or 32), the smallest that covers nsplit when it can (16 beyond
// 32 splits: the 32-split group's registers cost more than its saved round trips there).
template <int G>
__global__ __launch_bounds__(512) void mla_combine_kernel(MlaArgs a) {
  // 96 slots per row (attention wave, register octet), blockDim.x / 64 of them per workgroup: a
  // batch of few rows takes small workgroups, so that its loads are spread over many CUs
  const int row = blockIdx.x;
  const int slot = blockIdx.y * (int)(blockDim.x >> 6) + (int)(threadIdx.x >> 6);
  const int wave = slot >> 3;
  const int oc = slot & 7;
  const int lane = threadIdx.x & 63;
  const int head = 32 * (wave >> 2) + (lane & 31);
  const int d = 128 * (wave & 3) + 32 * (oc >> 1) + 16 * (oc & 1) + 4 * (lane >> 5);
  const int64_t hbase = (int64_t)row * a.split_slots * DSA_MLA_HEADS + head;
  const uint4* pbase = reinterpret_cast<const uint4*>(a.part_o) +
                       ((int64_t)row * a.split_slots * kWavesM + wave) * 8 * kWave + oc * kWave + lane;
  const int64_t pstride = (int64_t)kWavesM * 8 * kWave;  // one split
  // One pass over groups of G splits: every load of a group (log-sum-exp, exponent and partial)
  // is in flight before any is used, and a running maximum rescales what earlier groups added,
  // so up to G splits take one memory round trip.
  float M = -INFINITY, L = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < a.split_slots; s0 += G) {
    float ls[G];
    int ex[G];
    uint4 v[G];
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
    for (int i = 0; i < 8; ++i) acc[i] *= r;
    M = m_new;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const float wgt = (s0 + u < a.split_slots && ls[u] != -INFINITY) ? exp2f(ls[u] - M) : 0.f;
      L += wgt;
      const float w2 = ldexpf(wgt, -ex[u]);
      const uint32_t vw[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += w2 * (float)__builtin_bit_cast(_Float16, (uint16_t)(vw[i] & 0xFFFFu));
        acc[2 * i + 1] += w2 * (float)__builtin_bit_cast(_Float16, (uint16_t)(vw[i] >> 16));
      }
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  uint32_t b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t u = __float_as_uint(acc[i] * inv);
    b[i] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  }
  uint16_t* orow = a.out + ((int64_t)row * DSA_MLA_HEADS + head) * DSA_MLA_DV + d;
  *reinterpret_cast<uint2*>(orow) = uint2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
  *reinterpret_cast<uint2*>(orow + 8) = uint2{b[4] | (b[5] << 16), b[6] | (b[7] << 16)};
  if (a.lse && oc == 0 && (wave & 3) == 0 && lane < 32)
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

#ifndef DSA_COMBINE_ROWS8
#define DSA_COMBINE_ROWS8 32
#endif
#ifndef DSA_COMBINE_ROWS2
#define DSA_COMBINE_ROWS2 4
#endif
constexpr int kCombineRows8 = DSA_COMBINE_ROWS8, kCombineRows2 = DSA_COMBINE_ROWS2;

hipError_t launch_mla_combine(const MlaArgs& a, hipStream_t s) {
  if (a.batch.num_rows <= 0) return hipSuccess;
  // waves per workgroup: 8 (one attention wave's 8 octets) from 32 rows on, fewer below
  const int rows = a.batch.num_rows;
  const int wpg = rows >= kCombineRows8 ? 8 : rows >= kCombineRows2 ? 2 : 1;
  const dim3 cgrid((unsigned)rows, (unsigned)(kWavesM * 8 / wpg)), cblock((unsigned)(kWave * wpg));
  if (a.split_slots <= 4)
    hipLaunchKernelGGL(mla_combine_kernel<4>, cgrid, cblock, 0, s, a);
  else if (a.split_slots <= 8)
    hipLaunchKernelGGL(mla_combine_kernel<8>, cgrid, cblock, 0, s, a);
  else if (a.split_slots <= 16 || a.split_slots > 32)  // more slots: groups of 16 measured faster
    hipLaunchKernelGGL(mla_combine_kernel<16>, cgrid, cblock, 0, s, a);
  else
    hipLaunchKernelGGL(mla_combine_kernel<32>, cgrid, cblock, 0, s, a);
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
