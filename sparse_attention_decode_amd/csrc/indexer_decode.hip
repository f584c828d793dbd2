// Lightning-indexer scorer: decode, speculative verification and prefill.
//
// Source: "vLLM Delivers Day-0 Support for Kimi K3.1 Pro" — §Sparse Attention in K3.1 Pro (every
// earlier token is scored for each query by 32 light heads over one FP8 key of 132 bytes with its
// scale; long-context decode is bound by memory bandwidth); §AMD / Quantization: Native MXFP4
// indexer (68-byte MXFP4 keys, scored with the matrix cores in FP4 and summed in fp32 over the
// weighted heads; one read of the keys serves every query row of a speculative step).  Scoring rule (DeepSeek-V3.2 lightning indexer, which the page defers to):
//     score[r,s] = sum_h w[r,h] * ReLU(scale_s * q[r,h] . k[s])
// computed here as scale_s * sum_h w[r,h] * ReLU(q[r,h] . k[s]) (scale_s > 0).
//
// Design (gfx950): the key pages are the only large stream.  A workgroup owns a long run of one
// sequence's blocks; each wave pulls whole 64-token key pages straight from HBM into MFMA operand
// registers (no LDS staging: each key byte is used by exactly one lane) and scores every row of
// its row tile from that single read.  The query rows are the MFMA A operand (M = 16 heads, two
// tiles per row), keys the B operand (N = 16 tokens per tile, K = 128 dims in one instruction),
// so the head reduction (ReLU, x w, sum over 32 heads) is 8 lane-local terms (an integer max and
// an FMA each) per token tile, then one three-swap exchange that hands lane group g the sum of
// token tile g (in the order of a plain xor reduction).  The 11-bit radix histogram the exact select needs is built on the way
// (LDS atomics, one global atomic per non-empty bin per workgroup).
#include "dsa_kernels.h"

namespace dsa {

namespace {

constexpr int kThreads = 256;         // 4 waves
constexpr int kPrefillThreads = 512;  // the prefill tile with a histogram: 8 waves
constexpr int kBins = DSA_HIST_BINS;  // top 11 bits of the order-preserving key
constexpr int kPrefillRows = 16;      // rows per workgroup tile on the prefill path
// rows per tile of the prefill candidate pass: 16 rows with their candidate staging spill the
// page loop's registers; 8-row tiles read each key page twice as often (from the caches) and
// run the chunk's pass 1.9 ms faster at 8,192 rows on a 340K prefix
constexpr int kPrefillCandRows = 8;
constexpr int kMaxPagesPerWave = 64;  // one block-table entry per lane
constexpr int kMaxPagesSmallR = 8;    // one or two rows: the whole run's scores in registers

// Operand fragments of one 16-token tile.
struct KeyFrag {
  v8i b;       // MFMA B operand
  int escale;  // MXFP4: E8M0 scale of (token, K block l/16)
};

// Byte offsets, within a pool row, of what lane (g, c) reads: the key bytes of token c of a
// page's first 16-token tile (tile nt adds nt * 16 tokens), and its scale: FP8, the scale of token
// 16g + c, the one token whose score the lane produces; MXFP4, the E8M0 scale of token c's K
// block g (tile nt adds nt * 64 bytes).
// FP8 key pages are stored in load order: lane 16g + c of a wave needs bytes [16g, 16g + 16) and
// [64 + 16g, 64 + 16g + 16) of token c of each tile (its two 16-byte pieces of the MFMA B
// operand), and the pool puts piece (tile nt, half h) of all 64 lanes in one contiguous 1 KB run
// at 2048 nt + 1024 h, lane-ordered.  Each 16-byte load of a wave then reads 1 KB in one piece,
// where the token-major order made every load touch half of each of 16 key lines.
struct LaneOffsets {
  int key, scale;
};

template <int KFMT>
__device__ __forceinline__ LaneOffsets lane_offsets(const PoolView& p, int g, int c) {
  LaneOffsets o;
  if (KFMT == DSA_IKEY_FP8) {
    o.key = (int)p.ikey_off + 16 * (16 * g + c);
    o.scale = (int)p.ikey_scale_off + (16 * g + c) * 4;
  } else {
    o.key = (int)p.ikey_off + c * (DSA_INDEX_DIM / 2) + 16 * g;
    o.scale = (int)p.ikey_scale_off + c * 4 + g;
  }
  return o;
}

// A buffer resource over one pool row.  A page that does not exist (past the wave's run or the
// sequence) gets zero records: its loads are still issued, return zeros and touch no memory, so
// the compiler can count every outstanding page load and keep exactly one page in flight behind
// the one being scored.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint8_t* row, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(row), (short)0, bytes,
                                           0x00020000 /* gfx9: 32-bit data format */);
}

// AUX: the loads' cache policy, 0 or 2 (non-temporal: a key stream far larger than the
// memory-side cache is read once per step, so its lines are not worth allocating).
template <int AUX>
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t rs, int off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, AUX);
  return uint4{v[0], v[1], v[2], v[3]};
}

// max(x, 0) for finite x as one integer max on the bits: a negative float is a negative integer
// (and -0 becomes +0).  fmaxf would add a NaN-quieting max in front of it.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Head sums of four token tiles at once: lane (g, c) holds partials p[nt] of its four heads for
// token c of tile nt; it returns the sum over the four lane groups of p[g].  The additions are
// (g0 + g1) + (g2 + g3), the order of a 16-lane then a 32-lane xor reduction, in three lane swaps
// instead of eight.
__device__ __forceinline__ float group_sum_scatter(const float (&p)[4]) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[0]), __float_as_uint(p[1]), false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[2]), __float_as_uint(p[3]), false, false);
  const float s01 = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // rows: tiles 0, 1, 0, 1
  const float s23 = __uint_as_float(b[0]) + __uint_as_float(b[1]);  // rows: tiles 2, 3, 2, 3
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);            // rows: tiles 0, 1, 2, 3
}

template <int KFMT, int AUX>
__device__ __forceinline__ void load_key_page(KeyFrag* f, float& scale, __amdgpu_buffer_rsrc_t rs,
                                              const LaneOffsets& o) {
  // FP8: scale_s of the one token whose score this lane produces, token 16g + c of the page
  // (lane group g ends up with the head sum of token tile g); MXFP4 keys carry block scales only
  if (KFMT == DSA_IKEY_FP8)
    scale = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, o.scale, 0, AUX));
  else
    scale = 1.0f;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    if (KFMT == DSA_IKEY_FP8) {
      const int k = o.key + nt * 2048;
      const uint4 lo = ld16<AUX>(rs, k), hi = ld16<AUX>(rs, k + 1024);
      f[nt].b = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
                    (int)hi.w};
      f[nt].escale = 127;
    } else {
      const uint4 v = ld16<AUX>(rs, o.key + nt * 16 * (DSA_INDEX_DIM / 2));
      f[nt].b = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      f[nt].escale = __builtin_amdgcn_raw_buffer_load_b8(rs, o.scale + nt * 64, 0, AUX);
    }
  }
}

// Launch slot y (of T row tiles of a prefill chunk) -> row tile, in the balanced 16-piece order
// of token-sharded prefill ("vLLM Delivers Day-0 Support for Kimi K3.1 Pro", §Prefill: shard the
// attention by token, not by head): the tiles are cut into 16 contiguous pieces, piece p holding
// tiles [p T / 16, (p + 1) T / 16), and slot s = 0..7 takes pieces s and 15 - s.  Under the causal
// mask a tile's work grows with its position, so each slot, and so each stretch of dispatched
// workgroups, holds a light and a heavy piece.  A bijection on [0, T).
__device__ __forceinline__ int balanced_tile(int y, int T) {
  auto start = [&](int p) { return (int)(((int64_t)p * T) / 16); };
  int acc = 0;
  for (int sl = 0; sl < 8; ++sl) {
    const int p0 = sl, p1 = 15 - sl;
    const int n0 = start(p0 + 1) - start(p0), n1 = start(p1 + 1) - start(p1);
    if (y < acc + n0) return start(p0) + (y - acc);
    acc += n0;
    if (y < acc + n1) return start(p1) + (y - acc);
    acc += n1;
  }
  return y;  // not reached for y < T
}

// One workgroup scores the R query rows of one sequence (decode: 1 row; speculative
// verification: up to 8; prefill: a tile of 16 rows of the chunk) against a run of that
// sequence's key pages (at most 64 per wave).  The rows' queries and head weights sit in LDS
// (registers for 6-16 rows would leave one wave per SIMD).  Every key byte is read once per row
// tile.  Scores stay in registers for G pages and then leave as coalesced 256-byte streaming
// stores: for one or two rows G covers the whole run, so no store is pending while page loads are
// (gfx9 counts loads and stores on one counter, and a mix makes every later wait a full drain).
// NTH: threads per workgroup (the prefill tile with a histogram takes 8 waves, so that the one
// workgroup its LDS allows per CU still puts two waves on each SIMD).
// MODE: kScoreDense (every block, dense scores), kScoreSample (blocks 0, S, 2S, ..., dense
// scores in sample numbering), kScoreCand (the other blocks; tokens at or above the row's floor
// are staged in LDS and appended to the row's candidate list, one global atomic per row and
// workgroup).
template <int R, int KFMT, bool HIST, bool NT = false, int NTH = kThreads, int MODE = kScoreDense>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2)))
void indexer_kernel(IndexerArgs a) {
  static_assert(!(HIST && MODE != kScoreDense), "the candidate path counts no histogram");
  constexpr bool kCand = MODE == kScoreCand;
  // candidates staged in LDS per wave and row; a wave empties a row's slice into the row's global
  // list when a page might not fit, and at its end
  constexpr int kStage = !kCand ? 1 : (R <= 8 ? 128 : 64);
  constexpr int AUX = NT ? 2 : 0;  // cache policy of the key loads
  constexpr int G = R <= 2 ? kMaxPagesSmallR : (R <= 8 ? 4 : 2);  // pages per store group
  constexpr int NH = R <= 2 ? 2 : 1;  // histogram copies (lane parity): fewer same-address atomics
  constexpr int kWaves = NTH / kWave;
  // Three or more rows: two 16-bit bins per LDS word (a workgroup counts at most 64 pages x
  // kWaves x 64 tokens, at most 32,768, per row), which halves the histogram's LDS so that three
  // speculative workgroups, or a 16-row prefill tile with its queries, fit on a CU.
  constexpr int HB = R >= 3 ? 2 : 1;  // bins per LDS word
  static_assert(HB == 1 || kMaxPagesPerWave * kWaves * kBlock < 65536, "16-bit bins");
  constexpr int kHistWords = NH * R * kBins / HB;
  // The prefill tile reads each row's query a row ahead; fewer rows keep those registers, which
  // would cost a wave per SIMD.
  constexpr bool kPrefetchRow = R > 8;
  constexpr int kQRow = DSA_INDEX_DIM + 16;  // padded LDS row of one head's query
  constexpr int kQChunks = R * DSA_INDEX_HEADS * (DSA_INDEX_DIM / 16);  // 16-byte pieces
  constexpr int kQPer = (kQChunks + NTH - 1) / NTH;
  constexpr int kWPer = (R * DSA_INDEX_HEADS + NTH - 1) / NTH;
  __shared__ __attribute__((aligned(16))) uint8_t s_q[R * DSA_INDEX_HEADS * kQRow];
  __shared__ __attribute__((aligned(16))) float s_w[R * DSA_INDEX_HEADS];
  __shared__ uint32_t s_hist[HIST ? kHistWords : 1];
  __shared__ uint2 s_cand[kCand ? (NTH / kWave) * R * kStage : 1];
  // blockIdx.y = (sequence, tile of R consecutive rows of that sequence), the tiles in the
  // balanced order unless the plain one is asked for
  const int seq = blockIdx.y / a.tiles_per_seq;
  const int tile = a.plain_order ? blockIdx.y % a.tiles_per_seq
                                 : balanced_tile(blockIdx.y % a.tiles_per_seq, a.tiles_per_seq);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;

  const int r0 = __builtin_amdgcn_readfirstlane(a.batch.seq_row_start[seq] + tile * R);
  const int rows_left = __builtin_amdgcn_readfirstlane(a.batch.seq_row_start[seq + 1] - r0);
  const int nr = min(R, rows_left);
  // rows past the sequence's last tile are never scored: a broken max_rows_per_seq
  if (rows_left > R && tile == a.tiles_per_seq - 1 && blockIdx.x == 0 && tid == 0)
    atomicOr(a.status, DSA_DEVERR_ROWS_PER_SEQ);
  if (nr <= 0) return;
  const int ppw = a.pages_per_wave;  // <= 64: one block-table entry per lane
  const int blk0 = blockIdx.x * kWaves * ppw;
  // logical page lp of this launch -> block of the sequence
  const int S = a.sample_stride;
  auto map_block = [&](int lp) {
    if (MODE == kScoreSample) return lp * S;
    if (MODE == kScoreCand) return lp + lp / (S - 1) + 1;  // the blocks that are not multiples of S
    return lp;
  };

  // Loads that need only the sequence and the rows, issued together before the row positions are
  // read: the block-table entry of this wave's page `lane` (first, so the first page waits for it
  // alone; clamped into the table's row, unused lanes are discarded below), the rows' queries and
  // their head weights (rows past nr repeat the last row; their results are never used).
  const int32_t* bt = a.batch.block_table + (int64_t)seq * a.batch.ld_bt;
  const int my_blk = blk0 + wave + kWaves * lane;
  // lane i: the sequence block of this wave's page i (the candidate pass's mapping divides by
  // S - 1: done once per lane here, and its page loop reads it back with readlane)
  const int my_map = map_block(my_blk);
  const int bt_raw = bt[min((int64_t)my_map, a.batch.ld_bt - 1)];
  uint4 qv[kQPer];
  float wl[kWPer];
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int i = min(tid + NTH * j, kQChunks - 1);
    const int rh = i / (DSA_INDEX_DIM / 16), ch = i % (DSA_INDEX_DIM / 16);
    const int r = rh / DSA_INDEX_HEADS, h = rh % DSA_INDEX_HEADS;
    const int row = r0 + min(r, nr - 1);
    qv[j] = *reinterpret_cast<const uint4*>(a.q + ((int64_t)row * DSA_INDEX_HEADS + h) * DSA_INDEX_DIM + 16 * ch);
  }
#pragma unroll
  for (int j = 0; j < kWPer; ++j) {
    const int i = min(tid + NTH * j, R * DSA_INDEX_HEADS - 1);
    const int r = i / DSA_INDEX_HEADS;
    wl[j] = a.w[(int64_t)(r0 + min(r, nr - 1)) * DSA_INDEX_HEADS + i % DSA_INDEX_HEADS];
  }
  asm volatile("" ::: "memory");  // not to be sunk below the early exit
  int pos[R];
  uint32_t fT[kCand ? R : 1];
  int fI[kCand ? R : 1];
  int L = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pos[r] = r < nr ? a.batch.row_pos[r0 + r] : -1;
    L = max(L, pos[r] + 1);
    if constexpr (kCand) {
      fT[r] = r < nr ? a.floor[2 * (r0 + r)] : 0xFFFFFFFFu;
      fI[r] = r < nr ? (int)a.floor[2 * (r0 + r) + 1] : -1;
    }
  }
  // logical pages of this launch over the longest row's blocks
  const int nb_seq = (L + kBlock - 1) / kBlock;
  const int nblk = MODE == kScoreDense ? nb_seq
                   : MODE == kScoreSample ? (nb_seq + S - 1) / S
                                          : nb_seq - (nb_seq + S - 1) / S;
  if (blk0 >= nblk) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }
  // lane j: pool row of this wave's page j, or -1 where that page does not exist
  const int64_t pool_rows = a.pool.tokens / kBlock;
  const bool page_exists = lane < ppw && my_blk < nblk;
  const int btv = (page_exists && bt_raw >= 0 && bt_raw < pool_rows) ? bt_raw : -1;
  // a visible block outside the pool: its tokens score 0 (zero records), and the fact is recorded
  if (__builtin_amdgcn_readfirstlane(__ballot(page_exists && btv < 0) != 0) && lane == 0)
    atomicOr(a.status, DSA_DEVERR_BLOCK_ID);
  auto page_of = [&](int i) { return blk0 + wave + kWaves * i; };
  const int row_bytes = (int)a.pool.row_bytes;
  auto page_rsrc = [&](int i) {
    const int prow = __builtin_amdgcn_readlane(btv, i & 63);
    const bool ok = i < ppw && prow >= 0;  // wave-uniform
    return row_rsrc(a.pool.base + (int64_t)(ok ? prow : 0) * row_bytes, ok ? row_bytes : 0);
  };
  const LaneOffsets lo = lane_offsets<KFMT>(a.pool, g, c);
  KeyFrag buf[2][4];
  float bscale[2];
  load_key_page<KFMT, AUX>(buf[0], bscale[0], page_rsrc(0), lo);

  // queries and weights to LDS (the first page is on its way meanwhile)
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int i = tid + NTH * j;
    if (i < kQChunks) {
      const int rh = i / (DSA_INDEX_DIM / 16), ch = i % (DSA_INDEX_DIM / 16);
      *reinterpret_cast<uint4*>(&s_q[rh * kQRow + 16 * ch]) = qv[j];
    }
  }
#pragma unroll
  for (int j = 0; j < kWPer; ++j) {
    const int i = tid + NTH * j;
    if (i < R * DSA_INDEX_HEADS) s_w[i] = wl[j];
  }
  if (HIST)
    for (int i = tid; i < kHistWords; i += NTH) s_hist[i] = 0;
  lds_barrier();  // not a wait for the first page: the second is requested before that

  // Candidate slices of this wave (one per row) and their fill, wave-uniform: a wave appends
  // without atomics, and its slices are read back only by itself (its LDS operations complete in
  // order).  Emptying a slice: one global atomic reserves its place in the row's list, every
  // lane copies, and the slice's largest key raises the row's maximum.
  uint2* my_cand = s_cand + (kCand ? wave * R * kStage : 0);
  uint32_t ncand[kCand ? R : 1];
#pragma unroll
  for (int r = 0; r < (kCand ? R : 1); ++r) ncand[r] = 0;
  auto flush_row = [&](int r) {
    uint32_t base = 0;
    if (lane == 0) base = (uint32_t)atomicAdd(&a.cand_count[r0 + r], (int)ncand[r]);
    base = __builtin_amdgcn_readfirstlane(base);
    uint2* dst = a.cand + (int64_t)(r0 + r) * a.cand_cap;
    uint32_t kmax = 0;
    for (uint32_t i = lane; i < ncand[r]; i += kWave) {
      const uint2 v = my_cand[r * kStage + i];
      if (base + i < (uint64_t)a.cand_cap) dst[base + i] = v;
      kmax = max(kmax, v.x);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, d, 64));
    if (lane == 0) atomicMax(&a.cand_max[r0 + r], kmax);
    ncand[r] = 0;
  };

  // Scores of the group of G pages starting at page i0 into sbuf (and the histogram).
  auto score_group = [&](int i0, float (&sbuf)[R][G]) {
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int i = i0 + u;
      load_key_page<KFMT, AUX>(buf[(u + 1) & 1], bscale[(u + 1) & 1], page_rsrc(i + 1), lo);  // always issued
      if (i >= ppw || page_of(i) >= nblk) break;
      const KeyFrag* cur = buf[u & 1];
      const float cur_scale = bscale[u & 1];
      const int blk = MODE == kScoreCand ? __builtin_amdgcn_readlane(my_map, i & 63) : map_block(page_of(i));
      // The rows' queries and weights come from LDS one row ahead of their use, so each row's
      // reads are in flight while the previous row is scored.  Not hoisted further: out of the
      // page loop they would hold 24 registers per row for the whole kernel.
      auto load_row = [&](int r, v8i (&qa)[2], float (&wv)[2][4]) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const uint8_t* qr = &s_q[(r * DSA_INDEX_HEADS + 16 * mt + c) * kQRow];
          const uint4 ql = *reinterpret_cast<const uint4*>(qr + 16 * g);
          const uint4 qh = *reinterpret_cast<const uint4*>(qr + 64 + 16 * g);
          qa[mt] = v8i{(int)ql.x, (int)ql.y, (int)ql.z, (int)ql.w, (int)qh.x, (int)qh.y, (int)qh.z,
                       (int)qh.w};
          const float4 w4 = *reinterpret_cast<const float4*>(&s_w[r * DSA_INDEX_HEADS + 16 * mt + 4 * g]);
          wv[mt][0] = w4.x; wv[mt][1] = w4.y; wv[mt][2] = w4.z; wv[mt][3] = w4.w;
        }
      };
      asm volatile("" ::: "memory");
      v8i qa[2];
      float wv[2][4];
      load_row(0, qa, wv);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // a dense decode tile with fewer rows than R (a shorter sequence in a mixed batch) skips
        // the rest (nr is wave-uniform).  Not in the 16-row prefill tile, whose rows are all
        // present but in a chunk's last tile (the branch cost its pipelined row loop 7%), nor in
        // the candidate pass (measured slower with it).
        if (MODE == kScoreDense && !kPrefetchRow && r >= nr) break;
        asm volatile("" ::: "memory");  // at most two rows' queries live
        if (!kPrefetchRow && r > 0) load_row(r, qa, wv);
        v8i qn[2];
        float wn[2][4];
        if (kPrefetchRow && r + 1 < R) load_row(r + 1, qn, wn);
        float pt[4];  // lane-local part of token tile nt's head sum
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          v4f z = {0.f, 0.f, 0.f, 0.f};
          v4f acc0, acc1;
          if (KFMT == DSA_IKEY_FP8) {
            acc0 = mfma_fp8(qa[0], cur[nt].b, z);
            acc1 = mfma_fp8(qa[1], cur[nt].b, z);
          } else {
            acc0 = mfma_fp8_fp4(qa[0], cur[nt].b, z, 127, cur[nt].escale);
            acc1 = mfma_fp8_fp4(qa[1], cur[nt].b, z, 127, cur[nt].escale);
          }
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            part += wv[0][e] * relu(acc0[e]);
            part += wv[1][e] * relu(acc1[e]);
          }
          pt[nt] = part;
        }
        float mine = group_sum_scatter(pt) * cur_scale;
        // materialise the score here: left to the store, the page's whole computation (pure)
        // would be sunk there and every page's key fragments would stay live until then
        asm volatile("" : "+v"(mine));
        sbuf[r][u] = mine;
        if (HIST && r < nr && blk * kBlock + lane <= pos[r])
        {
          const uint32_t bin = order_key(mine) >> 21;
          atomicAdd(&s_hist[(((lane % NH) * R + r) * kBins + bin) / HB],
                    HB == 2 ? 1u << (16 * (bin & 1)) : 1u);
        }
        if (kPrefetchRow && r + 1 < R) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            qa[mt] = qn[mt];
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[mt][e] = wn[mt][e];
          }
        }
      }
      if constexpr (kCand) {
        // the page's tokens at or above their row's floor into this wave's slices, once every
        // row of the page is scored (each row's scoring chain runs undisturbed)
        const int tok = blk * kBlock + lane;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t key = order_key(sbuf[r][u]);
          const bool keep = r < nr && tok <= pos[r] &&
                            (key > fT[r] || (key == fT[r] && tok < fI[r]));
          const uint64_t m = __ballot(keep);
          const uint32_t add = (uint32_t)__popcll(m);
          if (ncand[r] + add > (uint32_t)kStage) flush_row(r);  // the slice is full (rare)
          const uint32_t p =
              ncand[r] + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if (keep) my_cand[r * kStage + p] = uint2{key, (uint32_t)tok};
          ncand[r] += add;
        }
      }
    }
  };
  // One coalesced 256-byte streaming store per (page, row) of the group starting at page i0.
  auto store_group = [&](int i0, const float (&sbuf)[R][G]) {
    if constexpr (kCand) return;  // candidates were appended page by page
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int i = i0 + u;
      if (i >= ppw || page_of(i) >= nblk) break;
      const int lp = page_of(i);
      const int s_tok = map_block(lp) * kBlock + lane;  // the token (visibility)
      const int s_at = lp * kBlock + lane;               // its place in this launch's scores
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // row offset kept scalar and computed here (hoisted, 16 rows of 64-bit VGPR addresses
        // would stay live through the whole page loop)
        int64_t off = (int64_t)(r0 + r) * a.ld;
        asm volatile("" : "+s"(off));
        if (r < nr && s_tok <= pos[r]) __builtin_nontemporal_store(sbuf[r][u], &a.scores[off + s_at]);
      }
    }
  };

  auto flush_hist = [&]() {
    lds_barrier();  // every wave's LDS counts are in; its global stores need not be
    for (int i = tid; i < nr * kBins; i += NTH) {
      uint32_t v = 0;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const uint32_t word = s_hist[(h * R * kBins + i) / HB];
        v += HB == 2 ? (word >> (16 * (i & 1))) & 0xFFFFu : word;
      }
      if (v) atomicAdd(&a.hist[(int64_t)(r0 + i / kBins) * kBins + (i % kBins)], v);
    }
  };

  if constexpr (G == kMaxPagesSmallR) {
    // The whole run is one group (pages per wave <= G): the histogram flush goes out before the
    // stores and neither waits for the other, so the kernel's tail is one round trip.
    float sbuf[R][G];
    score_group(0, sbuf);
    if (HIST) flush_hist();
    store_group(0, sbuf);
  } else {
#pragma unroll 1
    for (int i0 = 0; i0 < ppw; i0 += G) {
      if (page_of(i0) >= nblk) break;
      float sbuf[R][G];
      score_group(i0, sbuf);
      store_group(i0, sbuf);
    }
    if (HIST) flush_hist();
  }
  if constexpr (kCand) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (ncand[r]) flush_row(r);
  }
}

__global__ void zero_u32_kernel(uint32_t* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

// The sample and candidate passes of the candidates path (no histogram).  Decode rows stream
// their keys past the caches (the path is for long contexts); a prefill tile (the sample pass's
// 16 rows, the candidate pass's 8) keeps them cached for the next row tile.
template <int KFMT, int MODE>
hipError_t launch_cand_rows(const IndexerArgs& a, int rows, dim3 grid, hipStream_t s,
                            bool prefill) {
  static_assert(kPrefillCandRows == 8, "the case below");
  switch (rows) {
#define DSA_CASE(R)                                                                               \
  case R:                                                                                         \
    hipLaunchKernelGGL((indexer_kernel<R, KFMT, false, true, kThreads, MODE>), grid,              \
                       dim3(kThreads), 0, s, a);                                                  \
    break;
    DSA_CASE(1) DSA_CASE(2) DSA_CASE(3) DSA_CASE(4) DSA_CASE(5) DSA_CASE(6) DSA_CASE(7)
#undef DSA_CASE
    case 8:
      if (prefill && MODE == kScoreCand)
        hipLaunchKernelGGL((indexer_kernel<8, KFMT, false, false, kThreads, MODE>), grid,
                           dim3(kThreads), 0, s, a);
      else
        hipLaunchKernelGGL((indexer_kernel<8, KFMT, false, true, kThreads, MODE>), grid,
                           dim3(kThreads), 0, s, a);
      break;
    case kPrefillRows:
      if constexpr (MODE == kScoreSample)
        hipLaunchKernelGGL((indexer_kernel<kPrefillRows, KFMT, false, false, kThreads, MODE>),
                           grid, dim3(kThreads), 0, s, a);
      else
        return hipErrorInvalidValue;  // the candidate pass takes 8-row tiles
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// nt: stream the keys past the caches (decode with a histogram only).
template <int KFMT>
hipError_t launch_many_rows(const IndexerArgs& a, int rows, dim3 grid, hipStream_t s,
                            bool nt = false, int mode = kScoreDense, bool prefill = false) {
  if (mode == kScoreSample) return launch_cand_rows<KFMT, kScoreSample>(a, rows, grid, s, prefill);
  if (mode == kScoreCand) return launch_cand_rows<KFMT, kScoreCand>(a, rows, grid, s, prefill);
  switch (rows) {
#define DSA_CASE(R)                                                                              \
  case R:                                                                                        \
    if (a.hist && nt)                                                                            \
      hipLaunchKernelGGL((indexer_kernel<R, KFMT, true, true>), grid, dim3(kThreads), 0, s, a); \
    else if (a.hist)                                                                             \
      hipLaunchKernelGGL((indexer_kernel<R, KFMT, true>), grid, dim3(kThreads), 0, s, a);       \
    else                                                                                         \
      hipLaunchKernelGGL((indexer_kernel<R, KFMT, false>), grid, dim3(kThreads), 0, s, a);      \
    break;
    DSA_CASE(1) DSA_CASE(2) DSA_CASE(3) DSA_CASE(4) DSA_CASE(5) DSA_CASE(6) DSA_CASE(7) DSA_CASE(8)
#undef DSA_CASE
    case kPrefillRows:
      if (a.hist)
        hipLaunchKernelGGL((indexer_kernel<kPrefillRows, KFMT, true, false, kPrefillThreads>),
                           grid, dim3(kPrefillThreads), 0, s, a);
      else
        hipLaunchKernelGGL((indexer_kernel<kPrefillRows, KFMT, false>), grid, dim3(kThreads), 0,
                           s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

namespace {
// Pages one launch visits per sequence of max_context tokens: every block, the sample blocks
// (0, S, 2S, ...) or the others.
int64_t launch_pages(int64_t max_context, int mode, int S) {
  const int64_t nb = (max_context + kBlock - 1) / kBlock;
  if (mode == kScoreSample) return (nb + S - 1) / S;
  if (mode == kScoreCand) return nb - (nb + S - 1) / S;
  return nb;
}
}  // namespace

hipError_t launch_indexer_decode(const IndexerArgs& a0, int ikey_fmt, int rows_per_seq,
                                 int64_t max_context, hipStream_t s, int mode) {
  IndexerArgs a = a0;
  a.tiles_per_seq = 1;
  const int64_t nblk = launch_pages(max_context, mode, a.sample_stride);
  if (nblk <= 0) return hipSuccess;
  // Workgroups, from the longest sequence: about 1024 for one or two rows (4 to 8 pages per
  // wave; with three workgroups resident per CU that is about 1.3 rounds, so the score stores of
  // the first round overlap the key reads of the second: measured faster than one round of 688
  // or 2048 workgroups), about 2048 for more rows (pages per wave a multiple of the 4-page store
  // group, at most 64).
  constexpr int kWaves = kThreads / kWave;
  const bool small = rows_per_seq <= 2;
#ifndef DSA_IDX_TARGET_MANY
#define DSA_IDX_TARGET_MANY 2048
#endif
  const int64_t target = small ? 1024 : DSA_IDX_TARGET_MANY;
  const int64_t cap = small ? kMaxPagesSmallR : kMaxPagesPerWave;
  const int64_t want = (nblk * a.batch.num_seqs + target - 1) / target;
  int64_t ppw = (want + kWaves - 1) / kWaves;
  if (!small) ppw = (ppw + 3) / 4 * 4;
  if (ppw < 4) ppw = 4;
  if (ppw > cap) ppw = cap;
  a.pages_per_wave = (int32_t)ppw;
  const int64_t per_wg = ppw * kWaves;
  dim3 grid((unsigned)((nblk + per_wg - 1) / per_wg), (unsigned)a.batch.num_seqs);
  // A key stream much larger than the 256 MB memory-side cache cannot stay there between steps:
  // load it non-temporally, leaving the cache to the scores and latents the next kernels read.
  // A small one (a short context) is re-read from that cache on the next step: keep it there.
  const int64_t key_bytes = a.batch.num_seqs * max_context *
                            (ikey_fmt == DSA_IKEY_FP8 ? DSA_INDEX_DIM + 4 : DSA_INDEX_DIM / 2 + 4);
  const bool nt = key_bytes >= ((int64_t)64 << 20);
  return ikey_fmt == DSA_IKEY_FP8
             ? launch_many_rows<DSA_IKEY_FP8>(a, rows_per_seq, grid, s, nt, mode)
             : launch_many_rows<DSA_IKEY_MXFP4>(a, rows_per_seq, grid, s, nt, mode);
}

// Prefill: the rows of a sequence are cut into tiles of 16 (the candidate pass: 8) rows
// (queries in LDS); each workgroup
// contracts one row tile with a run of at most 64 key pages per wave, at least about 2048
// workgroups in all.  Key pages
// are re-read once per row tile, from L2 / the memory-side cache for a context that fits there.
hipError_t launch_indexer_prefill(const IndexerArgs& a0, int ikey_fmt, int64_t max_context,
                                  int32_t max_rows_per_seq, hipStream_t s, int mode) {
  IndexerArgs a = a0;
  const int R = mode == kScoreCand ? kPrefillCandRows : kPrefillRows;
  // with a histogram the tile's workgroup has 8 waves (the same waves per CU as two 4-wave ones)
  const int kWaves = (a.hist ? kPrefillThreads : kThreads) / kWave;
  a.tiles_per_seq = (max_rows_per_seq + R - 1) / R;
  const int64_t nblk = launch_pages(max_context, mode, a.sample_stride);
  if (nblk <= 0) return hipSuccess;
  const int64_t gy = (int64_t)a.batch.num_seqs * a.tiles_per_seq;
  if (gy > 65535) return hipErrorInvalidValue;
  int64_t chunks = (2048 + gy - 1) / gy;
  int64_t ppw = (nblk + chunks * kWaves - 1) / (chunks * kWaves);
  ppw = (ppw + 1) / 2 * 2;
  if (ppw < 2) ppw = 2;
  if (ppw > kMaxPagesPerWave) ppw = kMaxPagesPerWave;
  a.pages_per_wave = (int32_t)ppw;
  dim3 grid((unsigned)((nblk + ppw * kWaves - 1) / (ppw * kWaves)), (unsigned)gy);
  return ikey_fmt == DSA_IKEY_FP8
             ? launch_many_rows<DSA_IKEY_FP8>(a, R, grid, s, false, mode, true)
             : launch_many_rows<DSA_IKEY_MXFP4>(a, R, grid, s, false, mode, true);
}

}  // namespace dsa
