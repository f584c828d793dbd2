// Exact top-k select over materialised indexer scores.
//
// Source: "vLLM Delivers Day-0 Support for Kimi K3.1 Pro" — §Sparse Attention in K3.1 Pro (keep
// the 2,048 highest-scoring tokens); §Low-latency decode (an exact top-k select that emits the
// pool rows, which the attention then gathers); §An exact top-k merge (a radix select); §AMD /
// Communication (a consistent tie rule).  Tie rule used here: the lower token index wins; -0 and
// +0 tie.
//
// Keys: the order-preserving 32-bit image of each fp32 score.  Three kernels per call:
//   hist    (only when the scorer did not provide it) 11-bit radix histogram of each row's keys;
//   filter  many workgroups per row: each derives the threshold bin b1 (the 11-bit bin holding
//           the k-th largest key) from the histogram, streams one slice of the row's scores and
//           compacts the tokens whose key lies in a bin >= b1, in token order;
//   resolve one workgroup per row: gathers the survivors (k plus the members of bin b1, a few
//           thousand for long rows), refines bin b1 by two more radix levels (11 + 10 bits) to the
//           exact k-th key T and the number E of keys equal to T that make the cut, then selects
//           key > T, or key == T among the first E in token order.  A block prefix sum in token
//           order places each selected token, so the output is ascending with no sort.
#include "dsa_kernels.h"

namespace dsa {

namespace {

constexpr int kBins = DSA_HIST_BINS;
constexpr int kFilterThreads = 256;
constexpr int kPerThread = kTopkSlice / kFilterThreads;  // 16 scores per thread
constexpr int kHistChunk = 32768;                          // tokens per histogram workgroup
// Above this many filter slices per row (contexts beyond 256K) the threshold bin is found once
// per row by its own kernel instead of by every filter workgroup.
constexpr int kLevel1Slices = 64;
constexpr int kResolveThreads = 1024;
constexpr int kResolveWaves = kResolveThreads / kWave;
constexpr int kCap = 8192;  // survivors resolved in LDS
// Batches whose rows see at most kCap tokens skip the filter: the resolve reads each row's scores
// itself, kDirectPer per thread.
constexpr int kDirectPer = kCap / kResolveThreads;

__device__ __forceinline__ int row_seq(const BatchView& b, int row) {
  int lo = 0, hi = b.num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (b.seq_row_start[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Block-wide exclusive prefix sum in thread order; *total receives the block sum.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, uint32_t* wtot) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t t = wtot[i];
    before += (i < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Find the bin b of an nbins-bin histogram (bin index increasing with the key) that holds the
// need-th largest element: above(b) < need <= above(b) + hist[b].  Returns b; *rest = need -
// above(b).  hist is in LDS; every thread gets the result.  sc: LDS scratch of NT + 4 words.
template <int NT>
__device__ uint32_t select_bin(const uint32_t* hist, int nbins, uint32_t need, uint32_t* rest,
                               uint32_t* sc, uint32_t* wtot) {
  const int tid = threadIdx.x;
  const int per = nbins / NT;  // bins per thread (>= 1)
  uint32_t own = 0;
  for (int j = 0; j < per; ++j) own += hist[per * tid + j];
  // suffix sums: scan the per-thread totals in reverse thread order
  const int rt = NT - 1 - tid;
  sc[rt] = own;
  __syncthreads();
  const uint32_t mine = sc[tid];
  __syncthreads();
  uint32_t total;
  const uint32_t ex = block_excl_scan<NT>(mine, &total, wtot);
  sc[tid] = ex;
  __syncthreads();
  uint32_t above = sc[rt];  // elements in bins owned by threads after this one
  __syncthreads();
  for (int j = per - 1; j >= 0; --j) {
    const int b = per * tid + j;
    const uint32_t h = hist[b];
    if (h && above < need && need <= above + h) {
      sc[NT] = (uint32_t)b;
      sc[NT + 1] = need - above;
    }
    above += h;
  }
  __syncthreads();
  const uint32_t b = sc[NT];
  *rest = sc[NT + 1];
  __syncthreads();
  return b;
}

// ------------------------------------------------------------------ histogram (optional pass)
// One histogram copy per wave: a row's scores crowd into few bins, and four waves adding to one
// copy serialise on the same LDS words.
__global__ __launch_bounds__(256) void topk_hist_kernel(TopkArgs a, uint32_t* hist) {
  __shared__ uint32_t h[4][kBins];
  const int row = blockIdx.y;
  const int n = a.batch.row_pos[row] + 1;
  if (n <= a.k) return;
  const int s0 = blockIdx.x * kHistChunk;
  if (s0 >= n) return;
  const int s1 = min(n, s0 + kHistChunk);
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * kBins; i += 256) (&h[0][0])[i] = 0;
  __syncthreads();
  const float* sc = a.scores + (int64_t)row * a.ld;
  uint32_t* hw = h[wave];
  // four coalesced float4 loads per thread in flight before their counts are added
  constexpr int kU = 4;
  for (int base = s0; base < s1; base += 256 * 4 * kU) {
    float4 f[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = base + (u * 256 + (int)threadIdx.x) * 4;
      if (a.vec_ok && s + 3 < s1) f[u] = *reinterpret_cast<const float4*>(sc + s);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = base + (u * 256 + (int)threadIdx.x) * 4;
      if (a.vec_ok && s + 3 < s1) {
        atomicAdd(&hw[order_key(f[u].x) >> 21], 1u);
        atomicAdd(&hw[order_key(f[u].y) >> 21], 1u);
        atomicAdd(&hw[order_key(f[u].z) >> 21], 1u);
        atomicAdd(&hw[order_key(f[u].w) >> 21], 1u);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (s + j < s1) atomicAdd(&hw[order_key(sc[s + j]) >> 21], 1u);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += 256) {
    const uint32_t v = h[0][i] + h[1][i] + h[2][i] + h[3][i];
    if (v) atomicAdd(&hist[(int64_t)row * kBins + i], v);
  }
}

// ------------------------------------------------------------------ filter
// L1: the threshold bin was found before (topk_level1_kernel); else every workgroup finds it.
template <bool L1>
__global__ __launch_bounds__(kFilterThreads) void topk_filter_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sc[kFilterThreads + 4];
  __shared__ uint32_t wtot[kFilterThreads / kWave];
  const int row = blockIdx.y, slice = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = a.batch.row_pos[row] + 1;
  const int base = slice * kTopkSlice;
  if (n <= a.k || base >= n) return;

  // issue the slice loads first; they overlap the threshold search below
  const float* src = a.scores + (int64_t)row * a.ld + base + kPerThread * tid;
  const int avail = n - base - kPerThread * tid;  // valid scores of this thread's run
  float v[kPerThread];
  if (avail >= kPerThread && a.vec_ok) {
#pragma unroll
    for (int j = 0; j < kPerThread; j += 4) {
      const float4 f = *reinterpret_cast<const float4*>(src + j);
      v[j] = f.x; v[j + 1] = f.y; v[j + 2] = f.z; v[j + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) v[j] = (j < avail) ? src[j] : 0.f;
  }

  uint32_t b1, rest = 0;
  if constexpr (L1) {
    b1 = a.level1[2 * row];
  } else {
    // the histogram row: every load in flight before the first is used
    const uint32_t* gh = a.hist_in + (int64_t)row * kBins;
    uint32_t hv[kBins / kFilterThreads];
#pragma unroll
    for (int j = 0; j < kBins / kFilterThreads; ++j) hv[j] = gh[tid + kFilterThreads * j];
#pragma unroll
    for (int j = 0; j < kBins / kFilterThreads; ++j) hist[tid + kFilterThreads * j] = hv[j];
    __syncthreads();
    b1 = select_bin<kFilterThreads>(hist, kBins, (uint32_t)a.k, &rest, sc, wtot);
  }

  uint32_t mask = 0, cnt = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const bool keep = j < avail && (order_key(v[j]) >> 21) >= b1;
    mask |= keep ? (1u << j) : 0u;
    cnt += keep ? 1u : 0u;
  }
  uint32_t total;
  uint32_t pos = block_excl_scan<kFilterThreads>(cnt, &total, wtot);
  uint2* out = a.cand + (int64_t)row * a.cand_ld + base;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (mask & (1u << j)) out[pos++] = uint2{order_key(v[j]), (uint32_t)(base + kPerThread * tid + j)};
  if (tid == 0) a.slice_cnt[(int64_t)row * a.num_slices + slice] = total;
  if (!L1 && tid == 0 && slice == 0) {  // every slice found the same bin; the resolve starts
    a.level1[2 * row] = b1;              // from it
    a.level1[2 * row + 1] = rest;
  }
}

// The threshold bin of each row, once, for a filter with many slices per row (prefill): the
// same search every filter workgroup would otherwise repeat over the row's histogram.
__global__ __launch_bounds__(kFilterThreads) void topk_level1_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sc[kFilterThreads + 4];
  __shared__ uint32_t wtot[kFilterThreads / kWave];
  const int row = blockIdx.x, tid = threadIdx.x;
  if (a.batch.row_pos[row] + 1 <= a.k) return;
  const uint32_t* gh = a.hist_in + (int64_t)row * kBins;
  uint32_t hv[kBins / kFilterThreads];
#pragma unroll
  for (int j = 0; j < kBins / kFilterThreads; ++j) hv[j] = gh[tid + kFilterThreads * j];
#pragma unroll
  for (int j = 0; j < kBins / kFilterThreads; ++j) hist[tid + kFilterThreads * j] = hv[j];
  __syncthreads();
  uint32_t rest;
  const uint32_t b1 = select_bin<kFilterThreads>(hist, kBins, (uint32_t)a.k, &rest, sc, wtot);
  if (tid == 0) {
    a.level1[2 * row] = b1;
    a.level1[2 * row + 1] = rest;
  }
}

// ------------------------------------------------------------------ resolve
constexpr int kBtCache = 4096;  // block-table entries of a row cached in LDS (contexts to 256K)
constexpr int kBtPer = kBtCache / kResolveThreads;

struct ResolveShared {
  int32_t bt[kBtCache];
  uint32_t hist[kBins];
  uint32_t key[kCap];
  int32_t idx[kCap];
  uint32_t pre[kMaxSlices + 1];  // exclusive prefix of slice counts
  uint32_t sc[kResolveThreads + 4];
  uint32_t wtot[kResolveWaves];
};

// DIRECT: rows of at most kCap visible tokens, no filter pass before (see kDirectPer).
template <bool DIRECT>
__global__ __launch_bounds__(kResolveThreads) void topk_resolve_kernel(TopkArgs a) {
  __shared__ ResolveShared sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = a.k;
  const int n = a.batch.row_pos[row] + 1;
  int32_t* out = a.idx + (int64_t)row * k;
  int32_t* phys = a.phys ? a.phys + (int64_t)row * k : nullptr;
  const int32_t* bt = a.batch.block_table + (int64_t)row_seq(a.batch, row) * a.batch.ld_bt;
  auto phys_of = [&](int s) { return bt[s / kBlock] * kBlock + (s % kBlock); };

  uint32_t* hist_row = a.hist_in + (int64_t)row * kBins;
  if (*a.status & DSA_DEVERR_ROWS_PER_SEQ) {  // some scorer skipped rows: nothing is selected
    for (int i = tid; i < k; i += kResolveThreads) {
      out[i] = -1;
      if (phys) phys[i] = -1;
    }
    for (int i = tid; i < kBins; i += kResolveThreads) hist_row[i] = 0;
    if (tid == 0) a.count[row] = -1;
    return;
  }
  if (n <= k) {  // every visible token is selected
    for (int i = tid; i < k; i += kResolveThreads) {
      out[i] = i < n ? i : -1;
      if (phys) phys[i] = i < n ? phys_of(i) : -1;
    }
    for (int i = tid; i < kBins; i += kResolveThreads) hist_row[i] = 0;  // consumed
    if (tid == 0) a.count[row] = n;
    return;
  }
  // the row's block-table entries, for the pool rows of the selection at the end: loaded now
  // into registers (their latency overlaps the loads below), moved to LDS before they are used
  const int nblk = (n + kBlock - 1) / kBlock;
  const bool bt_cached = phys != nullptr && nblk <= kBtCache;
  int32_t btv[kBtPer];
#pragma unroll
  for (int j = 0; j < kBtPer; ++j) {
    const int i = tid + kResolveThreads * j;
    btv[j] = (bt_cached && i < nblk) ? bt[i] : 0;
  }
  const int nsl = DIRECT ? 0 : (n + kTopkSlice - 1) / kTopkSlice;
  uint32_t b1, need, M;
  if constexpr (DIRECT) {
    // The row's scores (kDirectPer consecutive tokens per thread) and its histogram are read at
    // once; level 1 (the top 11 key bits) comes from the histogram, and the keys in the threshold
    // bin or above are compacted into LDS in token order, as the filter would have left them.
    const int nr = min(n, a.max_n);  // max_n <= kCap
    const int t0 = kDirectPer * tid;
    const float* src = a.scores + (int64_t)row * a.ld + t0;
    float v[kDirectPer];
    if (t0 + kDirectPer <= nr && a.vec_ok) {
#pragma unroll
      for (int j = 0; j < kDirectPer; j += 4) {
        const float4 f = *reinterpret_cast<const float4*>(src + j);
        v[j] = f.x; v[j + 1] = f.y; v[j + 2] = f.z; v[j + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kDirectPer; ++j) v[j] = (t0 + j < nr) ? src[j] : 0.f;
    }
    uint32_t hv[kBins / kResolveThreads];
#pragma unroll
    for (int j = 0; j < kBins / kResolveThreads; ++j) hv[j] = hist_row[tid + kResolveThreads * j];
#pragma unroll
    for (int j = 0; j < kBins / kResolveThreads; ++j) sh.hist[tid + kResolveThreads * j] = hv[j];
    __syncthreads();
    uint32_t rest;
    b1 = select_bin<kResolveThreads>(sh.hist, kBins, (uint32_t)k, &rest, sh.sc, sh.wtot);
    need = rest;
    uint32_t keep = 0, cnt = 0;
#pragma unroll
    for (int j = 0; j < kDirectPer; ++j) {
      const bool in = t0 + j < nr && (order_key(v[j]) >> 21) >= b1;
      keep |= in ? (1u << j) : 0u;
      cnt += in ? 1u : 0u;
    }
    uint32_t pos = block_excl_scan<kResolveThreads>(cnt, &M, sh.wtot);
#pragma unroll
    for (int j = 0; j < kDirectPer; ++j)
      if (keep & (1u << j)) {
        sh.key[pos] = order_key(v[j]);
        sh.idx[pos] = t0 + j;
        ++pos;
      }
    __syncthreads();
  } else {
    // level 1 (the top 11 key bits) was resolved by the filter from the histogram
    b1 = a.level1[2 * row];
    need = a.level1[2 * row + 1];
    // survivors per slice -> exclusive prefix
    const uint32_t* cnt = a.slice_cnt + (int64_t)row * a.num_slices;
    uint32_t carry = 0;
    for (int s0 = 0; s0 < nsl; s0 += kResolveThreads) {
      const uint32_t c = (s0 + tid < nsl) ? cnt[s0 + tid] : 0u;
      uint32_t total;
      const uint32_t ex = block_excl_scan<kResolveThreads>(c, &total, sh.wtot);
      if (s0 + tid < nsl) sh.pre[s0 + tid] = carry + ex;
      carry += total;
    }
    if (tid == 0) sh.pre[nsl] = carry;
    __syncthreads();
    M = sh.pre[nsl];
  }
  const bool in_lds = DIRECT || M <= (uint32_t)kCap;
  const uint2* cand = a.cand + (int64_t)row * a.cand_ld;
  // survivor e (in token order) -> (key, token index)
  auto cand_at = [&](uint32_t e) -> uint2 {
    int lo = 0, hi = nsl - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (sh.pre[mid] <= e) lo = mid; else hi = mid - 1;
    }
    return cand[lo * kTopkSlice + (int)(e - sh.pre[lo])];
  };
  if (!DIRECT && in_lds) {  // survivors in batches of 4 per thread, every load of a batch in flight at once
    constexpr int kPer = 4;
    for (uint32_t e0 = 0; e0 < M; e0 += kPer * kResolveThreads) {
      uint2 kv[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const uint32_t e = e0 + tid + kResolveThreads * j;
        kv[j] = cand_at(e < M ? e : e0);  // e0 < M
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const uint32_t e = e0 + tid + kResolveThreads * j;
        if (e < M) {
          sh.key[e] = kv[j].x;
          sh.idx[e] = (int32_t)kv[j].y;
        }
      }
    }
  }
  auto key_of = [&](uint32_t e) -> uint32_t { return in_lds ? sh.key[e] : cand_at(e).x; };
  auto tok_of = [&](uint32_t e) -> int32_t { return in_lds ? sh.idx[e] : (int32_t)cand_at(e).y; };

  // the histogram is consumed: return it to zero for the next call
#pragma unroll
  for (int j = 0; j < kBins / kResolveThreads; ++j) hist_row[tid + kResolveThreads * j] = 0;

  // levels 2 and 3: key bits [20:10] and [9:0] among survivors sharing the chosen prefix.  When
  // the cut takes the whole level-2 bin (the usual case: a few hundred survivors share the top
  // 11 bits, spread over 2,048 level-2 bins), every key at or above that 21-bit prefix is in and
  // level 3 is skipped.
  uint32_t prefix = b1 << 21, mask = 0xFFE00000u;
  bool whole_bin = false;
#pragma unroll
  for (int lev = 0; lev < 2; ++lev) {
    const int shift = lev == 0 ? 10 : 0;
    const int nb = lev == 0 ? kBins : 1024;
    const uint32_t bmask = (uint32_t)nb - 1;
    for (int i = tid; i < kBins; i += kResolveThreads) sh.hist[i] = 0;
    __syncthreads();
    for (uint32_t e = tid; e < M; e += kResolveThreads) {
      const uint32_t key = key_of(e);
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & bmask], 1u);
    }
    __syncthreads();
    uint32_t rest;
    const uint32_t b = select_bin<kResolveThreads>(sh.hist, nb, need, &rest, sh.sc, sh.wtot);
    need = rest;
    prefix |= b << shift;
    mask |= bmask << shift;
    if (lev == 0 && prefix != 0u && need == sh.hist[b]) {  // uniform
      whole_bin = true;
      break;
    }
  }
  // The cut: keys above T, and of the keys equal to T the E with the lowest token index.  T is
  // the exact key of the k-th largest score, or, when the whole level-2 bin is taken, the key
  // just below that bin (and E = 0).
  const uint32_t T = whole_bin ? prefix - 1u : prefix;
  const uint32_t E = whole_bin ? 0u : need;
  if (bt_cached) {
#pragma unroll
    for (int j = 0; j < kBtPer; ++j) {
      const int i = tid + kResolveThreads * j;
      if (i < nblk) sh.bt[i] = btv[j];
    }
    __syncthreads();
  }
  auto phys_sel = [&](int s) {
    return (bt_cached ? sh.bt[s / kBlock] : bt[s / kBlock]) * kBlock + (s % kBlock);
  };

  // ordered selection over the survivors (token order)
  uint32_t gt_run = 0, eq_run = 0;
  for (uint32_t base = 0; base < M; base += 4 * kResolveThreads) {
    const uint32_t e0 = base + 4 * tid;
    uint32_t key[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = (e0 + j < M) ? key_of(e0 + j) : 0u;
    uint32_t cgt = 0, ceq = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool valid = e0 + j < M;
      cgt += (valid && key[j] > T) ? 1u : 0u;
      ceq += (valid && key[j] == T) ? 1u : 0u;
    }
    uint32_t total;
    const uint32_t ex = block_excl_scan<kResolveThreads>(cgt | (ceq << 16), &total, sh.wtot);
    uint32_t gt_before = gt_run + (ex & 0xFFFFu);
    uint32_t eq_before = eq_run + (ex >> 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (e0 + j >= M) break;
      uint32_t slot = 0xFFFFFFFFu;
      if (key[j] > T) {
        slot = gt_before + min(E, eq_before);
        ++gt_before;
      } else if (key[j] == T) {
        if (eq_before < E) slot = gt_before + eq_before;
        ++eq_before;
      }
      if (slot < (uint32_t)k) {
        const int32_t s = tok_of(e0 + j);
        out[slot] = s;
        if (phys) phys[slot] = phys_sel(s);
      }
    }
    gt_run += total & 0xFFFFu;
    eq_run += total >> 16;
    if (gt_run + min(E, eq_run) >= (uint32_t)k) break;
  }
  if (tid == 0) a.count[row] = k;
}

}  // namespace

size_t topk_workspace_bytes(int32_t num_rows, int64_t max_context) {
  const int64_t ns = (max_context + kTopkSlice - 1) / kTopkSlice;
  return (size_t)num_rows * (kBins + ns + 2 + 2 * ns * kTopkSlice + 2) * sizeof(uint32_t);
}

hipError_t launch_topk(const TopkArgs& a0, int64_t max_context, void* ws, hipStream_t s) {
  TopkArgs a = a0;
  if (a.batch.num_rows <= 0) return hipSuccess;
  const int64_t R = a.batch.num_rows;
  a.num_slices = (int32_t)((max_context + kTopkSlice - 1) / kTopkSlice);
  a.cand_ld = (int64_t)a.num_slices * kTopkSlice;
  uint32_t* w = static_cast<uint32_t*>(ws);
  uint32_t* hist_ws = w;
  a.slice_cnt = w + R * kBins;
  a.level1 = a.slice_cnt + R * a.num_slices;
  uint32_t* cand = a.level1 + 2 * R;
  cand += ((uintptr_t)cand & 7) ? 1 : 0;  // 8-byte alignment of the (key, index) pairs
  a.cand = reinterpret_cast<uint2*>(cand);
  a.vec_ok = ((a.ld & 3) == 0) && ((((uintptr_t)a.scores) & 15) == 0);
  a.max_n = (int32_t)std::min<int64_t>(max_context, kCap);
  const bool direct = max_context <= kCap;  // every row's survivors fit in LDS: no filter pass
  hipError_t e;
  if (a.hist_in == nullptr) {
    if ((e = launch_zero_u32(hist_ws, R * kBins, s)) != hipSuccess) return e;
    dim3 gh((unsigned)((max_context + kHistChunk - 1) / kHistChunk), (unsigned)R);
    hipLaunchKernelGGL(topk_hist_kernel, gh, dim3(256), 0, s, a, hist_ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    a.hist_in = hist_ws;
  }
  if (direct) {
    hipLaunchKernelGGL(topk_resolve_kernel<true>, dim3((unsigned)R), dim3(kResolveThreads), 0, s, a);
    return hipGetLastError();
  }
  const bool l1 = a.num_slices > kLevel1Slices;  // many slices per row: find each row's bin once
  if (l1) {
    hipLaunchKernelGGL(topk_level1_kernel, dim3((unsigned)R), dim3(kFilterThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (l1)
    hipLaunchKernelGGL(topk_filter_kernel<true>, dim3((unsigned)a.num_slices, (unsigned)R),
                       dim3(kFilterThreads), 0, s, a);
  else
    hipLaunchKernelGGL(topk_filter_kernel<false>, dim3((unsigned)a.num_slices, (unsigned)R),
                       dim3(kFilterThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_resolve_kernel<false>, dim3((unsigned)R), dim3(kResolveThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
