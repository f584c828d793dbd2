// Exact top-k select over materialised indexer scores.
//
// Source: "vLLM Delivers Day-0 Support for Kimi K3.1 Pro" — §Sparse Attention in K3.1 Pro (keep
// the 2,048 highest-scoring tokens); §Low-latency decode (an exact top-k select that emits the
// physical KV rows the attention reads); §An exact top-k merge (a radix select); §AMD /
// Communication (a consistent tie rule).  Tie rule used here: the lower token index wins; -0 and
// +0 tie.
//
// Per row, one 1024-thread workgroup:
//   1. 11-bit radix histogram of the order-preserving keys (given by the scorer, or one pass);
//   2. the bin holding the k-th largest key; its members are compacted into LDS and refined by
//      two more radix levels (11 + 10 bits) to the exact k-th key T and the number E of keys
//      equal to T that make the cut (falling back to passes over global memory when the bin does
//      not fit in LDS);
//   3. one ordered pass: a token is selected if key > T, or key == T and fewer than E keys equal
//      to T precede it.  A block-wide prefix sum in token order gives each selected token its
//      output slot, so the output comes out in ascending token order with no sort.
#include "dsa_kernels.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = DSA_HIST_BINS;
constexpr int kCap = 6144;  // LDS candidates of the threshold bin

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t cand_key[kCap];
  int32_t cand_idx[kCap];
  uint32_t wave_tot[kWaves];
  uint32_t bcast[4];
};

// Block-wide exclusive prefix sum of v in thread order; *total gets the sum over the block.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, TopkShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t incl = wave_incl_scan(v);
  if (lane == 63) sh.wave_tot[wave] = incl;
  __syncthreads();
  uint32_t wsum = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    uint32_t t = sh.wave_tot[i];
    wsum += (i < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return wsum + incl - v;
}

// Given a histogram of nbins bins (bin index increasing with the key), find the bin b holding the
// need-th largest element: above(b) < need <= above(b) + hist[b].  Returns b and, in *need_in_bin,
// need - above(b).  Every thread gets the result.
__device__ uint32_t select_bin(TopkShared& sh, int nbins, uint32_t need, uint32_t* need_in_bin) {
  const int tid = threadIdx.x;
  const int per = nbins / kThreads;  // 1 or 2 bins per thread
  // thread t owns bins [per*t, per*t + per); count elements in bins owned by higher threads
  uint32_t own = 0;
  for (int j = 0; j < per; ++j) own += sh.hist[per * tid + j];
  // exclusive scan in reverse thread order
  const int rt = kThreads - 1 - tid;
  uint32_t total;
  // reverse order: do the scan on a permuted index by exchanging through LDS
  __shared__ uint32_t tmp[kThreads];
  tmp[rt] = own;
  __syncthreads();
  uint32_t mine = tmp[tid];  // value of thread (kThreads-1-tid)
  __syncthreads();
  uint32_t ex = block_excl_scan(mine, &total, sh);  // sum over threads with larger index than rt
  tmp[tid] = ex;
  __syncthreads();
  uint32_t above = tmp[rt];  // elements in bins of threads > tid
  __syncthreads();
  for (int j = per - 1; j >= 0; --j) {
    const int b = per * tid + j;
    const uint32_t h = sh.hist[b];
    if (h && above < need && need <= above + h) {
      sh.bcast[0] = (uint32_t)b;
      sh.bcast[1] = need - above;
    }
    above += h;
  }
  __syncthreads();
  uint32_t b = sh.bcast[0];
  *need_in_bin = sh.bcast[1];
  __syncthreads();
  return b;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  __shared__ TopkShared sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = a.k;
  const int n = a.batch.row_pos[row] + 1;
  int32_t* out = a.idx + (int64_t)row * k;
  int32_t* phys = a.phys ? a.phys + (int64_t)row * k : nullptr;

  // sequence of this row (rows are grouped by sequence)
  if (tid == 0) {
    int lo = 0, hi = a.batch.num_seqs - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (a.batch.seq_row_start[mid] <= row) lo = mid; else hi = mid - 1;
    }
    sh.bcast[2] = (uint32_t)lo;
  }
  __syncthreads();
  const int seq = (int)sh.bcast[2];
  const int32_t* bt = a.batch.block_table + (int64_t)seq * a.batch.ld_bt;
  auto phys_of = [&](int s) { return bt[s / kBlock] * kBlock + (s % kBlock); };

  if (n <= k) {  // everything visible is selected
    for (int i = tid; i < k; i += kThreads) {
      out[i] = i < n ? i : -1;
      if (phys) phys[i] = i < n ? phys_of(i) : -1;
    }
    if (tid == 0) a.count[row] = n;
    return;
  }
  const float* sc = a.scores + (int64_t)row * a.ld;

  // ---- level 1: histogram of key bits [31:21]
  if (a.hist) {
    for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = a.hist[(int64_t)row * kBins + i];
  } else {
    for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int s = tid; s < n; s += kThreads) atomicAdd(&sh.hist[order_key(sc[s]) >> 21], 1u);
  }
  __syncthreads();
  uint32_t need;
  const uint32_t b1 = select_bin(sh, kBins, (uint32_t)k, &need);

  // ---- compact the threshold bin's members into LDS
  if (tid == 0) sh.bcast[3] = 0;
  __syncthreads();
  for (int s = tid; s < n; s += kThreads) {
    const uint32_t key = order_key(sc[s]);
    if ((key >> 21) == b1) {
      const uint32_t p = atomicAdd(&sh.bcast[3], 1u);
      if (p < kCap) {
        sh.cand_key[p] = key;
        sh.cand_idx[p] = s;
      }
    }
  }
  __syncthreads();
  const uint32_t ncand = sh.bcast[3];
  const bool in_lds = ncand <= (uint32_t)kCap;
  __syncthreads();

  // ---- levels 2 and 3: bits [20:10] and [9:0] among keys with the chosen prefix
  uint32_t prefix = b1 << 21, mask = 0xFFE00000u;
  const int shifts[2] = {10, 0};
  const int widths[2] = {kBins, 1024};
  for (int lev = 0; lev < 2; ++lev) {
    const int sh_ = shifts[lev];
    const uint32_t bmask = (uint32_t)widths[lev] - 1;
    for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    if (in_lds) {
      for (uint32_t c = tid; c < ncand; c += kThreads) {
        const uint32_t key = sh.cand_key[c];
        if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> sh_) & bmask], 1u);
      }
    } else {
      for (int s = tid; s < n; s += kThreads) {
        const uint32_t key = order_key(sc[s]);
        if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> sh_) & bmask], 1u);
      }
    }
    __syncthreads();
    uint32_t need2;
    const uint32_t b = select_bin(sh, widths[lev], need, &need2);
    need = need2;
    prefix |= b << sh_;
    mask |= bmask << sh_;
  }
  const uint32_t T = prefix;  // exact key of the k-th largest score
  const uint32_t E = need;    // keys equal to T that are selected (the lowest-index ones)

  // ---- ordered selection pass
  uint32_t gt_run = 0, eq_run = 0;
  const bool vec = ((a.ld & 3) == 0) && ((((uintptr_t)sc) & 15) == 0);
  for (int base = 0; base < n; base += 4 * kThreads) {
    const int s0 = base + 4 * tid;
    uint32_t key[4];
    if (vec && s0 + 3 < n) {
      const float4 v = *reinterpret_cast<const float4*>(sc + s0);
      key[0] = order_key(v.x);
      key[1] = order_key(v.y);
      key[2] = order_key(v.z);
      key[3] = order_key(v.w);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) key[j] = (s0 + j < n) ? order_key(sc[s0 + j]) : 0u;
    }
    uint32_t cgt = 0, ceq = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool valid = s0 + j < n;
      cgt += (valid && key[j] > T) ? 1u : 0u;
      ceq += (valid && key[j] == T) ? 1u : 0u;
    }
    uint32_t total;
    const uint32_t ex = block_excl_scan(cgt | (ceq << 16), &total, sh);
    uint32_t gt_before = gt_run + (ex & 0xFFFFu);
    uint32_t eq_before = eq_run + (ex >> 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = s0 + j;
      if (s >= n) break;
      if (key[j] > T) {
        const uint32_t slot = gt_before + min(E, eq_before);
        if (slot < (uint32_t)k) {
          out[slot] = s;
          if (phys) phys[slot] = phys_of(s);
        }
        ++gt_before;
      } else if (key[j] == T) {
        if (eq_before < E) {
          const uint32_t slot = gt_before + eq_before;
          if (slot < (uint32_t)k) {
            out[slot] = s;
            if (phys) phys[slot] = phys_of(s);
          }
        }
        ++eq_before;
      }
    }
    gt_run += total & 0xFFFFu;
    eq_run += total >> 16;
    if (gt_run + min(E, eq_run) >= (uint32_t)k) break;
  }
  if (tid == 0) a.count[row] = k;
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.batch.num_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.batch.num_rows), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
