// Exact top-k over candidate lists: the select half of the candidates path, where the indexer's
// scores are never stored in full.
//
// Source: "vLLM Delivers Day-0 Support for Kimi K3.1 Pro" — §Low-latency decode: a fused DSA
// decode path (a scorer and an exact top-k select in two kernels, the select emitting physical KV
// rows); §Sparse Attention in K3.1 Pro (keep the 2,048 highest-scoring tokens); §AMD /
// Communication (a consistent tie rule: here the lower token index wins, -0 ties +0).
//
// Why a candidate list is exact.  The scorer first scores a sample of each sequence (every S-th
// 64-token block).  If the sample holds at least k visible tokens, its k-th largest key T is a
// lower bound on the whole row's k-th largest: a token with a smaller key is beaten by k sample
// tokens.  With ties broken by index, a token whose key equals T is beaten by k sample tokens too
// when its index exceeds I, the index of the last sample token tied at T that the sample's own
// top-k takes.  So the sample's top-k plus every other token with key > T, or key == T and index
// < I, contains the row's top-k; the candidate pass appends exactly those.
//
// One workgroup per row (SRC 0: dense sample scores in; SRC 1: the candidate list in):
//   level 1  11-bit radix histogram of every entry's key -> the bin b1 holding the k-th largest;
//            the entries in bins >= b1 (the survivors) go to LDS when they fit;
//   level 2  bits [20:10] among the entries of bin b1; level 3, bits [9:0] -> the exact k-th key
//            T and the number E of entries equal to T that make the cut (level 3 is skipped when
//            the cut takes a whole level-2 bin);
//   ties     when only some of the entries equal to T are taken, a radix select over their token
//            indices (12 + 12 bits, ascending) finds the E-th lowest index I;
//   emit     key > T, or key == T and index <= I: exactly min(k, entries).  SRC 0 leaves them as
//            the row's first candidates, with the floor (T, I); SRC 1 sorts their token indices
//            ascending (bitonic, in LDS) and writes idx, count and the physical pool rows.
#include "dsa_kernels.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = DSA_HIST_BINS;  // 2048
constexpr int kTieBins = 4096;        // 12-bit digits of a token index (< 2^24)
constexpr int kLdsCap = 8192;         // survivors held in LDS
constexpr int kSort = DSA_MAX_TOPK;   // 2048 slots of the final sort

struct Shared {
  uint32_t hist[kTieBins];
  uint32_t key[kLdsCap];
  int32_t tok[kLdsCap];
  int32_t sel[kSort];
  uint32_t sc[kThreads + 4];
  uint32_t wtot[kWaves];
  uint32_t nsurv, nsel;
};

__device__ __forceinline__ int row_seq(const BatchView& b, int row) {
  int lo = 0, hi = b.num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (b.seq_row_start[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Block-wide exclusive prefix sum in thread order; *total receives the block sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, uint32_t* wtot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const uint32_t t = wtot[i];
    before += (i < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// The bin of an nbins-bin LDS histogram that holds the need-th element counted from the top bin
// down (desc) or from bin 0 up (!desc): before(b) < need <= before(b) + hist[b], where before(b)
// counts the bins met first.  Returns b; *rest = need - before(b).  Every thread gets both.
__device__ uint32_t find_bin(const uint32_t* hist, int nbins, uint32_t need, bool desc,
                             uint32_t* rest, Shared& sh) {
  const int tid = threadIdx.x;
  const int per = nbins / kThreads;  // 2 or 4 bins per thread
  // thread t owns the per bins met in position t of the walk
  auto bin_at = [&](int t, int j) { return desc ? nbins - 1 - (per * t + j) : per * t + j; };
  uint32_t own = 0;
  for (int j = 0; j < per; ++j) own += hist[bin_at(tid, j)];
  uint32_t total;
  uint32_t before = block_excl_scan(own, &total, sh.wtot);
  for (int j = 0; j < per; ++j) {
    const int b = bin_at(tid, j);
    const uint32_t h = hist[b];
    if (h && before < need && need <= before + h) {
      sh.sc[0] = (uint32_t)b;
      sh.sc[1] = need - before;
    }
    before += h;
  }
  __syncthreads();
  const uint32_t b = sh.sc[0];
  *rest = sh.sc[1];
  __syncthreads();
  return b;
}

template <int SRC>
struct Source {
  const float* samp;
  const uint2* cand;
  int S;
  __device__ __forceinline__ uint2 at(int64_t e) const {
    if constexpr (SRC == 0) {
      // sample token e is token 64 S (e / 64) + e % 64 of the sequence
      const uint32_t t = (uint32_t)(((e >> 6) * S) << 6) | (uint32_t)(e & 63);
      return uint2{order_key(samp[e]), t};
    } else {
      return cand[e];
    }
  }
};

// Visible sample tokens of a row at position p: the sample holds blocks 0, S, 2S, ...
__device__ __forceinline__ int sample_visible(int p, int S) {
  const int pb = p >> 6;
  const int last = S * (pb / S);
  return (pb / S) * 64 + (last == pb ? (p & 63) + 1 : 64);
}

template <int SRC>
__global__ __launch_bounds__(kThreads) void cand_select_kernel(CandArgs a) {
  __shared__ Shared sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = a.k;
  Source<SRC> src{a.samp + (int64_t)row * a.samp_ld, a.cand + (int64_t)row * a.cand_cap,
                  a.sample_stride};
  int32_t* out = a.idx + (int64_t)row * k;
  int32_t* phys = a.phys ? a.phys + (int64_t)row * k : nullptr;
  uint2* cand_out = a.cand + (int64_t)row * a.cand_cap;

  int64_t n;
  if constexpr (SRC == 0) {
    n = sample_visible(a.batch.row_pos[row], a.sample_stride);
  } else {
    const int64_t got = a.cand_count[row];
    bool bad = got > a.cand_cap;
    if (bad && tid == 0) atomicOr(a.status, DSA_DEVERR_CAND_OVERFLOW);
    bad = bad || (*a.status & DSA_DEVERR_ROWS_PER_SEQ);  // some scorer skipped rows
    if (bad) {  // candidates were lost: nothing is selected
      for (int i = tid; i < k; i += kThreads) {
        out[i] = -1;
        if (phys) phys[i] = -1;
      }
      if (tid == 0) a.count[row] = -1;
      return;
    }
    n = got;
  }
  const uint32_t need = (uint32_t)min<int64_t>(k, n);

  // T, E and I define the cut: key > T, or key == T and token <= I.
  uint32_t T = 0;
  int32_t I = -1;
  bool take_all = n <= k;
  bool in_lds = false;
  if (take_all) {
    T = 0;          // every key of a finite score is above 0
    I = 0x7FFFFFFF;
  } else {
    // level 1 over every entry
    for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0;
    if (tid == 0) sh.nsurv = 0;
    __syncthreads();
    for (int64_t e = tid; e < n; e += kThreads) atomicAdd(&sh.hist[src.at(e).x >> 21], 1u);
    __syncthreads();
    uint32_t rest;
    const uint32_t b1 = find_bin(sh.hist, kBins, need, true, &rest, sh);
    const uint32_t nsurv = need - rest + sh.hist[b1];  // entries in bins >= b1
    in_lds = nsurv <= (uint32_t)kLdsCap;
    if (in_lds) {
      for (int64_t e = tid; e < n; e += kThreads) {
        const uint2 v = src.at(e);
        if ((v.x >> 21) >= b1) {
          const uint32_t p = atomicAdd(&sh.nsurv, 1u);
          sh.key[p] = v.x;
          sh.tok[p] = (int32_t)v.y;
        }
      }
    }
    __syncthreads();
    const int64_t m = in_lds ? (int64_t)nsurv : n;
    auto get = [&](int64_t e) -> uint2 {
      return in_lds ? uint2{sh.key[e], (uint32_t)sh.tok[e]} : src.at(e);
    };
    // levels 2 and 3 within bin b1
    uint32_t prefix = b1 << 21, mask = 0xFFE00000u;
    bool whole_bin = false;
    uint32_t tied = 0;
    for (int lev = 0; lev < 2; ++lev) {
      const int shift = lev == 0 ? 10 : 0;
      const int nb = lev == 0 ? kBins : 1024;
      const uint32_t bmask = (uint32_t)nb - 1;
      for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0;
      __syncthreads();
      for (int64_t e = tid; e < m; e += kThreads) {
        const uint32_t key = get(e).x;
        if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & bmask], 1u);
      }
      __syncthreads();
      uint32_t r2;
      const uint32_t b = find_bin(sh.hist, kBins, rest, true, &r2, sh);
      const uint32_t hb = sh.hist[b];
      __syncthreads();
      rest = r2;
      prefix |= b << shift;
      mask |= bmask << shift;
      tied = hb;
      if (lev == 0 && prefix != 0u && rest == hb) {  // the cut takes the whole level-2 bin
        whole_bin = true;
        break;
      }
    }
    if (whole_bin) {
      T = prefix - 1u;  // every key from the bin up is in; nothing at T itself
      I = -1;
    } else {
      T = prefix;  // the exact k-th key; `rest` of the `tied` keys equal to it are taken
      if (rest == tied) {
        I = 0x7FFFFFFF;
      } else {
        // the rest-th lowest token index among the keys equal to T: two 12-bit digits
        uint32_t tp = 0, need_t = rest;
        for (int lev = 0; lev < 2; ++lev) {
          const int shift = lev == 0 ? 12 : 0;
          for (int i = tid; i < kTieBins; i += kThreads) sh.hist[i] = 0;
          __syncthreads();
          for (int64_t e = tid; e < m; e += kThreads) {
            const uint2 v = get(e);
            if (v.x == T && (lev == 0 || (v.y >> 12) == (tp >> 12)))
              atomicAdd(&sh.hist[(v.y >> shift) & 0xFFFu], 1u);
          }
          __syncthreads();
          uint32_t r3;
          const uint32_t b = find_bin(sh.hist, kTieBins, need_t, false, &r3, sh);
          need_t = r3;
          tp |= b << shift;
        }
        I = (int32_t)tp;
      }
    }
  }

  // emission: exactly `need` entries
  if (tid == 0) sh.nsel = 0;
  for (int i = tid; i < kSort; i += kThreads) sh.sel[i] = 0x7FFFFFFF;
  __syncthreads();
  {
    const int64_t m = take_all ? n : (in_lds ? (int64_t)sh.nsurv : n);
    for (int64_t e = tid; e < m; e += kThreads) {
      const uint2 v = (!take_all && in_lds) ? uint2{sh.key[e], (uint32_t)sh.tok[e]} : src.at(e);
      if (v.x > T || (v.x == T && (int32_t)v.y <= I)) {
        const uint32_t p = atomicAdd(&sh.nsel, 1u);
        if constexpr (SRC == 0)
          cand_out[p] = v;
        else
          sh.sel[p] = (int32_t)v.y;
      }
    }
  }
  __syncthreads();
  if constexpr (SRC == 0) {
    if (tid == 0) {
      a.cand_count[row] = (int32_t)need;
      // the floor the candidate pass applies to the other tokens: with the whole sample taken
      // (fewer than k visible sample tokens) nothing can be ruled out
      a.floor[2 * row] = take_all ? 0u : T;
      a.floor[2 * row + 1] = take_all ? 0x7FFFFFFFu : (uint32_t)I;
    }
    return;
  } else {
    // bitonic sort of the selected token indices, ascending (unused slots hold INT_MAX)
    for (int size = 2; size <= kSort; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = tid; t < kSort / 2; t += kThreads) {
          const int lo = 2 * t - (t & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const int32_t x = sh.sel[lo], y = sh.sel[hi];
          if ((x > y) == up) {
            sh.sel[lo] = y;
            sh.sel[hi] = x;
          }
        }
        __syncthreads();
      }
    }
    const int32_t* bt = a.batch.block_table + (int64_t)row_seq(a.batch, row) * a.batch.ld_bt;
    for (int i = tid; i < k; i += kThreads) {
      const int32_t s = i < (int)need ? sh.sel[i] : -1;
      out[i] = s;
      if (phys) phys[i] = s >= 0 ? bt[s / kBlock] * kBlock + (s % kBlock) : -1;
    }
    if (tid == 0) a.count[row] = (int32_t)need;
  }
}

}  // namespace

hipError_t launch_cand_select(const CandArgs& a, int src, hipStream_t s) {
  if (a.batch.num_rows <= 0) return hipSuccess;
  if (src == 0)
    hipLaunchKernelGGL(cand_select_kernel<0>, dim3((unsigned)a.batch.num_rows), dim3(kThreads), 0,
                       s, a);
  else
    hipLaunchKernelGGL(cand_select_kernel<1>, dim3((unsigned)a.batch.num_rows), dim3(kThreads), 0,
                       s, a);
  return hipGetLastError();
}

}  // namespace dsa
