// Exact top-k over candidate lists: the select half of the candidates path, where the indexer's
// scores are never stored in full.
//
// Source: "vLLM Delivers Day-0 Support for Kimi K3.1 Pro" — §Low-latency decode: a fused DSA
// decode path (two kernels: a scorer, then an exact top-k select whose output is the pool rows
// to gather); §Sparse Attention in K3.1 Pro (keep the 2,048 highest-scoring tokens); §AMD /
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
// One workgroup per row (SRC 0: dense sample scores in; SRC 1: the candidate list in), a radix
// select on d = key - base (SRC 0: base 0; SRC 1: the row's floor, so that the candidates, which
// sit in a narrow band of keys, spread over the first digit's bins):
//   digit 1  up to 11 top bits of d over every entry -> the bin b1 holding the k-th largest; the
//            entries in bins >= b1 (the survivors) go to LDS when they fit;
//   digits 2, 3  the next bits among the entries of bin b1 -> the exact k-th key T and the number
//            E of entries equal to T that make the cut (the last digit is skipped when the cut
//            takes a whole bin);
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

// Visible sample tokens of a row at position p: the sample holds blocks 0, S, 2S, ...
__device__ __forceinline__ int sample_visible(int p, int S) {
  const int pb = p >> 6;
  const int last = S * (pb / S);
  return (pb / S) * 64 + (last == pb ? (p & 63) + 1 : 64);
}

// Every entry of a row, in batches with all of a thread's loads of a batch in flight before the
// first is used: SRC 0, 16 sample scores per thread (four 16-byte loads), SRC 1, 8 candidates
// (four 16-byte loads).  f(e, key, token) for each entry e < n.
template <int SRC, class F>
__device__ __forceinline__ void for_each_entry(const float* samp, const uint2* cand, int S,
                                               int64_t n, F f) {
  const int tid = threadIdx.x;
  constexpr int kPer = SRC == 0 ? 4 : 2;  // entries per 16-byte load
  constexpr int kU = 4;                   // loads in flight per thread
  constexpr int64_t kStep = (int64_t)kThreads * kPer * kU;
  for (int64_t b0 = 0; b0 < n; b0 += kStep) {
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t e = b0 + ((int64_t)u * kThreads + tid) * kPer;
      if (e < n) {  // rows are 256-byte aligned and padded to whole loads
        if constexpr (SRC == 0)
          v[u] = *reinterpret_cast<const uint4*>(samp + e);
        else
          v[u] = *reinterpret_cast<const uint4*>(cand + e);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t e = b0 + ((int64_t)u * kThreads + tid) * kPer;
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if (e + j >= n) break;
        if constexpr (SRC == 0) {
          // sample token e is token 64 S (e / 64) + e % 64 of the sequence
          const int64_t x = e + j;
          f(x, order_key(__uint_as_float(w[j])),
            (uint32_t)((((x >> 6) * S) << 6) | (x & 63)));
        } else {
          f(e + j, w[2 * j], w[2 * j + 1]);
        }
      }
    }
  }
}

// The radix select works on d = key - base, in up to three digits from the top: bits
// [s0, s0 + 11), [s1, s0), [0, s1), s0 = max(0, bits(range) - 11), s1 = max(0, s0 - 11).  With
// base 0 and range 2^32 this is the plain 11 + 11 + 10 split of the key; for a candidate list
// base is the row's floor and range its largest key minus the floor, so that the candidates,
// which sit in a narrow band of keys, spread over the first digit's bins.
template <int SRC>
__global__ __launch_bounds__(kThreads) void cand_select_kernel(CandArgs a) {
  __shared__ Shared sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = a.k;
  const float* samp = a.samp + (int64_t)row * a.samp_ld;
  const uint2* cand = a.cand + (int64_t)row * a.cand_cap;
  const int S = a.sample_stride;
  int32_t* out = a.idx + (int64_t)row * k;
  int32_t* phys = a.phys ? a.phys + (int64_t)row * k : nullptr;
  uint2* cand_out = a.cand + (int64_t)row * a.cand_cap;

  int64_t n;
  uint32_t base = 0, range_bits = 32;
  if constexpr (SRC == 0) {
    n = sample_visible(a.batch.row_pos[row], S);
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
    base = a.floor[2 * row];
    const uint32_t range = a.cand_max[row] - base;  // every candidate key is >= the floor
    range_bits = range ? 32 - __builtin_clz(range) : 1;
  }
  const uint32_t need = (uint32_t)min<int64_t>(k, n);
  const int s0 = max(0, (int)range_bits - 11);
  const int s1 = max(0, s0 - 11);

  // The cut: key > T, or key == T and token <= I.
  uint32_t T = 0;
  int32_t I = 0x7FFFFFFF;
  const bool take_all = n <= k;
  bool in_lds = false;
  uint32_t nsurv = 0;
  if (!take_all) {
    // first digit over every entry
    for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0;
    if (tid == 0) sh.nsurv = 0;
    __syncthreads();
    for_each_entry<SRC>(samp, cand, S, n, [&](int64_t, uint32_t key, uint32_t) {
      atomicAdd(&sh.hist[(key - base) >> s0], 1u);
    });
    __syncthreads();
    uint32_t rest;
    const uint32_t b1 = find_bin(sh.hist, kBins, need, true, &rest, sh);
    nsurv = need - rest + sh.hist[b1];  // entries in bins >= b1
    in_lds = nsurv <= (uint32_t)kLdsCap;
    if (in_lds) {
      for_each_entry<SRC>(samp, cand, S, n, [&](int64_t, uint32_t key, uint32_t tok) {
        if (((key - base) >> s0) >= b1) {
          const uint32_t p = atomicAdd(&sh.nsurv, 1u);
          sh.key[p] = key;
          sh.tok[p] = (int32_t)tok;
        }
      });
    }
    __syncthreads();
    // the survivors (LDS), or every entry again; f(key, token) for each
    auto survivors = [&](auto f) {
      if (in_lds) {
        for (uint32_t e = tid; e < nsurv; e += kThreads) f(sh.key[e], (uint32_t)sh.tok[e]);
      } else {
        for_each_entry<SRC>(samp, cand, S, n, [&](int64_t, uint32_t key, uint32_t tok) {
          f(key, tok);
        });
      }
    };
    // the remaining digits within bin b1
    uint32_t prefix = b1 << s0;                      // of d
    uint32_t mask = range_bits >= 32 ? ~0u << s0 : ((1u << range_bits) - 1) & (~0u << s0);
    bool whole_bin = false;
    uint32_t tied = sh.hist[b1];
    int lo = s0;
    for (int lev = 0; lev < 2 && lo > 0; ++lev) {
      const int shift = lev == 0 ? s1 : 0;
      const int width = lo - shift;
      const uint32_t bmask = (1u << width) - 1;
      for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0;
      __syncthreads();
      survivors([&](uint32_t key, uint32_t) {
        const uint32_t d = key - base;
        if ((d & mask) == prefix) atomicAdd(&sh.hist[(d >> shift) & bmask], 1u);
      });
      __syncthreads();
      uint32_t r2;
      const uint32_t b = find_bin(sh.hist, kBins, rest, true, &r2, sh);
      const uint32_t hb = sh.hist[b];
      __syncthreads();
      rest = r2;
      prefix |= b << shift;
      mask |= bmask << shift;
      tied = hb;
      lo = shift;
      if (lo > 0 && prefix != 0u && rest == hb) {  // the cut takes the whole bin
        whole_bin = true;
        break;
      }
    }
    if (whole_bin) {
      T = base + prefix - 1u;  // every key from the bin up is in; nothing at T itself
      I = -1;
    } else {  // every digit resolved (lo == 0)
      T = base + prefix;  // the exact k-th key; `rest` of the `tied` keys equal to it are taken
      if (rest < tied) {
        // the rest-th lowest token index among the keys equal to T: two 12-bit digits
        uint32_t tp = 0, need_t = rest;
        for (int lev = 0; lev < 2; ++lev) {
          const int shift = lev == 0 ? 12 : 0;
          for (int i = tid; i < kTieBins; i += kThreads) sh.hist[i] = 0;
          __syncthreads();
          survivors([&](uint32_t key, uint32_t tok) {
            if (key == T && (lev == 0 || (tok >> 12) == (tp >> 12)))
              atomicAdd(&sh.hist[(tok >> shift) & 0xFFFu], 1u);
          });
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
  uint32_t kmax = 0;
  __syncthreads();
  auto emit = [&](uint32_t key, uint32_t tok) {
    if (key > T || (key == T && (int32_t)tok <= I)) {
      const uint32_t p = atomicAdd(&sh.nsel, 1u);
      if constexpr (SRC == 0) {
        cand_out[p] = uint2{key, tok};
        kmax = max(kmax, key);
      } else {
        sh.sel[p] = (int32_t)tok;
      }
    }
  };
  if (!take_all && in_lds) {
    for (uint32_t e = tid; e < nsurv; e += kThreads) emit(sh.key[e], (uint32_t)sh.tok[e]);
  } else {
    for_each_entry<SRC>(samp, cand, S, n, [&](int64_t, uint32_t key, uint32_t tok) {
      emit(key, tok);
    });
  }
  if constexpr (SRC == 0) {
    // the largest key among the row's first candidates (the candidate pass raises it)
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, d, 64));
    if ((tid & 63) == 0) sh.sc[tid >> 6] = kmax;
    __syncthreads();
    if (tid == 0) {
      uint32_t m = 0;
      for (int w = 0; w < kWaves; ++w) m = max(m, sh.sc[w]);
      a.cand_count[row] = (int32_t)need;
      a.cand_max[row] = m;
      // the floor the candidate pass applies to the other tokens: with the whole sample taken
      // (no more than k visible sample tokens) nothing can be ruled out
      a.floor[2 * row] = take_all ? 0u : T;
      a.floor[2 * row + 1] = take_all ? 0x7FFFFFFFu : (uint32_t)I;
    }
    return;
  } else {
    __syncthreads();
    // bitonic sort of the selected token indices, ascending (unused slots hold INT_MAX)
    for (int size = 2; size <= kSort; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = tid; t < kSort / 2; t += kThreads) {
          const int lo2 = 2 * t - (t & (stride - 1));
          const int hi2 = lo2 + stride;
          const bool up = (lo2 & size) == 0;
          const int32_t x = sh.sel[lo2], y = sh.sel[hi2];
          if ((x > y) == up) {
            sh.sel[lo2] = y;
            sh.sel[hi2] = x;
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
