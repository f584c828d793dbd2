// Decode context parallelism emulated on one GPU ("vLLM Delivers Day-0 Support for Kimi K3.1
// Pro", §Long context: decode context parallelism with a sparse indexer; §An exact top-k merge with
// 10x less traffic; §AMD / Communication: Efficient cross-GPU communication).
//
// Shard r of W holds tokens r, r + W, ... of each sequence in a pool of its own; its scorer and
// select give each row a local top-k.  Here:
//   publish  - each shard sorts its local top-k by (score desc, token index asc) into a mailbox
//              (the buffer a peer-mapped exchange would fill; the sorted list stays "local", and
//              the merge reads from it only what the chosen message carries);
//   merge    - the select every shard runs on the gathered messages: a block-wide radix select of
//              the k-th largest message key, a resend round for shards whose weakest sent
//              candidate reaches that threshold, and an exact tie round for entries equal to it;
//              it emits the global top-k (ascending) and each shard's own part of it;
// The shards' attention partials and their log-sum-exp combine are the attention's own split
// partials and split combine (sparse_mla.hip), over a buffer that holds every shard's splits.
// Message variants: PACKED (best ceil(1.5 k / W) candidates per shard, 32 bits each: the top 16
// bits of the score's order key and the candidate's 16-bit rank in its shard's list), SCORES (the
// whole local top-k as fp32 scores, indices kept local), GENERIC (the whole local top-k as (fp32
// score, index) pairs).  The result is the exact global top-k in every variant.
#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kMT = 1024;  // threads per row of the publish and merge kernels

struct Mailbox {
  uint32_t* key;  // [W][R][k] order keys, sorted descending per (shard, row)
  int32_t* gid;   // [W][R][k] global token indices
  int32_t* cnt;   // [W][R] list lengths
};

__device__ __forceinline__ Mailbox mailbox_view(void* mb, int W, int R, int k) {
  Mailbox m;
  const size_t n = (size_t)W * R * k;
  m.key = static_cast<uint32_t*>(mb);
  m.gid = reinterpret_cast<int32_t*>(m.key + n);
  m.cnt = m.gid + n;
  return m;
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int p = 64;
  while (p < n) p <<= 1;
  return p;
}

// Bitonic sort of 2,048 values, two per thread in registers (thread t holds elements 2t and
// 2t + 1), by the whole workgroup.  Compare-exchange stages of stride 1 stay in the thread, strides
// 2..64 pair lanes of one wave (a shuffle), and only strides of 128 and more go through LDS (xch,
// 2,048 values) with two barriers each: 10 of the 66 stages.
template <typename T>
__device__ __forceinline__ T shfl_xor_t(T v, int m) {
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = (uint64_t)v;
    const uint32_t lo = __shfl_xor((uint32_t)u, m, 64), hi = __shfl_xor((uint32_t)(u >> 32), m, 64);
    return (T)(((uint64_t)hi << 32) | lo);
  } else {
    return (T)__shfl_xor(v, m, 64);
  }
}

template <typename T, bool kDescending>
__device__ void block_sort2048(T& v0, T& v1, T* xch) {
  const int t = threadIdx.x;
  for (int size = 2; size <= 2048; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 128) {  // partners in other waves: through LDS
        xch[2 * t] = v0;
        xch[2 * t + 1] = v1;
        __syncthreads();
      }
      T e[2] = {v0, v1};
      if (stride == 1) {
        const bool up = ((2 * t) & size) == 0 ? !kDescending : kDescending;
        const bool sw = up ? (e[0] > e[1]) : (e[0] < e[1]);
        const T a = e[0];
        e[0] = sw ? e[1] : a;
        e[1] = sw ? a : e[1];
      } else {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          const int i = 2 * t + sl;
          const T other = stride <= 64 ? shfl_xor_t(e[sl], stride >> 1) : xch[i ^ stride];
          const bool up = (i & size) == 0 ? !kDescending : kDescending;
          const bool keep_small = ((i & stride) == 0) == up;  // lower index of an ascending pair
          e[sl] = keep_small ? (other < e[sl] ? other : e[sl]) : (other > e[sl] ? other : e[sl]);
        }
      }
      if (stride >= 128) __syncthreads();  // every read of xch done before the next write
      v0 = e[0];
      v1 = e[1];
    }
  }
}

__global__ __launch_bounds__(kMT) void dcp_publish_kernel(int R, int k, int W, int shard,
                                                          const float* __restrict__ scores,
                                                          int64_t ld, const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ count,
                                                          void* mb) {
  __shared__ uint64_t xch[2048];
  const int row = blockIdx.x, t = threadIdx.x;
  const Mailbox m = mailbox_view(mb, W, R, k);
  const int cnt = min(max(count[row], 0), k);
  // (order key, ~local index): descending = score descending, index ascending; 0 pads (no real
  // entry is 0) and sorts last
  uint64_t v[2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    const int i = 2 * t + sl;
    v[sl] = 0;
    if (i < cnt) {
      const uint32_t j = (uint32_t)idx[(int64_t)row * k + i];
      v[sl] = ((uint64_t)order_key(scores[(int64_t)row * ld + j]) << 32) | (0xFFFFFFFFu - j);
    }
  }
  block_sort2048<uint64_t, true>(v[0], v[1], xch);
  const size_t base = ((size_t)shard * R + row) * k;
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    const int i = 2 * t + sl;
    if (i < cnt) {
      m.key[base + i] = (uint32_t)(v[sl] >> 32);
      m.gid[base + i] = (int32_t)(0xFFFFFFFFu - (uint32_t)v[sl]) * W + shard;
    }
  }
  if (t == 0) m.cnt[(size_t)shard * R + row] = cnt;
}

constexpr int kMaxPer = 16;  // message entries per thread: up to 16,384 per row (8 shards x 2,048)

struct MergeShared {
  uint32_t hist[256];
  int32_t sel[2048];
  uint32_t wtot[16], wofs[16];
  int32_t cnt[16], n[16], flag[16], pre[17];
  uint32_t digit, above, eq;
  int32_t nsel;
};

// The want-th largest key (1 <= want <= number of active entries) among this workgroup's entries,
// all active keys sharing the bits above their low nbits (a multiple of 8), which equal those of
// `high`: 8-bit digits from bit nbits down, one histogram pass each over the entries that match the
// digits found so far.  key_of(j, act) gives the key of this thread's j-th entry.  Returns the key;
// *gt / *eq = active entries above / equal to it.
template <class KeyOf>
__device__ uint64_t block_select_desc(MergeShared& sh, int N, KeyOf key_of, int want, int nbits,
                                      int* gt, int* eq, uint64_t high = 0) {
  uint64_t mask = nbits >= 64 ? 0 : ~0ull << nbits;
  uint64_t T = high & mask;
  int rem = want;
  uint32_t last_eq = 0;
  const int lane = threadIdx.x & 63;
  for (int shift = nbits - 8; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) sh.hist[threadIdx.x] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j)
      if ((int)threadIdx.x + kMT * j < N) {
        bool act;
        const uint64_t kk = key_of(j, act);
        if (act && (kk & mask) == T) atomicAdd(&sh.hist[(kk >> shift) & 255u], 1u);
      }
    __syncthreads();
    if (threadIdx.x < 64) {
      const uint32_t h0 = sh.hist[4 * lane], h1 = sh.hist[4 * lane + 1],
                     h2 = sh.hist[4 * lane + 2], h3 = sh.hist[4 * lane + 3];
      const uint32_t s = h0 + h1 + h2 + h3;
      uint32_t suf = s;  // sum over lanes >= this one
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t t = __shfl_down(suf, d, 64);
        if (lane + d < 64) suf += t;
      }
      uint32_t above = suf - s;
      const uint32_t hb[4] = {h0, h1, h2, h3};
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < (uint32_t)rem && (uint32_t)rem <= above + hb[j]) {
          sh.digit = 4 * lane + j;
          sh.above = above;
          sh.eq = hb[j];
        }
        above += hb[j];
      }
    }
    __syncthreads();
    T |= (uint64_t)sh.digit << shift;
    mask |= (uint64_t)0xFF << shift;
    rem -= (int)sh.above;
    last_eq = sh.eq;
    __syncthreads();
  }
  *gt = want - rem;
  *eq = (int)last_eq;
  return T;
}

template <int variant>
__global__ __launch_bounds__(kMT) void dcp_merge_kernel(int R, int k, int W,
                                                        void* mb, int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ count,
                                                        int32_t* __restrict__ shard_idx,
                                                        int32_t* __restrict__ shard_count,
                                                        int32_t* __restrict__ stats) {
  __shared__ MergeShared sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Mailbox m = mailbox_view(mb, W, R, k);
  const int C = variant == DSA_MERGE_PACKED ? min(k, (3 * k + 2 * W - 1) / (2 * W)) : k;
  constexpr int wbytes = variant == DSA_MERGE_GENERIC ? 8 : 4;
  if (tid < W) {
    const int c = min(max(m.cnt[(size_t)tid * R + row], 0), k);  // a list holds at most k
    sh.cnt[tid] = c;
    sh.n[tid] = min(C, c);
  }
  __syncthreads();
  int payload = 0;
  for (int r = 0; r < W; ++r) payload += sh.n[r] * wbytes;

  auto at = [&](int r, int i) { return ((size_t)r * R + row) * k + i; };
  auto coarse_of = [&](uint32_t key, int32_t gid) -> uint64_t {
    if constexpr (variant == DSA_MERGE_PACKED) return key >> 16;
    else if constexpr (variant == DSA_MERGE_SCORES) return key;
    else return ((uint64_t)key << 32) | (0xFFFFFFFFu - (uint32_t)gid);
  };
  auto composite_of = [&](uint32_t key, int32_t gid) -> uint64_t {
    return ((uint64_t)key << 32) | (0xFFFFFFFFu - (uint32_t)gid);
  };
  constexpr int nbits = variant == DSA_MERGE_PACKED ? 16 : (variant == DSA_MERGE_SCORES ? 32 : 64);

  // this thread's message entries, e = tid + 1024 j over the shards' messages back to back
  uint32_t key[kMaxPer];
  int32_t gid[kMaxPer];
  int rounds = 1, resent = 0, N = 0, gt = 0, eq = 0;
  uint64_t T = 0;
  bool have_T = false;
  for (;;) {
    if (tid == 0) {
      int acc = 0;
      for (int r = 0; r < W; ++r) {
        sh.pre[r] = acc;
        acc += sh.n[r];
      }
      sh.pre[W] = acc;
    }
    __syncthreads();
    N = sh.pre[W];
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int e = tid + kMT * j;
      key[j] = 0;
      gid[j] = 0;
      if (e < N) {
        int r = 0;
        while (e >= sh.pre[r + 1]) ++r;
        key[j] = m.key[at(r, e - sh.pre[r])];
        gid[j] = m.gid[at(r, e - sh.pre[r])];
      }
    }
    have_T = N > k;
    if (have_T)
      T = block_select_desc(sh, N, [&](int j, bool& act) {
        act = true;
        return coarse_of(key[j], gid[j]);
      }, k, nbits, &gt, &eq);
    if (tid < W) {
      int f = 0;
      if (sh.n[tid] < sh.cnt[tid]) {
        const size_t o = at(tid, sh.n[tid] - 1);  // the shard's weakest sent candidate
        f = !have_T || coarse_of(m.key[o], m.gid[o]) >= T;
      }
      sh.flag[tid] = f;
    }
    __syncthreads();
    int nflag = 0;
    for (int r = 0; r < W; ++r) nflag += sh.flag[r];
    if (nflag == 0 || rounds == 2) break;  // a second resend cannot happen: the threshold only rises
    for (int r = 0; r < W; ++r)
      if (sh.flag[r]) payload += sh.cnt[r] * wbytes;  // the full local top-k, sent again
    __syncthreads();
    if (tid < W && sh.flag[tid]) sh.n[tid] = sh.cnt[tid];
    rounds = 2;
    resent = nflag;
    __syncthreads();
  }

  // entries tied with the threshold on the message key: all of them, or the best `need` by the
  // exact (score, index) order, learnt in a second small exchange
  bool take_all_eq = true;
  int tie = 0;
  uint64_t T2 = 0;
  if (have_T) {
    const int need = k - gt;
    if (need != eq) {
      take_all_eq = false;
      tie = eq;
      payload += eq * (variant == DSA_MERGE_SCORES ? 4 : 8);
      // within the tie bucket the top bits of the exact key are the message key itself: only the
      // rest of the score key (packed) or the index (scores) is left to select on
      constexpr int tbits = variant == DSA_MERGE_PACKED ? 48 : 32;
      int g2, e2;
      T2 = block_select_desc(sh, N, [&](int j, bool& act) {
        act = coarse_of(key[j], gid[j]) == T;
        return composite_of(key[j], gid[j]);
      }, need, tbits, &g2, &e2, T << tbits);
    }
  }

  if (tid == 0) sh.nsel = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j)
    if (tid + kMT * j < N) {
      bool s = !have_T;
      if (!s) {
        const uint64_t c = coarse_of(key[j], gid[j]);
        s = c > T || (c == T && (take_all_eq || composite_of(key[j], gid[j]) >= T2));
      }
      if (s) {
        const int p = atomicAdd(&sh.nsel, 1);
        if (p < k) sh.sel[p] = gid[j];
      }
    }
  __syncthreads();
  const int nsel = min(sh.nsel, k);
  int32_t g0 = 2 * tid < nsel ? sh.sel[2 * tid] : 0x7FFFFFFF;
  int32_t g1 = 2 * tid + 1 < nsel ? sh.sel[2 * tid + 1] : 0x7FFFFFFF;
  __syncthreads();  // sel becomes the sort's exchange buffer
  block_sort2048<int32_t, false>(g0, g1, sh.sel);
  {
    int32_t* orow = idx + (int64_t)row * k;
    if (2 * tid < k) orow[2 * tid] = 2 * tid < nsel ? g0 : -1;
    if (2 * tid + 1 < k) orow[2 * tid + 1] = 2 * tid + 1 < nsel ? g1 : -1;
  }
  if (tid == 0) {
    count[row] = nsel;
    if (stats) {
      stats[4 * row + 0] = rounds;
      stats[4 * row + 1] = resent;
      stats[4 * row + 2] = tie;
      stats[4 * row + 3] = payload;
    }
  }

  // each shard's part, in ascending order: a stable partition of the sorted list by residue
  const int i0 = 2 * tid, i1 = 2 * tid + 1;
  if (i0 >= nsel) g0 = -1;
  if (i1 >= nsel) g1 = -1;
  for (int r = 0; r < W; ++r) {
    const uint32_t f0 = g0 >= 0 && g0 % W == r, f1 = g1 >= 0 && g1 % W == r;
    const uint32_t c = f0 + f1;
    const uint32_t incl = wave_incl_scan(c);
    if (lane == 63) sh.wtot[wave] = incl;
    __syncthreads();
    if (tid < 64) {
      const uint32_t tt = tid < kMT / 64 ? sh.wtot[tid] : 0u;
      const uint32_t sc = wave_incl_scan(tt);
      if (tid < kMT / 64) sh.wofs[tid] = sc - tt;
    }
    __syncthreads();
    const int total = (int)(sh.wofs[kMT / 64 - 1] + sh.wtot[kMT / 64 - 1]);
    int32_t* out = shard_idx + ((int64_t)r * R + row) * k;
    int pos = (int)(sh.wofs[wave] + incl - c);
    if (f0) out[pos++] = g0 / W;
    if (f1) out[pos] = g1 / W;
    for (int j = total + tid; j < k; j += kMT) out[j] = -1;
    if (tid == 0) shard_count[(int64_t)r * R + row] = total;
    __syncthreads();
  }
}

}  // namespace

size_t dcp_mailbox_bytes(int32_t num_rows, int32_t k, int32_t num_shards) {
  const size_t n = (size_t)num_shards * num_rows * k;
  return (n * 8 + (size_t)num_shards * num_rows * 4 + 15) / 16 * 16;
}

hipError_t launch_dcp_publish(int32_t R, int32_t k, int32_t W, int32_t shard, const float* scores,
                              int64_t ld, const int32_t* idx, const int32_t* count, void* mb,
                              hipStream_t s) {
  dcp_publish_kernel<<<dim3(R), dim3(kMT), 0, s>>>(R, k, W, shard, scores, ld, idx, count, mb);
  return hipGetLastError();
}

hipError_t launch_dcp_merge(int32_t R, int32_t k, int32_t W, int32_t variant, void* mb,
                            int32_t* idx, int32_t* count, int32_t* shard_idx,
                            int32_t* shard_count, int32_t* stats, hipStream_t s) {
  if (variant == DSA_MERGE_PACKED)
    dcp_merge_kernel<DSA_MERGE_PACKED><<<dim3(R), dim3(kMT), 0, s>>>(R, k, W, mb, idx, count,
                                                                    shard_idx, shard_count, stats);
  else if (variant == DSA_MERGE_SCORES)
    dcp_merge_kernel<DSA_MERGE_SCORES><<<dim3(R), dim3(kMT), 0, s>>>(R, k, W, mb, idx, count,
                                                                    shard_idx, shard_count, stats);
  else
    dcp_merge_kernel<DSA_MERGE_GENERIC><<<dim3(R), dim3(kMT), 0, s>>>(R, k, W, mb, idx, count,
                                                                     shard_idx, shard_count, stats);
  return hipGetLastError();
}

}  // namespace dsa
