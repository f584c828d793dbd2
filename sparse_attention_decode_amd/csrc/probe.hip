// Read-bandwidth probe: the rate at which this GPU streams a given set of pool pages (the key
// pages the scorer reads, in the block tables' order) or a contiguous span, with no arithmetic
// behind the loads.  It is the measured ceiling the scorer's bandwidth is compared with; it
// computes nothing of the method.
#include "dsa_kernels.h"

namespace dsa {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeWaves = kProbeThreads / kWave;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// One wave per page at a time, two pages in flight: lane l loads 16-byte pieces l, l + 64, ...
// of the page.  The XOR of everything read goes to one word per workgroup, so no load is dead.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(ProbeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * kProbeWaves;
  const int pieces = a.bytes_per_page / 16;
  uint32_t acc = 0;
  auto page_base = [&](int64_t i) -> const uint8_t* {
    const int64_t r = a.rows ? (int64_t)a.rows[i] : i;
    return a.base + r * a.row_bytes + a.offset;
  };
  for (int64_t i = (int64_t)blockIdx.x * kProbeWaves + wave; i < a.num_pages; i += 2 * nw) {
    const uint8_t* p0 = page_base(i);
    const bool two = i + nw < a.num_pages;
    const uint8_t* p1 = two ? page_base(i + nw) : p0;
    v4u v0[kProbeMaxPieces / 64], v1[kProbeMaxPieces / 64];
#pragma unroll
    for (int j = 0; j < kProbeMaxPieces / 64; ++j) {
      const int piece = lane + 64 * j;
      if (piece < pieces) {
        v0[j] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p0) + piece);
        v1[j] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p1) + piece);
      }
    }
#pragma unroll
    for (int j = 0; j < kProbeMaxPieces / 64; ++j) {
      const int piece = lane + 64 * j;
      if (piece < pieces) {
        acc ^= v0[j][0] ^ v0[j][1] ^ v0[j][2] ^ v0[j][3];
        if (two) acc ^= v1[j][0] ^ v1[j][1] ^ v1[j][2] ^ v1[j][3];
      }
    }
  }
  // reduce the workgroup's words and leave one
  __shared__ uint32_t red[kProbeThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int t = 0; t < kProbeThreads; ++t) x ^= red[t];
    a.sink[blockIdx.x] = x;
  }
}

}  // namespace

hipError_t launch_probe_read(const ProbeArgs& a, hipStream_t s) {
  if (a.num_pages <= 0) return hipSuccess;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)a.grid), dim3(kProbeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
