// C ABI of the DSA layer: argument validation, pool layout, and kernel dispatch on the caller's
// stream.  Declarations and argument contracts are in include/dsa.h.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "dsa_kernels.h"

// The device status word (DSA_DEVERR_* bits): one per device, set by the kernels with atomic ORs
// where they meet device data outside the contract, read and cleared by dsa_device_status.  Host
// code never uses this name as an address: each device's address comes from hipGetSymbolAddress.
static __device__ uint32_t dev_status;

// Scratch of sparse_mla_decode_noalloc (its split partials): a fixed array in each device's
// memory, held until the process ends.  As with the status word, host code never passes this
// name to a kernel or a copy; it uses the address hipGetSymbolAddress gives for the device.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {

thread_local char g_err[512] = "";

dsa_status fail(dsa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

dsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kMaxDevices = 64;
std::atomic<uint32_t*> g_status[kMaxDevices];
std::mutex g_symbol_mu;

// The current device, checked against the device of `stream` (kernels get addresses of this
// device's status word, so they must run on it).
dsa_status current_device(hipStream_t stream, int* dev) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (*dev < 0 || *dev >= kMaxDevices)
    return fail(DSA_ERR_UNSUPPORTED, "device %d beyond the %d this build tracks", *dev, kMaxDevices);
  if (stream) {
    hipDevice_t sd;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if ((int)sd != *dev)
      return fail(DSA_ERR_INVALID_ARG, "stream belongs to device %d, the current device is %d",
                  (int)sd, *dev);
  }
  return DSA_OK;
}

// Address of the current device's status word, looked up once per device.
dsa_status status_word(hipStream_t stream, uint32_t** out) {
  int dev;
  dsa_status st = current_device(stream, &dev);
  if (st != DSA_OK) return st;
  uint32_t* p = g_status[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_symbol_mu);
    p = g_status[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(dev_status));
      if (e != hipSuccess || !addr)
        return fail(DSA_ERR_HIP, "hipGetSymbolAddress(status word): %s", hipGetErrorString(e));
      p = static_cast<uint32_t*>(addr);
      g_status[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return DSA_OK;
}

std::atomic<void*> g_scratch[kMaxDevices];

// Address of the current device's scratch array, looked up once per device (with that device
// current) on the first sparse_mla_decode_noalloc call there.
dsa_status scratch_address(hipStream_t stream, void** out) {
  int dev;
  dsa_status st = current_device(stream, &dev);
  if (st != DSA_OK) return st;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_symbol_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return DSA_OK;
}

dsa_status check_layout(const dsa_kv_layout* kv, const void* pool) {
  if (!kv) return fail(DSA_ERR_INVALID_ARG, "kv layout is NULL");
  if (!pool) return fail(DSA_ERR_INVALID_ARG, "pool is NULL");
  if (!aligned(pool, 256)) return fail(DSA_ERR_INVALID_ARG, "pool must be 256-byte aligned");
  if (kv->block_size != 64)
    return fail(DSA_ERR_UNSUPPORTED, "block_size %d (only 64 is built)", kv->block_size);
  if (kv->ikey_format != DSA_IKEY_FP8 && kv->ikey_format != DSA_IKEY_MXFP4)
    return fail(DSA_ERR_INVALID_ARG, "unknown ikey_format %d", kv->ikey_format);
  if (kv->latent_format != DSA_LATENT_FP8 && kv->latent_format != DSA_LATENT_NVFP4)
    return fail(DSA_ERR_INVALID_ARG, "unknown latent_format %d", kv->latent_format);
  const int64_t offs[4] = {kv->latent_off, kv->latent_scale_off, kv->ikey_off, kv->ikey_scale_off};
  for (int i = 0; i < 4; ++i)
    if (offs[i] < 0 || offs[i] % 16 || offs[i] >= kv->row_bytes)
      return fail(DSA_ERR_INVALID_ARG, "page offset %lld not 16-aligned inside the row",
                  (long long)offs[i]);
  if (kv->row_bytes <= 0 || kv->row_bytes % 256)
    return fail(DSA_ERR_INVALID_ARG, "row_bytes %lld must be a positive multiple of 256",
                (long long)kv->row_bytes);
  {
    // every page inside the row; the attention gathers a token's latent scales as whole 16-byte
    // pieces, reading up to 12 bytes past its scales, so the latent-scale page needs 12 bytes of
    // the row behind it
    const bool fp8l = kv->latent_format == DSA_LATENT_FP8, fp8k = kv->ikey_format == DSA_IKEY_FP8;
    const int64_t bs = kv->block_size;
    const int64_t ends[4] = {kv->latent_off + bs * (fp8l ? DSA_MLA_DQK : DSA_MLA_DQK / 2),
                             kv->latent_scale_off + bs * (fp8l ? 4 : DSA_MLA_DQK / 16) + 12,
                             kv->ikey_off + bs * (fp8k ? DSA_INDEX_DIM : DSA_INDEX_DIM / 2),
                             kv->ikey_scale_off + bs * (fp8k ? 4 : DSA_INDEX_DIM / 32)};
    for (int i = 0; i < 4; ++i)
      if (ends[i] > kv->row_bytes)
        return fail(DSA_ERR_INVALID_ARG, "page at offset %lld extends past row_bytes %lld%s",
                    (long long)offs[i], (long long)kv->row_bytes,
                    i == 1 ? " (the latent scales need 12 bytes of the row behind them)" : "");
  }
  if (kv->num_blocks <= 0) return fail(DSA_ERR_INVALID_ARG, "num_blocks must be positive");
  if (kv->latent_format == DSA_LATENT_NVFP4 &&
      !(kv->latent_tensor_scale > 0.f && isfinite(kv->latent_tensor_scale)))
    return fail(DSA_ERR_INVALID_ARG, "NVFP4 tensor scale must be finite and positive");
  return DSA_OK;
}

dsa_status check_batch(const dsa_batch* b) {
  if (!b) return fail(DSA_ERR_INVALID_ARG, "batch is NULL");
  if (b->num_seqs < 1) return fail(DSA_ERR_INVALID_ARG, "num_seqs must be >= 1");
  if (b->num_rows < 0) return fail(DSA_ERR_INVALID_ARG, "num_rows must be >= 0");
  if (b->max_rows_per_seq < (b->num_rows > 0 ? 1 : 0))
    return fail(DSA_ERR_INVALID_ARG, "max_rows_per_seq must be >= 1 when num_rows > 0");
  if (b->max_context < 1) return fail(DSA_ERR_INVALID_ARG, "max_context must be >= 1");
  if (b->max_context > (int64_t)1 << 30) return fail(DSA_ERR_UNSUPPORTED, "max_context too large");
  if ((int64_t)b->max_blocks_per_seq * 64 < b->max_context)
    return fail(DSA_ERR_INVALID_ARG, "max_blocks_per_seq * 64 < max_context");
  if (!b->block_table || !b->seq_row_start || !b->row_pos)
    return fail(DSA_ERR_INVALID_ARG, "block_table, seq_row_start and row_pos must be non-NULL");
  if (b->flags & ~(DSA_BATCH_INVARIANT | DSA_BATCH_PLAIN_ORDER))
    return fail(DSA_ERR_INVALID_ARG, "unknown batch flags");
  return DSA_OK;
}

dsa::PoolView pool_view(const dsa_kv_layout* kv, const void* pool) {
  dsa::PoolView p;
  p.base = static_cast<const uint8_t*>(pool);
  p.row_bytes = kv->row_bytes;
  p.lat_off = kv->latent_off;
  p.lat_scale_off = kv->latent_scale_off;
  p.ikey_off = kv->ikey_off;
  p.ikey_scale_off = kv->ikey_scale_off;
  p.tokens = kv->num_blocks * kv->block_size;
  return p;
}

dsa::BatchView batch_view(const dsa_batch* b) {
  dsa::BatchView v;
  v.block_table = b->block_table;
  v.ld_bt = b->max_blocks_per_seq;
  v.seq_row_start = b->seq_row_start;
  v.row_pos = b->row_pos;
  v.num_seqs = b->num_seqs;
  v.num_rows = b->num_rows;
  return v;
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Split count and split size of the decode attention for num_rows rows and top-k k.
void mla_splits(int32_t num_rows, int32_t k, bool invariant, int32_t* nsplit, int32_t* per) {
  int32_t ns = dsa::mla_num_splits(num_rows, k, invariant);
  *per = (int32_t)align_up((k + ns - 1) / ns, 32);
  *nsplit = (k + *per - 1) / *per;
}

// Splits of one shard's attention under decode context parallelism: sized for the shard's
// expected share of the selection (k / num_shards), since each shard's entries are compacted at
// the front of its list and spread over its splits by count.
void shard_splits(int32_t num_rows, int32_t k, int32_t num_shards, bool invariant,
                  int32_t* nsplit, int32_t* per) {
  int32_t ns, unused;
  if (invariant)
    mla_splits(num_rows, k, true, &ns, &unused);
  else
    mla_splits(num_rows, std::max(32, (k + num_shards - 1) / num_shards), false, &ns, &unused);
  *per = (int32_t)align_up((k + ns - 1) / ns, 32);  // ranges covering all k when no count is given
  *nsplit = (k + *per - 1) / *per;
}

size_t partial_bytes(int32_t num_rows, int32_t slots) {
  return (size_t)num_rows * slots * DSA_MLA_HEADS *
         (DSA_MLA_DV * sizeof(uint16_t) + 2 * sizeof(float));
}

void partial_views(dsa::MlaArgs& a, void* buf, int32_t num_rows) {
  const size_t nslot = (size_t)num_rows * a.split_slots * DSA_MLA_HEADS;
  a.part_o = static_cast<uint16_t*>(buf);
  a.part_lse = reinterpret_cast<float*>(a.part_o + nslot * DSA_MLA_DV);
  a.part_exp = reinterpret_cast<int32_t*>(a.part_lse + nslot);
}

// shard < 0: the whole attention of each row (decode or prefill variant).  shard >= 0: the part of
// decode context parallelism one shard runs: its splits go to partial slots [shard * nsplit,
// (shard + 1) * nsplit) of a buffer holding num_shards * nsplit slots per row (workspace), and no
// output is written (dsa_lse_combine writes it).
dsa_status mla_common(const dsa_kv_layout* kv, const void* pool, const dsa_batch* batch,
                      const uint16_t* q, const int32_t* idx, const int32_t* phys, int32_t k,
                      float softmax_scale,
                      uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                      hipStream_t stream, bool prefill, int32_t shard = -1,
                      int32_t num_shards = 1, const int32_t* count = nullptr,
                      bool noalloc = false) {
  dsa_status st = check_layout(kv, pool);
  if (st != DSA_OK) return st;
  if ((st = check_batch(batch)) != DSA_OK) return st;
  if (shard >= 0) {
    if (num_shards < 1 || num_shards > DSA_MAX_SHARDS || shard >= num_shards)
      return fail(DSA_ERR_INVALID_ARG, "shard %d of %d shards out of range", shard, num_shards);
    if (!q || !idx) return fail(DSA_ERR_INVALID_ARG, "q and idx must be non-NULL");
    if (!aligned(q, 16)) return fail(DSA_ERR_INVALID_ARG, "q must be 16-byte aligned");
  } else {
    if (!q || !idx || !out) return fail(DSA_ERR_INVALID_ARG, "q, idx and out must be non-NULL");
    if (!aligned(q, 16) || !aligned(out, 16))
      return fail(DSA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(DSA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  }
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID_ARG, "k %d not in [1, 2048]", k);
  if (!isfinite(softmax_scale)) return fail(DSA_ERR_INVALID_ARG, "softmax_scale not finite");
  if (batch->num_rows == 0) return DSA_OK;
  dsa::MlaArgs a;
  a.pool = pool_view(kv, pool);
  a.batch = batch_view(batch);
  a.q = q;
  a.idx = idx;
  a.phys = phys;
  a.k = k;
  a.softmax_scale = softmax_scale;
  a.tensor_scale = kv->latent_format == DSA_LATENT_NVFP4 ? kv->latent_tensor_scale : 1.f;
  a.out = out;
  a.lse = lse;
  const bool invariant = (batch->flags & DSA_BATCH_INVARIANT) != 0;
  a.count = count;
  if (shard >= 0) {
    shard_splits(batch->num_rows, k, num_shards, invariant, &a.nsplit, &a.tokens_per_split);
  } else if (prefill && !invariant) {
    a.nsplit = 1;
    a.tokens_per_split = (int32_t)align_up(k, 32);
  } else {
    mla_splits(batch->num_rows, k, invariant, &a.nsplit, &a.tokens_per_split);
  }
  a.split_base = shard >= 0 ? shard * a.nsplit : 0;
  a.split_slots = shard >= 0 ? num_shards * a.nsplit : a.nsplit;
  a.out_direct = shard < 0 && a.nsplit == 1;
  a.part_o = nullptr;
  a.part_lse = nullptr;
  a.part_exp = nullptr;
  a.nt_partials = 0;
  if (!a.out_direct && noalloc) {
    // the split partials go to the device's static scratch; every split writes its whole slot
    // before the combine reads it, so nothing there has to start at zero
    const size_t need = partial_bytes(batch->num_rows, a.split_slots);
    if (need > kNoallocScratchBytes)
      return fail(DSA_ERR_WORKSPACE,
                  "%d rows at top-k %d need %zu bytes of split partials; the static scratch "
                  "holds %zu (use sparse_mla_decode with a workspace)",
                  batch->num_rows, k, need, kNoallocScratchBytes);
    if ((st = scratch_address(stream, &workspace)) != DSA_OK) return st;
    workspace_bytes = kNoallocScratchBytes;
  }
  if (!a.out_direct) {
    const size_t need = partial_bytes(batch->num_rows, a.split_slots);
    // 16 MB and more: the set would evict as dirty lines during the next step's key stream
    a.nt_partials = need >= ((size_t)16 << 20);
    if (!workspace || workspace_bytes < need)
      return fail(DSA_ERR_WORKSPACE, "%s of %zu bytes needed, %zu given",
                  shard >= 0 ? "partials buffer" : "workspace", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-aligned");
    partial_views(a, workspace, batch->num_rows);
  }
  if ((st = status_word(stream, &a.status)) != DSA_OK) return st;
  return hip_status(dsa::launch_sparse_mla(a, kv->latent_format, shard < 0, stream),
                    shard >= 0 ? "sparse_mla_decode_shard launch"
                               : (prefill ? "sparse_mla_prefill launch" : "sparse_mla_decode launch"));
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_ERR_UNKNOWN";
}

const char* dsa_last_error(void) { return g_err; }

dsa_status dsa_probe_read(const void* base, int64_t row_bytes, int64_t offset,
                          int32_t bytes_per_page, const int32_t* rows, int64_t num_pages,
                          uint32_t* sink, int32_t grid, void* stream) {
  g_err[0] = 0;
  if (!base || !sink) return fail(DSA_ERR_INVALID_ARG, "base and sink must be non-NULL");
  if (bytes_per_page < 16 || bytes_per_page % 16 || bytes_per_page > 16 * dsa::kProbeMaxPieces)
    return fail(DSA_ERR_INVALID_ARG, "bytes_per_page %d not a multiple of 16 in [16, %d]",
                bytes_per_page, 16 * dsa::kProbeMaxPieces);
  if (offset < 0 || row_bytes < 0 || row_bytes % 16 || !aligned((const uint8_t*)base + offset, 16))
    return fail(DSA_ERR_INVALID_ARG, "base + offset and row_bytes must be 16-byte aligned");
  if (num_pages < 0) return fail(DSA_ERR_INVALID_ARG, "num_pages must be >= 0");
  if (grid < 1 || grid > 65535) return fail(DSA_ERR_INVALID_ARG, "grid %d not in [1, 65535]", grid);
  if (rows && !aligned(rows, 4)) return fail(DSA_ERR_INVALID_ARG, "rows must be 4-byte aligned");
  if (num_pages == 0) return DSA_OK;
  dsa::ProbeArgs a;
  a.base = static_cast<const uint8_t*>(base);
  a.row_bytes = row_bytes;
  a.offset = offset;
  a.bytes_per_page = bytes_per_page;
  a.rows = rows;
  a.num_pages = num_pages;
  a.sink = sink;
  a.grid = grid;
  return hip_status(dsa::launch_probe_read(a, static_cast<hipStream_t>(stream)),
                    "dsa_probe_read launch");
}

dsa_status dsa_device_status(uint32_t* status, int32_t clear, void* stream) {
  g_err[0] = 0;
  if (!status) return fail(DSA_ERR_INVALID_ARG, "status is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* word;
  dsa_status st = status_word(s, &word);
  if (st != DSA_OK) return st;
  if ((st = hip_status(hipStreamSynchronize(s), "hipStreamSynchronize")) != DSA_OK) return st;
  if ((st = hip_status(hipMemcpy(status, word, sizeof(uint32_t), hipMemcpyDeviceToHost),
                       "reading the status word")) != DSA_OK)
    return st;
  if (clear) {
    static const uint32_t zero = 0;
    if ((st = hip_status(hipMemcpy(word, &zero, sizeof(uint32_t), hipMemcpyHostToDevice),
                         "clearing the status word")) != DSA_OK)
      return st;
  }
  return DSA_OK;
}

dsa_status dsa_kv_layout_init(dsa_kv_layout* out, int32_t ikey_format, int32_t latent_format,
                              int32_t block_size, int64_t num_blocks, float latent_tensor_scale) {
  g_err[0] = 0;
  if (!out) return fail(DSA_ERR_INVALID_ARG, "out is NULL");
  if (block_size != 64) return fail(DSA_ERR_UNSUPPORTED, "block_size %d (only 64 is built)", block_size);
  if (ikey_format != DSA_IKEY_FP8 && ikey_format != DSA_IKEY_MXFP4)
    return fail(DSA_ERR_INVALID_ARG, "unknown ikey_format %d", ikey_format);
  if (latent_format != DSA_LATENT_FP8 && latent_format != DSA_LATENT_NVFP4)
    return fail(DSA_ERR_INVALID_ARG, "unknown latent_format %d", latent_format);
  if (num_blocks <= 0) return fail(DSA_ERR_INVALID_ARG, "num_blocks must be positive");
  if (latent_format == DSA_LATENT_NVFP4 && !(latent_tensor_scale > 0.f && isfinite(latent_tensor_scale)))
    return fail(DSA_ERR_INVALID_ARG, "NVFP4 tensor scale must be finite and positive");
  memset(out, 0, sizeof(*out));
  const int64_t bs = block_size;
  int64_t off = 0;
  out->block_size = block_size;
  out->ikey_format = ikey_format;
  out->latent_format = latent_format;
  out->latent_off = off;
  off += bs * (latent_format == DSA_LATENT_FP8 ? DSA_MLA_DQK : DSA_MLA_DQK / 2);
  out->latent_scale_off = off = align_up(off, 16);
  off += bs * (latent_format == DSA_LATENT_FP8 ? 4 : DSA_MLA_DQK / 16);
  out->ikey_off = off = align_up(off, 16);
  off += bs * (ikey_format == DSA_IKEY_FP8 ? DSA_INDEX_DIM : DSA_INDEX_DIM / 2);
  out->ikey_scale_off = off = align_up(off, 16);
  off += bs * (ikey_format == DSA_IKEY_FP8 ? 4 : DSA_INDEX_DIM / 32);
  out->row_bytes = align_up(off, 256);
  out->num_blocks = num_blocks;
  out->latent_tensor_scale = latent_format == DSA_LATENT_NVFP4 ? latent_tensor_scale : 1.f;
  return DSA_OK;
}

dsa_status dsa_indexer_scores(const dsa_kv_layout* kv, const void* pool, const dsa_batch* batch,
                              const uint8_t* q_idx, const float* w, float* scores,
                              int64_t ld_scores, uint32_t* hist, void* stream) {
  g_err[0] = 0;
  dsa_status st = check_layout(kv, pool);
  if (st != DSA_OK) return st;
  if ((st = check_batch(batch)) != DSA_OK) return st;
  if (!q_idx || !w || !scores) return fail(DSA_ERR_INVALID_ARG, "q_idx, w and scores must be non-NULL");
  if (!aligned(q_idx, 16) || !aligned(w, 4) || !aligned(scores, 4))
    return fail(DSA_ERR_INVALID_ARG, "q_idx must be 16-byte aligned");
  if (ld_scores < batch->max_context)
    return fail(DSA_ERR_INVALID_ARG, "ld_scores %lld < max_context %lld", (long long)ld_scores,
                (long long)batch->max_context);
  if (hist && !aligned(hist, 4)) return fail(DSA_ERR_INVALID_ARG, "hist must be 4-byte aligned");
  if (batch->num_rows == 0) return DSA_OK;
  dsa::IndexerArgs a;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = status_word(s, &a.status)) != DSA_OK) return st;
  a.pool = pool_view(kv, pool);
  a.batch = batch_view(batch);
  a.q = q_idx;
  a.w = w;
  a.scores = scores;
  a.ld = ld_scores;
  a.hist = hist;
  a.plain_order = (batch->flags & DSA_BATCH_PLAIN_ORDER) != 0;
  a.sample_stride = 1;
  a.cand = nullptr;
  a.cand_count = nullptr;
  a.cand_max = nullptr;
  a.floor = nullptr;
  a.cand_cap = 0;
  if (batch->max_rows_per_seq <= DSA_MAX_ROWS_PER_SEQ)
    return hip_status(dsa::launch_indexer_decode(a, kv->ikey_format, batch->max_rows_per_seq,
                                                 batch->max_context, s),
                      "indexer launch");
  return hip_status(dsa::launch_indexer_prefill(a, kv->ikey_format, batch->max_context,
                                                batch->max_rows_per_seq, s),
                    "prefill indexer launch");
}

size_t dsa_topk_workspace_bytes(int32_t num_rows, int64_t max_context) {
  if (num_rows <= 0 || max_context <= 0) return 0;
  return dsa::topk_workspace_bytes(num_rows, max_context);
}

dsa_status dsa_topk(const dsa_kv_layout* kv, const dsa_batch* batch, const float* scores,
                    int64_t ld_scores, uint32_t* hist, int32_t k, int32_t* idx,
                    int32_t* count, int32_t* phys, void* workspace, size_t workspace_bytes,
                    void* stream) {
  g_err[0] = 0;
  dsa_status st = check_batch(batch);
  if (st != DSA_OK) return st;
  if (!scores || !idx || !count) return fail(DSA_ERR_INVALID_ARG, "scores, idx and count must be non-NULL");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID_ARG, "k %d not in [1, 2048]", k);
  if (ld_scores < batch->max_context)
    return fail(DSA_ERR_INVALID_ARG, "ld_scores %lld < max_context", (long long)ld_scores);
  if (batch->max_context > (int64_t)dsa::kMaxSlices * dsa::kTopkSlice)
    return fail(DSA_ERR_UNSUPPORTED, "top-k is built for contexts up to %d tokens",
                dsa::kMaxSlices * dsa::kTopkSlice);
  if (hist && !aligned(hist, 4)) return fail(DSA_ERR_INVALID_ARG, "hist must be 4-byte aligned");
  if (phys) {
    if (!kv) return fail(DSA_ERR_INVALID_ARG, "kv layout is required for phys rows");
    if (kv->block_size != 64) return fail(DSA_ERR_UNSUPPORTED, "block_size must be 64");
  }
  if (batch->num_rows == 0) return DSA_OK;
  const size_t need = dsa::topk_workspace_bytes(batch->num_rows, batch->max_context);
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "top-k workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-aligned");
  dsa::TopkArgs a = {};
  uint32_t* status;
  if ((st = status_word(static_cast<hipStream_t>(stream), &status)) != DSA_OK) return st;
  a.status = status;
  a.batch = batch_view(batch);
  a.scores = scores;
  a.ld = ld_scores;
  a.hist_in = hist;
  a.k = k;
  a.idx = idx;
  a.count = count;
  a.phys = phys;
  return hip_status(dsa::launch_topk(a, batch->max_context, workspace,
                                     static_cast<hipStream_t>(stream)),
                    "topk launch");
}

}  // extern "C"

namespace {

// Layout of the candidates path's workspace: the sample's dense scores, each row's candidate
// list, its count and its floor.
struct CandLayout {
  int32_t S;
  int64_t samp_ld, cap;
  size_t off_samp, off_cand, off_count, off_max, off_floor, total;
};

constexpr int64_t kCandMaxContext = (int64_t)1 << 23;

CandLayout cand_layout(int32_t num_rows, int64_t max_context, int32_t k) {
  CandLayout c;
  const int64_t nb = (max_context + 63) / 64;
  // the largest power of two S <= 32 with S^2 <= N / (2k) rounded to the nearer power: the
  // sample's N / S scores (4 bytes) and the about S k candidates (8 bytes) then cost alike
  int32_t S = 1;
  while (S < 32 && 2 * S <= nb && (int64_t)(2 * S) * (2 * S) * k <= max_context) S *= 2;
  c.S = S;
  c.samp_ld = (nb + S - 1) / S * 64;
  const int64_t room = 2 * (int64_t)S * (k + 64) + k;
  c.cap = align_up(std::max<int64_t>(k, std::min<int64_t>(align_up(max_context, 64), room)), 64);
  const size_t R = (size_t)num_rows;
  size_t off = 0;
  c.off_samp = off;
  off = align_up(off + R * c.samp_ld * sizeof(float), 256);
  c.off_cand = off;
  off = align_up(off + R * c.cap * 8, 256);
  c.off_count = off;
  off = align_up(off + R * sizeof(int32_t), 256);
  c.off_max = off;
  off = align_up(off + R * sizeof(uint32_t), 256);
  c.off_floor = off;
  off = align_up(off + R * 2 * sizeof(uint32_t), 256);
  c.total = off;
  return c;
}

dsa_status check_cand_call(const dsa_batch* batch, int32_t k, const void* workspace,
                           size_t workspace_bytes, CandLayout* c) {
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID_ARG, "k %d not in [1, 2048]", k);
  if (batch->max_context > kCandMaxContext)
    return fail(DSA_ERR_UNSUPPORTED, "the candidates path is built for contexts up to %lld tokens",
                (long long)kCandMaxContext);
  *c = cand_layout(batch->num_rows, batch->max_context, k);
  if (batch->num_rows == 0) return DSA_OK;
  if (!workspace || workspace_bytes < c->total)
    return fail(DSA_ERR_WORKSPACE, "candidates workspace of %zu bytes needed, %zu given", c->total,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return DSA_OK;
}

dsa::CandArgs cand_args(const dsa_batch* batch, int32_t k, void* ws, const CandLayout& c) {
  dsa::CandArgs a = {};
  uint8_t* base = static_cast<uint8_t*>(ws);
  a.batch = batch_view(batch);
  a.k = k;
  a.sample_stride = c.S;
  a.samp = reinterpret_cast<const float*>(base + c.off_samp);
  a.samp_ld = c.samp_ld;
  a.cand = reinterpret_cast<uint2*>(base + c.off_cand);
  a.cand_count = reinterpret_cast<int32_t*>(base + c.off_count);
  a.cand_max = reinterpret_cast<uint32_t*>(base + c.off_max);
  a.floor = reinterpret_cast<uint32_t*>(base + c.off_floor);
  a.cand_cap = c.cap;
  return a;
}

}  // namespace

extern "C" {

size_t dsa_candidates_workspace_bytes(int32_t num_rows, int64_t max_context, int32_t k) {
  if (num_rows <= 0 || max_context <= 0 || max_context > kCandMaxContext || k < 1 ||
      k > DSA_MAX_TOPK)
    return 0;
  return cand_layout(num_rows, max_context, k).total;
}

dsa_status dsa_indexer_candidates(const dsa_kv_layout* kv, const void* pool, const dsa_batch* batch,
                                  const uint8_t* q_idx, const float* w, int32_t k, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  dsa_status st = check_layout(kv, pool);
  if (st != DSA_OK) return st;
  if ((st = check_batch(batch)) != DSA_OK) return st;
  if (!q_idx || !w) return fail(DSA_ERR_INVALID_ARG, "q_idx and w must be non-NULL");
  if (!aligned(q_idx, 16) || !aligned(w, 4))
    return fail(DSA_ERR_INVALID_ARG, "q_idx must be 16-byte and w 4-byte aligned");
  CandLayout c;
  if ((st = check_cand_call(batch, k, workspace, workspace_bytes, &c)) != DSA_OK) return st;
  if (batch->num_rows == 0) return DSA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* status;
  if ((st = status_word(s, &status)) != DSA_OK) return st;
  dsa::CandArgs ca = cand_args(batch, k, workspace, c);
  ca.status = status;
  dsa::IndexerArgs a = {};
  a.pool = pool_view(kv, pool);
  a.batch = batch_view(batch);
  a.q = q_idx;
  a.w = w;
  a.hist = nullptr;
  a.status = status;
  a.plain_order = (batch->flags & DSA_BATCH_PLAIN_ORDER) != 0;
  a.sample_stride = c.S;
  a.cand = ca.cand;
  a.cand_count = ca.cand_count;
  a.cand_max = ca.cand_max;
  a.floor = ca.floor;
  a.cand_cap = c.cap;
  const bool decode = batch->max_rows_per_seq <= DSA_MAX_ROWS_PER_SEQ;
  auto score = [&](int mode) {
    return decode ? dsa::launch_indexer_decode(a, kv->ikey_format, batch->max_rows_per_seq,
                                               batch->max_context, s, mode)
                  : dsa::launch_indexer_prefill(a, kv->ikey_format, batch->max_context,
                                                batch->max_rows_per_seq, s, mode);
  };
  // the sample blocks, dense, in sample numbering
  a.scores = const_cast<float*>(ca.samp);
  a.ld = c.samp_ld;
  if ((st = hip_status(score(dsa::kScoreSample), "sample scorer launch")) != DSA_OK) return st;
  // the sample's top-k and floor
  if ((st = hip_status(dsa::launch_cand_select(ca, 0, s), "sample select launch")) != DSA_OK)
    return st;
  // the other blocks, into the candidate lists
  a.scores = nullptr;
  a.ld = 0;
  return hip_status(score(dsa::kScoreCand), "candidate scorer launch");
}

dsa_status dsa_topk_candidates(const dsa_kv_layout* kv, const dsa_batch* batch, int32_t k,
                               void* workspace, size_t workspace_bytes, int32_t* idx,
                               int32_t* count, int32_t* phys, void* stream) {
  g_err[0] = 0;
  dsa_status st = check_batch(batch);
  if (st != DSA_OK) return st;
  if (!idx || !count) return fail(DSA_ERR_INVALID_ARG, "idx and count must be non-NULL");
  if (phys) {
    if (!kv) return fail(DSA_ERR_INVALID_ARG, "kv layout is required for phys rows");
    if (kv->block_size != 64) return fail(DSA_ERR_UNSUPPORTED, "block_size must be 64");
  }
  CandLayout c;
  if ((st = check_cand_call(batch, k, workspace, workspace_bytes, &c)) != DSA_OK) return st;
  if (batch->num_rows == 0) return DSA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  dsa::CandArgs ca = cand_args(batch, k, workspace, c);
  if ((st = status_word(s, &ca.status)) != DSA_OK) return st;
  ca.idx = idx;
  ca.count = count;
  ca.phys = phys;
  return hip_status(dsa::launch_cand_select(ca, 1, s), "candidate select launch");
}

size_t sparse_mla_workspace_bytes(int32_t num_rows, int32_t k, uint32_t flags) {
  if (num_rows <= 0 || k < 1) return 0;
  return dsa::mla_workspace_bytes(num_rows, k > DSA_MAX_TOPK ? DSA_MAX_TOPK : k,
                                  (flags & DSA_BATCH_INVARIANT) != 0);
}

dsa_status sparse_mla_decode(const dsa_kv_layout* kv, const void* pool, const dsa_batch* batch,
                             const uint16_t* q, const int32_t* idx, const int32_t* phys, int32_t k,
                             float softmax_scale, uint16_t* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  return mla_common(kv, pool, batch, q, idx, phys, k, softmax_scale, out, lse, workspace,
                    workspace_bytes, static_cast<hipStream_t>(stream), false);
}

dsa_status sparse_mla_decode_noalloc(const dsa_kv_layout* kv, const void* pool,
                                     const dsa_batch* batch, const uint16_t* q, const int32_t* idx,
                                     const int32_t* phys, int32_t k, float softmax_scale,
                                     uint16_t* out, float* lse, void* stream) {
  g_err[0] = 0;
  return mla_common(kv, pool, batch, q, idx, phys, k, softmax_scale, out, lse, nullptr, 0,
                    static_cast<hipStream_t>(stream), false, -1, 1, nullptr, true);
}

dsa_status sparse_mla_prefill(const dsa_kv_layout* kv, const void* pool, const dsa_batch* batch,
                              const uint16_t* q, const int32_t* idx, const int32_t* phys, int32_t k,
                              float softmax_scale, uint16_t* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  return mla_common(kv, pool, batch, q, idx, phys, k, softmax_scale, out, lse, workspace,
                    workspace_bytes, static_cast<hipStream_t>(stream), true);
}

dsa_status dsa_cache_append(const dsa_kv_layout* kv, void* pool, int32_t num_tokens,
                            const int64_t* slot, const uint16_t* index_key, const uint16_t* latent,
                            void* stream) {
  g_err[0] = 0;
  dsa_status st = check_layout(kv, pool);
  if (st != DSA_OK) return st;
  if (num_tokens < 0) return fail(DSA_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (num_tokens == 0 || (!index_key && !latent)) return DSA_OK;
  if (!slot) return fail(DSA_ERR_INVALID_ARG, "slot must be non-NULL");
  if (!aligned(slot, 8) || (index_key && !aligned(index_key, 4)) ||
      (latent && !aligned(latent, 8)))
    return fail(DSA_ERR_INVALID_ARG,
                "slot must be 8-byte, index_key 4-byte and latent 8-byte aligned");
  const float ts = kv->latent_format == DSA_LATENT_NVFP4 ? kv->latent_tensor_scale : 1.f;
  return hip_status(dsa::launch_cache_write(pool_view(kv, pool), static_cast<uint8_t*>(pool),
                                            kv->ikey_format, kv->latent_format, ts, num_tokens,
                                            slot, index_key, latent,
                                            static_cast<hipStream_t>(stream)),
                    "dsa_cache_append launch");
}

dsa_status dsa_quantize_query(int32_t num_rows, const uint16_t* q, const float* w, uint8_t* q_idx,
                              float* w_out, void* stream) {
  g_err[0] = 0;
  if (num_rows < 0) return fail(DSA_ERR_INVALID_ARG, "num_rows must be >= 0");
  if (num_rows > (1 << 25)) return fail(DSA_ERR_INVALID_ARG, "num_rows too large");
  if (num_rows == 0) return DSA_OK;
  if (!q || !w || !q_idx || !w_out)
    return fail(DSA_ERR_INVALID_ARG, "q, w, q_idx and w_out must be non-NULL");
  if (!aligned(q, 4) || !aligned(w, 4) || !aligned(q_idx, 2) || !aligned(w_out, 4))
    return fail(DSA_ERR_INVALID_ARG, "q, w, w_out must be 4-byte and q_idx 2-byte aligned");
  return hip_status(dsa::launch_quantize_query(num_rows, q, w, q_idx, w_out,
                                               static_cast<hipStream_t>(stream)),
                    "dsa_quantize_query launch");
}

dsa_status dsa_indexer_front(const dsa_kv_layout* kv, void* pool, int32_t num_tokens,
                             const int64_t* slot, const uint16_t* index_key, int32_t num_rows,
                             const uint16_t* q, const float* w, uint8_t* q_idx, float* w_out,
                             void* stream) {
  g_err[0] = 0;
  dsa_status st = check_layout(kv, pool);
  if (st != DSA_OK) return st;
  if (num_tokens < 0 || num_rows < 0)
    return fail(DSA_ERR_INVALID_ARG, "num_tokens and num_rows must be >= 0");
  if (num_rows > (1 << 25)) return fail(DSA_ERR_INVALID_ARG, "num_rows too large");
  if (num_tokens > 0 && (!slot || !index_key))
    return fail(DSA_ERR_INVALID_ARG, "slot and index_key must be non-NULL when num_tokens > 0");
  if (num_rows > 0 && (!q || !w || !q_idx || !w_out))
    return fail(DSA_ERR_INVALID_ARG, "q, w, q_idx and w_out must be non-NULL when num_rows > 0");
  if (num_tokens > 0 && (!aligned(slot, 8) || !aligned(index_key, 4)))
    return fail(DSA_ERR_INVALID_ARG, "slot must be 8-byte and index_key 4-byte aligned");
  if (num_rows > 0 &&
      (!aligned(q, 4) || !aligned(w, 4) || !aligned(q_idx, 2) || !aligned(w_out, 4)))
    return fail(DSA_ERR_INVALID_ARG, "q, w, w_out must be 4-byte and q_idx 2-byte aligned");
  if (num_tokens == 0 && num_rows == 0) return DSA_OK;
  return hip_status(dsa::launch_indexer_front(pool_view(kv, pool), static_cast<uint8_t*>(pool),
                                              kv->ikey_format, num_tokens, slot, index_key,
                                              num_rows, q, w, q_idx, w_out,
                                              static_cast<hipStream_t>(stream)),
                    "dsa_indexer_front launch");
}

size_t dsa_dcp_mailbox_bytes(int32_t num_rows, int32_t k, int32_t num_shards) {
  if (num_rows <= 0 || k < 1 || k > DSA_MAX_TOPK || num_shards < 1 ||
      num_shards > DSA_MAX_SHARDS)
    return 0;
  return dsa::dcp_mailbox_bytes(num_rows, k, num_shards);
}

static dsa_status check_dcp(int32_t num_rows, int32_t k, int32_t num_shards, const void* mailbox,
                            size_t mailbox_bytes) {
  if (num_rows < 0) return fail(DSA_ERR_INVALID_ARG, "num_rows must be >= 0");
  if (num_rows > (1 << 20)) return fail(DSA_ERR_INVALID_ARG, "num_rows too large");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID_ARG, "k %d not in [1, 2048]", k);
  if (num_shards < 1 || num_shards > DSA_MAX_SHARDS)
    return fail(DSA_ERR_INVALID_ARG, "num_shards %d not in [1, %d]", num_shards, DSA_MAX_SHARDS);
  if (num_rows == 0) return DSA_OK;
  const size_t need = dsa::dcp_mailbox_bytes(num_rows, k, num_shards);
  if (!mailbox || mailbox_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "mailbox of %zu bytes needed, %zu given", need,
                mailbox ? mailbox_bytes : (size_t)0);
  if (!aligned(mailbox, 16)) return fail(DSA_ERR_INVALID_ARG, "mailbox must be 16-byte aligned");
  return DSA_OK;
}

dsa_status dsa_dcp_publish(int32_t num_rows, int32_t k, int32_t num_shards, int32_t shard,
                           const float* scores, int64_t ld_scores, const int32_t* idx,
                           const int32_t* count, void* mailbox, size_t mailbox_bytes,
                           void* stream) {
  g_err[0] = 0;
  dsa_status st = check_dcp(num_rows, k, num_shards, mailbox, mailbox_bytes);
  if (st != DSA_OK || num_rows == 0) return st;
  if (shard < 0 || shard >= num_shards)
    return fail(DSA_ERR_INVALID_ARG, "shard %d not in [0, %d)", shard, num_shards);
  if (!scores || !idx || !count)
    return fail(DSA_ERR_INVALID_ARG, "scores, idx and count must be non-NULL");
  if (ld_scores < 1) return fail(DSA_ERR_INVALID_ARG, "ld_scores must be positive");
  return hip_status(dsa::launch_dcp_publish(num_rows, k, num_shards, shard, scores, ld_scores, idx,
                                            count, mailbox, static_cast<hipStream_t>(stream)),
                    "dsa_dcp_publish launch");
}

dsa_status dsa_dcp_merge(int32_t num_rows, int32_t k, int32_t num_shards, int32_t variant,
                         void* mailbox, size_t mailbox_bytes, int32_t* idx, int32_t* count,
                         int32_t* shard_idx, int32_t* shard_count, int32_t* stats, void* stream) {
  g_err[0] = 0;
  dsa_status st = check_dcp(num_rows, k, num_shards, mailbox, mailbox_bytes);
  if (st != DSA_OK || num_rows == 0) return st;
  if (variant != DSA_MERGE_PACKED && variant != DSA_MERGE_SCORES && variant != DSA_MERGE_GENERIC)
    return fail(DSA_ERR_INVALID_ARG, "unknown merge variant %d", variant);
  if (!idx || !count || !shard_idx || !shard_count)
    return fail(DSA_ERR_INVALID_ARG, "idx, count, shard_idx and shard_count must be non-NULL");
  return hip_status(dsa::launch_dcp_merge(num_rows, k, num_shards, variant, mailbox, idx, count,
                                          shard_idx, shard_count, stats,
                                          static_cast<hipStream_t>(stream)),
                    "dsa_dcp_merge launch");
}

size_t dsa_dcp_partials_bytes(int32_t num_rows, int32_t k, int32_t num_shards, uint32_t flags) {
  if (num_rows <= 0 || k < 1 || k > DSA_MAX_TOPK || num_shards < 1 ||
      num_shards > DSA_MAX_SHARDS)
    return 0;
  int32_t ns, per;
  shard_splits(num_rows, k, num_shards, (flags & DSA_BATCH_INVARIANT) != 0, &ns, &per);
  return partial_bytes(num_rows, num_shards * ns);
}

dsa_status sparse_mla_decode_shard(const dsa_kv_layout* kv, const void* pool,
                                   const dsa_batch* batch, const uint16_t* q, const int32_t* idx,
                                   const int32_t* count, const int32_t* phys, int32_t k,
                                   float softmax_scale, int32_t shard, int32_t num_shards,
                                   void* partials, size_t partials_bytes, void* stream) {
  g_err[0] = 0;
  if (shard < 0) return fail(DSA_ERR_INVALID_ARG, "shard %d out of range", shard);
  return mla_common(kv, pool, batch, q, idx, phys, k, softmax_scale, nullptr, nullptr, partials,
                    partials_bytes, static_cast<hipStream_t>(stream), false, shard, num_shards,
                    count);
}

dsa_status dsa_lse_combine(int32_t num_rows, int32_t k, int32_t num_shards, uint32_t flags,
                           const void* partials, size_t partials_bytes, uint16_t* out, float* lse,
                           void* stream) {
  g_err[0] = 0;
  if (num_rows < 0 || num_rows > (1 << 20))
    return fail(DSA_ERR_INVALID_ARG, "num_rows out of range");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID_ARG, "k %d not in [1, 2048]", k);
  if (num_shards < 1 || num_shards > DSA_MAX_SHARDS)
    return fail(DSA_ERR_INVALID_ARG, "num_shards %d not in [1, %d]", num_shards, DSA_MAX_SHARDS);
  if (flags & ~(DSA_BATCH_INVARIANT | DSA_BATCH_PLAIN_ORDER))
    return fail(DSA_ERR_INVALID_ARG, "unknown batch flags");
  if (num_rows == 0) return DSA_OK;
  if (!out) return fail(DSA_ERR_INVALID_ARG, "out must be non-NULL");
  if (!aligned(out, 16) || (lse && !aligned(lse, 4)))
    return fail(DSA_ERR_INVALID_ARG, "out must be 16-byte aligned");
  dsa::MlaArgs a = {};
  a.batch.num_rows = num_rows;
  a.k = k;
  int32_t ns, per;
  shard_splits(num_rows, k, num_shards, (flags & DSA_BATCH_INVARIANT) != 0, &ns, &per);
  a.nsplit = ns;
  a.tokens_per_split = per;
  a.split_slots = num_shards * ns;
  a.out = out;
  a.lse = lse;
  const size_t need = partial_bytes(num_rows, a.split_slots);
  if (!partials || partials_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "partials buffer of %zu bytes needed, %zu given", need,
                partials ? partials_bytes : (size_t)0);
  if (!aligned(partials, 16)) return fail(DSA_ERR_INVALID_ARG, "partials must be 16-byte aligned");
  partial_views(a, const_cast<void*>(partials), num_rows);
  return hip_status(dsa::launch_mla_combine(a, static_cast<hipStream_t>(stream)),
                    "dsa_lse_combine launch");
}

}  // extern "C"
