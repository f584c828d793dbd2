// Internal launch interface between the C ABI layer (dsa_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa_device.h"

namespace dsa {

struct BatchView {
  const int32_t* block_table;
  int64_t ld_bt;
  const int32_t* seq_row_start;
  const int32_t* row_pos;
  int32_t num_seqs, num_rows;
};

struct IndexerArgs {
  PoolView pool;
  BatchView batch;
  const uint8_t* q;  // [R][32][128] e4m3
  const float* w;    // [R][32]
  float* scores;     // [R][ld]
  int64_t ld;
  uint32_t* hist;    // [R][2048] or null
  int32_t tiles_per_seq;  // row tiles per sequence (1 on the decode path)
  int32_t plain_order;    // prefill row tiles in ascending order instead of the balanced one
  int32_t pages_per_wave; // multi-row scorer: key pages per wave (a multiple of 4)
  uint32_t* status;       // the device status word (DSA_DEVERR_* bits)
  // Candidates path (scores never stored in full).  The sample pass scores blocks 0, S, 2S, ...
  // of each sequence into `scores` in sample numbering (sample token 64 j + t is token
  // 64 S j + t); the candidate pass scores the other blocks and appends (order key, token) of
  // each token at or above its row's floor to the row's candidate list.
  int32_t sample_stride;   // S (>= 1)
  uint2* cand;             // [R][cand_cap]
  int32_t* cand_count;     // [R] entries appended so far (may exceed cand_cap: overflow)
  uint32_t* cand_max;      // [R] the largest key in the row's list
  const uint32_t* floor;   // [R][2]: key T and tie cutoff I: keep key > T, or key == T and token < I
  int64_t cand_cap;
};
// Scorer modes: every block into dense scores; the sample blocks into dense sample scores; the
// other blocks into candidate lists.
enum { kScoreDense = 0, kScoreSample = 1, kScoreCand = 2 };

// Decode / speculative decode scorer: grid (chunks, num_seqs).
hipError_t launch_indexer_decode(const IndexerArgs& a, int ikey_fmt, int rows_per_seq,
                                 int64_t max_context, hipStream_t s, int mode = kScoreDense);
// Prefill scorer (dense contraction of row tiles x key tiles; FP8 or MXFP4 keys).
hipError_t launch_indexer_prefill(const IndexerArgs& a, int ikey_fmt, int64_t max_context,
                                  int32_t max_rows_per_seq, hipStream_t s, int mode = kScoreDense);

// Candidate selects (one workgroup per row): SRC 0 reads a row's dense sample scores and leaves
// its exact top-k as the row's first candidates plus the floor; SRC 1 selects the row's top-k
// from its candidate list and writes idx / count / phys.
struct CandArgs {
  BatchView batch;
  int32_t k;
  int32_t sample_stride;
  const float* samp;  // [R][samp_ld] sample scores (SRC 0)
  int64_t samp_ld;
  uint2* cand;        // [R][cand_cap]
  int32_t* cand_count;
  uint32_t* cand_max; // [R]
  uint32_t* floor;    // [R][2]
  int64_t cand_cap;
  int32_t* idx;       // [R][k] (SRC 1)
  int32_t* count;     // [R]
  int32_t* phys;      // [R][k] or null
  uint32_t* status;
};
hipError_t launch_cand_select(const CandArgs& a, int src, hipStream_t s);
hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s);

constexpr int kTopkSlice = 4096;   // scores per filter workgroup
constexpr int kMaxSlices = 2048;   // => contexts up to 8M tokens

struct TopkArgs {
  BatchView batch;
  const float* scores;
  int64_t ld;
  uint32_t* hist_in;  // [R][2048] key histogram (from the scorer or the hist pass); zeroed once consumed
  int32_t k;
  int32_t* idx;
  int32_t* count;
  int32_t* phys;  // or null
  // workspace views (set by launch_topk)
  uint32_t* slice_cnt;  // [R][num_slices] survivors per slice
  uint32_t* level1;     // [R][2] threshold bin of the top 11 key bits, and how many of k it holds
  uint2* cand;          // [R][cand_ld] survivors (order key, token index), slice-major
  int64_t cand_ld;
  int32_t num_slices;
  int32_t vec_ok;       // scores rows are 16-byte aligned
  int32_t max_n;        // the batch's bound on visible tokens per row (direct select: reads stop there)
  const uint32_t* status;  // the device status word: a row-count violation poisons the select
};
size_t topk_workspace_bytes(int32_t num_rows, int64_t max_context);
hipError_t launch_topk(const TopkArgs& a, int64_t max_context, void* workspace, hipStream_t s);

struct MlaArgs {
  PoolView pool;
  BatchView batch;
  const uint16_t* q;  // [R][96][576] bf16
  const int32_t* idx; // [R][k]
  const int32_t* phys; // [R][k] pool rows of idx, or null
  const int32_t* count; // [R] selected entries at the front of each idx row, or null (all k)
  int32_t k;
  float softmax_scale;
  float tensor_scale;  // NVFP4 latent tensor scale (1 for FP8)
  uint16_t* out;       // [R][96][512] bf16
  float* lse;          // [R][96] or null
  uint16_t* part_o;    // [R][split_slots][12 waves][8][64 lanes][8] fp16 normalised split outputs
                       // * 2^part_exp, in the attention kernel's accumulator layout
  float* part_lse;     // [R][split_slots][96] base-2 log-sum-exp of each split
  int32_t* part_exp;   // [R][split_slots][96] power-of-two scale exponent of each split output
  int32_t nsplit;           // splits of this call (grid y)
  int32_t tokens_per_split;
  int32_t split_base;       // first partial slot of this call's splits in each row
  int32_t split_slots;      // partial slots per row (nsplit, or shards x nsplit across shards)
  int32_t out_direct;       // one split, no partials: the attention writes out and lse itself
  int32_t nt_partials;      // store the partials non-temporally (a large set)
  uint32_t* status;         // the device status word (DSA_DEVERR_* bits), or null
};
int mla_num_splits(int32_t num_rows, int32_t k, bool invariant);
size_t mla_workspace_bytes(int32_t num_rows, int32_t k, bool invariant);
// Attention (grid rows x nsplit), then, unless out_direct or !combine, the split combine.
hipError_t launch_sparse_mla(const MlaArgs& a, int lat_fmt, bool combine, hipStream_t s);
// The log-sum-exp combine of split_slots partial slots per row into out / lse.
hipError_t launch_mla_combine(const MlaArgs& a, hipStream_t s);

// The step before the path: quantise new tokens into their pool rows, and the indexer query.
hipError_t launch_cache_write(const PoolView& pool, uint8_t* base, int ikey_fmt, int lat_fmt,
                              float tensor_scale, int32_t n, const int64_t* slot,
                              const uint16_t* ikey, const uint16_t* latent, hipStream_t s);
hipError_t launch_quantize_query(int32_t num_rows, const uint16_t* q, const float* w, uint8_t* qo,
                                 float* wo, hipStream_t s);
// Both index-key writes and query quantisation in one launch (latents not touched).
hipError_t launch_indexer_front(const PoolView& pool, uint8_t* base, int ikey_fmt, int32_t n,
                                const int64_t* slot, const uint16_t* ikey, int32_t num_rows,
                                const uint16_t* q, const float* w, uint8_t* qo, float* wo,
                                hipStream_t s);

// Read-bandwidth probe (measurement only): page i is bytes_per_page bytes at
// base + (rows ? rows[i] : i) * row_bytes + offset.
constexpr int kProbeMaxPieces = 576;  // 16-byte pieces per page (9,216 bytes)
struct ProbeArgs {
  const uint8_t* base;
  int64_t row_bytes, offset;
  int32_t bytes_per_page;
  const int32_t* rows;
  int64_t num_pages;
  uint32_t* sink;  // [grid] one word per workgroup
  int32_t grid;
};
hipError_t launch_probe_read(const ProbeArgs& a, hipStream_t s);

// Decode context parallelism emulated on one GPU: shard lists and the exact merge.
size_t dcp_mailbox_bytes(int32_t num_rows, int32_t k, int32_t num_shards);
hipError_t launch_dcp_publish(int32_t R, int32_t k, int32_t W, int32_t shard, const float* scores,
                              int64_t ld, const int32_t* idx, const int32_t* count, void* mb,
                              hipStream_t s);
hipError_t launch_dcp_merge(int32_t R, int32_t k, int32_t W, int32_t variant, void* mb,
                            int32_t* idx, int32_t* count, int32_t* shard_idx,
                            int32_t* shard_count, int32_t* stats, hipStream_t s);

}  // namespace dsa
