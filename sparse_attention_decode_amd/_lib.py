"""ctypes binding of libdsa.so (include/dsa.h).  Argument marshalling only: every step of the
layer runs in the HIP kernels behind the C ABI.  Tensors are torch tensors on the GPU; streams
are torch CUDA(HIP) streams (the current stream by default)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
IKEY_FP8, IKEY_MXFP4 = 0, 1
LATENT_FP8, LATENT_NVFP4 = 0, 1
INDEX_HEADS, INDEX_DIM, MLA_HEADS, MLA_DQK, MLA_DV = 32, 128, 96, 576, 512
MAX_TOPK, HIST_BINS, MAX_ROWS_PER_SEQ = 2048, 2048, 8

# Every symbol include/dsa.h declares.
EXPORTS = ("dsa_kv_layout_init", "dsa_indexer_scores", "dsa_topk_workspace_bytes", "dsa_topk",
           "dsa_candidates_workspace_bytes", "dsa_indexer_candidates", "dsa_topk_candidates",
           "sparse_mla_workspace_bytes",
           "sparse_mla_decode", "sparse_mla_prefill", "sparse_mla_decode_noalloc",
           "dsa_cache_append", "dsa_quantize_query",
           "dsa_indexer_front",
           "dsa_dcp_mailbox_bytes", "dsa_dcp_publish", "dsa_dcp_merge", "dsa_dcp_partials_bytes",
           "sparse_mla_decode_shard", "dsa_lse_combine", "dsa_device_status", "dsa_probe_read", "dsa_status_string",
           "dsa_last_error")
MERGE_PACKED, MERGE_SCORES, MERGE_GENERIC, MAX_SHARDS = 0, 1, 2, 8
# bits of the device status word (include/dsa.h)
DEVERR_ROWS_PER_SEQ, DEVERR_BLOCK_ID, DEVERR_POOL_ROW, DEVERR_CAND_OVERFLOW = 1, 2, 4, 8


class DSAError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


class KVLayout(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("ikey_format", ctypes.c_int32),
                ("latent_format", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("row_bytes", ctypes.c_int64), ("latent_off", ctypes.c_int64),
                ("latent_scale_off", ctypes.c_int64), ("ikey_off", ctypes.c_int64),
                ("ikey_scale_off", ctypes.c_int64), ("num_blocks", ctypes.c_int64),
                ("latent_tensor_scale", ctypes.c_float)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


class Batch(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_rows", ctypes.c_int32),
                ("max_rows_per_seq", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("max_context", ctypes.c_int64), ("block_table", ctypes.c_void_p),
                ("seq_row_start", ctypes.c_void_p), ("row_pos", ctypes.c_void_p),
                ("flags", ctypes.c_uint32)]


BATCH_INVARIANT = 1  # dsa_batch.flags: attention split count from k alone (see include/dsa.h)
BATCH_PLAIN_ORDER = 2  # dsa_batch.flags: prefill row tiles in ascending order, not balanced


_lib = None


def lib():
    """Load libdsa.so (raises if it has not been built: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.dsa_kv_layout_init.restype = i32
        L.dsa_kv_layout_init.argtypes = [ctypes.POINTER(KVLayout), i32, i32, i32, i64, f32]
        L.dsa_indexer_scores.restype = i32
        L.dsa_indexer_scores.argtypes = [ctypes.POINTER(KVLayout), vp, ctypes.POINTER(Batch), vp,
                                         vp, vp, i64, vp, vp]
        L.dsa_topk_workspace_bytes.restype = ctypes.c_size_t
        L.dsa_topk_workspace_bytes.argtypes = [i32, i64]
        L.dsa_topk.restype = i32
        L.dsa_topk.argtypes = [ctypes.POINTER(KVLayout), ctypes.POINTER(Batch), vp, i64, vp, i32,
                               vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.dsa_candidates_workspace_bytes.restype = ctypes.c_size_t
        L.dsa_candidates_workspace_bytes.argtypes = [i32, i64, i32]
        L.dsa_indexer_candidates.restype = i32
        L.dsa_indexer_candidates.argtypes = [ctypes.POINTER(KVLayout), vp, ctypes.POINTER(Batch),
                                             vp, vp, i32, vp, ctypes.c_size_t, vp]
        L.dsa_topk_candidates.restype = i32
        L.dsa_topk_candidates.argtypes = [ctypes.POINTER(KVLayout), ctypes.POINTER(Batch), i32, vp,
                                          ctypes.c_size_t, vp, vp, vp, vp]
        L.sparse_mla_workspace_bytes.restype = ctypes.c_size_t
        L.sparse_mla_workspace_bytes.argtypes = [i32, i32, ctypes.c_uint32]
        for fn in ("sparse_mla_decode", "sparse_mla_prefill"):
            f = getattr(L, fn)
            f.restype = i32
            f.argtypes = [ctypes.POINTER(KVLayout), vp, ctypes.POINTER(Batch), vp, vp, vp, i32,
                          f32, vp, vp, vp, ctypes.c_size_t, vp]
        L.sparse_mla_decode_noalloc.restype = i32
        L.sparse_mla_decode_noalloc.argtypes = [ctypes.POINTER(KVLayout), vp, ctypes.POINTER(Batch),
                                                vp, vp, vp, i32, f32, vp, vp, vp]
        L.dsa_cache_append.restype = i32
        L.dsa_cache_append.argtypes = [ctypes.POINTER(KVLayout), vp, i32, vp, vp, vp, vp]
        L.dsa_quantize_query.restype = i32
        L.dsa_quantize_query.argtypes = [i32, vp, vp, vp, vp, vp]
        L.dsa_indexer_front.restype = i32
        L.dsa_indexer_front.argtypes = [ctypes.POINTER(KVLayout), vp, i32, vp, vp, i32, vp, vp, vp,
                                        vp, vp]
        sz = ctypes.c_size_t
        L.dsa_dcp_mailbox_bytes.restype = sz
        L.dsa_dcp_mailbox_bytes.argtypes = [i32, i32, i32]
        L.dsa_dcp_publish.restype = i32
        L.dsa_dcp_publish.argtypes = [i32, i32, i32, i32, vp, i64, vp, vp, vp, sz, vp]
        L.dsa_dcp_merge.restype = i32
        L.dsa_dcp_merge.argtypes = [i32, i32, i32, i32, vp, sz, vp, vp, vp, vp, vp, vp]
        L.dsa_dcp_partials_bytes.restype = sz
        L.dsa_dcp_partials_bytes.argtypes = [i32, i32, i32, ctypes.c_uint32]
        L.sparse_mla_decode_shard.restype = i32
        L.sparse_mla_decode_shard.argtypes = [ctypes.POINTER(KVLayout), vp, ctypes.POINTER(Batch),
                                              vp, vp, vp, vp, i32, f32, i32, i32, vp, sz, vp]
        L.dsa_lse_combine.restype = i32
        L.dsa_lse_combine.argtypes = [i32, i32, i32, ctypes.c_uint32, vp, sz, vp, vp, vp]
        L.dsa_probe_read.restype = i32
        L.dsa_probe_read.argtypes = [vp, i64, i64, i32, vp, i64, vp, i32, vp]
        L.dsa_device_status.restype = i32
        L.dsa_device_status.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32, vp]
        L.dsa_status_string.restype = ctypes.c_char_p
        L.dsa_status_string.argtypes = [i32]
        L.dsa_last_error.restype = ctypes.c_char_p
        L.dsa_last_error.argtypes = []
        _lib = L
    return _lib


def _check(status: int, fn: str):
    if status != DSA_OK:
        raise DSAError(status, fn, lib().dsa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def kv_layout(ikey_format: int, latent_format: int, num_blocks: int,
              latent_tensor_scale: float = 1.0, block_size: int = 64) -> KVLayout:
    kv = KVLayout()
    _check(lib().dsa_kv_layout_init(ctypes.byref(kv), ikey_format, latent_format, block_size,
                                    num_blocks, latent_tensor_scale), "dsa_kv_layout_init")
    return kv


class DeviceBatch:
    """A dsa_batch plus the device tensors it points at (kept alive here)."""

    def __init__(self, block_table, seq_row_start, row_pos, max_rows_per_seq: int,
                 max_context: int, flags: int = 0):
        self.block_table, self.seq_row_start, self.row_pos = block_table, seq_row_start, row_pos
        b = Batch()
        b.num_seqs = seq_row_start.numel() - 1
        b.num_rows = row_pos.numel()
        b.max_rows_per_seq = int(max_rows_per_seq)
        b.max_blocks_per_seq = block_table.shape[1]
        b.max_context = int(max_context)
        b.block_table = block_table.data_ptr()
        b.seq_row_start = seq_row_start.data_ptr()
        b.row_pos = row_pos.data_ptr()
        b.flags = int(flags)
        self.c = b

    @property
    def num_rows(self) -> int:
        return self.c.num_rows


def dsa_indexer_scores(kv: KVLayout, pool, batch: DeviceBatch, q_idx, w, scores, hist=None,
                       stream=None):
    _check(lib().dsa_indexer_scores(ctypes.byref(kv), _ptr(pool), ctypes.byref(batch.c),
                                    _ptr(q_idx), _ptr(w), _ptr(scores), scores.stride(0),
                                    _ptr(hist), _stream(stream)), "dsa_indexer_scores")


def dsa_topk_workspace_bytes(num_rows: int, max_context: int) -> int:
    return int(lib().dsa_topk_workspace_bytes(num_rows, max_context))


def dsa_topk(kv: KVLayout | None, batch: DeviceBatch, scores, hist, k: int, idx, count,
             workspace, phys=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsa_topk(ctypes.byref(kv) if kv is not None else None, ctypes.byref(batch.c),
                          _ptr(scores), scores.stride(0), _ptr(hist), k, _ptr(idx), _ptr(count),
                          _ptr(phys), _ptr(workspace), ws_bytes, _stream(stream)), "dsa_topk")


def dsa_candidates_workspace_bytes(num_rows: int, max_context: int, k: int) -> int:
    return int(lib().dsa_candidates_workspace_bytes(num_rows, max_context, k))


def dsa_indexer_candidates(kv: KVLayout, pool, batch: DeviceBatch, q_idx, w, k: int, workspace,
                           stream=None):
    """Scores without storing them: the sample pass, its select and the candidate pass."""
    _check(lib().dsa_indexer_candidates(ctypes.byref(kv), _ptr(pool), ctypes.byref(batch.c),
                                        _ptr(q_idx), _ptr(w), k, _ptr(workspace),
                                        _nbytes(workspace), _stream(stream)),
           "dsa_indexer_candidates")


def dsa_topk_candidates(kv: KVLayout | None, batch: DeviceBatch, k: int, workspace, idx, count,
                        phys=None, stream=None):
    """The exact top-k of each row from its candidates (after dsa_indexer_candidates)."""
    _check(lib().dsa_topk_candidates(ctypes.byref(kv) if kv is not None else None,
                                     ctypes.byref(batch.c), k, _ptr(workspace),
                                     _nbytes(workspace), _ptr(idx), _ptr(count), _ptr(phys),
                                     _stream(stream)), "dsa_topk_candidates")


def sparse_mla_workspace_bytes(num_rows: int, k: int, flags: int = 0) -> int:
    return int(lib().sparse_mla_workspace_bytes(num_rows, k, flags))


def _mla(fn: str, kv, pool, batch, q, idx, phys, k, softmax_scale, out, lse, workspace, stream):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(getattr(lib(), fn)(ctypes.byref(kv), _ptr(pool), ctypes.byref(batch.c), _ptr(q),
                              _ptr(idx), _ptr(phys), k, softmax_scale, _ptr(out), _ptr(lse),
                              _ptr(workspace), ws_bytes, _stream(stream)), fn)


def sparse_mla_decode(kv, pool, batch, q, idx, k, softmax_scale, out, lse=None, workspace=None,
                      stream=None, phys=None):
    _mla("sparse_mla_decode", kv, pool, batch, q, idx, phys, k, softmax_scale, out, lse,
         workspace, stream)


def sparse_mla_prefill(kv, pool, batch, q, idx, k, softmax_scale, out, lse=None, workspace=None,
                       stream=None, phys=None):
    _mla("sparse_mla_prefill", kv, pool, batch, q, idx, phys, k, softmax_scale, out, lse,
         workspace, stream)


def sparse_mla_decode_noalloc(kv, pool, batch, q, idx, k, softmax_scale, out, lse=None,
                              stream=None, phys=None):
    """sparse_mla_decode with its split partials in the library's static per-device scratch (no
    workspace argument; nothing is allocated)."""
    _check(lib().sparse_mla_decode_noalloc(ctypes.byref(kv), _ptr(pool), ctypes.byref(batch.c),
                                           _ptr(q), _ptr(idx), _ptr(phys), k, softmax_scale,
                                           _ptr(out), _ptr(lse), _stream(stream)),
           "sparse_mla_decode_noalloc")


def dsa_cache_append(kv: KVLayout, pool, slot, index_key=None, latent=None, stream=None):
    """Quantise new tokens into their pool rows.  slot: int64 [n] physical rows; index_key: bf16
    [n, 128] or None; latent: bf16 [n, 576] or None."""
    _check(lib().dsa_cache_append(ctypes.byref(kv), _ptr(pool), slot.numel(), _ptr(slot),
                                  _ptr(index_key), _ptr(latent), _stream(stream)),
           "dsa_cache_append")


def dsa_quantize_query(q, w, q_idx, w_out, stream=None):
    """q: bf16 [R, 32, 128], w: f32 [R, 32] -> q_idx: uint8 E4M3 [R, 32, 128], w_out: f32 [R, 32]
    (w_out may be w)."""
    _check(lib().dsa_quantize_query(q.shape[0], _ptr(q), _ptr(w), _ptr(q_idx), _ptr(w_out),
                                    _stream(stream)), "dsa_quantize_query")


def dsa_indexer_front(kv: KVLayout, pool, slot, index_key, q, w, q_idx, w_out, stream=None):
    """One launch of dsa_cache_append(index keys only) and dsa_quantize_query.  slot: int64 [n];
    index_key: bf16 [n, 128]; q: bf16 [R, 32, 128]; w: f32 [R, 32]; q_idx: uint8 [R, 32, 128];
    w_out: f32 [R, 32] (may be w).  slot/index_key may be None with n = 0, the query tensors
    None with R = 0."""
    n = 0 if slot is None else slot.numel()
    R = 0 if q is None else q.shape[0]
    _check(lib().dsa_indexer_front(ctypes.byref(kv), _ptr(pool), n, _ptr(slot), _ptr(index_key),
                                   R, _ptr(q), _ptr(w), _ptr(q_idx), _ptr(w_out),
                                   _stream(stream)), "dsa_indexer_front")


def dsa_dcp_mailbox_bytes(num_rows: int, k: int, num_shards: int) -> int:
    return int(lib().dsa_dcp_mailbox_bytes(num_rows, k, num_shards))


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def dsa_dcp_publish(k: int, num_shards: int, shard: int, scores, idx, count, mailbox,
                    stream=None):
    """Shard `shard` publishes its rows' sorted local top-k (scores [R, ld] f32, idx [R, k] and
    count [R] from dsa_topk on that shard) into the mailbox (uint8 device tensor)."""
    _check(lib().dsa_dcp_publish(count.numel(), k, num_shards, shard, _ptr(scores),
                                 scores.stride(0), _ptr(idx), _ptr(count), _ptr(mailbox),
                                 _nbytes(mailbox), _stream(stream)), "dsa_dcp_publish")


def dsa_dcp_merge(k: int, num_shards: int, variant: int, mailbox, idx, count, shard_idx,
                  shard_count, stats=None, stream=None):
    """The exact merge: idx [R, k], count [R], shard_idx [W, R, k], shard_count [W, R] (int32),
    stats [R, 4] int32 or None."""
    _check(lib().dsa_dcp_merge(count.numel(), k, num_shards, variant, _ptr(mailbox),
                               _nbytes(mailbox), _ptr(idx), _ptr(count), _ptr(shard_idx),
                               _ptr(shard_count), _ptr(stats), _stream(stream)), "dsa_dcp_merge")


def dsa_dcp_partials_bytes(num_rows: int, k: int, num_shards: int, flags: int = 0) -> int:
    return int(lib().dsa_dcp_partials_bytes(num_rows, k, num_shards, flags))


def sparse_mla_decode_shard(kv, pool, batch, q, idx, k, softmax_scale, shard: int,
                            num_shards: int, partials, count=None, stream=None, phys=None):
    """One shard's attention over its part of the selection (idx / count: its shard_idx /
    shard_count rows), into its slots of `partials`."""
    _check(lib().sparse_mla_decode_shard(ctypes.byref(kv), _ptr(pool), ctypes.byref(batch.c),
                                         _ptr(q), _ptr(idx), _ptr(count), _ptr(phys), k,
                                         softmax_scale, shard,
                                         num_shards, _ptr(partials), _nbytes(partials),
                                         _stream(stream)), "sparse_mla_decode_shard")


def dsa_lse_combine(num_rows: int, k: int, num_shards: int, partials, out, lse=None, flags=0,
                    stream=None):
    """Merge every shard's partials into out bf16 [R, 96, 512] (and lse f32 [R, 96])."""
    _check(lib().dsa_lse_combine(num_rows, k, num_shards, flags, _ptr(partials),
                                 _nbytes(partials), _ptr(out), _ptr(lse), _stream(stream)),
           "dsa_lse_combine")


def dsa_device_status(clear: bool = True, stream=None) -> int:
    """The device status word (DEVERR_* bits) after the work enqueued on `stream`; synchronises
    that stream, and resets the word to 0 when `clear`."""
    v = ctypes.c_uint32(0)
    _check(lib().dsa_device_status(ctypes.byref(v), 1 if clear else 0, _stream(stream)),
           "dsa_device_status")
    return int(v.value)


def dsa_probe_read(base, row_bytes: int, offset: int, bytes_per_page: int, rows, num_pages: int,
                   sink, stream=None):
    """Measurement only: stream num_pages pages (see include/dsa.h); sink: uint32/int32 device
    tensor with one word per workgroup (its length is the grid)."""
    _check(lib().dsa_probe_read(_ptr(base), row_bytes, offset, bytes_per_page, _ptr(rows),
                                num_pages, _ptr(sink), sink.numel(), _stream(stream)),
           "dsa_probe_read")
