"""Seeded synthetic inputs for the DSA layer (shared by the GPU path and the CPU oracle).

Holds no part of the method's arithmetic: it draws counter-based random numbers, encodes them
into the storage formats, lays them out in a paged pool and describes workloads.  Values are a
pure function of (seed, tensor, sequence or row, element index), so the oracle regenerates just
the sequences it checks.

Workload shapes follow the layer described in "vLLM Delivers Day-0 Support for Kimi K3.1 Pro"
(§Sparse Attention in K3.1 Pro: 32 indexer heads x 128 dims, top-2048, 96 MLA heads; §A KV cache
for three kinds of state: paged blocks of a power-of-two size, FP8 or NVFP4 latents, FP8 or
MXFP4 index keys).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

IKEY_FP8, IKEY_MXFP4 = 0, 1
LATENT_FP8, LATENT_NVFP4 = 0, 1
IDX_HEADS, IDX_DIM = 32, 128
MLA_HEADS, MLA_DQK, MLA_DV = 96, 576, 512


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so (host C, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.synth_hash.restype = u64
        L.synth_hash.argtypes = [u64, ctypes.c_uint32, u64, u64]
        L.synth_enc_e4m3.restype = ctypes.c_uint8
        L.synth_enc_e4m3.argtypes = [ctypes.c_double]
        L.synth_enc_e2m1.restype = ctypes.c_uint8
        L.synth_enc_e2m1.argtypes = [ctypes.c_double]
        L.synth_enc_bf16.restype = ctypes.c_uint16
        L.synth_enc_bf16.argtypes = [ctypes.c_float]
        for fn in ("synth_ikey_fp8", "synth_ikey_mxfp4", "synth_latent_fp8", "synth_latent_nvfp4"):
            getattr(L, fn).restype = None
            getattr(L, fn).argtypes = [u64, i64, i64, i64, vp, vp]
        L.synth_qidx.restype = None
        L.synth_qidx.argtypes = [u64, i64, i64, i32, vp, vp]
        L.synth_qmla.restype = None
        L.synth_qmla.argtypes = [u64, i64, i64, vp]
        L.synth_fill_pool.restype = None
        L.synth_fill_pool.argtypes = [u64, i32, i32, i32, i64, i64, i64, i64, i64, i64, vp, i32,
                                      vp, i64, vp, vp, i64, i64]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


# ----------------------------------------------------------------------------- logical tensors

def ikey_fp8(seed: int, seq: int, tok0: int, ntok: int):
    codes = np.empty((ntok, IDX_DIM), np.uint8)
    scale = np.empty((ntok,), np.float32)
    lib().synth_ikey_fp8(seed, seq, tok0, ntok, _p(codes), _p(scale))
    return codes, scale


def ikey_mxfp4(seed: int, seq: int, tok0: int, ntok: int):
    packed = np.empty((ntok, IDX_DIM // 2), np.uint8)
    e8m0 = np.empty((ntok, IDX_DIM // 32), np.uint8)
    lib().synth_ikey_mxfp4(seed, seq, tok0, ntok, _p(packed), _p(e8m0))
    return packed, e8m0


def latent_fp8(seed: int, seq: int, tok0: int, ntok: int):
    codes = np.empty((ntok, MLA_DQK), np.uint8)
    scale = np.empty((ntok,), np.float32)
    lib().synth_latent_fp8(seed, seq, tok0, ntok, _p(codes), _p(scale))
    return codes, scale


def latent_nvfp4(seed: int, seq: int, tok0: int, ntok: int):
    packed = np.empty((ntok, MLA_DQK // 2), np.uint8)
    bscale = np.empty((ntok, MLA_DQK // 16), np.uint8)
    lib().synth_latent_nvfp4(seed, seq, tok0, ntok, _p(packed), _p(bscale))
    return packed, bscale


def qidx(seed: int, row0: int, nrows: int, wq: int = 8):
    q = np.empty((nrows, IDX_HEADS, IDX_DIM), np.uint8)
    w = np.empty((nrows, IDX_HEADS), np.float32)
    lib().synth_qidx(seed, row0, nrows, wq, _p(q), _p(w))
    return q, w


def qmla(seed: int, row0: int, nrows: int):
    q = np.empty((nrows, MLA_HEADS, MLA_DQK), np.uint16)
    lib().synth_qmla(seed, row0, nrows, _p(q))
    return q


def enc_e4m3(x) -> np.ndarray:
    L = lib()
    x = np.asarray(x, np.float64)
    return np.array([L.synth_enc_e4m3(float(v)) for v in x.ravel()], np.uint8).reshape(x.shape)


def enc_e2m1(x) -> np.ndarray:
    L = lib()
    x = np.asarray(x, np.float64)
    return np.array([L.synth_enc_e2m1(float(v)) for v in x.ravel()], np.uint8).reshape(x.shape)


def enc_bf16(x) -> np.ndarray:
    L = lib()
    x = np.asarray(x, np.float32)
    return np.array([L.synth_enc_bf16(float(v)) for v in x.ravel()], np.uint16).reshape(x.shape)


# ----------------------------------------------------------------------------- workloads

@dataclass
class Workload:
    """One batch of query rows over a paged, block-packed KV pool.

    seq_len[b]: cached tokens of sequence b (its rows see prefixes of these);
    row_seq/row_pos: rows sorted by sequence, row r sees tokens [0, row_pos[r]];
    block_table[b, j]: pool block holding tokens [64 j, 64 j + 64) of sequence b.
    seq_id/row_id: generator ids (so replicas and sub-batches get distinct data).
    """
    name: str
    seed: int
    seq_len: np.ndarray
    row_seq: np.ndarray
    row_pos: np.ndarray
    ikey_fmt: int = IKEY_FP8
    lat_fmt: int = LATENT_FP8
    block_size: int = 64
    k: int = 2048
    softmax_scale: float = 1.0 / math.sqrt(192.0)
    lat_tensor_scale: float = 1.0
    spare_blocks: int = 8
    wq: int = 8
    seq_id: np.ndarray = None
    row_id: np.ndarray = None
    block_table: np.ndarray = field(default=None, repr=False)
    num_blocks: int = 0
    tok_stride: int = 1   # token t of a pool sequence is generator token t * stride + offset
    tok_offset: int = 0

    def __post_init__(self):
        self.seq_len = np.asarray(self.seq_len, np.int64)
        self.row_seq = np.asarray(self.row_seq, np.int32)
        self.row_pos = np.asarray(self.row_pos, np.int32)
        assert np.all(np.diff(self.row_seq) >= 0), "rows must be grouped by sequence"
        if self.seq_id is None:
            self.seq_id = np.arange(len(self.seq_len), dtype=np.int64)
        if self.row_id is None:
            self.row_id = np.arange(len(self.row_pos), dtype=np.int64)
        for r, (b, p) in enumerate(zip(self.row_seq, self.row_pos)):
            assert 0 <= p < self.seq_len[b], (r, b, p)
        if self.block_table is None:
            self.block_table, self.num_blocks = shuffled_block_table(
                self.seed, self.seq_len, self.block_size, self.spare_blocks)

    @property
    def num_seqs(self) -> int:
        return len(self.seq_len)

    @property
    def num_rows(self) -> int:
        return len(self.row_pos)

    @property
    def seq_row_start(self) -> np.ndarray:
        return np.searchsorted(self.row_seq, np.arange(self.num_seqs + 1)).astype(np.int32)

    def rows_of(self, b: int) -> np.ndarray:
        return np.nonzero(self.row_seq == b)[0]


def shuffled_block_table(seed: int, seq_len, block_size: int, spare: int):
    """Block tables of all sequences as one random permutation of a shared pool (plus `spare`
    poisoned blocks no table points at)."""
    nb = [(int(L) + block_size - 1) // block_size for L in seq_len]
    total = sum(nb) + spare
    perm = np.random.Generator(np.random.PCG64(seed)).permutation(total).astype(np.int32)
    width = max(nb) if nb else 1
    bt = np.full((len(nb), width), -1, np.int32)
    at = 0
    for b, n in enumerate(nb):
        bt[b, :n] = perm[at:at + n]
        at += n
    return bt, total


def shard_workload(w: Workload, W: int, r: int) -> Workload:
    """Shard r of W of workload w under token-interleaved sharding: token j of a shard sequence
    is token j*W + r of the original sequence (same data), and a row at position p sees the
    shard's tokens [0, (p - r) // W] (p >= r).  The shard's pool has its own shuffled block table;
    the rows keep their generator ids, so their queries are those of w."""
    assert w.tok_stride == 1 and w.tok_offset == 0 and 0 <= r < W
    assert np.all(w.row_pos >= r), "every row must see at least one token of every shard"
    lens = np.array([(int(L) - r + W - 1) // W for L in w.seq_len], np.int64)
    bt, nb = shuffled_block_table(w.seed * 1000003 + 7919 * (r + 1) + W, lens, w.block_size,
                                  w.spare_blocks)
    return Workload(f"{w.name}-shard{r}of{W}", w.seed, lens, w.row_seq.copy(),
                    (w.row_pos - r) // W, ikey_fmt=w.ikey_fmt, lat_fmt=w.lat_fmt,
                    block_size=w.block_size, k=w.k, softmax_scale=w.softmax_scale,
                    lat_tensor_scale=w.lat_tensor_scale, spare_blocks=w.spare_blocks, wq=w.wq,
                    seq_id=w.seq_id.copy(), row_id=w.row_id.copy(), block_table=bt,
                    num_blocks=nb, tok_stride=W, tok_offset=r)


def fill_pool(w: Workload, layout) -> np.ndarray:
    """Pool bytes [num_blocks * row_bytes] for workload `w`.  `layout` gives row_bytes and the
    four in-row byte offsets (from the library's layout descriptor)."""
    row_bytes = int(layout["row_bytes"])
    pool = np.empty(w.num_blocks * row_bytes, np.uint8)
    bt = np.ascontiguousarray(w.block_table, np.int32)
    lens = np.ascontiguousarray(w.seq_len, np.int64)
    sid = np.ascontiguousarray(w.seq_id, np.int64)
    lib().synth_fill_pool(w.seed, w.ikey_fmt, w.lat_fmt, w.block_size, row_bytes,
                          int(layout["latent_off"]), int(layout["latent_scale_off"]),
                          int(layout["ikey_off"]), int(layout["ikey_scale_off"]), w.num_blocks,
                          _p(pool), w.num_seqs, _p(bt), bt.shape[1], _p(lens), _p(sid),
                          w.tok_stride, w.tok_offset)
    return pool


def row_queries(w: Workload):
    """(q_idx [R,32,128] e4m3 codes, w [R,32] f32, q [R,96,576] bf16 bits) of the workload."""
    R = w.num_rows
    qi = np.empty((R, IDX_HEADS, IDX_DIM), np.uint8)
    hw = np.empty((R, IDX_HEADS), np.float32)
    qm = np.empty((R, MLA_HEADS, MLA_DQK), np.uint16)
    for r in range(R):
        a, b = qidx(w.seed, int(w.row_id[r]), 1, w.wq)
        qi[r], hw[r] = a[0], b[0]
        qm[r] = qmla(w.seed, int(w.row_id[r]), 1)[0]
    return qi, hw, qm


def seq_tensors(w: Workload, b: int, ntok: int | None = None):
    """Logical (unpaged) keys and latents of sequence b: (keys, key_scale, lat, lat_scale)."""
    n = int(w.seq_len[b]) if ntok is None else ntok
    sid = int(w.seq_id[b])
    if w.ikey_fmt == IKEY_FP8:
        keys, kscale = ikey_fp8(w.seed, sid, 0, n)
    else:
        keys, kscale = ikey_mxfp4(w.seed, sid, 0, n)
    if w.lat_fmt == LATENT_FP8:
        lat, lscale = latent_fp8(w.seed, sid, 0, n)
    else:
        lat, lscale = latent_nvfp4(w.seed, sid, 0, n)
    return keys, kscale, lat, lscale


# ----------------------------------------------------------------------------- named shapes

def decode_config(i: int, seed: int | None = None, replica: int = 0) -> Workload:
    """The layer shapes this project measures: 0 decode 8K, 1 batched decode 16 x 128K,
    2 speculative decode 16 x (1+5) at 1M, 3 chunked prefill 8192 on 339,968, 4 mixed-length
    64 x log-uniform[4K, 256K] with MXFP4 keys and NVFP4 latents, 5 short-append prefill
    2048 on 150,000, 6 the first 16,384-row chunk of a prompt (positions 0 .. 16,383)."""
    seed = (1000 + i + 7919 * replica) if seed is None else seed
    if i == 0:
        return Workload("decode-1x8K", seed, [8192], [0], [8191])
    if i == 1:
        L = 131072
        return Workload("decode-16x128K", seed, [L] * 16, list(range(16)), [L - 1] * 16)
    if i == 2:
        L = 1048576
        rs = [b for b in range(16) for _ in range(6)]
        rp = [L - 6 + j for _ in range(16) for j in range(6)]
        return Workload("specdec-16x6-1M", seed, [L] * 16, rs, rp)
    if i == 3:
        P, T = 339968, 8192
        return Workload("prefill-8192-on-339968", seed, [P + T], [0] * T,
                        [P + t for t in range(T)])
    if i == 5:
        P, T = 150000, 2048
        return Workload("prefill-2048-on-150000", seed, [P + T], [0] * T,
                        [P + t for t in range(T)])
    if i == 6:
        # the first chunk of a prompt: rows at every position from 0, so the causal work of a row
        # grows along the chunk
        T = 16384
        return Workload("prefill-16384-from-0", seed, [T], [0] * T, list(range(T)))
    if i == 4:
        g = np.random.Generator(np.random.PCG64(seed + 1))
        Ls = np.floor(np.exp(g.uniform(math.log(4096), math.log(262144), 64))).astype(np.int64)
        return Workload("mixed-64-mxfp4-nvfp4", seed, Ls, list(range(64)), list(Ls - 1),
                        ikey_fmt=IKEY_MXFP4, lat_fmt=LATENT_NVFP4, wq=4, lat_tensor_scale=0.75)
    raise ValueError(i)
