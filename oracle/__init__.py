"""CPU oracle of the DSA layer (lightning-indexer scores -> exact top-k -> exact sparse MLA).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  It shares no code with the GPU path; the arithmetic lives in oracle.c
(plain loops, double precision) and this module only marshals numpy arrays.

Source: "vLLM Delivers Day-0 Support for Kimi K3.1 Pro" (§Sparse Attention in K3.1 Pro; §A KV
cache for three kinds of state; §AMD / Quantization: Native MXFP4 indexer).  The indexer rule is
DeepSeek-V3.2's lightning indexer, to which the pages defer:
    score[s] = sum_h w[h] * ReLU(scale_s * q[h] . k[s]).
The quantisers (the step before the path, §Low-latency decode: a fused DSA decode path) quantise
the new token's index key and latent and the indexer query.
Parity pins: see tests/test_oracle.py, tests/test_codecs.py and tests/test_oracle_quant.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile oracle.c (host C, OpenMP, no FMA contraction) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               "-Wall", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        d, vp, i64, i32 = ctypes.c_double, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_e4m3.restype = d
        L.orc_e4m3.argtypes = [ctypes.c_uint8]
        L.orc_e2m1.restype = d
        L.orc_e2m1.argtypes = [ctypes.c_uint8]
        L.orc_e8m0.restype = d
        L.orc_e8m0.argtypes = [ctypes.c_uint8]
        L.orc_bf16.restype = d
        L.orc_bf16.argtypes = [ctypes.c_uint16]
        L.orc_indexer_scores.restype = i64
        L.orc_indexer_scores.argtypes = [i32, i32, i32, vp, vp, i64, vp, vp, vp, vp]
        L.orc_topk.restype = None
        L.orc_topk.argtypes = [i64, vp, i32, vp, vp]
        L.orc_dequant_latent_fp8.restype = None
        L.orc_dequant_latent_fp8.argtypes = [i32, vp, ctypes.c_float, vp]
        L.orc_dequant_latent_nvfp4.restype = None
        L.orc_dequant_latent_nvfp4.argtypes = [i32, vp, vp, ctypes.c_float, vp]
        L.orc_sparse_mla.restype = None
        L.orc_sparse_mla.argtypes = [i32, i32, i32, vp, i64, vp, d, vp, vp]
        L.orc_dsa_rows.restype = i64
        L.orc_dsa_rows.argtypes = [i32, i32, i32, vp, vp, vp, vp, i64, vp, vp, vp, vp,
                                   ctypes.c_float, i32, d, vp, vp, vp, vp, vp]
        L.orc_quant_e4m3.restype = ctypes.c_uint8
        L.orc_quant_e4m3.argtypes = [ctypes.c_float]
        L.orc_quant_e2m1.restype = ctypes.c_uint8
        L.orc_quant_e2m1.argtypes = [ctypes.c_float]
        for f in (L.orc_quant_fp8_token, L.orc_quant_mxfp4_key, L.orc_quant_nvfp4_latent,
                  L.orc_quantize_query):
            f.restype = None
        L.orc_quant_fp8_token.argtypes = [i32, vp, vp, vp]
        L.orc_quant_mxfp4_key.argtypes = [i32, vp, vp, vp]
        L.orc_quant_nvfp4_latent.argtypes = [i32, vp, ctypes.c_float, vp, vp]
        L.orc_quantize_query.argtypes = [i32, i32, vp, vp, vp, vp]
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype)


def _p(a):
    return ctypes.c_void_p(a.ctypes.data)


# ----------------------------------------------------------------------------- codecs

def e4m3(codes) -> np.ndarray:
    c = np.asarray(codes, np.uint8)
    L = lib()
    return np.array([L.orc_e4m3(int(v)) for v in c.ravel()], np.float64).reshape(c.shape)


def e2m1(nibbles) -> np.ndarray:
    c = np.asarray(nibbles, np.uint8)
    L = lib()
    return np.array([L.orc_e2m1(int(v)) for v in c.ravel()], np.float64).reshape(c.shape)


def e8m0(codes) -> np.ndarray:
    c = np.asarray(codes, np.uint8)
    L = lib()
    return np.array([L.orc_e8m0(int(v)) for v in c.ravel()], np.float64).reshape(c.shape)


def bf16(bits) -> np.ndarray:
    c = np.asarray(bits, np.uint16)
    L = lib()
    return np.array([L.orc_bf16(int(v)) for v in c.ravel()], np.float64).reshape(c.shape)


# ----------------------------------------------------------------------------- steps

def indexer_scores(q, w, keys, key_scale, key_fmt: int = 0):
    """Scores of one row.  q [H,D] e4m3 codes, w [H] f32, keys [n,D] e4m3 (fmt 0) or [n,D/2]
    packed e2m1 (fmt 1), key_scale f32 [n] (fmt 0) or e8m0 [n,D/32] (fmt 1).
    Returns (score64 [n], score32 [n], number of tokens where fp32 != fp64)."""
    q = _c(q, np.uint8)
    H, D = q.shape
    w = _c(w, np.float32)
    keys = _c(keys, np.uint8)
    n = keys.shape[0]
    ks = _c(key_scale, np.float32 if key_fmt == 0 else np.uint8)
    s64 = np.empty(n, np.float64)
    s32 = np.empty(n, np.float32)
    mism = lib().orc_indexer_scores(H, D, key_fmt, _p(q), _p(w), n, _p(keys), _p(ks), _p(s64),
                                    _p(s32))
    return s64, s32, int(mism)


def topk(scores, k: int):
    """(idx [k] ascending, -1 padded; count) of the exact top-k of one row."""
    s = _c(scores, np.float64)
    idx = np.empty(k, np.int32)
    cnt = np.zeros(1, np.int32)
    lib().orc_topk(s.shape[0], _p(s), k, _p(idx), _p(cnt))
    return idx, int(cnt[0])


def dequant_latent_fp8(codes, scale) -> np.ndarray:
    codes = _c(codes, np.uint8)
    n, D = codes.shape
    scale = _c(scale, np.float32)
    out = np.empty((n, D), np.float64)
    for j in range(n):
        lib().orc_dequant_latent_fp8(D, _p(codes[j]), float(scale[j]), _p(out[j]))
    return out


def dequant_latent_nvfp4(packed, bscale, tensor_scale: float) -> np.ndarray:
    packed = _c(packed, np.uint8)
    n, half = packed.shape
    bscale = _c(bscale, np.uint8)
    out = np.empty((n, 2 * half), np.float64)
    for j in range(n):
        lib().orc_dequant_latent_nvfp4(2 * half, _p(packed[j]), _p(bscale[j]),
                                       float(tensor_scale), _p(out[j]))
    return out


def sparse_mla(q_bf16, c, softmax_scale: float, dv: int):
    """Exact attention of one row: q [H,Dqk] bf16 bits, c [nsel,Dqk] dequantised latents.
    Returns (out [H,dv] float64, lse [H])."""
    q = _c(q_bf16, np.uint16)
    H, Dqk = q.shape
    c = _c(c, np.float64).reshape(-1, Dqk)
    out = np.empty((H, dv), np.float64)
    lse = np.empty(H, np.float64)
    lib().orc_sparse_mla(H, Dqk, dv, _p(q), c.shape[0], _p(c), float(softmax_scale), _p(out),
                         _p(lse))
    return out, lse


def dsa_rows(key_fmt, lat_fmt, row_pos, qidx, w, qmla, keys, key_scale, lat, lat_scale,
             lat_tensor_scale, k, softmax_scale, want_scores=False):
    """The whole layer for the rows of one sequence (logical inputs).  Returns a dict with idx
    [R,k], count [R], out [R,96,512], lse [R,96], mism (inexact fp32 scores) and, on request,
    scores [R,ntok] (-inf past each row's position)."""
    rp = _c(row_pos, np.int64)
    R = rp.shape[0]
    qidx = _c(qidx, np.uint8)
    w = _c(w, np.float32)
    qmla = _c(qmla, np.uint16)
    keys = _c(keys, np.uint8)
    ntok = keys.shape[0]
    ks = _c(key_scale, np.float32 if key_fmt == 0 else np.uint8)
    lat = _c(lat, np.uint8)
    ls = _c(lat_scale, np.float32 if lat_fmt == 0 else np.uint8)
    idx = np.empty((R, k), np.int32)
    cnt = np.empty(R, np.int32)
    out = np.empty((R, 96, 512), np.float64)
    lse = np.empty((R, 96), np.float64)
    sc = np.empty((R, ntok), np.float64) if want_scores else None
    mism = lib().orc_dsa_rows(key_fmt, lat_fmt, R, _p(rp), _p(qidx), _p(w), _p(qmla), ntok,
                              _p(keys), _p(ks), _p(lat), _p(ls), float(lat_tensor_scale), k,
                              float(softmax_scale), _p(idx), _p(cnt), _p(out), _p(lse),
                              _p(sc) if sc is not None else None)
    res = dict(idx=idx, count=cnt, out=out, lse=lse, mism=int(mism))
    if sc is not None:
        res["scores"] = sc
    return res


def workload_rows(wl, b: int, rows=None, ntok=None, want_scores=False):
    """Oracle result for sequence b of a synth.Workload (all its rows, or the listed ones).
    The logical inputs are regenerated from the seed; the paged pool is never read."""
    import synth
    rows = wl.rows_of(b) if rows is None else np.asarray(rows)
    need = int(wl.row_pos[rows].max()) + 1 if ntok is None else ntok
    keys, ks, lat, ls = synth.seq_tensors(wl, b, need)
    qi = np.empty((len(rows), 32, 128), np.uint8)
    hw = np.empty((len(rows), 32), np.float32)
    qm = np.empty((len(rows), 96, 576), np.uint16)
    for i, r in enumerate(rows):
        a, c = synth.qidx(wl.seed, int(wl.row_id[r]), 1, wl.wq)
        qi[i], hw[i] = a[0], c[0]
        qm[i] = synth.qmla(wl.seed, int(wl.row_id[r]), 1)[0]
    return dsa_rows(wl.ikey_fmt, wl.lat_fmt, wl.row_pos[rows], qi, hw, qm, keys, ks, lat, ls,
                    wl.lat_tensor_scale, wl.k, wl.softmax_scale, want_scores)


# ----------------------------------------------------------------------------- quantisers
# (the step before the path: writing the new token into its paged row, quantising the query)

def quant_e4m3(x) -> np.ndarray:
    """e4m3 codes of fp32 values: nearest, ties to even, saturating at 448."""
    a = np.asarray(x, np.float32)
    L = lib()
    return np.array([L.orc_quant_e4m3(float(v)) for v in a.ravel()], np.uint8).reshape(a.shape)


def quant_e2m1(x) -> np.ndarray:
    """e2m1 nibbles of fp32 values: nearest, ties to even, saturating at 6."""
    a = np.asarray(x, np.float32)
    L = lib()
    return np.array([L.orc_quant_e2m1(float(v)) for v in a.ravel()], np.uint8).reshape(a.shape)


def quant_fp8_token(x_bf16):
    """[D] bf16 bits -> (codes [D] e4m3, scale f32)."""
    x = _c(x_bf16, np.uint16)
    codes = np.empty(x.size, np.uint8)
    s = np.empty(1, np.float32)
    lib().orc_quant_fp8_token(x.size, _p(x), _p(codes), _p(s))
    return codes, float(s[0])


def quant_mxfp4_key(x_bf16):
    """[D] bf16 bits -> (packed e2m1 [D/2], e8m0 scales [D/32])."""
    x = _c(x_bf16, np.uint16)
    packed = np.empty(x.size // 2, np.uint8)
    sc = np.empty(x.size // 32, np.uint8)
    lib().orc_quant_mxfp4_key(x.size, _p(x), _p(packed), _p(sc))
    return packed, sc


def quant_nvfp4_latent(x_bf16, tensor_scale: float):
    """[D] bf16 bits -> (packed e2m1 [D/2], e4m3 block scales [D/16])."""
    x = _c(x_bf16, np.uint16)
    packed = np.empty(x.size // 2, np.uint8)
    sc = np.empty(x.size // 16, np.uint8)
    lib().orc_quant_nvfp4_latent(x.size, _p(x), float(tensor_scale), _p(packed), _p(sc))
    return packed, sc


def quantize_query(q_bf16, w):
    """q [H,D] bf16 bits, w [H] f32 -> (codes [H,D] e4m3, w' [H] f32)."""
    q = _c(q_bf16, np.uint16)
    w = _c(w, np.float32)
    H, D = q.shape
    codes = np.empty((H, D), np.uint8)
    wout = np.empty(H, np.float32)
    lib().orc_quantize_query(H, D, _p(q), _p(w), _p(codes), _p(wout))
    return codes, wout
