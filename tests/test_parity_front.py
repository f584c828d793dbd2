"""Parity of the step before the path: dsa_cache_append (new tokens quantised into their pool
rows), dsa_quantize_query (the FP8 indexer query with its scale folded into the head weight) and
dsa_indexer_front (the keys and the query in one launch), against the oracle's quantisers, bit for
bit.

The pool starts as random bytes; after the calls the whole pool must equal the same random bytes
with exactly the oracle's codes and scales written at the given slots, so a stray write anywhere
fails too.  Inputs are seeded bf16 values of widely varying magnitude per token, plus tokens built
so that every element sits exactly on a rounding midpoint of its format (ties to even), an
all-zero token with negative zeros, a padding slot (-1) and a slot past the end of the pool."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_decode_amd as sad
from pool_layout import fp8_key_positions

pytestmark = pytest.mark.gpu

_E4M3_POS = np.array([m * 2.0 ** -9 for m in range(8)] +
                     [2.0 ** (e - 7) * (1 + m / 8) for e in range(1, 16) for m in range(8)][:-1])
E4M3_MID = (_E4M3_POS[:-1] + _E4M3_POS[1:]) / 2          # every rounding midpoint below 448
E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _bf16(x):
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _tokens(rng, n, D):
    """bf16 bits [n, D]: random magnitudes, then the special tokens 0..2."""
    x = rng.standard_normal((n, D)) * 10.0 ** rng.uniform(-3, 2, (n, 1))
    x *= rng.uniform(0.05, 1.5, (n, D))
    x[0] = 0.0
    t = _bf16(x)
    t[0, 1::3] = 0x8000                                    # negative zeros
    # token 1: every element an E4M3 midpoint times 2^-3 with amax 448 * 2^-3, so the FP8 token
    # scale is exactly 2^-3 and every code is a tie
    v = rng.choice(E4M3_MID, D) * np.where(rng.random(D) < 0.5, -1, 1)
    v[0] = 448.0
    t[1] = _bf16(v * 2.0 ** -3)
    # token 2: every 16-block holds 6 P and E2M1 midpoints times P (P = 2^-2): MXFP4 X = P and,
    # with a tensor scale of 2^-4, the NVFP4 block scale is exactly P / 2^-4 -- all ties again
    v = rng.choice(E2M1_MID, D) * np.where(rng.random(D) < 0.5, -1, 1)
    v[::16] = 6.0
    t[2] = _bf16(v * 0.25)
    back = (t[1:3].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert back[0, 0] == 56.0 and back[1, 0] == 1.5      # the ties survive the bf16 rounding
    assert np.all(np.isin(np.abs(back[0]) * 8, np.append(E4M3_MID, 448.0)))
    assert np.all(np.isin(np.abs(back[1]) * 4, np.append(E2M1_MID, 6.0)))
    return t


def _expected_rows(kv, pool, slots, ikey, lat, write_keys=True, write_lat=True):
    """Write the oracle's encodings of tokens at `slots` into the host pool copy `pool`."""
    rb, bs = kv.row_bytes, kv.block_size
    for t, s in enumerate(slots):
        if s < 0 or s >= kv.num_blocks * bs:
            continue
        base = (s // bs) * rb
        j = s % bs
        if write_keys and kv.ikey_format == sad.IKEY_FP8:
            codes, sc = oracle.quant_fp8_token(ikey[t])
            pool[base + kv.ikey_off + fp8_key_positions(j)] = codes
            pool[base + kv.ikey_scale_off + 4 * j:][:4] = np.frombuffer(np.float32(sc).tobytes(),
                                                                         np.uint8)
        elif write_keys:
            packed, e = oracle.quant_mxfp4_key(ikey[t])
            pool[base + kv.ikey_off + j * 64:][:64] = packed
            pool[base + kv.ikey_scale_off + 4 * j:][:4] = e
        if write_lat and kv.latent_format == sad.LATENT_FP8:
            codes, sc = oracle.quant_fp8_token(lat[t])
            pool[base + kv.latent_off + j * 576:][:576] = codes
            pool[base + kv.latent_scale_off + 4 * j:][:4] = np.frombuffer(
                np.float32(sc).tobytes(), np.uint8)
        elif write_lat:
            packed, bsc = oracle.quant_nvfp4_latent(lat[t], kv.latent_tensor_scale)
            pool[base + kv.latent_off + j * 288:][:288] = packed
            pool[base + kv.latent_scale_off + 36 * j:][:36] = bsc


def _first_diff(a, b):
    d = np.nonzero(a != b)[0]
    return "" if d.size == 0 else f"{d.size} bytes differ, first at {d[0]}: {a[d[0]]} vs {b[d[0]]}"


@pytest.mark.parametrize("ikey_fmt,lat_fmt,ts", [
    (sad.IKEY_FP8, sad.LATENT_FP8, 1.0),
    (sad.IKEY_MXFP4, sad.LATENT_FP8, 1.0),
    (sad.IKEY_FP8, sad.LATENT_NVFP4, 2.0 ** -4),
    (sad.IKEY_MXFP4, sad.LATENT_NVFP4, 0.37),
])
def test_cache_append_bit_exact(ikey_fmt, lat_fmt, ts):
    print(f"\n[case] cache_append ikey={ikey_fmt} lat={lat_fmt} ts={ts}", flush=True)
    rng = np.random.default_rng(1000 + 10 * ikey_fmt + lat_fmt)
    nblk = 12
    kv = sad.kv_layout(ikey_fmt, lat_fmt, nblk, ts)
    n = 103
    slots = rng.choice(nblk * 64, n, replace=False).astype(np.int64)
    slots[7] = -1
    slots[50] = nblk * 64 + 5
    ikey = _tokens(rng, n, 128)
    lat = _tokens(rng, n, 576)
    host = rng.integers(0, 256, nblk * kv.row_bytes, dtype=np.uint8)
    pool = torch.from_numpy(host.copy()).cuda()
    d_slot = torch.from_numpy(slots).cuda()
    d_ikey = torch.from_numpy(ikey.view(np.int16)).cuda()
    d_lat = torch.from_numpy(lat.view(np.int16)).cuda()
    # keys first (the scorer needs them), then the latents by themselves
    sad.dsa_cache_append(kv, pool, d_slot, index_key=d_ikey)
    torch.cuda.synchronize()
    want = host.copy()
    _expected_rows(kv, want, slots, ikey, lat, write_lat=False)
    got = pool.cpu().numpy()
    assert np.array_equal(got, want), "keys only: " + _first_diff(got, want)
    sad.dsa_cache_append(kv, pool, d_slot, latent=d_lat)
    torch.cuda.synchronize()
    _expected_rows(kv, want, slots, ikey, lat, write_keys=False)
    got = pool.cpu().numpy()
    assert np.array_equal(got, want), "latents: " + _first_diff(got, want)
    # both at once into a fresh pool gives the same bytes
    pool2 = torch.from_numpy(host.copy()).cuda()
    sad.dsa_cache_append(kv, pool2, d_slot, index_key=d_ikey, latent=d_lat)
    torch.cuda.synchronize()
    assert torch.equal(pool, pool2)


def test_cache_append_prefill_chunk():
    # a full prefill chunk of 8,192 new tokens (FP8 keys and latents) into a 160-block pool;
    # 256 sampled tokens are checked against the oracle, every other row must be untouched
    print("\n[case] cache_append prefill 8192", flush=True)
    rng = np.random.default_rng(77)
    nblk = 160
    kv = sad.kv_layout(sad.IKEY_FP8, sad.LATENT_FP8, nblk)
    n = 8192
    blocks = rng.permutation(nblk)[:n // 64]
    slots = (blocks[:, None] * 64 + np.arange(64)[None]).reshape(-1).astype(np.int64)
    ikey = _tokens(rng, n, 128)
    lat = _tokens(rng, n, 576)
    host = rng.integers(0, 256, nblk * kv.row_bytes, dtype=np.uint8)
    pool = torch.from_numpy(host.copy()).cuda()
    sad.dsa_cache_append(kv, pool, torch.from_numpy(slots).cuda(),
                         index_key=torch.from_numpy(ikey.view(np.int16)).cuda(),
                         latent=torch.from_numpy(lat.view(np.int16)).cuda())
    torch.cuda.synchronize()
    got = pool.cpu().numpy().reshape(nblk, kv.row_bytes)
    host = host.reshape(nblk, kv.row_bytes)
    untouched = np.setdiff1d(np.arange(nblk), blocks)
    assert np.array_equal(got[untouched], host[untouched])
    sample = set([0, 1, 2, n - 1] + rng.choice(n, 252, replace=False).tolist())
    want = got.reshape(-1).copy()
    _expected_rows(kv, want, [int(slots[t]) if t in sample else -1 for t in range(n)], ikey, lat)
    assert np.array_equal(got.reshape(-1), want), _first_diff(got.reshape(-1), want)
    # bytes of the written rows outside the four pages (row padding) are untouched
    pad = np.ones(kv.row_bytes, bool)
    for off, size in ((kv.latent_off, 64 * 576), (kv.latent_scale_off, 64 * 4),
                      (kv.ikey_off, 64 * 128), (kv.ikey_scale_off, 64 * 4)):
        pad[off:off + size] = False
    assert np.array_equal(got[blocks][:, pad], host[blocks][:, pad])


@pytest.mark.parametrize("rows", [1, 16, 37])
def test_quantize_query_bit_exact(rows):
    print(f"\n[case] quantize_query rows={rows}", flush=True)
    rng = np.random.default_rng(500 + rows)
    q = _tokens(rng, rows * 32, 128).reshape(rows, 32, 128)
    w = (rng.standard_normal((rows, 32)) * 0.3).astype(np.float32)
    d_q = torch.from_numpy(q.view(np.int16)).cuda()
    d_w = torch.from_numpy(w).cuda()
    q_idx = torch.full((rows, 32, 128), 0x5A, dtype=torch.uint8, device="cuda")
    w_out = torch.full((rows, 32), 7.0, dtype=torch.float32, device="cuda")
    sad.dsa_quantize_query(d_q, d_w, q_idx, w_out)
    torch.cuda.synchronize()
    gq, gw = q_idx.cpu().numpy(), w_out.cpu().numpy()
    for r in range(rows):
        codes, w2 = oracle.quantize_query(q[r], w[r])
        assert np.array_equal(gq[r], codes), f"row {r}: {_first_diff(gq[r].ravel(), codes.ravel())}"
        assert np.array_equal(gw[r].view(np.uint32), w2.view(np.uint32)), f"row {r} weights"
    # in place: w_out may be w
    sad.dsa_quantize_query(d_q, d_w, q_idx, d_w)
    torch.cuda.synchronize()
    assert np.array_equal(d_w.cpu().numpy().view(np.uint32), gw.view(np.uint32))


@pytest.mark.parametrize("ikey_fmt,n,rows", [
    (sad.IKEY_FP8, 77, 16),
    (sad.IKEY_MXFP4, 5, 37),
    (sad.IKEY_FP8, 0, 3),       # query half only
    (sad.IKEY_MXFP4, 9, 0),     # key half only
])
def test_indexer_front_bit_exact(ikey_fmt, n, rows):
    """The fused front writes exactly the oracle's index keys (latent bytes untouched) and the
    oracle's query codes and weights; a latent-only dsa_cache_append afterwards gives the same
    pool as one dsa_cache_append of both."""
    print(f"\n[case] indexer_front ikey={ikey_fmt} n={n} rows={rows}", flush=True)
    rng = np.random.default_rng(3000 + 100 * ikey_fmt + n + rows)
    nblk = 6
    kv = sad.kv_layout(ikey_fmt, sad.LATENT_NVFP4, nblk, 0.37)
    slots = rng.choice(nblk * 64, max(n, 1), replace=False).astype(np.int64)[:n]
    if n > 3:
        slots[1] = -1
        slots[3] = nblk * 64 + 2
    ikey = _tokens(rng, max(n, 3), 128)[:n]
    lat = _tokens(rng, max(n, 3), 576)[:n]
    q = _tokens(rng, max(rows, 1) * 32, 128)[:rows * 32].reshape(rows, 32, 128)
    w = (rng.standard_normal((rows, 32)) * 0.3).astype(np.float32)
    host = rng.integers(0, 256, nblk * kv.row_bytes, dtype=np.uint8)
    pool = torch.from_numpy(host.copy()).cuda()
    d_slot = torch.from_numpy(slots).cuda() if n else None
    d_ikey = torch.from_numpy(ikey.view(np.int16)).cuda() if n else None
    d_q = torch.from_numpy(q.view(np.int16)).cuda() if rows else None
    d_w = torch.from_numpy(w).cuda() if rows else None
    q_idx = torch.full((rows, 32, 128), 0x5A, dtype=torch.uint8, device="cuda") if rows else None
    w_out = torch.full((rows, 32), 7.0, dtype=torch.float32, device="cuda") if rows else None
    sad.dsa_indexer_front(kv, pool, d_slot, d_ikey, d_q, d_w, q_idx, w_out)
    torch.cuda.synchronize()
    want = host.copy()
    _expected_rows(kv, want, slots, ikey, lat, write_lat=False)
    got = pool.cpu().numpy()
    assert np.array_equal(got, want), "keys: " + _first_diff(got, want)
    if rows:
        gq, gw = q_idx.cpu().numpy(), w_out.cpu().numpy()
        for r in range(rows):
            codes, w2 = oracle.quantize_query(q[r], w[r])
            assert np.array_equal(gq[r], codes), f"row {r}: " + _first_diff(gq[r].ravel(),
                                                                             codes.ravel())
            assert np.array_equal(gw[r].view(np.uint32), w2.view(np.uint32)), f"row {r} weights"
    if n:
        d_lat = torch.from_numpy(lat.view(np.int16)).cuda()
        sad.dsa_cache_append(kv, pool, d_slot, latent=d_lat)
        pool2 = torch.from_numpy(host.copy()).cuda()
        sad.dsa_cache_append(kv, pool2, d_slot, index_key=d_ikey, latent=d_lat)
        torch.cuda.synchronize()
        assert torch.equal(pool, pool2)
