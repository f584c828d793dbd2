"""Pins of the CPU oracle against values and properties fixed by the pages and by mathematics.

Each check is chosen so that a plausible slip in the oracle (a dropped term, a wrong sign or
index, a transposed operand, a wrong tie rule) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- indexer

def test_indexer_fp8_hand_worked():
    g = _load("indexer_fp8_tiny.json")
    q = np.array(g["q_codes"], np.uint8)
    keys = np.array(g["key_codes"], np.uint8)
    assert np.array_equal(oracle.e4m3(q), np.array(g["q_values"]))
    assert np.array_equal(oracle.e4m3(keys), np.array(g["key_values"]))
    s64, s32, mism = oracle.indexer_scores(q, np.array(g["w"], np.float32), keys,
                                           np.array(g["key_scale"], np.float32), 0)
    assert list(s64) == g["scores"] and mism == 0


def test_indexer_mxfp4_hand_worked():
    g = _load("indexer_mxfp4_tiny.json")
    H, D = g["H"], g["D"]
    q = np.zeros((H, D), np.uint8)
    for h, d, c in g["q_nonzero"]:
        q[h, d] = c
    keys = np.zeros((len(g["tokens"]), D // 2), np.uint8)
    sc = np.zeros((len(g["tokens"]), D // 32), np.uint8)
    for t, tok in enumerate(g["tokens"]):
        for j, b in tok["bytes_nonzero"]:
            keys[t, j] = b
        sc[t] = tok["e8m0"]
    s64, _, mism = oracle.indexer_scores(q, np.array(g["w"], np.float32), keys, sc, 1)
    assert list(s64) == g["scores"] and mism == 0


def test_indexer_one_hot_closed_form():
    # q[h] = a e_d for one head h, k = b e_d  =>  score = w[h] * max(0, scale * a * b)
    rng = np.random.default_rng(3)
    vals = [0.25, 0.5, 1.0, 1.5, 2.0, 3.0, -0.5, -1.0, -2.0]
    for _ in range(40):
        h, d = rng.integers(32), rng.integers(128)
        a, b = rng.choice(vals), rng.choice(vals)
        wv = rng.choice([-1.5, -0.25, 0.75, 2.0])
        scale = 2.0 ** -int(rng.integers(0, 7))
        q = np.zeros((32, 128), np.uint8)
        q[h, d] = synth.enc_e4m3([a])[0]
        w = np.zeros(32, np.float32)
        w[h] = wv
        k = np.zeros((1, 128), np.uint8)
        k[0, d] = synth.enc_e4m3([b])[0]
        s64, _, _ = oracle.indexer_scores(q, w, k, np.array([scale], np.float32), 0)
        assert s64[0] == wv * max(0.0, scale * a * b)


def test_indexer_zero_query_and_relu_sign():
    keys, ks = synth.ikey_fp8(7, 0, 0, 64)
    q, w = synth.qidx(7, 0, 1)
    s64, _, _ = oracle.indexer_scores(np.zeros((32, 128), np.uint8), w[0], keys, ks, 0)
    assert np.all(s64 == 0)
    # With all head weights positive the score is a sum of non-negative terms; flipping the sign
    # of every query element turns each head's ReLU input into its negative.
    wp = np.abs(w[0]) + 0.25
    pos, _, _ = oracle.indexer_scores(q[0], wp, keys, ks, 0)
    neg, _, _ = oracle.indexer_scores(q[0] ^ 0x80, wp, keys, ks, 0)
    assert np.all(pos >= 0) and np.all(neg >= 0)
    # per head: ReLU(x) - ReLU(-x) = x, so pos - neg = sum_h w_h * scale * q_h.k
    qv = oracle.e4m3(q[0])
    kv = oracle.e4m3(keys)
    lin = (kv @ qv.T) * ks[:, None].astype(np.float64) @ wp.astype(np.float64)
    assert np.allclose(pos - neg, lin, rtol=0, atol=1e-9)


def test_indexer_head_permutation_and_token_independence():
    keys, ks = synth.ikey_fp8(11, 2, 0, 200)
    q, w = synth.qidx(11, 5, 1)
    base, _, _ = oracle.indexer_scores(q[0], w[0], keys, ks, 0)
    perm = np.random.default_rng(0).permutation(32)
    s2, _, _ = oracle.indexer_scores(q[0][perm], w[0][perm], keys, ks, 0)
    assert np.array_equal(base, s2)
    tp = np.random.default_rng(1).permutation(200)
    s3, _, _ = oracle.indexer_scores(q[0], w[0], keys[tp], ks[tp], 0)
    assert np.array_equal(base[tp], s3)
    # Swapping q and w between two heads must change the score unless the heads are identical.
    q2 = q[0].copy()
    q2[[0, 1]] = q2[[1, 0]]
    s4, _, _ = oracle.indexer_scores(q2, w[0], keys, ks, 0)
    assert not np.array_equal(base, s4)


def test_indexer_scale_enters_each_head_positively():
    # scale_s = 2^-e > 0: doubling it doubles the score exactly.
    keys, ks = synth.ikey_fp8(5, 1, 0, 100)
    q, w = synth.qidx(5, 1, 1)
    a, _, _ = oracle.indexer_scores(q[0], w[0], keys, ks, 0)
    b, _, _ = oracle.indexer_scores(q[0], w[0], keys, ks * 2, 0)
    assert np.array_equal(2 * a, b)


def test_indexer_exact_grid_fp32_equals_fp64():
    for seed in (1, 2):
        keys, ks = synth.ikey_fp8(seed, 0, 0, 4096)
        q, w = synth.qidx(seed, 0, 2)
        for r in range(2):
            _, _, mism = oracle.indexer_scores(q[r], w[r], keys, ks, 0)
            assert mism == 0
        mk, me = synth.ikey_mxfp4(seed, 0, 0, 4096)
        q4, w4 = synth.qidx(seed, 0, 2, wq=4)
        for r in range(2):
            _, _, mism = oracle.indexer_scores(q4[r], w4[r], mk, me, 1)
            assert mism == 0


def test_indexer_exact_grid_worst_case_magnitude():
    # Largest grid magnitudes everywhere: |q|=|k|=4, |w|=2 (FP8) -> still exact in fp32.
    q = np.full((32, 128), synth.enc_e4m3([4.0])[0], np.uint8)
    q[:, 1::2] = synth.enc_e4m3([3.75])[0]
    keys = np.full((3, 128), synth.enc_e4m3([4.0])[0], np.uint8)
    keys[1, ::3] = synth.enc_e4m3([0.25])[0]
    w = np.full(32, 2.0, np.float32)
    w[::2] = -1.75
    _, _, mism = oracle.indexer_scores(q, w, keys, np.array([1, 2.0 ** -6, 0.5], np.float32), 0)
    assert mism == 0
    # MXFP4 bound: |k| <= 6 * 1, |w| <= 1
    mk = np.full((2, 64), 0x77, np.uint8)
    me = np.full((2, 4), 127, np.uint8)
    me[1] = [125, 126, 127, 125]
    _, _, mism = oracle.indexer_scores(q, np.full(32, 1.0, np.float32), mk, me, 1)
    assert mism == 0


# ----------------------------------------------------------------------------- top-k

def test_topk_hand_worked_ties():
    for case in _load("topk_ties.json")["cases"]:
        idx, cnt = oracle.topk(np.array(case["scores"], np.float64), case["k"])
        assert list(idx) == case["idx"], case["why"]
        assert cnt == case["count"]


def _check_topk_property(s, k, idx, cnt):
    n = len(s)
    assert cnt == min(k, n)
    sel = idx[:cnt]
    assert np.all(idx[cnt:] == -1)
    assert np.all(np.diff(sel) > 0)  # ascending, distinct
    mask = np.zeros(n, bool)
    mask[sel] = True
    if cnt < n:
        lo = s[mask].min()
        hi = s[~mask].max()
        assert lo >= hi
        if lo == hi:  # at the threshold value the lowest indices are the ones taken
            tied_sel = np.nonzero(mask & (s == lo))[0]
            tied_out = np.nonzero(~mask & (s == lo))[0]
            assert tied_sel.max() < tied_out.min()


def test_topk_defining_property_random_with_ties():
    rng = np.random.default_rng(4)
    for n, k in [(10, 3), (300, 64), (5000, 2048), (2048, 2048), (2049, 2048), (1, 2048)]:
        s = rng.integers(-20, 20, n).astype(np.float64) / 4  # many ties
        s[rng.random(n) < 0.1] = -0.0
        idx, cnt = oracle.topk(s, k)
        _check_topk_property(s, k, idx, cnt)


def test_topk_brute_force_tiny():
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = int(rng.integers(1, 9))
        k = int(rng.integers(1, 10))
        s = rng.integers(-2, 3, n).astype(np.float64)
        idx, cnt = oracle.topk(s, k)
        # brute force: a token is selected iff fewer than k tokens beat it, where j beats i when
        # s[j] > s[i] or (s[j] == s[i] and j < i)
        want = [i for i in range(n)
                if sum(1 for j in range(n) if s[j] > s[i] or (s[j] == s[i] and j < i)) < k]
        assert list(idx[:cnt]) == want


def test_topk_zero_query_selects_first_tokens():
    idx, cnt = oracle.topk(np.zeros(10000), 2048)
    assert cnt == 2048 and np.array_equal(idx, np.arange(2048))


# ----------------------------------------------------------------------------- attention

def test_mla_hand_worked():
    g = _load("mla_tiny.json")
    out, lse = oracle.sparse_mla(np.array([g["q_bf16"]], np.uint16),
                                 np.array(g["latents"], np.float64), g["softmax_scale"], g["dv"])
    assert out[0, 0] == pytest.approx(g["out"][0], rel=1e-15)
    assert lse[0] == pytest.approx(g["lse"][0], rel=1e-15)


def _rand_q(rng, H=96, D=576):
    return synth.enc_bf16(rng.normal(size=(H, D)).astype(np.float32))


def test_mla_matches_torch_sdpa_float64():
    rng = np.random.default_rng(6)
    codes, sc = synth.latent_fp8(9, 0, 0, 300)
    c = oracle.dequant_latent_fp8(codes, sc)
    q = _rand_q(rng)
    scale = 1 / math.sqrt(192)
    out, lse = oracle.sparse_mla(q, c, scale, 512)
    qt = torch.from_numpy(oracle.bf16(q))[None, :, None, :]  # [1,96,1,576]
    kt = torch.from_numpy(c)[None, None].expand(1, 96, 300, 576)
    vt = torch.from_numpy(c[:, :512])[None, None].expand(1, 96, 300, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    ref = ref[0, :, 0].numpy()
    ref_lse = torch.logsumexp(torch.from_numpy(oracle.bf16(q)) @ torch.from_numpy(c).T * scale,
                              dim=-1).numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_mla_closed_forms():
    rng = np.random.default_rng(7)
    codes, sc = synth.latent_fp8(10, 0, 0, 50)
    c = oracle.dequant_latent_fp8(codes, sc)
    q = _rand_q(rng)
    s = 1 / math.sqrt(192)
    # one token: out = its value exactly, lse = its logit
    out, lse = oracle.sparse_mla(q, c[3:4], s, 512)
    assert np.array_equal(out, np.broadcast_to(c[3, :512], (96, 512)))
    assert np.allclose(lse, s * oracle.bf16(q) @ c[3], rtol=1e-13)
    # identical latents: out = value, lse = logit + ln n
    same = np.repeat(c[5:6], 17, axis=0)
    out, lse = oracle.sparse_mla(q, same, s, 512)
    assert np.allclose(out, np.broadcast_to(c[5, :512], (96, 512)), rtol=1e-13, atol=1e-13)
    assert np.allclose(lse, s * oracle.bf16(q) @ c[5] + math.log(17), rtol=1e-13)
    # q = 0: uniform weights -> mean of the values, lse = ln n
    out, lse = oracle.sparse_mla(np.zeros((96, 576), np.uint16), c, s, 512)
    assert np.allclose(out, np.broadcast_to(c[:, :512].mean(0), (96, 512)), rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, math.log(50))


def test_mla_selected_order_invariance():
    rng = np.random.default_rng(8)
    codes, sc = synth.latent_fp8(12, 0, 0, 64)
    c = oracle.dequant_latent_fp8(codes, sc)
    q = _rand_q(rng)
    a, la = oracle.sparse_mla(q, c, 0.1, 512)
    p = rng.permutation(64)
    b, lb = oracle.sparse_mla(q, c[p], 0.1, 512)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14) and np.allclose(la, lb, rtol=1e-13)


def test_fp8_latent_dequant_hand_worked():
    # distinct per-token scales: a dropped or inverted scale, or one taken from the wrong token,
    # changes the values written out by hand in the fixture
    g = _load("latent_fp8_tiny.json")
    v = oracle.dequant_latent_fp8(np.array(g["codes"], np.uint8),
                                  np.array(g["scales"], np.float32))
    want = np.array(g["values"], np.float64)
    assert np.array_equal(v, want)
    assert np.array_equal(np.signbit(v), np.signbit(want))


def test_nvfp4_latent_dequant_hand_worked():
    # byte 0x53: element 0 = nibble 3 (1.5), element 1 = nibble 5 (3.0); block scale 0x38 = 1.0;
    # byte 0xF8: element 2 = nibble 8 (-0), element 3 = nibble 0xF (-6); tensor scale 0.5.
    packed = np.zeros((1, 8), np.uint8)
    packed[0, 0], packed[0, 1] = 0x53, 0xF8
    bs = np.array([[0x38]], np.uint8)
    v = oracle.dequant_latent_nvfp4(packed, bs, 0.5)
    assert list(v[0, :4]) == [0.75, 1.5, 0.0, -3.0] and np.all(v[0, 4:] == 0)
    bs2 = np.array([[0x30]], np.uint8)  # block scale 0.5
    assert list(oracle.dequant_latent_nvfp4(packed, bs2, 1.0)[0, :4]) == [0.75, 1.5, 0.0, -3.0]


# ----------------------------------------------------------------------------- whole layer

def _tiny_workload(seed, L, rows, k, ikey=0, lat=0):
    wl = synth.Workload("tiny", seed, [L], [0] * len(rows), rows, ikey_fmt=ikey, lat_fmt=lat,
                        k=k, wq=4 if ikey else 8, lat_tensor_scale=0.75 if lat else 1.0)
    return wl


@pytest.mark.parametrize("ikey,lat", [(0, 0), (1, 1)])
def test_layer_equals_dense_attention_when_k_covers_context(ikey, lat):
    # top-k >= visible tokens: the sparse layer is dense causal attention over all tokens.
    wl = _tiny_workload(21, 150, [40, 149], 2048, ikey, lat)
    res = oracle.workload_rows(wl, 0)
    keys, ks, latc, ls = synth.seq_tensors(wl, 0)
    c = (oracle.dequant_latent_fp8(latc, ls) if lat == 0
         else oracle.dequant_latent_nvfp4(latc, ls, wl.lat_tensor_scale))
    _, _, qm = synth.row_queries(wl)
    for i, p in enumerate(wl.row_pos):
        assert res["count"][i] == p + 1
        assert np.array_equal(res["idx"][i, :p + 1], np.arange(p + 1))
        qt = torch.from_numpy(oracle.bf16(qm[i]))[None, :, None, :]  # [1,96,1,576]
        kt = torch.from_numpy(c[:p + 1])[None, None].expand(1, 96, p + 1, 576)
        vt = torch.from_numpy(c[:p + 1, :512])[None, None].expand(1, 96, p + 1, 512)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=wl.softmax_scale)
        assert np.allclose(res["out"][i], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_layer_causal_invariance():
    # Changing tokens after a row's position leaves that row's result unchanged.
    wl = _tiny_workload(22, 3000, [2500], 256)
    keys, ks, lat, ls = synth.seq_tensors(wl, 0)
    qi, hw, qm = synth.row_queries(wl)
    a = oracle.dsa_rows(0, 0, wl.row_pos, qi, hw, qm, keys, ks, lat, ls, 1.0, 256, wl.softmax_scale)
    keys2, lat2 = keys.copy(), lat.copy()
    keys2[2501:] = keys2[2501:][::-1]
    lat2[2501:] = 0x38
    b = oracle.dsa_rows(0, 0, wl.row_pos, qi, hw, qm, keys2, ks, lat2, ls, 1.0, 256,
                        wl.softmax_scale)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["out"], b["out"])


def test_layer_selected_set_is_the_defining_top_k():
    wl = _tiny_workload(23, 5000, [4999, 3000], 2048)
    res = oracle.workload_rows(wl, 0, want_scores=True)
    assert res["mism"] == 0
    for i, p in enumerate(wl.row_pos):
        s = res["scores"][i, :p + 1]
        _check_topk_property(s, 2048, res["idx"][i], res["count"][i])


_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _latents_from_codes(wl, lat, ls, sel):
    """Dequantised latents of the tokens `sel`, built here from the stored codes with torch's
    E4M3 cast and the OCP E2M1 table (not through the oracle's decoders): FP8, code times the
    token's own scale; NVFP4, E2M1 element times its block's E4M3 scale times the tensor scale."""
    f8 = lambda c: torch.from_numpy(np.ascontiguousarray(c, np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()
    if wl.lat_fmt == 0:
        return f8(lat[sel]) * ls[sel].astype(np.float64)[:, None]
    packed = lat[sel]
    nib = np.empty((len(sel), 576), np.uint8)
    nib[:, 0::2] = packed & 0xF
    nib[:, 1::2] = packed >> 4
    val = np.where(nib & 8, -1.0, 1.0) * _E2M1[nib & 7]
    bs = np.repeat(f8(ls[sel]), 16, axis=1)
    return val * bs * float(wl.lat_tensor_scale)


@pytest.mark.parametrize("ikey,lat", [(0, 0), (1, 1)])
def test_layer_attention_over_a_strict_subset(ikey, lat):
    # k < visible tokens at interior positions: the attention runs over exactly the selected
    # tokens, each latent taken at its own token index with its own scale.  The reference is
    # float64 SDPA over latents gathered at the oracle's own idx and decoded independently.
    wl = _tiny_workload(24, 3000, [1500, 2999, 2203], 256, ikey, lat)
    res = oracle.workload_rows(wl, 0)
    _, _, latc, ls = synth.seq_tensors(wl, 0)
    _, _, qm = synth.row_queries(wl)
    for i, p in enumerate(wl.row_pos):
        cnt = int(res["count"][i])
        sel = res["idx"][i, :cnt]
        assert cnt == 256 and np.all(res["idx"][i, cnt:] == -1)
        # a strict, non-trivial subset: slot j does not hold token j
        assert sel.max() <= p and np.count_nonzero(sel != np.arange(cnt)) > cnt // 2
        c = _latents_from_codes(wl, latc, ls, sel)
        qf = torch.from_numpy(oracle.bf16(qm[i]))  # [96, 576]
        ct = torch.from_numpy(c)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qf[None, :, None, :], ct[None, None].expand(1, 96, cnt, 576),
            ct[None, None, :, :512].expand(1, 96, cnt, 512), scale=wl.softmax_scale)[0, :, 0]
        ref_lse = torch.logsumexp(qf @ ct.T * wl.softmax_scale, dim=-1)
        assert np.allclose(res["out"][i], ref.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(res["lse"][i], ref_lse.numpy(), rtol=1e-12, atol=1e-12)
