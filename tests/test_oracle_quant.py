"""Pins of the oracle's quantisers (the step before the path: the new token's index key and latent
written into its paged row, and the indexer query quantised with its per-head scale folded into
the head weight).

The oracle rounds by exhaustive nearest search over the codes of a format.  These tests pin it to
what the formats fix independently of that search:
  - an arithmetic formulation of round-to-nearest-even on the format's grid (the spacing of each
    binade, numpy's half-to-even rint), with saturation at the largest finite value;
  - exact round trips of every code and of tokens made of representable values;
  - the scale rules (FP8 token scale amax/448, OCP MX E8M0 scale with amax/X in [4, 8), NVFP4
    E4M3 block scale of amax/6) and the error bounds they imply;
  - the fold of the query scale into the head weight, through the scoring rule.
"""
import numpy as np
import pytest

import oracle

E4M3_MAX = 448.0


def _e4m3_value(c):
    return oracle.e4m3(np.array([c], np.uint8))[0]


def _rne_e4m3(v):
    """|v| -> e4m3 magnitude on the grid (3 mantissa bits, min normal 2^-6, subnormal step
    2^-9), round half to even, saturating at 448."""
    v = abs(float(v))
    e = max(int(np.floor(np.log2(v))) if v > 0 else -6, -6)
    step = 2.0 ** (e - 3)
    return min(float(np.rint(v / step)) * step, E4M3_MAX)


def _rne_e2m1(v):
    """|v| -> e2m1 magnitude on {0, .5, 1, 1.5, 2, 3, 4, 6}, round half to even code."""
    v = abs(float(v))
    if v < 2:
        return float(np.rint(v * 2)) / 2
    if v < 4:
        return float(np.rint(v))
    return min(float(np.rint(v / 2)) * 2, 6.0)


E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])


def _bf16(x):
    """fp32 -> bf16 bits, round to nearest even (test-side helper)."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def _f(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_e4m3_every_code_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    vals = oracle.e4m3(finite).astype(np.float32)
    got = oracle.quant_e4m3(vals)
    assert np.array_equal(got, finite)


def test_e2m1_every_code_round_trips():
    nib = np.arange(16, dtype=np.uint8)
    vals = np.where(nib & 8, -1.0, 1.0) * E2M1[nib & 7]
    assert np.array_equal(oracle.quant_e2m1(vals.astype(np.float32)), nib)


def test_e4m3_midpoints_go_to_even_code():
    for c in range(0, 0x7E):
        lo, hi = _e4m3_value(c), _e4m3_value(c + 1)
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.quant_e4m3([mid])[0] == even, c
        assert oracle.quant_e4m3([np.nextafter(mid, np.float32(0))])[0] == c
        assert oracle.quant_e4m3([np.nextafter(mid, np.float32(1e9))])[0] == c + 1
        assert oracle.quant_e4m3([-mid])[0] == 0x80 | even


def test_e2m1_midpoints_go_to_even_code():
    for c in range(7):
        mid = np.float32((E2M1[c] + E2M1[c + 1]) / 2)
        even = c if c % 2 == 0 else c + 1
        assert oracle.quant_e2m1([mid])[0] == even
        assert oracle.quant_e2m1([np.nextafter(mid, np.float32(0))])[0] == c
        assert oracle.quant_e2m1([np.nextafter(mid, np.float32(9))])[0] == c + 1


def test_saturation_and_signed_zero():
    assert list(oracle.quant_e4m3([448.0, 464.0, 1e6, np.inf, -1e30])) == [0x7E, 0x7E, 0x7E, 0x7E,
                                                                          0xFE]
    assert list(oracle.quant_e2m1([6.0, 7.0, 100.0, -1e9, 5.0])) == [7, 7, 7, 15, 6]
    assert list(oracle.quant_e4m3([0.0, -0.0, 2.0 ** -11, -2.0 ** -11])) == [0, 0x80, 0, 0x80]
    assert list(oracle.quant_e2m1([0.0, -0.0, 0.25, -0.2])) == [0, 8, 0, 8]


def test_rounding_matches_arithmetic_formulation():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.uniform(-4, 3, 3000),
                        rng.uniform(-8, 8, 1000)]).astype(np.float32)
    q4 = oracle.quant_e4m3(x)
    got4 = oracle.e4m3(q4)
    want4 = np.array([np.copysign(_rne_e4m3(v), v) for v in x])
    assert np.array_equal(got4, want4)
    q2 = oracle.quant_e2m1(x)
    got2 = np.where(q2 & 8, -1.0, 1.0) * E2M1[q2 & 7]
    want2 = np.array([np.copysign(_rne_e2m1(v), v) for v in x])
    assert np.array_equal(got2, want2)


def test_fp8_token_scale_and_error_bound():
    rng = np.random.default_rng(5)
    for D, spread in ((128, 1.0), (576, 30.0), (576, 1e-3)):
        x = _bf16(rng.standard_normal(D) * spread)
        codes, s = oracle.quant_fp8_token(x)
        xf = _f(x).astype(np.float64)
        amax = np.abs(xf).max()
        assert s == np.float32(np.float32(amax) / np.float32(448))
        deq = oracle.e4m3(codes) * s
        # e4m3 keeps 3 mantissa bits: relative error <= 2^-4 for normals, absolute <= 2^-10 * s
        # on the subnormal grid; the largest element lands on 448 within one rounding of s
        assert np.all(np.abs(deq - xf) <= np.maximum(np.abs(xf) * 2.0 ** -4, s * 2.0 ** -10))
        assert codes[np.argmax(np.abs(xf))] & 0x7F == 0x7E
    zero = np.zeros(128, np.uint16)
    codes, s = oracle.quant_fp8_token(zero)
    assert s == 1.0 and not codes.any()


def test_fp8_token_exact_round_trip():
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 256, 576).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10
    codes[17] = 0xFE                                   # -448 sets amax exactly
    s = 2.0 ** -5
    x = _bf16(oracle.e4m3(codes) * s)
    assert np.array_equal(_f(x).astype(np.float64), oracle.e4m3(codes) * s)
    got, gs = oracle.quant_fp8_token(x)
    assert gs == s
    # +0 and -0 codes are both exact encodings of a zero value
    same = (got == codes) | (((got & 0x7F) == 0) & ((codes & 0x7F) == 0))
    assert same.all()


def _unpack(packed, D):
    out = np.empty(D, np.uint8)
    out[0::2] = packed & 0xF
    out[1::2] = packed >> 4
    return out


def test_mxfp4_key_scale_rule_and_bound():
    rng = np.random.default_rng(7)
    for spread in (1.0, 1e-3, 200.0):
        x = _bf16(rng.standard_normal(128) * spread * rng.uniform(0.1, 10, 128))
        packed, sc = oracle.quant_mxfp4_key(x)
        xf = _f(x).astype(np.float64)
        nib = _unpack(packed, 128)
        val = np.where(nib & 8, -1.0, 1.0) * E2M1[nib & 7]
        for b in range(4):
            blk = np.abs(xf[32 * b:32 * b + 32])
            X = 2.0 ** (int(sc[b]) - 127)
            assert 4 <= blk.max() / X < 8, (b, blk.max(), X)
            assert int(sc[b]) - 127 == int(np.floor(np.log2(blk.max()))) - 2
            # grid step at most 2X below 8X, saturation at 6X costs < 2X
            err = np.abs(val[32 * b:32 * b + 32] * X - xf[32 * b:32 * b + 32])
            assert np.all(err <= 2 * X)
            assert np.all(err[blk < 4 * X] <= X)


def test_mxfp4_key_exact_round_trip_and_zero_block():
    rng = np.random.default_rng(8)
    nib = rng.integers(0, 16, 128).astype(np.uint8)
    nib[5] = 7                                         # every block holds a 6 or a 4
    nib[40] = 14
    nib[64 + 3] = 6
    nib[96 + 31] = 15
    E = np.array([120, 127, 131, 100])
    X = 2.0 ** (E - 127).astype(np.float64)
    vals = np.where(nib & 8, -1.0, 1.0) * E2M1[nib & 7] * np.repeat(X, 32)
    x = _bf16(vals)
    assert np.array_equal(_f(x).astype(np.float64), vals)
    packed, sc = oracle.quant_mxfp4_key(x)
    assert np.array_equal(sc, E.astype(np.uint8))
    got = _unpack(packed, 128)
    assert np.all((got == nib) | (((got & 7) == 0) & ((nib & 7) == 0)))
    zero = np.zeros(128, np.uint16)
    packed, sc = oracle.quant_mxfp4_key(zero)
    assert np.all(sc == 127) and not packed.any()


def test_nvfp4_latent_scale_rule_bound_and_round_trip():
    rng = np.random.default_rng(9)
    ts = np.float32(2.0 ** -8)
    x = _bf16(rng.standard_normal(576) * rng.uniform(0.01, 3, 576))
    packed, bs = oracle.quant_nvfp4_latent(x, float(ts))
    xf = _f(x).astype(np.float64)
    deq = oracle.dequant_latent_nvfp4(packed[None], bs[None], float(ts))[0]
    for b in range(36):
        blk = xf[16 * b:16 * b + 16]
        want_bs = oracle.quant_e4m3([np.float32(np.float32(np.abs(blk).max()) / np.float32(6)) /
                                     ts])[0]
        assert bs[b] == want_bs
        sd = oracle.e4m3(bs[b:b + 1])[0] * float(ts)
        # the block scale is within one e4m3 rounding of amax/6, so amax/sd is within 6(1 +- 2^-4)
        # and every element is on the grid {0..6} * sd up to half a step (1 * sd) or saturation
        assert np.all(np.abs(deq[16 * b:16 * b + 16] - blk) <= 1.0 * sd + 1e-12 + 0.4 * sd)
    # exact round trip: blocks built from representable values with a 6 in each block
    nib = rng.integers(0, 16, 576).astype(np.uint8)
    nib[::16] = 7
    bsc = rng.integers(0x30, 0x60, 36).astype(np.uint8)
    vals = (np.where(nib & 8, -1.0, 1.0) * E2M1[nib & 7] *
            np.repeat(oracle.e4m3(bsc), 16) * float(ts))
    xr = _bf16(vals)
    assert np.array_equal(_f(xr).astype(np.float64), vals)
    packed, bs = oracle.quant_nvfp4_latent(xr, float(ts))
    assert np.array_equal(bs, bsc)
    got = _unpack(packed, 576)
    assert np.all((got == nib) | (((got & 7) == 0) & ((nib & 7) == 0)))


def test_query_fold_preserves_scores_within_quantisation_bound():
    rng = np.random.default_rng(10)
    H, D = 32, 128
    q = _bf16(rng.standard_normal((H, D)) * rng.uniform(0.1, 5, (H, 1)))
    w = (rng.standard_normal(H) * 0.2).astype(np.float32)
    codes, w2 = oracle.quantize_query(q, w)
    qf = _f(q).astype(np.float64).reshape(H, D)
    s = np.array([oracle.quant_fp8_token(q[h])[1] for h in range(H)])
    assert np.array_equal(w2, (w * s.astype(np.float32)).astype(np.float32))
    deq = oracle.e4m3(codes).reshape(H, D)
    keys = rng.standard_normal((50, D))
    exact = (np.maximum(qf @ keys.T, 0) * w[:, None]).sum(0)
    folded = (np.maximum(deq @ keys.T, 0) * w2.astype(np.float64)[:, None]).sum(0)
    # per head the dequantised query (codes * s_h) differs from q by at most
    # max(2^-4 |q|, 2^-10 s_h) per element; ReLU is 1-Lipschitz
    err_q = np.maximum(np.abs(qf) * 2.0 ** -4, s[:, None] * 2.0 ** -10)
    bound = np.abs(w.astype(np.float64)) @ (err_q @ np.abs(keys).T) * (1 + 1e-6) + 1e-9
    assert np.all(np.abs(exact - folded) <= bound)
    # and the bound is not vacuous: the fold is tight to a few per cent of the score scale
    assert np.abs(exact - folded).max() < 0.1 * np.abs(exact).max()


@pytest.mark.parametrize("H", [1, 32])
def test_query_fold_zero_head(H):
    q = np.zeros((H, 128), np.uint16)
    w = np.full(H, 0.5, np.float32)
    codes, w2 = oracle.quantize_query(q, w)
    assert not codes.any() and np.all(w2 == 0.5)
