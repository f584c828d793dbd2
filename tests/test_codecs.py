"""Pins of the oracle's number-format decoders and of the generator's encoders.

Decoders are pinned to torch's float8 casts (a library routine independent of the oracle) and,
for E2M1, to the value table of the OCP Microscaling Formats v1.0 specification.
"""
import numpy as np
import torch

import oracle
import synth


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # S.1111.111 for both signs; no infinities
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e8m0_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e8m0(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[125] == 0.25


def test_e2m1_decode_matches_ocp_table():
    # OCP MX v1.0, FP4 E2M1: magnitudes for codes 0..7, bit 3 is the sign.
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    ours = oracle.e2m1(np.arange(16, dtype=np.uint8))
    assert list(ours[:8]) == table
    assert list(ours[8:]) == [-v for v in table]


def test_e2m1_decode_agrees_with_rebased_e4m3():
    # Every E2M1 value is an E4M3 value: rebias the exponent (1 -> 7) and widen the mantissa.
    for c in range(8):
        e, m = c >> 1, c & 1
        if e == 0:
            code8 = 0 if m == 0 else (6 << 3)  # 0 or 0.5 = 2^-1
        else:
            code8 = ((e - 1 + 7) << 3) | (m << 2)
        ref = torch.tensor([code8], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
        assert oracle.e2m1(np.array([c], np.uint8))[0] == ref


def test_bf16_decode_matches_torch():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x0001, 0x7F7F, 0x3C00], np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.bf16(bits), ref)


def test_generator_e4m3_encoder_matches_torch_cast():
    g = np.random.default_rng(0)
    x = np.concatenate([g.normal(size=4000), g.normal(size=2000) * 40, g.normal(size=1000) * 1e-2,
                        # exact midpoints between neighbouring codes exercise ties-to-even
                        (oracle.e4m3(np.arange(0, 125, dtype=np.uint8))
                         + oracle.e4m3(np.arange(1, 126, dtype=np.uint8))) / 2])
    x = x[np.abs(x) < 448]
    ours = synth.enc_e4m3(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    assert synth.enc_e4m3([500.0, -1e6])[0] == 0x7E  # saturates instead of NaN


def test_generator_bf16_encoder_matches_torch_cast():
    x = np.random.default_rng(1).normal(size=5000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.enc_bf16(x), ref)


def test_generator_e2m1_encoder_is_nearest_even():
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    xs = np.concatenate([np.linspace(-7, 7, 2801), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]])
    for x in xs:
        code = int(synth.enc_e2m1([x])[0])
        v = oracle.e2m1(np.array([code], np.uint8))[0]
        a = min(abs(x), 6.0)
        d = np.abs(mags - a)
        best = np.nonzero(d == d.min())[0]
        if len(best) == 1:
            assert abs(v) == mags[best[0]], x
        else:  # tie: the even mantissa (code bit 0 clear)
            even = [i for i in best if i % 2 == 0]
            assert abs(v) == mags[even[0]], x
        if a > 0 and abs(v) > 0:
            assert np.sign(v) == np.sign(x)
