"""Parity of the HIP path with the oracle at the full sizes of the six measured workloads, in the
launch configurations the benchmark times (dense: scorer with its fused histogram, select
emitting physical rows, attention reading them; candidates: scores never stored, the sample and
candidate passes and the candidate select; prefill variants for the 8,192-row chunk).  The whole
batch runs on the GPU; sampled rows are recomputed by the oracle one by one and compared element
by element: scores and indices bit-exact, attention outputs within rtol 2e-2 / atol 2e-3."""
import gc

import numpy as np
import pytest
import torch

import sparse_attention_decode_amd as sad
import synth
from gpu_harness import check_rows, oracle_seq, run_gpu

pytestmark = pytest.mark.gpu


def _sample_rows(wl, picks):
    out = []
    for r in picks:
        r = int(r) % wl.num_rows
        if r not in out:
            out.append(r)
    return out


def _check_sampled(wl, layer, rows):
    for r in rows:
        b = int(wl.row_seq[r])
        print(f"[parity] {wl.name}{' candidates' if layer.candidates else ''}: oracle row {r} "
              f"(sequence {b}, position {wl.row_pos[r]})", flush=True)
        ref = oracle_seq(wl, b, rows=[r])
        check_rows(wl, layer, ref, [r])


@pytest.fixture(autouse=True)
def _free_device_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def test_full_decode_1x8k():
    wl = synth.decode_config(0)
    layer, _, _ = run_gpu(wl)
    _check_sampled(wl, layer, [0])


@pytest.mark.parametrize("candidates", [False, True])
def test_full_decode_16x128k(candidates):
    wl = synth.decode_config(1)
    layer, _, _ = run_gpu(wl, candidates=candidates)
    _check_sampled(wl, layer, _sample_rows(wl, [0, 7, 15]))


@pytest.mark.parametrize("candidates", [False, True])
def test_full_specdec_16x6_1m(candidates):
    # 96 rows, six per sequence at positions L-6 .. L-1, sharing each sequence's 1M keys
    wl = synth.decode_config(2)
    layer, _, _ = run_gpu(wl, candidates=candidates)
    assert not layer.prefill
    _check_sampled(wl, layer, _sample_rows(wl, [0, 5, 50, 95]))


@pytest.mark.parametrize("candidates", [False, True])
def test_full_prefill_8192_on_339968(candidates):
    wl = synth.decode_config(3)
    layer, _, _ = run_gpu(wl, candidates=candidates)
    assert layer.prefill
    _check_sampled(wl, layer, _sample_rows(wl, [0, 4095, 8191]))
    # every row has more than 2048 visible tokens: a full selection
    assert int(layer.count.min().item()) == wl.k


@pytest.mark.parametrize("candidates", [False, True])
def test_full_prefill_2048_on_150000(candidates):
    # the short-append prefill: 2,048 rows after a 150,000-token prefix
    wl = synth.decode_config(5)
    layer, _, _ = run_gpu(wl, candidates=candidates)
    assert layer.prefill
    _check_sampled(wl, layer, _sample_rows(wl, [0, 1023, 2047]))
    assert int(layer.count.min().item()) == wl.k


@pytest.mark.parametrize("candidates", [False, True])
def test_full_mixed_64_mxfp4_nvfp4(candidates):
    wl = synth.decode_config(4)
    layer, _, _ = run_gpu(wl, candidates=candidates)
    shortest = int(np.argmin(wl.row_pos))
    longest = int(np.argmax(wl.row_pos))
    _check_sampled(wl, layer, _sample_rows(wl, [shortest, longest, 17, 40]))


@pytest.mark.parametrize("plain", [False, True])
def test_full_prefill_16384_from_0(plain):
    # the first chunk of a prompt, its row tiles scored in the balanced 16-piece order or in plain
    # ascending order: the same results either way, against the oracle on sampled rows
    wl = synth.decode_config(6)
    layer, _, _ = run_gpu(wl, flags=sad.BATCH_PLAIN_ORDER if plain else 0)
    assert layer.prefill
    _check_sampled(wl, layer, _sample_rows(wl, [0, 1, 2047, 2048, 9000, 16383]))
    counts = layer.count.cpu().numpy()
    assert np.array_equal(counts, np.minimum(wl.k, wl.row_pos + 1))
