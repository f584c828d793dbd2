"""Batch invariance: a row's results do not depend on which other rows share its batch.

Every score is computed from the row's own query and its sequence's keys, in a fixed order, so
the selected indices are identical in any batch.  The attention of a row depends only on its
selected set and on the number of splits of the selected set, which is a function of the row
count and k alone, so the outputs are bit-identical between batches of equal row count (even with
a differently shuffled pool) and within the oracle tolerance otherwise.  The rows keep their data
across batches through the generator ids (seq_id, row_id)."""
import numpy as np
import pytest
import torch

import sparse_attention_decode_amd as sad
import synth
from gpu_harness import ATOL, RTOL, check_rows, oracle_seq, run_gpu

pytestmark = pytest.mark.gpu

SEED = 4242
LENS = {1: 5000, 2: 70000, 4: 33000, 6: 1500, 7: 20000, 8: 12000, 9: 2100, 10: 48000, 11: 9000}


def _batch(name, ids):
    lens = [LENS[i] for i in ids]
    return synth.Workload(name, SEED, lens, list(range(len(ids))), [L - 1 for L in lens],
                          seq_id=np.array(ids), row_id=np.array(ids))


def _results(layer, rows):
    """(idx, count, output bits, lse, output as float64) of the given rows."""
    out = layer.out[rows]
    return (layer.idx[rows].cpu().numpy(), layer.count[rows].cpu().numpy(),
            out.view(torch.int16).cpu().numpy(), layer.lse[rows].cpu().numpy(),
            out.float().cpu().numpy().astype(np.float64))


def test_rows_independent_of_batch():
    base = _batch("invariance-base", [1, 2, 4, 6, 7, 8])
    mixed = _batch("invariance-mixed", [4, 9, 1, 10, 2, 11])      # 3 shared rows, new order
    alone = _batch("invariance-alone", [2, 4, 1])                  # the shared rows only
    shared = [1, 2, 4]
    where = lambda wl: [int(np.nonzero(wl.seq_id == i)[0][0]) for i in shared]

    lb, _, _ = run_gpu(base)
    ref = _results(lb, where(base))
    del lb
    torch.cuda.empty_cache()
    lm, _, _ = run_gpu(mixed)
    got = _results(lm, where(mixed))
    del lm
    torch.cuda.empty_cache()
    for a, b, what in zip(ref[:4], got[:4], ("idx", "count", "output bits", "lse")):
        assert np.array_equal(a, b), f"{what} differ between batches of equal row count"

    la, _, _ = run_gpu(alone)
    got = _results(la, where(alone))
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1]), \
        "selected indices depend on the batch"
    assert np.all(np.abs(ref[4] - got[4]) <= ATOL + RTOL * np.abs(ref[4])), \
        "outputs beyond tolerance between batches of different row count"
    # the rows of the smaller batch still match the oracle (one row per sequence)
    for r in where(alone):
        check_rows(alone, la, oracle_seq(alone, r, rows=[r]), [r])


def test_batch_invariant_flag():
    inv = sad.BATCH_INVARIANT
    base = _batch("invariance-base", [1, 2, 4, 6, 7, 8])
    alone = _batch("invariance-alone", [2, 4, 1])
    shared = [1, 2, 4]
    where = lambda wl: [int(np.nonzero(wl.seq_id == i)[0][0]) for i in shared]
    runs = []
    for wl, prefill in ((base, False), (alone, False), (alone, True)):
        layer, _, _ = run_gpu(wl, flags=inv, prefill=prefill)
        assert layer.prefill == prefill
        runs.append(_results(layer, where(wl)))
        del layer
        torch.cuda.empty_cache()
    for other, what in ((runs[1], "a smaller batch"), (runs[2], "the prefill entry point")):
        for a, b, name in zip(runs[0][:4], other[:4], ("idx", "count", "output bits", "lse")):
            assert np.array_equal(a, b), f"{name} differ on {what} with DSA_BATCH_INVARIANT"
