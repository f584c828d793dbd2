"""Parity of the HIP path (through the C ABI) with the CPU oracle, on seeded synthetic inputs:
indexer scores and top-k indices bit-exact (inputs on the exact grid), attention outputs and
log-sum-exp within rtol 2e-2 / atol 2e-3."""
import numpy as np
import pytest
import torch

import sparse_attention_decode_amd as sad
import synth
from gpu_harness import check_rows, check_workload, oracle_seq, run_gpu

pytestmark = pytest.mark.gpu

RAGGED = [1, 63, 64, 65, 2047, 2048, 2049, 5000, 9001]


def _one_row_per_seq(name, seed, lens, **kw):
    lens = list(lens)
    return synth.Workload(name, seed, lens, list(range(len(lens))), [L - 1 for L in lens], **kw)


def test_decode_single_8k():
    wl = synth.decode_config(0)
    layer, _, _ = run_gpu(wl)
    check_workload(wl, layer)


@pytest.mark.parametrize("k", [2048, 100])
def test_decode_ragged_lengths_fp8(k):
    wl = _one_row_per_seq("ragged", 41, RAGGED, k=k)
    layer, _, _ = run_gpu(wl)
    check_workload(wl, layer)


@pytest.mark.parametrize("lat,phys", [(0, True), (0, False), (1, True)])
def test_attention_never_reads_poisoned_rows_into_the_output(lat, phys):
    # Nearly the whole pool is spare blocks filled with 0xFF bytes (an E4M3 NaN code), and so are
    # the slots past each sequence's end.  Tiles that end part-way (visible tokens not a multiple of
    # 32) gather such rows into their unused slots; a NaN there must never reach the output, even
    # though its probability is zero.
    print(f"\n[case] poisoned pool lat={lat} phys={phys}", flush=True)
    kw = dict(lat_fmt=1, lat_tensor_scale=0.75) if lat else {}
    wl = _one_row_per_seq(f"poison{lat}{int(phys)}", 47 + lat, [700, 1500, 70, 2100], k=2048,
                          spare_blocks=1000, **kw)
    layer, _, _ = run_gpu(wl, phys=phys)
    assert bool(torch.isfinite(layer.out.float()).all()) and bool(torch.isfinite(layer.lse).all())
    check_workload(wl, layer)


@pytest.mark.parametrize("k", [2048, 100, 7, 1])
def test_short_rows_select_in_one_pass(k):
    # Every row sees at most 8,192 tokens, so the select reads the scores in its resolve pass and
    # runs no filter; the same rows under a context bound of 8,193 take the filter path.  Both
    # against the oracle, and bit-identical to each other.
    print(f"\n[case] short rows k={k}", flush=True)
    wl = _one_row_per_seq(f"short{k}", 60 + k, [1, 63, 65, 2047, 2049, 5000, 8191, 8192], k=k)
    direct, _, _ = run_gpu(wl)
    check_workload(wl, direct)
    filtered, _, _ = run_gpu(wl, context_bound=8193)
    assert torch.equal(direct.count, filtered.count)
    assert torch.equal(direct.idx, filtered.idx)
    assert torch.equal(direct.phys, filtered.phys)
    assert torch.equal(direct.out.view(torch.int16), filtered.out.view(torch.int16))


def test_short_rows_all_scores_tied():
    # q = 0 on rows of at most 8,192 tokens: every key ties, and the lowest indices are selected
    print("\n[case] short rows all tied", flush=True)
    wl = _one_row_per_seq("shortties", 71, [3000, 8192, 2100])
    layer, _, _ = run_gpu(wl, zero_qidx=True)
    check_workload(wl, layer, zero_qidx=True)
    idx = layer.idx.cpu().numpy()
    assert np.array_equal(idx[0], np.arange(2048)) and np.array_equal(idx[1], np.arange(2048))


@pytest.mark.parametrize("rows", [3, 4, 31, 32])
def test_split_combine_at_its_workgroup_size_boundaries(rows):
    # the split combine runs one-wave workgroups below 4 rows, two-wave ones below 32 and
    # eight-wave ones from 32 on: batches on each side of both boundaries, against the oracle
    print(f"\n[case] combine boundary rows={rows}", flush=True)
    rng = np.random.default_rng(700 + rows)
    lens = [int(x) for x in rng.integers(2100, 12000, rows)]
    wl = _one_row_per_seq(f"cmb{rows}", 700 + rows, lens)
    layer, _, _ = run_gpu(wl)
    check_workload(wl, layer)


def test_decode_without_scorer_histogram():
    wl = _one_row_per_seq("nohist", 42, [3000, 70000, 129])
    layer, _, _ = run_gpu(wl, use_hist=False)
    check_workload(wl, layer)


def test_speculative_rows_share_keys():
    # 6 rows per sequence at positions L-6..L-1 (causal within the step); one sequence has 1 row.
    lens = [3000, 7000, 4100, 2500]
    rs, rp = [], []
    for b, L in enumerate(lens):
        n = 1 if b == 3 else 6
        rs += [b] * n
        rp += [L - n + j for j in range(n)]
    wl = synth.Workload("spec", 43, lens, rs, rp)
    layer, _, _ = run_gpu(wl)
    check_workload(wl, layer)


@pytest.mark.parametrize("rows,ikey", [(2, 0), (3, 1), (5, 0), (7, 1), (8, 0)])
def test_speculative_rows_per_sequence(rows, ikey):
    # Each row count is its own scorer instance (rows 3-8 count the histogram in 16-bit halves
    # of LDS words); the last sequence has fewer rows than the others, one sequence starts its
    # rows on a block boundary.
    lens = [3000, 9000 + rows, 64 * 40 + max(1, rows - 2)]
    rs, rp = [], []
    for b, L in enumerate(lens):
        n = rows if b < 2 else max(1, rows - 2)
        rs += [b] * n
        rp += [L - n + j for j in range(n)]
    wl = synth.Workload(f"spec{rows}", 60 + rows, lens, rs, rp, ikey_fmt=ikey, wq=4 if ikey else 8)
    layer, _, _ = run_gpu(wl)
    check_workload(wl, layer)


@pytest.mark.parametrize("ikey,lat", [(1, 1), (0, 1), (1, 0)])
def test_decode_low_precision_formats(ikey, lat):
    wl = _one_row_per_seq("lp", 44 + 2 * ikey + lat, [5000, 65, 2049, 12000], ikey_fmt=ikey,
                          lat_fmt=lat, wq=4 if ikey else 8, lat_tensor_scale=0.75)
    layer, _, _ = run_gpu(wl)
    check_workload(wl, layer)


def test_all_scores_tied_selects_lowest_indices():
    # q = 0 makes every score 0: the tie rule alone decides, and the threshold bin holds every
    # token (more than the LDS candidate buffer), exercising the global-memory fallback.
    wl = _one_row_per_seq("ties", 45, [9000, 2000, 40000])
    layer, _, _ = run_gpu(wl, zero_qidx=True)
    check_workload(wl, layer, zero_qidx=True)
    idx = layer.idx.cpu().numpy()
    assert np.array_equal(idx[0], np.arange(2048)) and np.array_equal(idx[2], np.arange(2048))


def test_physical_rows_and_determinism():
    wl = _one_row_per_seq("phys", 46, [5000, 300, 10000], k=512)
    layer, d, kv = run_gpu(wl, phys=True)
    idx = layer.idx.cpu().numpy()
    ph = layer.phys.cpu().numpy()
    for r in range(wl.num_rows):
        bt = wl.block_table[wl.row_seq[r]]
        ok = idx[r] >= 0
        want = np.where(ok, bt[np.where(ok, idx[r], 0) // 64] * 64 + np.where(ok, idx[r], 0) % 64, -1)
        assert np.array_equal(ph[r], want)
    out1 = layer.out.clone()
    layer.run(d["pool"], d["q_idx"], d["w"], d["q"])
    torch.cuda.synchronize()
    assert torch.equal(out1, layer.out)


@pytest.mark.parametrize("ikey,lat,hist", [(0, 0, False), (1, 1, False), (0, 0, True), (1, 0, True)])
def test_prefill_chunk_rows(ikey, lat, hist):
    # 40 rows of one sequence (prefill path: row tiles x key chunks), plus a second sequence;
    # FP8 keys and latents, or MXFP4 keys and NVFP4 latents.
    P = 6000
    rs = [0] * 40 + [1] * 12
    rp = [P - 40 + i for i in range(40)] + [900 + i for i in range(12)]
    # hist: the scorer counts the select's histogram itself (8-wave prefill tiles)
    kw = dict(ikey_fmt=1, wq=4) if ikey else {}
    if lat:
        kw.update(lat_fmt=1, lat_tensor_scale=0.75)
    wl = synth.Workload("prefill", 47 + 3 * ikey + lat, [P, 912], rs, rp, **kw)
    layer, _, _ = run_gpu(wl, use_hist=hist)
    assert layer.prefill and (layer.hist is not None) == hist
    check_workload(wl, layer)


def test_prefill_attention_matches_decode_attention():
    wl = _one_row_per_seq("pvd", 48, [7000, 3000])
    a, _, _ = run_gpu(wl, prefill=False)
    b, _, _ = run_gpu(wl, prefill=True)
    assert torch.equal(a.idx, b.idx)
    ao, bo = a.out.float(), b.out.float()
    assert bool(((ao - bo).abs() <= 2 * (2e-3 + 2e-2 * bo.abs())).all())
    check_workload(wl, a)
    check_workload(wl, b)


@pytest.mark.parametrize("k", [1, 7])
def test_decode_small_k(k):
    # the smallest selections: k = 1 (the single best token; ties to the lowest index) and an odd
    # k, over the ragged lengths (a row at position 0 sees one token)
    print(f"\n[case] small k={k}", flush=True)
    wl = _one_row_per_seq(f"smallk{k}", 49 + k, RAGGED, k=k)
    layer, _, _ = run_gpu(wl)
    check_workload(wl, layer)


def test_prefill_first_chunk_from_position_zero():
    # the first chunk of a prompt: rows 0..47 of one sequence, so the early rows see fewer
    # tokens than k and row 0 sees only itself
    print("\n[case] prefill from position 0", flush=True)
    wl = synth.Workload("prefill0", 51, [48], [0] * 48, list(range(48)), k=16)
    layer, _, _ = run_gpu(wl)
    assert layer.prefill
    check_workload(wl, layer)


@pytest.mark.parametrize("case", range(8))
def test_random_batches(case):
    """Seeded random batches: 1-5 sequences of 1-20,000 tokens, 1-8 rows per sequence (or a
    prefill chunk of 9-40 rows), k from {1, 63, 512, 2048}, every key and latent format, with or
    without the scorer's histogram, all against the oracle."""
    rng = np.random.default_rng(9000 + case)
    nseq = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.integers(1, 20001, nseq)]
    prefill = case % 4 == 3
    rs, rp = [], []
    for b, L in enumerate(lens):
        n = int(rng.integers(9, 41)) if (prefill and b == 0) else int(rng.integers(1, 9))
        n = min(n, L)
        rs += [b] * n
        rp += [L - n + j for j in range(n)]
    ikey, lat = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    kw = dict(ikey_fmt=ikey, lat_fmt=lat, wq=4 if ikey else 8,
              lat_tensor_scale=0.75 if lat else 1.0, k=int(rng.choice([1, 63, 512, 2048])))
    wl = synth.Workload(f"rand{case}", 9000 + case, lens, rs, rp, **kw)
    hist = bool(rng.integers(0, 2))
    print(f"\n[case] random {case}: lens={lens} rows={len(rs)} ikey={ikey} lat={lat} "
          f"k={kw['k']} hist={hist}", flush=True)
    layer, _, _ = run_gpu(wl, use_hist=hist)
    check_workload(wl, layer)
