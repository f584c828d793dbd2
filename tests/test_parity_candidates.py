"""Parity of the candidates path (scores never stored in full: a pass over every S-th block fixes
each row's floor, the other blocks append only the tokens at or above it, and an exact select
takes the top-k of the candidates) with the oracle, and with the dense path on the same inputs:
indices, counts and physical rows bit-identical, attention outputs bit-identical (the attention is
the same call on the same selection).  A pool built so that the sample sees only zero scores makes
the candidates outgrow their capacity; that must be reported, never silently wrong."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_decode_amd as sad
import synth
from gpu_harness import check_workload, run_gpu

pytestmark = pytest.mark.gpu

RAGGED = [1, 63, 64, 65, 2047, 2048, 2049, 5000, 9001, 40000]


@pytest.fixture(autouse=True)
def clean_status():
    sad.dsa_device_status(clear=True)
    yield
    sad.dsa_device_status(clear=True)


def _one_row_per_seq(name, seed, lens, **kw):
    lens = list(lens)
    return synth.Workload(name, seed, lens, list(range(len(lens))), [L - 1 for L in lens], **kw)


def _both(wl, **kw):
    """The candidates path, checked against the dense path run on the same inputs."""
    dense, _, _ = run_gpu(wl, **kw)
    cand, _, _ = run_gpu(wl, candidates=True, **kw)
    assert cand.scores is None
    assert torch.equal(dense.count, cand.count)
    assert torch.equal(dense.idx, cand.idx)
    assert torch.equal(dense.phys, cand.phys)
    assert torch.equal(dense.out.view(torch.int16), cand.out.view(torch.int16))
    assert sad.dsa_device_status() == 0
    return cand


@pytest.mark.parametrize("k", [2048, 100, 7, 1])
def test_candidates_ragged_lengths(k):
    print(f"\n[case] candidates ragged k={k}", flush=True)
    wl = _one_row_per_seq(f"cragged{k}", 81 + k, RAGGED, k=k)
    check_workload(wl, _both(wl))


@pytest.mark.parametrize("rows,ikey", [(1, 1), (2, 0), (3, 1), (6, 0), (8, 1)])
def test_candidates_speculative_rows(rows, ikey):
    print(f"\n[case] candidates speculative rows={rows} ikey={ikey}", flush=True)
    lens = [30000, 9000 + rows, 64 * 40 + max(1, rows - 2)]
    rs, rp = [], []
    for b, L in enumerate(lens):
        n = rows if b < 2 else max(1, rows - 2)
        rs += [b] * n
        rp += [L - n + j for j in range(n)]
    wl = synth.Workload(f"cspec{rows}", 90 + rows, lens, rs, rp, ikey_fmt=ikey,
                        wq=4 if ikey else 8)
    check_workload(wl, _both(wl))


def test_candidates_all_scores_tied():
    # q = 0: every score is 0; the floor is the sample's tie cutoff on the token index, and the
    # selection is the lowest indices
    print("\n[case] candidates all tied", flush=True)
    wl = _one_row_per_seq("cties", 95, [9000, 2000, 70000])
    layer = _both(wl, zero_qidx=True)
    check_workload(wl, layer, zero_qidx=True)
    idx = layer.idx.cpu().numpy()
    assert np.array_equal(idx[0], np.arange(2048)) and np.array_equal(idx[2], np.arange(2048))


@pytest.mark.parametrize("ikey,lat", [(0, 0), (1, 1)])
def test_candidates_prefill_chunk(ikey, lat):
    # 40 rows of one sequence (the prefill scorer's 16-row tiles) plus a short second sequence
    print(f"\n[case] candidates prefill ikey={ikey} lat={lat}", flush=True)
    P = 26000
    rs = [0] * 40 + [1] * 12
    rp = [P - 40 + i for i in range(40)] + [900 + i for i in range(12)]
    kw = dict(ikey_fmt=1, wq=4) if ikey else {}
    if lat:
        kw.update(lat_fmt=1, lat_tensor_scale=0.75)
    wl = synth.Workload("cprefill", 96 + ikey, [P, 912], rs, rp, **kw)
    layer = _both(wl)
    assert layer.prefill
    check_workload(wl, layer)


def test_candidates_prefill_from_position_zero():
    print("\n[case] candidates prefill from 0", flush=True)
    wl = synth.Workload("cprefill0", 98, [48], [0] * 48, list(range(48)), k=16)
    check_workload(wl, _both(wl))


@pytest.mark.parametrize("case", range(6))
def test_candidates_random_batches(case):
    rng = np.random.default_rng(9100 + case)
    nseq = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(1, 60001, nseq)]
    prefill = case % 3 == 2
    rs, rp = [], []
    for b, L in enumerate(lens):
        n = int(rng.integers(9, 41)) if (prefill and b == 0) else int(rng.integers(1, 9))
        n = min(n, L)
        rs += [b] * n
        rp += [L - n + j for j in range(n)]
    ikey, lat = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    kw = dict(ikey_fmt=ikey, lat_fmt=lat, wq=4 if ikey else 8,
              lat_tensor_scale=0.75 if lat else 1.0, k=int(rng.choice([1, 63, 512, 2048])))
    wl = synth.Workload(f"crand{case}", 9100 + case, lens, rs, rp, **kw)
    print(f"\n[case] candidates random {case}: lens={lens} rows={len(rs)} ikey={ikey} lat={lat} "
          f"k={kw['k']}", flush=True)
    check_workload(wl, _both(wl))


def _zero_even_blocks(wl):
    """A pool edit: the index keys of every even block of every sequence become 0 (so the
    sample, which holds blocks 0, S, 2S, ... for a power of two S, scores only zeros)."""
    def edit(pool, kv):
        rows = pool.view(-1, kv.row_bytes)  # one pool row per block
        for b in range(wl.num_seqs):
            nb = (int(wl.seq_len[b]) + 63) // 64
            phys = torch.from_numpy(wl.block_table[b, 0:nb:2].astype(np.int64)).to(pool.device)
            rows[phys, kv.ikey_off:kv.ikey_off + 64 * 128] = 0
    return edit


def test_candidates_overflow_is_reported_and_dense_path_stays_exact():
    print("\n[case] candidates overflow", flush=True)
    L = 262144
    wl = synth.Workload("coverflow", 99, [L], [0, 0], [L - 2, L - 1])
    edit = _zero_even_blocks(wl)
    cand, _, _ = run_gpu(wl, candidates=True, pool_edit=edit)
    assert np.all(cand.count.cpu().numpy() == -1)
    assert torch.all(cand.idx == -1) and torch.all(cand.phys == -1)
    assert sad.dsa_device_status(clear=True) == sad.DEVERR_CAND_OVERFLOW
    # the dense path on the same pool, against the oracle on the same edited keys
    dense, _, _ = run_gpu(wl, pool_edit=edit)
    keys, ks, lat, ls = synth.seq_tensors(wl, 0)
    keys = keys.copy()
    blk = np.arange(L) // 64
    keys[blk % 2 == 0] = 0
    qi, hw, qm = synth.row_queries(wl)
    ref = oracle.dsa_rows(0, 0, wl.row_pos, qi, hw, qm, keys, ks, lat, ls, 1.0, wl.k,
                          wl.softmax_scale)
    assert ref["mism"] == 0
    assert np.array_equal(dense.idx.cpu().numpy(), ref["idx"])
    assert np.array_equal(dense.count.cpu().numpy(), ref["count"])
