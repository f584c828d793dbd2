"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI on a synthetic
workload and compare it with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sparse_attention_decode_amd as sad
import synth
import synth.device

RTOL, ATOL = 2e-2, 2e-3  # bf16 outputs and fp32 log-sum-exp against the float64 oracle


def run_gpu(wl: synth.Workload, use_hist=None, prefill=None, zero_qidx=False, phys=True, flags=0,
            candidates=False, pool_edit=None, context_bound=None):
    """Run the layer through the C ABI on workload wl.  candidates: scores are never stored (the
    candidates path); pool_edit(pool, kv): a change made to the staged pool before the run;
    context_bound: a larger bound on the rows' visible tokens than the batch's own (the block table
    is padded with -1 to match), which only changes how the library sizes its passes."""
    kv = sad.kv_layout(wl.ikey_fmt, wl.lat_fmt, wl.num_blocks, wl.lat_tensor_scale)
    d = synth.device.stage(wl, kv.as_dict())
    if zero_qidx:
        d["q_idx"].zero_()
    if pool_edit is not None:
        pool_edit(d["pool"], kv)
    bt, max_context = d["block_table"], d["max_context"]
    if context_bound is not None:
        assert context_bound >= max_context
        nb = (context_bound + 63) // 64
        if nb > bt.shape[1]:
            pad = torch.full((bt.shape[0], nb - bt.shape[1]), -1, dtype=bt.dtype, device=bt.device)
            bt = torch.cat([bt, pad], dim=1).contiguous()
        max_context = context_bound
    batch = sad.DeviceBatch(bt, d["seq_row_start"], d["row_pos"], d["max_rows_per_seq"],
                            max_context, flags)
    if prefill is None:
        prefill = d["max_rows_per_seq"] > sad.MAX_ROWS_PER_SEQ
    layer = sad.DSALayer(kv, batch, wl.k, wl.softmax_scale, prefill=prefill, use_hist=use_hist,
                         candidates=candidates)
    layer.scores_step(d["pool"], d["q_idx"], d["w"])
    if phys:
        layer.phys.fill_(-7)
    layer.topk_step(phys=phys)
    layer.attention_step(d["pool"], d["q"])
    torch.cuda.synchronize()
    if layer.hist is not None:  # dsa_topk returns the scorer's histogram to zero
        assert int(layer.hist.abs().sum().item()) == 0
    return layer, d, kv


def oracle_seq(wl: synth.Workload, b: int, rows=None, zero_qidx=False, want_scores=True):
    if not zero_qidx:
        return oracle.workload_rows(wl, b, rows=rows, want_scores=want_scores)
    rows = wl.rows_of(b) if rows is None else np.asarray(rows)
    need = int(wl.row_pos[rows].max()) + 1
    keys, ks, lat, ls = synth.seq_tensors(wl, b, need)
    qi, hw, qm = synth.row_queries(wl)
    return oracle.dsa_rows(wl.ikey_fmt, wl.lat_fmt, wl.row_pos[rows],
                           np.zeros_like(qi[rows]), hw[rows], qm[rows], keys, ks, lat, ls,
                           wl.lat_tensor_scale, wl.k, wl.softmax_scale, want_scores)


def check_rows(wl, layer, ref, rows, check_scores=True):
    """Element-wise parity of the rows `rows` (global row ids) against the oracle result `ref`
    (computed for the same rows, in order)."""
    rows = list(rows)
    idx = layer.idx[rows].cpu().numpy()
    cnt = layer.count[rows].cpu().numpy()
    assert ref["mism"] == 0, "inputs off the exact grid"
    check_scores = check_scores and layer.scores is not None  # the candidates path stores none
    for i, r in enumerate(rows):
        p = int(wl.row_pos[r])
        if check_scores:
            gs = layer.scores[r, :p + 1].cpu().numpy().astype(np.float64)
            rs = ref["scores"][i, :p + 1]
            bad = np.nonzero(gs != rs)[0]
            assert bad.size == 0, f"row {r}: {bad.size} scores differ, first at {bad[:5]}: " \
                                  f"{gs[bad[:5]]} vs {rs[bad[:5]]}"
        assert cnt[i] == ref["count"][i], (r, cnt[i], ref["count"][i])
        diff = np.nonzero(idx[i] != ref["idx"][i])[0]
        assert diff.size == 0, f"row {r}: {diff.size} indices differ, first at {diff[:5]}"
    out = layer.out[rows].float().cpu().numpy().astype(np.float64)
    err = np.abs(out - ref["out"]) - (ATOL + RTOL * np.abs(ref["out"]))
    assert err.max() <= 0, f"out off by {err.max():.3g} beyond tolerance"
    lse = layer.lse[rows].cpu().numpy().astype(np.float64)
    err = np.abs(lse - ref["lse"]) - (ATOL + RTOL * np.abs(ref["lse"]))
    assert err.max() <= 0, f"lse off by {err.max():.3g} beyond tolerance"


def check_workload(wl, layer, seqs=None, zero_qidx=False, check_scores=True):
    seqs = range(wl.num_seqs) if seqs is None else seqs
    for b in seqs:
        rows = wl.rows_of(b)
        ref = oracle_seq(wl, b, zero_qidx=zero_qidx, want_scores=check_scores)
        check_rows(wl, layer, ref, rows, check_scores)
