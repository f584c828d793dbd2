"""Parity of decode context parallelism emulated on one GPU: W token-interleaved shards, the exact
cross-shard merge (dsa_dcp_publish + dsa_dcp_merge) and the LSE combine (dsa_lse_combine).

1. The merge on crafted score rows (random, tied, one shard holding the top, all equal, fewer
   than k visible, scores sharing their top 16 bits) against the oracle's protocol, for every
   message variant: global indices, each shard's part, and the protocol counts (rounds, resends,
   tie-round entries, bytes) bit for bit; the oracle's result is itself pinned to the plain top-k.
2. A whole sharded decode step (per-shard scorer and select on shard pools, merge, per-shard
   attention, combine) on a synthetic workload: indices bit-identical to the unsharded GPU path
   and to the oracle, outputs within the oracle tolerance."""
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import dcp
import sparse_attention_decode_amd as sad
import synth
import synth.device
from gpu_harness import ATOL, RTOL, check_rows, oracle_seq, run_gpu

pytestmark = pytest.mark.gpu

VARIANTS = [sad.MERGE_PACKED, sad.MERGE_SCORES, sad.MERGE_GENERIC]


def _rows(rng, W):
    """Global fp32 score rows of varied shape (each row has at least W tokens)."""
    rows = []
    rows.append(rng.standard_normal(20000))
    rows.append(np.round(rng.standard_normal(9000) * 4) / 4)            # coarse grid: ties
    s = rng.standard_normal(30000)
    s[::W] += 3.0                                                        # shard 0 holds the top
    rows.append(s)
    rows.append(np.zeros(5000))                                          # all equal
    z = np.where(rng.random(4000) < 0.3, 1.0, 0.0)
    z[(np.arange(4000) % 2 == 1) & (z == 0)] = -0.0
    rows.append(z)                                                       # +-0 ties and ones
    rows.append(rng.standard_normal(1000))                               # fewer than k visible
    rows.append(rng.standard_normal(3 * W))                              # 3 tokens per shard
    rows.append(1000.0 + rng.random(12000) * 0.05)                       # one 16-bit prefix
    return [np.asarray(r, np.float32) for r in rows]


def _shard_topk(rows, W, r, k):
    """Shard r's local scores of every row, and its dsa_topk output (idx, count)."""
    local = [row[r::W] for row in rows]
    R = len(rows)
    n = np.array([len(x) for x in local])
    ld = int((n.max() + 63) // 64 * 64)
    sc = np.zeros((R, ld), np.float32)
    for i, x in enumerate(local):
        sc[i, :len(x)] = x
    scores = torch.from_numpy(sc).cuda()
    maxb = ld // 64
    bt = torch.zeros((R, maxb), dtype=torch.int32, device="cuda")
    batch = sad.DeviceBatch(bt, torch.arange(R + 1, dtype=torch.int32, device="cuda"),
                            torch.from_numpy((n - 1).astype(np.int32)).cuda(), 1, int(n.max()))
    idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(R, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(sad.dsa_topk_workspace_bytes(R, int(n.max())), 16) // 4 + 4,
                     dtype=torch.float32, device="cuda")
    sad.dsa_topk(None, batch, scores, None, k, idx, cnt, ws)
    return scores, idx, cnt


@pytest.mark.parametrize("W,k", [(2, 2048), (5, 2048), (8, 2048), (8, 100)])
def test_merge_matches_oracle_protocol(W, k):
    print(f"\n[case] dcp merge W={W} k={k}", flush=True)
    rng = np.random.default_rng(900 + W + k)
    rows = _rows(rng, W)
    R = len(rows)
    mb = torch.zeros(sad.dsa_dcp_mailbox_bytes(R, k, W), dtype=torch.uint8, device="cuda")
    keep = []
    for r in range(W):
        scores, idx, cnt = _shard_topk(rows, W, r, k)
        sad.dsa_dcp_publish(k, W, r, scores, idx, cnt, mb)
        keep.append((scores, idx, cnt))
    torch.cuda.synchronize()
    lists = [dcp.shard_lists(row, W, k) for row in rows]
    for v in VARIANTS:
        idx = torch.full((R, k), -5, dtype=torch.int32, device="cuda")
        cnt = torch.full((R,), -5, dtype=torch.int32, device="cuda")
        sidx = torch.full((W, R, k), -5, dtype=torch.int32, device="cuda")
        scnt = torch.full((W, R), -5, dtype=torch.int32, device="cuda")
        stats = torch.full((R, 4), -5, dtype=torch.int32, device="cuda")
        sad.dsa_dcp_merge(k, W, v, mb, idx, cnt, sidx, scnt, stats)
        torch.cuda.synchronize()
        gi, gc, gs, gsc, gst = (t.cpu().numpy() for t in (idx, cnt, sidx, scnt, stats))
        for i, row in enumerate(rows):
            chosen, per_shard, st = dcp.merge(lists[i], k, v)
            want, wc = oracle.topk(row.astype(np.float64), k)
            assert np.array_equal(chosen, want[:wc])
            assert gc[i] == len(chosen), (v, i)
            assert np.array_equal(gi[i, :gc[i]], chosen) and np.all(gi[i, gc[i]:] == -1), (v, i)
            assert tuple(gst[i]) == st, (v, i, tuple(gst[i]), st)
            for r in range(W):
                loc = per_shard[r] // W
                assert gsc[r, i] == len(loc), (v, i, r)
                assert np.array_equal(gs[r, i, :len(loc)], loc) and np.all(gs[r, i, len(loc):] == -1)


@pytest.mark.parametrize("W,variant,lowp", [(4, sad.MERGE_PACKED, False),
                                             (3, sad.MERGE_SCORES, False),
                                             (8, sad.MERGE_GENERIC, True)])
def test_sharded_decode_step(W, variant, lowp):
    print(f"\n[case] dcp decode step W={W} variant={variant} lowp={lowp}", flush=True)
    if lowp:  # MXFP4 keys, NVFP4 latents, a small k
        wl = synth.Workload("dcp-step-lowp", 37, [30000, 5000], [0, 0, 1], [29990, 29999, 4999],
                            ikey_fmt=sad.IKEY_MXFP4, lat_fmt=sad.LATENT_NVFP4,
                            lat_tensor_scale=0.5, k=100)
    else:
        wl = synth.Workload("dcp-step", 31, [40000, 9000, 26000], [0, 1, 1, 2],
                            [39999, 8990, 8999, 25999])
    k, R = wl.k, wl.num_rows
    full, _, _ = run_gpu(wl)
    ref_idx = full.idx.cpu().numpy()
    ref_cnt = full.count.cpu().numpy()
    del full
    mb = torch.zeros(sad.dsa_dcp_mailbox_bytes(R, k, W), dtype=torch.uint8, device="cuda")
    shards = []
    for r in range(W):
        sw = synth.shard_workload(wl, W, r)
        kv = sad.kv_layout(sw.ikey_fmt, sw.lat_fmt, sw.num_blocks, sw.lat_tensor_scale)
        d = synth.device.stage(sw, kv.as_dict())
        batch = sad.DeviceBatch(d["block_table"], d["seq_row_start"], d["row_pos"],
                                d["max_rows_per_seq"], d["max_context"])
        layer = sad.DSALayer(kv, batch, k, wl.softmax_scale)
        layer.scores_step(d["pool"], d["q_idx"], d["w"])
        layer.topk_step(phys=False)
        sad.dsa_dcp_publish(k, W, r, layer.scores, layer.idx, layer.count, mb)
        shards.append((kv, d, batch, layer))
    idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(R, dtype=torch.int32, device="cuda")
    sidx = torch.empty((W, R, k), dtype=torch.int32, device="cuda")
    scnt = torch.empty((W, R), dtype=torch.int32, device="cuda")
    stats = torch.empty((R, 4), dtype=torch.int32, device="cuda")
    sad.dsa_dcp_merge(k, W, variant, mb, idx, cnt, sidx, scnt, stats)
    parts = torch.empty(sad.dsa_dcp_partials_bytes(R, k, W), dtype=torch.uint8, device="cuda")
    for r, (kv, d, batch, layer) in enumerate(shards):
        sad.sparse_mla_decode_shard(kv, d["pool"], batch, d["q"], sidx[r], k, wl.softmax_scale,
                                    r, W, parts, count=scnt[r] if r % 2 == 0 else None)
    out = torch.empty((R, 96, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((R, 96), dtype=torch.float32, device="cuda")
    sad.dsa_lse_combine(R, k, W, parts, out, lse)
    torch.cuda.synchronize()
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    assert np.array_equal(gc, ref_cnt) and np.array_equal(gi, ref_idx), \
        "sharded selection differs from the unsharded select"
    gs, gsc = sidx.cpu().numpy(), scnt.cpu().numpy()
    for r in range(W):
        for i in range(R):
            mine = gi[i, :gc[i]][gi[i, :gc[i]] % W == r] // W
            assert gsc[r, i] == len(mine) and np.array_equal(gs[r, i, :len(mine)], mine)
    print("[stats]", stats.cpu().numpy().tolist(), flush=True)
    fake = types.SimpleNamespace(idx=idx, count=cnt, out=out, lse=lse)
    for b in range(wl.num_seqs):
        rows = wl.rows_of(b)
        check_rows(wl, fake, oracle_seq(wl, b, rows=rows, want_scores=False), rows,
                   check_scores=False)


def test_lse_combine_one_shard_and_empty_shards():
    # One shard over the whole selection, then the combine: the same splits and the same merge as
    # sparse_mla_decode, so bit-identical outputs.  With two shards the split count is sized for
    # half the selection (other splits, other rounding): a second shard that selected nothing
    # (all -1) adds slots of weight 0, and the result matches within the oracle tolerance.
    wl = synth.Workload("dcp-one", 17, [12000, 3000], [0, 1], [11999, 2999])
    layer, d, kv = run_gpu(wl)
    R, k = wl.num_rows, wl.k
    for W in (1, 2):
        parts = torch.empty(sad.dsa_dcp_partials_bytes(R, k, W), dtype=torch.uint8, device="cuda")
        sad.sparse_mla_decode_shard(kv, d["pool"], layer.batch, d["q"], layer.idx, k,
                                    wl.softmax_scale, 0, W, parts)
        if W == 2:
            none = torch.full_like(layer.idx, -1)
            sad.sparse_mla_decode_shard(kv, d["pool"], layer.batch, d["q"], none, k,
                                        wl.softmax_scale, 1, W, parts)
        out = torch.empty_like(layer.out)
        lse = torch.empty_like(layer.lse)
        sad.dsa_lse_combine(R, k, W, parts, out, lse)
        torch.cuda.synchronize()
        if W == 1:
            assert torch.equal(out, layer.out) and torch.equal(lse, layer.lse)
        else:
            a, b = out.float(), layer.out.float()
            assert torch.all((a - b).abs() <= ATOL + RTOL * b.abs())
            assert torch.all((lse - layer.lse).abs() <= ATOL + RTOL * layer.lse.abs())
    # every shard empty: 0 and -inf
    parts = torch.empty(sad.dsa_dcp_partials_bytes(R, k, 2), dtype=torch.uint8, device="cuda")
    none = torch.full_like(layer.idx, -1)
    for r in range(2):
        sad.sparse_mla_decode_shard(kv, d["pool"], layer.batch, d["q"], none, k, wl.softmax_scale,
                                    r, 2, parts)
    out = torch.ones_like(layer.out)
    lse = torch.zeros_like(layer.lse)
    sad.dsa_lse_combine(R, k, 2, parts, out, lse)
    torch.cuda.synchronize()
    assert not out.float().abs().sum().item() and torch.all(lse == -float("inf"))
