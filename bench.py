#!/usr/bin/env python3
"""Benchmark of one DSA layer step (indexer scores -> exact top-2048 -> sparse MLA) on one MI355X.

Default workload (the largest decode shape): speculative decode, 16 sequences x 6 query rows
(1 + 5 draft tokens, causal within the step) at a context of 1,048,576 tokens each, FP8 index keys
(132 B/token) and FP8 latents (576 B + 4 B scale per token) in 64-token paged blocks from one
shuffled 11.95 GB pool, 96 MLA heads, top-k 2048 per row.  The 2.2 GB of keys a step reads are far
larger than the 256 MB memory-side cache, so every step streams them from HBM.  Other workloads (--config): 0 decode-1x8K, 1 decode-16x128K (four rotated
batches), 3 prefill-8192-on-339968, 4 mixed-64-mxfp4-nvfp4, 5 prefill-2048-on-150000.  Inputs are
resident in HBM before the timed region.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 0..5] [--graph]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA decode layer query-tokens/s + achieved HBM TB/s (fraction of peak)"
# workloads where the candidates path (scores never stored) measured faster than the dense one
AUTO_CANDIDATES = (3,)
PEAK_HBM_GBPS = 8000.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_BF16_TFLOPS = 2500.0


def algorithmic_bytes(wl):
    """Bytes the method must move per step: keys of every visible
    token once per sequence, latents (+scales) of the selected tokens, the queries, the output
    and its log-sum-exp, and the block table.  Returns (total, indexer share)."""
    import numpy as np
    key_b = 132 if wl.ikey_fmt == 0 else 68
    lat_b = 580 if wl.lat_fmt == 0 else 324
    idx_bytes = 0
    total = 0
    for b in range(wl.num_seqs):
        rows = wl.rows_of(b)
        L = int(wl.row_pos[rows].max()) + 1
        nblk = (L + 63) // 64
        seq_idx = L * key_b + 4 * nblk + len(rows) * (32 * 128 + 32 * 4)
        idx_bytes += seq_idx
        total += seq_idx
        for r in rows:
            nsel = min(wl.k, int(wl.row_pos[r]) + 1)
            total += nsel * lat_b + 96 * 576 * 2 + 96 * 512 * 2 + 96 * 4
    return total, idx_bytes


def indexer_flops(wl):
    f = 0
    for b in range(wl.num_seqs):
        for r in wl.rows_of(b):
            f += 2 * 32 * 128 * (int(wl.row_pos[r]) + 1)
    return f


# Sources that determine the scorer kernel's code: counter readings recorded for it are only
# reported while these files are unchanged.
SCORER_SOURCES = ("sparse_attention_decode_amd/csrc/indexer_decode.hip",
                  "sparse_attention_decode_amd/csrc/dsa_device.h",
                  "sparse_attention_decode_amd/csrc/dsa_kernels.h")


def scorer_fingerprint() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in SCORER_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per scorer launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary in
    profiles/ (KiB per dispatch, scaled by the copy-kernel calibration), or None when there is
    none for this workload or the scorer has changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_indexer_decode_{workload}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    try:
        if vals["scorer fingerprint"] != scorer_fingerprint():
            return None
        return (float(vals["FETCH_SIZE KiB per launch"]) * float(vals["FETCH_SIZE scale"]) +
                float(vals["WRITE_SIZE KiB per launch"]) * float(vals["WRITE_SIZE scale"])) * 1024.0
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg: int, wl, budget_s: float = 15.0):
    """The oracle, as it stands, on a bounded sample of the workload: whole sequences spread over
    the batch with at most 16 rows in all (decode-16x128K: its 16 single-row sequences;
    specdec-16x6-1M: one sequence with its 6 rows), each sequence's inputs generated once and its
    rows evaluated together by the oracle (whole layer: fp64 + fp32 scores, sort, fp64
    attention), repeated until the sequence's share of the budget is used.  Returns query rows per
    second on the host's cores."""
    import numpy as np
    import oracle
    import synth
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    per_seq = max(len(wl.rows_of(b)) for b in range(wl.num_seqs))
    nseq = min(wl.num_seqs, 16) if per_seq == 1 else 1
    seqs = list(range(wl.num_seqs))[::max(1, wl.num_seqs // nseq)][:nseq]
    share = budget_s / len(seqs)
    rows_done, spent, picked = 0, 0.0, []
    for b in seqs:
        rows = wl.rows_of(b)
        if len(rows) > 16:  # a prefill chunk: 16 rows spread over it
            rows = rows[::max(1, len(rows) // 16)][:16]
        picked += [int(r) for r in rows]
        need = int(wl.row_pos[rows].max()) + 1
        keys, ks, lat, ls = synth.seq_tensors(wl, b, need)
        qi = np.empty((len(rows), 32, 128), np.uint8)
        hw = np.empty((len(rows), 32), np.float32)
        qm = np.empty((len(rows), 96, 576), np.uint16)
        for i, r in enumerate(rows):
            a, c = synth.qidx(wl.seed, int(wl.row_id[r]), 1, wl.wq)
            qi[i], hw[i] = a[0], c[0]
            qm[i] = synth.qmla(wl.seed, int(wl.row_id[r]), 1)[0]
        seq_spent = 0.0
        while seq_spent < share or seq_spent == 0.0:
            t0 = time.perf_counter()
            oracle.dsa_rows(wl.ikey_fmt, wl.lat_fmt, wl.row_pos[rows], qi, hw, qm, keys, ks, lat,
                            ls, wl.lat_tensor_scale, wl.k, wl.softmax_scale)
            seq_spent += time.perf_counter() - t0
            rows_done += len(rows)
        spent += seq_spent
    return {"value": rows_done / spent, "unit": "query-tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rows_done} row evaluations of {len(picked)} of the {wl.num_rows} rows of "
                      f"{wl.name} (rows {picked[:16]}), whole layer per row (scores in fp64 and "
                      f"fp32, top-k by sort, fp64 attention; inputs generated once, outside the timing), "
                      f"{spent:.1f} s on {threads} threads"}


def time_front(wl, d, kv, steps: int):
    """Event time of the step before the path for one batch: every row's own new token quantised
    into its pool row and the rows' indexer queries quantised with the scale folded into the head
    weights.  The index keys and the queries go in one launch (dsa_indexer_front), the latents in
    a second (dsa_cache_append with latents only).  Inputs are seeded N(0, 1) bf16 values already
    on the device."""
    import torch
    import sparse_attention_decode_amd as sad
    R = wl.num_rows
    pos = wl.row_pos.astype(np.int64)
    slots = wl.block_table[wl.row_seq, pos // wl.block_size].astype(np.int64) * wl.block_size \
        + pos % wl.block_size
    g = torch.Generator(device="cuda").manual_seed(wl.seed + 17)
    bf = lambda *shape: torch.randn(*shape, generator=g, device="cuda").to(torch.bfloat16)
    d_slot = torch.from_numpy(slots).cuda()
    ikey, lat, q = bf(R, 128), bf(R, 576), bf(R, 32, 128)
    w = torch.randn(R, 32, generator=g, device="cuda")
    q_idx = torch.empty(R, 32, 128, dtype=torch.uint8, device="cuda")
    w_out = torch.empty_like(w)
    stream = torch.cuda.current_stream()

    def run():
        sad.dsa_indexer_front(kv, d["pool"], d_slot, ikey, q, w, q_idx, w_out)
        sad.dsa_cache_append(kv, d["pool"], d_slot, latent=lat)

    for _ in range(5):
        run()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * a.elapsed_time(b) / steps
    key_b = 132 if wl.ikey_fmt == 0 else 68
    lat_b = 580 if wl.lat_fmt == 0 else 324
    nbytes = R * (8 + 2 * 128 + 2 * 576 + key_b + lat_b) + R * 32 * (2 * 128 + 4 + 128 + 4)
    return {"entry_points": "dsa_indexer_front + dsa_cache_append(latents)", "new_tokens": R,
            "query_rows": R, "us_per_step": us, "algorithmic_bytes_per_step": nbytes,
            "achieved_GBps": nbytes / (us * 1e-6) / 1e9}


def time_front_overlap(wl, layers, devs, kvs, reps: int, steps: int):
    """The step before the path together with the layer, by the host clock over `steps` steps:
    the layer alone; the front then the layer on one stream; and the front with its latent write
    (dsa_cache_append, latents only) on a second stream beside the scorer and the select, the
    attention waiting for it (an event).  Both streams keep the default priority.  The side stream
    also waits for the previous step's attention before it rewrites the new tokens' latents."""
    import torch
    import sparse_attention_decode_amd as sad
    R = wl.num_rows
    pos = wl.row_pos.astype(np.int64)
    slots = wl.block_table[wl.row_seq, pos // wl.block_size].astype(np.int64) * wl.block_size \
        + pos % wl.block_size
    g = torch.Generator(device="cuda").manual_seed(wl.seed + 29)
    bf = lambda *shape: torch.randn(*shape, generator=g, device="cuda").to(torch.bfloat16)
    d_slot = torch.from_numpy(slots).cuda()
    ikey, lat, q = bf(R, 128), bf(R, 576), bf(R, 32, 128)
    w = torch.randn(R, 32, generator=g, device="cuda")
    q_idx = torch.empty(R, 32, 128, dtype=torch.uint8, device="cuda")
    w_out = torch.empty_like(w)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ev_start = [torch.cuda.Event() for _ in range(4)]
    ev_lat = [torch.cuda.Event() for _ in range(4)]

    def layer_only(i):
        j = i % reps
        layers[j].scores_step(devs[j]["pool"], devs[j]["q_idx"], devs[j]["w"])
        layers[j].topk_step()
        layers[j].attention_step(devs[j]["pool"], devs[j]["q"])

    def serial(i):
        j = i % reps
        sad.dsa_indexer_front(kvs[j], devs[j]["pool"], d_slot, ikey, q, w, q_idx, w_out)
        sad.dsa_cache_append(kvs[j], devs[j]["pool"], d_slot, latent=lat)
        layer_only(i)

    def overlapped(i):
        j = i % reps
        e0, e1 = ev_start[i % 4], ev_lat[i % 4]
        e0.record(main)
        side.wait_event(e0)
        with torch.cuda.stream(side):
            sad.dsa_cache_append(kvs[j], devs[j]["pool"], d_slot, latent=lat, stream=side)
        e1.record(side)
        sad.dsa_indexer_front(kvs[j], devs[j]["pool"], d_slot, ikey, q, w, q_idx, w_out)
        layers[j].scores_step(devs[j]["pool"], devs[j]["q_idx"], devs[j]["w"])
        layers[j].topk_step()
        main.wait_event(e1)
        layers[j].attention_step(devs[j]["pool"], devs[j]["q"])

    out = {}
    for name, fn in (("layer_ms_per_step", layer_only), ("serial_ms_per_step", serial),
                     ("overlapped_ms_per_step", overlapped)):
        for i in range(5):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        out[name] = 1e3 * (time.perf_counter() - t0) / steps
    out["front_serial_us"] = 1e3 * (out["serial_ms_per_step"] - out["layer_ms_per_step"])
    out["front_overlapped_us"] = 1e3 * (out["overlapped_ms_per_step"] - out["layer_ms_per_step"])
    out["steps"] = steps
    return out


def read_ceiling(wls, devs, kvs, reps: int = 10):
    """Measured read ceilings after the timed region (dsa_probe_read: loads only, no
    arithmetic): (a) exactly the scorer's key pages, block by block in the block tables' order,
    rotating over the same batches as the timed steps; (b) a contiguous read of as many bytes from
    the start of each pool.  Returns GB/s of each (event-timed, `reps` launches)."""
    import torch
    from sparse_attention_decode_amd._lib import dsa_probe_read
    key_page = 64 * (132 if wls[0].ikey_fmt == 0 else 68)
    rows_list, npages = [], 0
    for wl, d in zip(wls, devs):
        bt = []
        for b in range(wl.num_seqs):
            L = int(wl.row_pos[wl.rows_of(b)].max()) + 1
            bt.append(np.asarray(wl.block_table[b, :(L + 63) // 64], np.int32))
        r = np.concatenate(bt)
        rows_list.append(torch.from_numpy(r).cuda())
        npages = r.size
    sink = torch.empty(2048, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for name in ("pages", "sequential"):
        def run(j):
            kv, d = kvs[j], devs[j]
            if name == "pages":
                dsa_probe_read(d["pool"], kv.row_bytes, kv.ikey_off, key_page, rows_list[j],
                               rows_list[j].numel(), sink)
            else:
                dsa_probe_read(d["pool"], key_page, 0, key_page, None, rows_list[j].numel(),
                               sink)
        for i in range(3):
            run(i % len(devs))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(reps):
            run(i % len(devs))
        b.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / reps
        res[name + "_GBps"] = npages * key_page / (us * 1e-6) / 1e9
    res["bytes_per_launch"] = npages * key_page
    res["launches"] = reps
    return res


def bench_dcp(args):
    """The decode step under emulated decode context parallelism: the workload's sequences split
    into W token-interleaved shards (each its own pool), per shard the scorer and the local
    select, then the publish of the sorted local lists, the exact merge, per shard the attention
    over its part, and the LSE combine.  On one GPU the shards run one after another; `value` is
    rows/s of the whole emulated step, and the merge and combine are timed with events."""
    import torch
    import sparse_attention_decode_amd as sad
    import synth
    import synth.device
    W = args.dcp
    if not 1 <= W <= sad.MAX_SHARDS:
        sys.exit(f"--dcp must be in [1, {sad.MAX_SHARDS}]")
    variant = {"packed": sad.MERGE_PACKED, "scores": sad.MERGE_SCORES,
               "generic": sad.MERGE_GENERIC}[args.dcp_variant]
    wl = synth.decode_config(args.config)
    if int(np.diff(wl.seq_row_start).max()) > sad.MAX_ROWS_PER_SEQ:
        sys.exit("--dcp emulates the decode path (up to 8 rows per sequence)")
    R, k = wl.num_rows, wl.k
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    shards = []
    for r in range(W):
        sw = synth.shard_workload(wl, W, r)
        kv = sad.kv_layout(sw.ikey_fmt, sw.lat_fmt, sw.num_blocks, sw.lat_tensor_scale)
        d = synth.device.stage(sw, kv.as_dict())
        batch = sad.DeviceBatch(d["block_table"], d["seq_row_start"], d["row_pos"],
                                d["max_rows_per_seq"], d["max_context"])
        shards.append((kv, d, batch, sad.DSALayer(kv, batch, k, wl.softmax_scale)))
        log(f"[bench] staged shard {r} of {W}: pool {d['pool'].numel() / 2**30:.2f} GiB")
    dev = dict(device="cuda")
    mb = torch.empty(sad.dsa_dcp_mailbox_bytes(R, k, W), dtype=torch.uint8, **dev)
    parts = torch.empty(sad.dsa_dcp_partials_bytes(R, k, W), dtype=torch.uint8, **dev)
    idx = torch.empty((R, k), dtype=torch.int32, **dev)
    cnt = torch.empty(R, dtype=torch.int32, **dev)
    sidx = torch.empty((W, R, k), dtype=torch.int32, **dev)
    scnt = torch.empty((W, R), dtype=torch.int32, **dev)
    stats = torch.empty((R, 4), dtype=torch.int32, **dev)
    out = torch.empty((R, sad.MLA_HEADS, sad.MLA_DV), dtype=torch.bfloat16, **dev)
    lse = torch.empty((R, sad.MLA_HEADS), dtype=torch.float32, **dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        for r, (kv, d, batch, layer) in enumerate(shards):
            layer.scores_step(d["pool"], d["q_idx"], d["w"])
            layer.topk_step(phys=False)
            sad.dsa_dcp_publish(k, W, r, layer.scores, layer.idx, layer.count, mb)
        if ev is not None:
            ev[0].record(stream)
        sad.dsa_dcp_merge(k, W, variant, mb, idx, cnt, sidx, scnt, stats)
        if ev is not None:
            ev[1].record(stream)
        for r, (kv, d, batch, layer) in enumerate(shards):
            sad.sparse_mla_decode_shard(kv, d["pool"], batch, d["q"], sidx[r], k,
                                        wl.softmax_scale, r, W, parts, count=scnt[r])
        if ev is not None:
            ev[2].record(stream)
        sad.dsa_lse_combine(R, k, W, parts, out, lse)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    merge_us = 1e3 * sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    comb_us = 1e3 * sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    st = stats.cpu().numpy()
    generic = W * np.minimum(k, np.ceil((wl.row_pos + 1) / W)) * 8
    print(json.dumps({
        "metric": "DSA decode layer query-tokens/s under emulated decode context parallelism "
                  "(all shards on one GPU, exact merge)",
        "value": R * args.steps / elapsed, "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True, "data": "synthetic (seeded, exact-grid FP8 keys)",
        "config": {"workload": wl.name, "shards": W, "variant": args.dcp_variant, "rows": R,
                   "context": int(wl.seq_len.max()), "top_k": k},
        "merge": {"us": merge_us, "rounds_max": int(st[:, 0].max()),
                  "resending_shards": int(st[:, 1].sum()), "tie_entries": int(st[:, 2].sum()),
                  "bytes_per_row_mean": float(st[:, 3].mean()),
                  "bytes_per_row_per_shard_mean": float(st[:, 3].mean() / W),
                  "generic_bytes_per_row_mean": float(generic.mean())},
        "combine_us": comb_us,
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--replicas", type=int, default=0, help="independent batches (0: auto)")
    ap.add_argument("--graph", action="store_true",
                    help="replay select + attention from a HIP graph per batch (slower on this "
                         "stack than five eager launches: the replay adds GPU-side time)")
    ap.add_argument("--no-graph", action="store_true", help="the default; kept for old commands")
    ap.add_argument("--event-every", type=int, default=1,
                    help="time the scorer with a pair of events on every n-th timed step (each "
                         "pair costs the step a few microseconds: under 1%% of a speculative "
                         "step, about 5%% of a decode-16x128K step)")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the read-ceiling probe after the timed region")
    ap.add_argument("--plain-order", action="store_true",
                    help="score a prefill chunk's row tiles in ascending order instead of the "
                         "balanced 16-piece order (for comparison)")
    ap.add_argument("--path", choices=["auto", "dense", "candidates"], default="auto",
                    help="dense: scores stored, then dsa_topk; candidates: scores never stored "
                         "(dsa_indexer_candidates + dsa_topk_candidates); auto: the faster one "
                         "for the workload as measured (candidates for the 8,192-row prefill "
                         "chunk, dense elsewhere)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip timing the step before the path together with the layer")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--dcp", type=int, default=0,
                    help="emulate decode context parallelism: the workload split into this many "
                         "token-interleaved shards on the one GPU, merged exactly (prints its own "
                         "JSON line instead of the layer's)")
    ap.add_argument("--dcp-variant", choices=["packed", "scores", "generic"], default="packed")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run three 1 GiB device-to-device copies (the reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_per_copy": 1 << 30, "copies": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): this build runs "
              "on a single GPU; sharding across GPUs is a design, not a measured path (the "
              "cross-shard merge itself is measured on one GPU with --dcp W).", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_decode_amd as sad
    import synth
    import synth.device

    if args.dcp:
        bench_dcp(args)
        return

    cfg = args.config
    reps = args.replicas or {0: 8, 1: 4, 2: 1, 3: 1, 4: 4, 5: 2, 6: 1}[cfg]
    use_cand = {"dense": False, "candidates": True}.get(args.path, cfg in AUTO_CANDIDATES)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    t_setup = time.perf_counter()
    wls, devs, layers, kvs = [], [], [], []
    for rep in range(reps):
        wl = synth.decode_config(cfg, replica=rep)
        kv = sad.kv_layout(wl.ikey_fmt, wl.lat_fmt, wl.num_blocks, wl.lat_tensor_scale)
        d = synth.device.stage(wl, kv.as_dict())
        batch = sad.DeviceBatch(d["block_table"], d["seq_row_start"], d["row_pos"],
                                d["max_rows_per_seq"], d["max_context"],
                                sad.BATCH_PLAIN_ORDER if args.plain_order else 0)
        layer = sad.DSALayer(kv, batch, wl.k, wl.softmax_scale,
                             prefill=d["max_rows_per_seq"] > sad.MAX_ROWS_PER_SEQ,
                             candidates=use_cand)
        wls.append(wl)
        devs.append(d)
        layers.append(layer)
        kvs.append(kv)
        log(f"[bench] staged replica {rep} of {wl.name}: pool {d['pool'].numel() / 2**30:.2f} GiB")
    torch.cuda.synchronize()
    log(f"[bench] setup {time.perf_counter() - t_setup:.1f} s")

    stream = torch.cuda.current_stream()
    graphs = []
    use_graph = args.graph and not args.no_graph
    if use_graph:
        s = torch.cuda.Stream()
        for layer, d in zip(layers, devs):
            layer.run(d["pool"], d["q_idx"], d["w"], d["q"])  # eager reference first
        torch.cuda.synchronize()
        ref_out = [l.out.clone() for l in layers]
        # The scorer is one launch per step and runs eagerly (so the events around it time the
        # kernel alone); select + attention (four kernels) replay from one graph per batch.
        for layer, d in zip(layers, devs):
            gb = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gb, stream=s):
                layer.topk_step()
                layer.attention_step(d["pool"], d["q"])
            graphs.append(gb)
        for gb, layer, d, ref in zip(graphs, layers, devs, ref_out):
            layer.scores_step(d["pool"], d["q_idx"], d["w"])
            gb.replay()
            torch.cuda.synchronize()
            assert torch.equal(layer.out, ref), "graph replay differs from eager run"

    def step(i, ev=None):
        j = i % reps
        if ev is not None:
            ev[0].record(stream)
        layers[j].scores_step(devs[j]["pool"], devs[j]["q_idx"], devs[j]["w"])
        if ev is not None:
            ev[1].record(stream)
        if use_graph:
            graphs[j].replay()
        else:
            layers[j].topk_step()
            layers[j].attention_step(devs[j]["pool"], devs[j]["q"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the scorer's launches are timed by events on its stream on a sample of the timed steps
    every = max(1, args.event_every)
    evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for i in range(0, args.steps, every)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    idx_samples = sorted(a.elapsed_time(b) for a, b in evs.values())
    idx_ms = sum(idx_samples) / len(idx_samples)

    wl = wls[0]
    rows = wl.num_rows
    ms_step = 1e3 * elapsed / args.steps
    value = rows * args.steps / elapsed
    total_b, idx_b = algorithmic_bytes(wl)
    layer_gbps = total_b / (ms_step * 1e-3) / 1e9
    idx_gbps = idx_b / (idx_ms * 1e-3) / 1e9
    flops = indexer_flops(wl)
    prefill = cfg in (3, 5, 6)
    if prefill:
        roof = {"bound": "mfma", "achieved": flops / (idx_ms * 1e-3) / 1e12,
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": idx_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None if (prefill or use_cand) else recorded_traffic(wl.name)
    roof["kernel"] = ("indexer_kernel sample + candidate passes with the sample select "
                      "(dsa_indexer_candidates)" if use_cand else
                      "indexer_kernel (dsa_indexer_scores)")
    roof["ms_per_launch"] = idx_ms
    roof["ms_per_launch_median"] = idx_samples[len(idx_samples) // 2]
    roof["timed_launches"] = len(evs)
    roof["timing"] = "hip events on the scorer's stream around its launch in the timed steps"
    roof["algorithmic_bytes_per_launch"] = idx_b
    roof["layer_frac"] = layer_gbps / PEAK_HBM_GBPS
    if not prefill and not args.no_probe:
        ceil = read_ceiling(wls, devs, kvs)
        roof["measured_ceiling"] = ceil
        roof["frac_of_page_ceiling"] = roof["achieved"] / ceil["pages_GBps"]

    result = {
        "metric": METRIC, "value": value, "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3 (indexer) / bf16+fp16 (attention), fp32 accumulate",
        "data": "synthetic (seeded, exact-grid FP8 keys)",
        "config": {"workload": wl.name, "seqs": wl.num_seqs, "rows": rows,
                   "context": int(wl.seq_len.max()), "top_k": wl.k,
                   "index_keys": "fp8" if wl.ikey_fmt == 0 else "mxfp4",
                   "latent": "fp8" if wl.lat_fmt == 0 else "nvfp4", "block": 64,
                   "batches_rotated": reps, "hip_graph": use_graph,
                   "path": "candidates" if use_cand else "dense",
                   "prefill_tile_order": "plain" if args.plain_order else "balanced"},
        "layer_hbm": {"algorithmic_bytes_per_step": total_b, "achieved_GBps": layer_gbps,
                      "frac_of_8TBps": layer_gbps / PEAK_HBM_GBPS},
        "roofline": roof,
    }
    # the step before the path, timed on its own after the layer (not part of `value`)
    result["front"] = time_front(wl, devs[0], kvs[0], max(10, min(args.steps, 100)))
    if not use_graph and not args.no_overlap:
        result["front"]["with_layer"] = time_front_overlap(wl, layers, devs, kvs, reps,
                                                           max(10, min(args.steps, 50)))
    if not args.no_cpu:
        log("[bench] timing the oracle on a CPU sample ...")
        result["cpu_baseline"] = cpu_baseline(cfg, wl, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
