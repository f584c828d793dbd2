"""Oracle of the exact cross-shard top-k merge and the log-sum-exp combine (decode context
parallelism, emulated: W token-interleaved shards of one sequence).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module.  It shares no code with the GPU path.  Plain numpy, small inputs.

Source: "vLLM Delivers Day-0 Support for Kimi K3.1 Pro", §Long context: decode context
parallelism with a sparse indexer (token-interleaved shards; the shards' partial attention
results are merged by log-sum-exp), §An exact top-k merge with 10x less traffic (a message of
1.5 k / W candidates per shard, each a 32-bit word carrying score and identity; the same global
select on every shard; a resend of the whole local top-k by a shard whose share of the global
top-k may exceed what it sent; as the baseline, whole local top-k lists of fp32 scores with
indices), and §AMD / Communication: Efficient cross-GPU communication (a message of scores alone,
token indices kept on their shard, ties settled by one rule applied everywhere).

The merge reaches exactly the plain top-k of the whole sequence (score descending, token index
ascending), so its result is pinned to oracle.topk; what this module adds is the protocol itself
(message sizes, rounds, resends, the tie round), followed step by step so the GPU's counts of
those can be compared too.  Readings where the page leaves a step open:
  - packed word: the upper 16 bits of the score's order-preserving 32-bit key (a truncation: a
    larger score never gets a smaller prefix) and a 16-bit rank of the candidate in its shard's
    sorted list (the id stays local: the rank names it);
  - the global select runs on what a message carries (the 16-bit prefix, or the fp32 score);
    entries that tie there at the threshold are resolved exactly (score, then token index) from
    their fp32 score and token index, sent in a second small exchange only when some but not all
    of them are needed;
  - a shard is told to resend when it sent a full message (it holds more) and its weakest sent
    candidate reaches the threshold; the resent message is its full local top-k, and the select
    is redone (a second resend is impossible: the threshold can only rise);
  - the score-only variant sends each shard's whole local top-k as fp32 scores (8 KiB at k =
    2,048, the page's figure) and exchanges the indices of threshold ties only;
  - C = min(k, ceil(1.5 k / W)) candidates per shard and row.
"""
from __future__ import annotations

import math

import numpy as np

PACKED, SCORES, GENERIC = 0, 1, 2


def order_key(scores) -> np.ndarray:
    """fp32 scores -> uint32 keys with the same order (-0 maps to +0's key)."""
    u = np.asarray(scores, np.float32).view(np.uint32).copy()
    u[u == 0x80000000] = 0
    neg = (u & 0x80000000) != 0
    return np.where(neg, ~u, u | 0x80000000).astype(np.uint32)


def candidates_per_shard(k: int, W: int) -> int:
    return min(k, math.ceil(1.5 * k / W))


def shard_lists(scores, W: int, k: int):
    """One row's shard-local exact top-k lists.  `scores` are the fp32 scores of the row's
    visible tokens [0, n).  Shard r holds tokens r, r + W, ...; its list is sorted by score
    descending, token index ascending.  Returns [(keys uint32, token indices int64)] per shard."""
    s = np.asarray(scores, np.float32)
    out = []
    for r in range(W):
        gid = np.arange(r, s.shape[0], W, dtype=np.int64)
        key = order_key(s[gid])
        order = np.lexsort((gid, -key.astype(np.int64)))[:k]
        out.append((key[order], gid[order]))
    return out


def merge(lists, k: int, variant: int = PACKED):
    """The exact merge of one row.  Returns (selected token indices ascending, per-shard selected
    token indices ascending, stats) with stats = (rounds, resending shards, entries of the tie
    exchange, message bytes of all shards over all rounds)."""
    W = len(lists)
    cnt = [len(g) for _, g in lists]
    C = candidates_per_shard(k, W) if variant == PACKED else k
    n = [min(C, c) for c in cnt]
    word_bytes = 8 if variant == GENERIC else 4
    payload = sum(n) * word_bytes
    rounds, resent = 1, 0

    def coarse(key, gid):
        if variant == PACKED:
            return key.astype(np.uint64) >> np.uint64(16)
        if variant == SCORES:
            return key.astype(np.uint64)
        return (key.astype(np.uint64) << np.uint64(32)) | (np.uint64(0xFFFFFFFF) -
                                                           gid.astype(np.uint64))

    while True:
        keys = np.concatenate([lists[r][0][:n[r]] for r in range(W)])
        gids = np.concatenate([lists[r][1][:n[r]] for r in range(W)])
        ck = coarse(keys, gids)
        N = ck.shape[0]
        if N > k:
            T = np.sort(ck)[::-1][k - 1]
        else:
            T = None  # everything sent is selected
        flagged = []
        for r in range(W):
            if n[r] < cnt[r]:
                weakest = coarse(lists[r][0][n[r] - 1:n[r]], lists[r][1][n[r] - 1:n[r]])[0]
                if T is None or weakest >= T:
                    flagged.append(r)
        if flagged and rounds == 1:
            for r in flagged:
                n[r] = cnt[r]
                payload += cnt[r] * word_bytes     # the full local top-k, sent again
            rounds, resent = 2, len(flagged)
            continue
        assert not flagged, "a second resend cannot happen"
        break

    tie = 0
    if T is None:
        sel = np.ones(N, bool)
    else:
        gt = ck > T
        eq = ck == T
        need = k - int(gt.sum())
        sel = gt.copy()
        if need == int(eq.sum()):
            sel |= eq
        else:
            # the tie round: the tied entries' exact (score, index), best `need` of them
            tie = int(eq.sum())
            payload += tie * (4 if variant == SCORES else 8)
            ties = np.nonzero(eq)[0]
            order = np.lexsort((gids[ties], -keys[ties].astype(np.int64)))[:need]
            sel[ties[order]] = True
    chosen = np.sort(gids[sel])
    per_shard = [chosen[chosen % W == r] for r in range(W)]
    return chosen, per_shard, (rounds, resent, tie, payload)


def lse_combine(outs, lses):
    """Merge W partial attention results of one row: outs [W,H,D], lses [W,H] (natural log;
    -inf for a shard with no selected token).  Returns (out [H,D], lse [H]) in float64: with M
    the largest lse, out = sum_r e^(lse_r - M) out_r / sum_r e^(lse_r - M), lse = M + ln(sum)."""
    outs = np.asarray(outs, np.float64)
    lses = np.asarray(lses, np.float64)
    M = lses.max(axis=0)
    H, D = outs.shape[1:]
    out = np.zeros((H, D))
    lse = np.full(H, -np.inf)
    ok = np.isfinite(M)
    wgt = np.exp(lses[:, ok] - M[ok])                       # [W, h]
    tot = wgt.sum(axis=0)
    out[ok] = (wgt[:, :, None] * outs[:, ok]).sum(axis=0) / tot[:, None]
    lse[ok] = M[ok] + np.log(tot)
    return out, lse
