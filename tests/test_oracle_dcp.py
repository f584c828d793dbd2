"""Pins of the oracle's cross-shard merge and log-sum-exp combine (oracle/dcp.py).

The merge must reach exactly the plain top-k of the whole row, computed independently by the C
oracle (a full sort); its protocol counts are pinned on hand-worked cases (a resend when one shard
holds more than it sent, none when the top-k is spread, the tie round when every score is equal,
nothing to do when fewer than k tokens are visible).  The combine of per-shard attention results
must equal the attention over the union of the shards' tokens (the identity behind decode context
parallelism), checked against the C oracle's attention in float64."""
import numpy as np
import pytest

import oracle
from oracle import dcp

VARIANTS = (dcp.PACKED, dcp.SCORES, dcp.GENERIC)


def _check(scores, W, k, variant):
    lists = dcp.shard_lists(scores, W, k)
    chosen, per_shard, stats = dcp.merge(lists, k, variant)
    want, cnt = oracle.topk(np.asarray(scores, np.float64), k)
    assert np.array_equal(chosen, want[:cnt]), (W, k, variant)
    assert np.array_equal(np.sort(np.concatenate(per_shard)), chosen)
    for r, s in enumerate(per_shard):
        assert np.all(s % W == r) and np.all(np.diff(s) > 0)
    return stats


@pytest.mark.parametrize("variant", VARIANTS)
def test_merge_equals_global_topk_random(variant):
    rng = np.random.default_rng(11)
    for trial in range(40):
        n = int(rng.integers(1, 6000))
        W = int(rng.choice([1, 2, 3, 4, 8]))
        k = int(rng.choice([1, 5, 64, 700, 2048]))
        s = rng.standard_normal(n).astype(np.float32)
        if trial % 3 == 0:                 # coarse grid: many exact ties
            s = np.round(s * 4) / 4
        if trial % 5 == 1:                 # one shard dominates
            s[::W] += 3.0
        _check(s, W, k, variant)


def test_resend_hand_worked():
    # W = 2, k = 4, C = ceil(1.5 * 4 / 2) = 3.  Shard 0 (tokens 0, 2, ..., 8) scores 9..5, shard 1
    # (tokens 1, 3, ..., 9) scores .1...5.  First exchange: shard 0 sends 9, 8, 7, shard 1 sends
    # .5, .4, .3; the 4th largest is .5 and shard 0's weakest sent (7) reaches it, so shard 0
    # resends its full local top-4; the second select takes tokens 0, 2, 4, 6.  Bytes: 6 words +
    # 4 resent words.
    s = np.zeros(10, np.float32)
    s[0::2] = [9, 8, 7, 6, 5]
    s[1::2] = [.1, .2, .3, .4, .5]
    lists = dcp.shard_lists(s, 2, 4)
    chosen, per_shard, stats = dcp.merge(lists, 4, dcp.PACKED)
    assert list(chosen) == [0, 2, 4, 6]
    assert stats == (2, 1, 0, (3 + 3) * 4 + 4 * 4)
    assert [list(p) for p in per_shard] == [[0, 2, 4, 6], []]
    # the generic merge sends full lists of (score, id) pairs: 8 pairs, one round
    assert dcp.merge(lists, 4, dcp.GENERIC)[2] == (1, 0, 0, 8 * 8)


def test_spread_top_k_needs_no_resend():
    # i.i.d. scores over 8 shards: each holds about 256 of the top 2,048 (sd ~15), far below the
    # 384 it sends
    rng = np.random.default_rng(12)
    s = rng.standard_normal(60000).astype(np.float32)
    stats = _check(s, 8, 2048, dcp.PACKED)
    assert stats[0] == 1 and stats[1] == 0
    assert stats[3] == 8 * 384 * 4 + stats[2] * 8      # 12 KiB of candidates (+ the tie round)
    assert _check(s, 8, 2048, dcp.SCORES)[3] == 8 * 2048 * 4 + _check(s, 8, 2048,
                                                                       dcp.SCORES)[2] * 4


def test_all_equal_scores_tie_round():
    # every score is 0 (a zero query): the lowest 2,048 indices win.  Packed: every shard's
    # weakest candidate sits on the threshold, so all four resend their full lists (1,250 each),
    # then the 5,000 tied entries go through the tie round.  Scores only: no resend, same tie round.
    s = np.zeros(5000, np.float32)
    s[7] = -0.0
    st = _check(s, 4, 2048, dcp.PACKED)
    assert st == (2, 4, 5000, 4 * 768 * 4 + 4 * 1250 * 4 + 5000 * 8)
    st = _check(s, 4, 2048, dcp.SCORES)
    assert st == (1, 0, 5000, 4 * 1250 * 4 + 5000 * 4)
    assert _check(s, 4, 2048, dcp.GENERIC) == (1, 0, 0, 4 * 1250 * 8)


def test_fewer_than_k_visible():
    rng = np.random.default_rng(13)
    s = rng.standard_normal(1000).astype(np.float32)
    for v in VARIANTS:
        assert _check(s, 8, 2048, v)[:3] == (1, 0, 0)
    # a shard holding more than it may send while the messages total fewer than k (shard 1 holds
    # nothing): shard 0 must resend, and then everything it holds is selected
    keys = dcp.order_key(np.arange(10, 0, -1).astype(np.float32))
    lists = [(keys, np.arange(0, 20, 2)), (keys[:0], np.arange(0))]
    chosen, _, stats = dcp.merge(lists, 12, dcp.PACKED)     # C = 9 < 10
    assert list(chosen) == list(range(0, 20, 2)) and stats == (2, 1, 0, 9 * 4 + 10 * 4)


def test_order_key_is_monotone():
    rng = np.random.default_rng(14)
    a = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.uniform(-30, 30, 2000),
                        [0.0, -0.0, np.inf, -np.inf]]).astype(np.float32)
    ka = dcp.order_key(a)
    i, j = rng.integers(0, a.size, (2, 20000))
    assert np.all((a[i] < a[j]) == (ka[i] < ka[j]))
    assert np.all((a[i] == a[j]) == (ka[i] == ka[j]))


def _bf16(x):
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def test_lse_combine_equals_attention_over_the_union():
    rng = np.random.default_rng(15)
    H, D, dv = 96, 576, 512
    q = _bf16(rng.standard_normal((H, D)))
    c = rng.standard_normal((300, D)) * 0.5
    scale = 1 / np.sqrt(192)
    ref_out, ref_lse = oracle.sparse_mla(q, c, scale, dv)
    for W in (1, 2, 5):
        part = rng.integers(0, W, 300)
        part[:W] = np.arange(W)                # no part is empty
        outs, lses = [], []
        for r in range(W):
            o, l = oracle.sparse_mla(q, c[part == r], scale, dv)
            outs.append(o)
            lses.append(l)
        out, lse = dcp.lse_combine(outs, lses)
        assert np.allclose(out, ref_out, rtol=1e-11, atol=1e-12)
        assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)
    # a shard that selected nothing contributes lse = -inf and nothing else
    o, l = oracle.sparse_mla(q, c, scale, dv)
    out, lse = dcp.lse_combine([o, np.zeros_like(o)], [l, np.full(H, -np.inf)])
    assert np.array_equal(out, o) and np.array_equal(lse, l)
    out, lse = dcp.lse_combine([np.zeros_like(o)] * 2, [np.full(H, -np.inf)] * 2)
    assert not out.any() and np.all(lse == -np.inf)
