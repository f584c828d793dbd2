"""One DSA layer step on one stream: scores -> top-k -> sparse MLA, with its device buffers."""
from __future__ import annotations

import math

from . import _lib as L


class DSALayer:
    """Owns the per-call device buffers for a fixed batch shape and runs the three C-ABI steps.

    kv: KVLayout of the pool; batch: DeviceBatch; k: top-k; prefill: use the prefill variant of
    sparse MLA (one workgroup per row, no split).  Buffers are allocated once here (torch), never
    inside run()."""

    def __init__(self, kv: L.KVLayout, batch: L.DeviceBatch, k: int = 2048,
                 softmax_scale: float = 1.0 / math.sqrt(192.0), prefill: bool = False,
                 use_hist: bool | None = None, device="cuda", candidates: bool = False):
        import torch
        self.kv, self.batch, self.k, self.softmax_scale = kv, batch, k, softmax_scale
        self.prefill = prefill
        R = batch.num_rows
        self.ld = (batch.c.max_context + 63) // 64 * 64
        # candidates: scores are never stored; the scorer leaves each row's candidates in a
        # workspace the select reads (dsa_indexer_candidates / dsa_topk_candidates)
        self.candidates = bool(candidates)
        if self.candidates:
            nb = L.dsa_candidates_workspace_bytes(R, batch.c.max_context, k)
            self.cand_ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=device)
            self.scores = self.hist = self.topk_ws = None
            use_hist = False
        # By default the scorer counts the select's histogram on the decode path only: at prefill
        # the count inside the scorer (8-wave tiles, shared LDS bins) costs about what the
        # select's own pass saves (prefill-8192: -2%, prefill-2048: +5%).
        decode_path = batch.c.max_rows_per_seq <= L.MAX_ROWS_PER_SEQ
        self.use_hist = decode_path if use_hist is None else bool(use_hist)
        if not self.candidates:
            self.scores = torch.empty((R, self.ld), dtype=torch.float32, device=device)
            # zero on entry to the scorer; dsa_topk returns it to zero after consuming it
            self.hist = (torch.zeros((R, L.HIST_BINS), dtype=torch.int32, device=device)
                         if self.use_hist else None)
        self.idx = torch.empty((R, k), dtype=torch.int32, device=device)
        # pool rows of the selection, handed from the select to the attention
        self.phys = torch.empty((R, k), dtype=torch.int32, device=device)
        self.count = torch.empty((R,), dtype=torch.int32, device=device)
        self.out = torch.empty((R, L.MLA_HEADS, L.MLA_DV), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((R, L.MLA_HEADS), dtype=torch.float32, device=device)
        if not self.candidates:
            tb = L.dsa_topk_workspace_bytes(R, batch.c.max_context)
            self.topk_ws = torch.empty((tb + 15) // 16 * 4, dtype=torch.float32, device=device)
        flags = batch.c.flags
        nbytes = 0 if (prefill and not flags & L.BATCH_INVARIANT) else \
            L.sparse_mla_workspace_bytes(R, k, flags)
        self.workspace = (torch.empty((max(nbytes, 16) + 15) // 16 * 4, dtype=torch.float32,
                                      device=device) if nbytes else None)

    def scores_step(self, pool, q_idx, w, stream=None):
        if self.candidates:
            L.dsa_indexer_candidates(self.kv, pool, self.batch, q_idx, w, self.k, self.cand_ws,
                                     stream)
        else:
            L.dsa_indexer_scores(self.kv, pool, self.batch, q_idx, w, self.scores, self.hist,
                                 stream)

    def topk_step(self, stream=None, phys=True):
        if self.candidates:
            L.dsa_topk_candidates(self.kv, self.batch, self.k, self.cand_ws, self.idx,
                                  self.count, self.phys if phys else None, stream)
        else:
            L.dsa_topk(self.kv, self.batch, self.scores, self.hist, self.k, self.idx, self.count,
                       self.topk_ws, self.phys if phys else None, stream)
        self.phys_valid = bool(phys)

    def attention_step(self, pool, q, stream=None, use_phys=None):
        fn = L.sparse_mla_prefill if self.prefill else L.sparse_mla_decode
        use_phys = getattr(self, "phys_valid", False) if use_phys is None else use_phys
        fn(self.kv, pool, self.batch, q, self.idx, self.k, self.softmax_scale, self.out,
           self.lse, self.workspace, stream, phys=self.phys if use_phys else None)

    def run(self, pool, q_idx, w, q, stream=None):
        self.scores_step(pool, q_idx, w, stream)
        self.topk_step(stream)
        self.attention_step(pool, q, stream)
        return self.out
