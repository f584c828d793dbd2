"""Stage a synth.Workload in device memory (torch tensors).  No method arithmetic."""
from __future__ import annotations

import numpy as np

from . import Workload, fill_pool, row_queries


def stage(w: Workload, layout: dict, device="cuda", with_queries=True):
    """Device tensors of workload w for a pool laid out as `layout` (the library's layout
    descriptor as a dict).  Returns a dict: pool (uint8), block_table (int32 [S, maxb]),
    seq_row_start (int32 [S+1]), row_pos (int32 [R]), and, with_queries, q_idx (uint8
    [R,32,128]), w (f32 [R,32]), q (bf16 [R,96,576]); plus max_context and max_rows_per_seq."""
    import torch
    pool = torch.from_numpy(fill_pool(w, layout)).to(device)
    out = dict(
        pool=pool,
        block_table=torch.from_numpy(np.ascontiguousarray(w.block_table, np.int32)).to(device),
        seq_row_start=torch.from_numpy(w.seq_row_start).to(device),
        row_pos=torch.from_numpy(np.ascontiguousarray(w.row_pos, np.int32)).to(device),
        max_context=int(w.row_pos.max()) + 1,
        max_rows_per_seq=int(np.diff(w.seq_row_start).max()),
    )
    if with_queries:
        qi, hw, qm = row_queries(w)
        out["q_idx"] = torch.from_numpy(qi).to(device)
        out["w"] = torch.from_numpy(hw).to(device)
        out["q"] = torch.from_numpy(qm.view(np.int16)).to(device).view(torch.bfloat16)
    return out
