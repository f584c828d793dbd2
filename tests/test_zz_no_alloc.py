"""sparse_mla_decode_noalloc (split partials in the library's static per-device scratch) against
sparse_mla_decode (caller's workspace): two calls in a row, the second on a smaller batch, each
bit-identical to the workspace entry point and within the oracle tolerance; a batch whose
partials exceed the scratch is refused before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_attention_decode_amd as sad
from sparse_attention_decode_amd import _lib as L
import synth
from gpu_harness import check_workload, run_gpu

pytestmark = pytest.mark.gpu


def _noalloc_matches(wl):
    layer, d, kv = run_gpu(wl)  # scorer, select, sparse_mla_decode with a workspace
    assert layer.workspace is not None, "the batch should use split partials"
    out = torch.full_like(layer.out, float("nan"))
    lse = torch.full_like(layer.lse, float("nan"))
    sad.sparse_mla_decode_noalloc(kv, d["pool"], layer.batch, d["q"], layer.idx, layer.k,
                                  layer.softmax_scale, out, lse, phys=layer.phys)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), layer.out.view(torch.int16))
    assert torch.equal(lse, layer.lse)
    layer.out.copy_(out)
    layer.lse.copy_(lse)
    check_workload(wl, layer)


def test_noalloc_matches_workspace_entry_point_twice():
    big = synth.Workload("noalloc-a", 71, [20000 + 97 * i for i in range(16)], list(range(16)),
                         [20000 + 97 * i - 1 for i in range(16)])
    small = synth.Workload("noalloc-b", 72, [3000, 5000, 2100], [0, 1, 2], [2999, 4999, 2099])
    _noalloc_matches(big)
    _noalloc_matches(small)


def test_noalloc_refuses_partials_beyond_the_scratch():
    lib = L.lib()
    kv = sad.kv_layout(sad.IKEY_FP8, sad.LATENT_FP8, 10)
    b = L.Batch()
    b.num_seqs, b.num_rows, b.max_rows_per_seq, b.max_blocks_per_seq = 1, 64, 64, 2
    b.max_context = 100
    b.block_table = b.seq_row_start = b.row_pos = 0x1000
    b.flags = sad.BATCH_INVARIANT  # 16 splits per row: 64 rows need 97 MiB of partials
    assert sad.sparse_mla_workspace_bytes(64, 2048, sad.BATCH_INVARIANT) > 64 << 20
    p = ctypes.c_void_p(0x2000)
    st = lib.sparse_mla_decode_noalloc(ctypes.byref(kv), ctypes.c_void_p(0x100000),
                                       ctypes.byref(b), p, p, None, 2048, 0.1, p, None, None)
    assert st == L.DSA_ERR_WORKSPACE and b"static scratch" in lib.dsa_last_error()
