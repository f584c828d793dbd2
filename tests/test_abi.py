"""The C-ABI library loads, exports every symbol include/dsa.h declares, and its host-side
validation and layout logic behave as documented (no GPU needed: nothing here launches)."""
import ctypes
import os
import re

import pytest

import sparse_attention_decode_amd as sad
from sparse_attention_decode_amd import _lib as L
from conftest import ROOT


def _header_functions():
    with open(os.path.join(ROOT, "include", "dsa.h")) as f:
        text = f.read()
    return re.findall(r"DSA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_library_exports_every_declared_symbol():
    names = _header_functions()
    assert len(names) >= 8
    assert set(names) == set(L.EXPORTS)
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_layout_rows_match_page_byte_counts():
    # Page (KV cache footprint / A KV cache for three kinds of state): FP8 index key 132 B per
    # token including its scale, MXFP4 key 68 B, FP8 latent 576 B.
    kv = sad.kv_layout(sad.IKEY_FP8, sad.LATENT_FP8, 10)
    assert kv.ikey_scale_off - kv.ikey_off == 64 * 128
    assert (kv.ikey_scale_off - kv.ikey_off) // 64 + 4 == 132
    assert kv.latent_scale_off - kv.latent_off == 64 * 576
    assert kv.row_bytes == 64 * (576 + 4 + 128 + 4) == 45568
    kv4 = sad.kv_layout(sad.IKEY_MXFP4, sad.LATENT_NVFP4, 10, 0.5)
    assert (kv4.ikey_scale_off - kv4.ikey_off) // 64 + 128 // 32 == 68
    assert kv4.latent_scale_off - kv4.latent_off == 64 * 288
    assert kv4.row_bytes == 64 * (288 + 36 + 64 + 4) == 25088
    assert abs(kv4.latent_tensor_scale - 0.5) < 1e-7
    for k in (kv, kv4):
        for off in (k.latent_off, k.latent_scale_off, k.ikey_off, k.ikey_scale_off):
            assert off % 16 == 0
        assert k.row_bytes % 256 == 0


def test_layout_rejects_bad_arguments():
    with pytest.raises(sad.DSAError) as e:
        sad.kv_layout(sad.IKEY_FP8, sad.LATENT_FP8, 10, block_size=32)
    assert e.value.status == L.DSA_ERR_UNSUPPORTED
    with pytest.raises(sad.DSAError) as e:
        sad.kv_layout(7, sad.LATENT_FP8, 10)
    assert e.value.status == L.DSA_ERR_INVALID_ARG
    with pytest.raises(sad.DSAError):
        sad.kv_layout(sad.IKEY_FP8, sad.LATENT_NVFP4, 10, 0.0)


def test_layout_pages_must_fit_in_the_row():
    # a hand-made layout whose latent-scale page sits at the very end of the row: the attention's
    # 16-byte scale gathers would read past it, so every entry point rejects the layout
    lib = L.lib()
    b = _fake_batch()
    p = ctypes.c_void_p(0x2000)
    for ikey, lat in ((sad.IKEY_FP8, sad.LATENT_FP8), (sad.IKEY_MXFP4, sad.LATENT_NVFP4)):
        kv = sad.kv_layout(ikey, lat, 10, 0.5 if lat else 1.0)
        scale_bytes = 64 * (4 if lat == sad.LATENT_FP8 else 36)
        kv.latent_off, kv.latent_scale_off, kv.ikey_off, kv.ikey_scale_off = (
            0, kv.row_bytes - (scale_bytes + 15) // 16 * 16, kv.latent_scale_off, kv.ikey_off)
        assert lib.dsa_indexer_scores(ctypes.byref(kv), ctypes.c_void_p(0x100000), ctypes.byref(b),
                                      p, p, p, 128, None, None) == L.DSA_ERR_INVALID_ARG
        assert b"12 bytes" in lib.dsa_last_error()
        # a page running past the row
        kv2 = sad.kv_layout(ikey, lat, 10, 0.5 if lat else 1.0)
        kv2.ikey_off = kv2.row_bytes - 16
        assert lib.dsa_indexer_scores(ctypes.byref(kv2), ctypes.c_void_p(0x100000), ctypes.byref(b),
                                      p, p, p, 128, None, None) == L.DSA_ERR_INVALID_ARG
        assert b"extends past" in lib.dsa_last_error()


def _fake_batch(**over):
    b = L.Batch()
    b.num_seqs, b.num_rows, b.max_rows_per_seq, b.max_blocks_per_seq = 1, 1, 1, 2
    b.max_context = 100
    b.block_table = b.seq_row_start = b.row_pos = 0x1000
    for k, v in over.items():
        setattr(b, k, v)
    return b


def test_entry_points_validate_before_launch():
    lib = L.lib()
    kv = sad.kv_layout(sad.IKEY_FP8, sad.LATENT_FP8, 10)
    pool = ctypes.c_void_p(0x100000)
    p = ctypes.c_void_p(0x2000)
    b = _fake_batch()
    # null pool
    assert lib.dsa_indexer_scores(ctypes.byref(kv), None, ctypes.byref(b), p, p, p, 128, None,
                                  None) == L.DSA_ERR_INVALID_ARG
    assert b"pool" in lib.dsa_last_error()
    # misaligned pool
    assert lib.dsa_indexer_scores(ctypes.byref(kv), ctypes.c_void_p(0x100010), ctypes.byref(b),
                                  p, p, p, 128, None, None) == L.DSA_ERR_INVALID_ARG
    # ld below max_context
    assert lib.dsa_indexer_scores(ctypes.byref(kv), pool, ctypes.byref(b), p, p, p, 64, None,
                                  None) == L.DSA_ERR_INVALID_ARG
    # block table too narrow for max_context
    b2 = _fake_batch(max_context=200)
    assert lib.dsa_indexer_scores(ctypes.byref(kv), pool, ctypes.byref(b2), p, p, p, 256, None,
                                  None) == L.DSA_ERR_INVALID_ARG
    # k out of range
    for k in (0, 2049):
        assert lib.dsa_topk(ctypes.byref(kv), ctypes.byref(b), p, 128, None, k, p, p, None,
                            p, 1 << 30, None) == L.DSA_ERR_INVALID_ARG
        assert lib.sparse_mla_decode(ctypes.byref(kv), pool, ctypes.byref(b), p, p, None, k, 0.1,
                                     p, None, None, 0, None) == L.DSA_ERR_INVALID_ARG
    # phys rows need the layout
    assert lib.dsa_topk(None, ctypes.byref(b), p, 128, None, 16, p, p, p, p, 1 << 30, None) == \
        L.DSA_ERR_INVALID_ARG
    # top-k needs its workspace
    need = lib.dsa_topk_workspace_bytes(1, 100)
    assert need > 0
    assert lib.dsa_topk(ctypes.byref(kv), ctypes.byref(b), p, 128, None, 16, p, p, None, p,
                        need - 1, None) == L.DSA_ERR_WORKSPACE
    # decode MLA with several splits needs its workspace
    b3 = _fake_batch(num_rows=1)
    need = lib.sparse_mla_workspace_bytes(1, 2048, 0)
    assert need > 0
    assert lib.sparse_mla_decode(ctypes.byref(kv), pool, ctypes.byref(b3), p, p, None, 2048, 0.1,
                                 p, None, None, 0, None) == L.DSA_ERR_WORKSPACE
    assert lib.sparse_mla_decode(ctypes.byref(kv), pool, ctypes.byref(b3), p, p, p, 2048, 0.1,
                                 p, None, p, need - 1, None) == L.DSA_ERR_WORKSPACE
    # the prefill path checks the histogram's alignment like the decode path
    kv4 = sad.kv_layout(sad.IKEY_MXFP4, sad.LATENT_FP8, 10)
    b4 = _fake_batch(max_rows_per_seq=64, num_rows=64)
    assert lib.dsa_indexer_scores(ctypes.byref(kv4), pool, ctypes.byref(b4), p, p, p, 128,
                                  ctypes.c_void_p(0x2002), None) == L.DSA_ERR_INVALID_ARG
    assert lib.dsa_status_string(L.DSA_ERR_WORKSPACE) == b"DSA_ERR_WORKSPACE"


def test_batch_flags():
    # Unknown flag bits are rejected before any launch; the batch-invariant split count depends
    # on k alone, so its workspace is rows x 16 splits for k = 2048, also on the prefill path.
    lib = L.lib()
    kv = sad.kv_layout(sad.IKEY_FP8, sad.LATENT_FP8, 10)
    pool = ctypes.c_void_p(0x100000)
    p = ctypes.c_void_p(0x2000)
    bad = _fake_batch(flags=4)  # bits 0 and 1 are DSA_BATCH_INVARIANT and DSA_BATCH_PLAIN_ORDER
    assert lib.dsa_indexer_scores(ctypes.byref(kv), pool, ctypes.byref(bad), p, p, p, 128, None,
                                  None) == L.DSA_ERR_INVALID_ARG
    assert lib.sparse_mla_decode(ctypes.byref(kv), pool, ctypes.byref(bad), p, p, p, 2048, 0.1,
                                 p, None, p, 1 << 30, None) == L.DSA_ERR_INVALID_ARG
    per_slot = sad.MLA_DV * 2 + 8
    assert lib.sparse_mla_workspace_bytes(8192, 2048, 0) == 0
    assert lib.sparse_mla_workspace_bytes(8192, 2048, sad.BATCH_INVARIANT) == 8192 * 16 * 96 * per_slot
    assert lib.sparse_mla_workspace_bytes(3, 2048, sad.BATCH_INVARIANT) == 3 * 16 * 96 * per_slot
    inv = _fake_batch(flags=sad.BATCH_INVARIANT, num_rows=64, max_rows_per_seq=64)
    assert lib.sparse_mla_prefill(ctypes.byref(kv), pool, ctypes.byref(inv), p, p, p, 2048, 0.1,
                                  p, None, None, 0, None) == L.DSA_ERR_WORKSPACE


def test_empty_batch_is_a_no_op():
    # A batch with no query rows validates and returns DSA_OK without launching anything.
    lib = L.lib()
    kv = sad.kv_layout(sad.IKEY_FP8, sad.LATENT_FP8, 10)
    pool = ctypes.c_void_p(0x100000)
    p = ctypes.c_void_p(0x2000)
    b = _fake_batch(num_rows=0, max_rows_per_seq=0)
    assert lib.dsa_indexer_scores(ctypes.byref(kv), pool, ctypes.byref(b), p, p, p, 128, p,
                                  None) == L.DSA_OK
    assert lib.dsa_topk_workspace_bytes(0, 100) == 0
    assert lib.dsa_topk(ctypes.byref(kv), ctypes.byref(b), p, 128, p, 16, p, p, p, None, 0,
                        None) == L.DSA_OK
    assert lib.sparse_mla_workspace_bytes(0, 2048, 0) == 0
    for fn in (lib.sparse_mla_decode, lib.sparse_mla_prefill):
        assert fn(ctypes.byref(kv), pool, ctypes.byref(b), p, p, p, 2048, 0.1, p, None, None, 0,
                  None) == L.DSA_OK


def test_front_entry_points_validate_before_launch():
    # dsa_cache_append / dsa_quantize_query / dsa_indexer_front: bad arguments are rejected on the host and nothing-to-
    # do calls return DSA_OK, all without a launch (no GPU here).
    lib = L.lib()
    kv = sad.kv_layout(sad.IKEY_MXFP4, sad.LATENT_NVFP4, 10, 0.5)
    pool = ctypes.c_void_p(0x100000)
    p = ctypes.c_void_p(0x2000)
    ok, bad = L.DSA_OK, L.DSA_ERR_INVALID_ARG
    assert lib.dsa_cache_append(ctypes.byref(kv), None, 4, p, p, p, None) == bad
    assert lib.dsa_cache_append(None, pool, 4, p, p, p, None) == bad
    assert lib.dsa_cache_append(ctypes.byref(kv), pool, -1, p, p, p, None) == bad
    assert lib.dsa_cache_append(ctypes.byref(kv), pool, 4, None, p, p, None) == bad
    assert b"slot" in lib.dsa_last_error()
    assert lib.dsa_cache_append(ctypes.byref(kv), pool, 4, ctypes.c_void_p(0x2004), p, p,
                                None) == bad
    assert lib.dsa_cache_append(ctypes.byref(kv), pool, 4, p, ctypes.c_void_p(0x2002), None,
                                None) == bad
    assert lib.dsa_cache_append(ctypes.byref(kv), pool, 4, p, None, ctypes.c_void_p(0x2004),
                                None) == bad
    assert lib.dsa_cache_append(ctypes.byref(kv), pool, 0, None, p, p, None) == ok
    assert lib.dsa_cache_append(ctypes.byref(kv), pool, 4, p, None, None, None) == ok
    kvb = sad.kv_layout(sad.IKEY_FP8, sad.LATENT_FP8, 10)
    kvb.block_size = 32
    assert lib.dsa_cache_append(ctypes.byref(kvb), pool, 4, p, p, p, None) == L.DSA_ERR_UNSUPPORTED
    assert lib.dsa_quantize_query(-1, p, p, p, p, None) == bad
    assert lib.dsa_quantize_query(2, None, p, p, p, None) == bad
    assert lib.dsa_quantize_query(2, p, p, p, None, None) == bad
    assert lib.dsa_quantize_query(2, ctypes.c_void_p(0x2002), p, p, p, None) == bad
    assert lib.dsa_quantize_query(2, p, p, ctypes.c_void_p(0x2001), p, None) == bad
    assert lib.dsa_quantize_query(0, None, None, None, None, None) == ok
    # dsa_indexer_front: each half is checked as its own call is, and an empty half needs no
    # pointers
    f = lib.dsa_indexer_front
    assert f(None, pool, 4, p, p, 2, p, p, p, p, None) == bad
    assert f(ctypes.byref(kv), pool, -1, p, p, 2, p, p, p, p, None) == bad
    assert f(ctypes.byref(kv), pool, 4, p, p, -1, p, p, p, p, None) == bad
    assert f(ctypes.byref(kv), pool, 4, None, p, 2, p, p, p, p, None) == bad
    assert f(ctypes.byref(kv), pool, 4, p, None, 2, p, p, p, p, None) == bad
    assert f(ctypes.byref(kv), pool, 4, p, p, 2, p, None, p, p, None) == bad
    assert f(ctypes.byref(kv), pool, 4, ctypes.c_void_p(0x2004), p, 2, p, p, p, p, None) == bad
    assert f(ctypes.byref(kv), pool, 4, p, p, 2, p, p, ctypes.c_void_p(0x2001), p, None) == bad
    assert f(ctypes.byref(kv), pool, 0, None, None, 0, None, None, None, None, None) == ok
    assert f(ctypes.byref(kvb), pool, 4, p, p, 2, p, p, p, p, None) == L.DSA_ERR_UNSUPPORTED


def test_dcp_entry_points_validate_before_launch():
    # mailbox sizing, bad arguments and missing buffers are rejected before any launch
    lib = L.lib()
    p = ctypes.c_void_p(0x2000)
    mb = ctypes.c_void_p(0x10000)
    ok, bad, ws = L.DSA_OK, L.DSA_ERR_INVALID_ARG, L.DSA_ERR_WORKSPACE
    need = lib.dsa_dcp_mailbox_bytes(16, 2048, 8)
    assert need == (8 * 16 * 2048 * 8 + 8 * 16 * 4 + 15) // 16 * 16
    assert lib.dsa_dcp_mailbox_bytes(16, 2049, 8) == 0 and lib.dsa_dcp_mailbox_bytes(16, 8, 9) == 0
    assert lib.dsa_dcp_publish(16, 2048, 8, 0, p, 4096, p, p, mb, need - 1, None) == ws
    assert lib.dsa_dcp_publish(16, 2048, 8, 8, p, 4096, p, p, mb, need, None) == bad
    assert lib.dsa_dcp_publish(16, 2048, 8, -1, p, 4096, p, p, mb, need, None) == bad
    assert lib.dsa_dcp_publish(16, 2048, 8, 0, None, 4096, p, p, mb, need, None) == bad
    assert lib.dsa_dcp_publish(16, 2048, 8, 0, p, 4096, p, p, ctypes.c_void_p(0x10004), need,
                               None) == bad
    assert lib.dsa_dcp_publish(16, 0, 8, 0, p, 4096, p, p, mb, need, None) == bad
    assert lib.dsa_dcp_publish(16, 2048, 0, 0, p, 4096, p, p, mb, need, None) == bad
    assert lib.dsa_dcp_merge(16, 2048, 8, 3, mb, need, p, p, p, p, None, None) == bad
    assert lib.dsa_dcp_merge(16, 2048, 8, 0, mb, need, p, p, None, p, None, None) == bad
    assert lib.dsa_dcp_merge(16, 2048, 8, 0, None, 0, p, p, p, p, None, None) == ws
    assert lib.dsa_dcp_merge(0, 2048, 8, 0, None, 0, None, None, None, None, None, None) == ok
    pb = lib.dsa_dcp_partials_bytes(4, 2048, 2, 0)
    # the shard split count is sized for k / shards = 1,024 tokens: at 4 rows, 32 splits per shard
    assert pb == 4 * 2 * 32 * 96 * (512 * 2 + 8)
    assert lib.dsa_dcp_partials_bytes(4, 2048, 9, 0) == 0
    assert lib.dsa_lse_combine(4, 2048, 0, 0, mb, pb, p, None, None) == bad
    assert lib.dsa_lse_combine(4, 2048, 2, 4, mb, pb, p, None, None) == bad
    assert lib.dsa_lse_combine(4, 2048, 2, 0, mb, pb - 1, p, None, None) == ws
    assert lib.dsa_lse_combine(4, 2048, 2, 0, mb, pb, ctypes.c_void_p(0x2008), None, None) == bad
    assert lib.dsa_lse_combine(4, 2048, 2, 0, mb, pb, None, None, None) == bad
    assert lib.dsa_lse_combine(0, 2048, 2, 0, None, 0, None, None, None) == ok
    kv = sad.kv_layout(sad.IKEY_FP8, sad.LATENT_FP8, 10)
    b = _fake_batch(num_rows=4)
    pool = ctypes.c_void_p(0x100000)
    assert lib.sparse_mla_decode_shard(ctypes.byref(kv), pool, ctypes.byref(b), p, p, None, None,
                                       2048, 0.1, 2, 2, mb, pb, None) == bad
    assert lib.sparse_mla_decode_shard(ctypes.byref(kv), pool, ctypes.byref(b), p, p, None, None,
                                       2048, 0.1, 0, 2, mb, pb - 1, None) == ws
    assert lib.sparse_mla_decode_shard(ctypes.byref(kv), pool, ctypes.byref(b), None, p, None,
                                       None, 2048, 0.1, 0, 2, mb, pb, None) == bad
