"""The generator's pool writer puts each token's pages where the library's layout descriptor
says, unused slots and rows are poisoned, and the byte identities of the pages hold."""
import numpy as np

import sparse_attention_decode_amd as sad
import synth
from pool_layout import fp8_key_positions


def _unpack_token(pool, kv, bt, s, wl):
    row = int(bt[s // 64])
    slot = s % 64
    base = row * kv.row_bytes
    if wl.lat_fmt == 0:
        lat = pool[base + kv.latent_off + slot * 576: base + kv.latent_off + slot * 576 + 576]
        ls = pool[base + kv.latent_scale_off + 4 * slot: base + kv.latent_scale_off + 4 * slot + 4].view(np.float32)
    else:
        lat = pool[base + kv.latent_off + slot * 288: base + kv.latent_off + slot * 288 + 288]
        ls = pool[base + kv.latent_scale_off + slot * 36: base + kv.latent_scale_off + slot * 36 + 36]
    if wl.ikey_fmt == 0:
        key = pool[base + kv.ikey_off + fp8_key_positions(slot)]
        ks = pool[base + kv.ikey_scale_off + 4 * slot: base + kv.ikey_scale_off + 4 * slot + 4].view(np.float32)
    else:
        key = pool[base + kv.ikey_off + slot * 64: base + kv.ikey_off + slot * 64 + 64]
        ks = pool[base + kv.ikey_scale_off + slot * 4: base + kv.ikey_scale_off + slot * 4 + 4]
    return lat, ls, key, ks


def test_pool_round_trip_all_formats():
    for ik, lf in [(0, 0), (1, 1), (0, 1), (1, 0)]:
        wl = synth.Workload("t", 31 + ik + 2 * lf, [130, 64, 1], [0, 1, 2], [129, 63, 0],
                            ikey_fmt=ik, lat_fmt=lf, lat_tensor_scale=0.5)
        kv = sad.kv_layout(ik, lf, wl.num_blocks, 0.5)
        pool = synth.fill_pool(wl, kv.as_dict())
        assert pool.size == wl.num_blocks * kv.row_bytes
        used = set()
        for b in range(wl.num_seqs):
            keys, kscale, lat, lscale = synth.seq_tensors(wl, b)
            bt = wl.block_table[b]
            used.update(int(x) for x in bt[bt >= 0])
            for s in range(int(wl.seq_len[b])):
                la, lsc, ke, ksc = _unpack_token(pool, kv, bt, s, wl)
                assert np.array_equal(la, lat[s].ravel())
                assert np.array_equal(ke, keys[s].ravel())
                assert np.array_equal(lsc.ravel(), np.asarray(lscale[s]).ravel().view(lsc.dtype))
                assert np.array_equal(ksc.ravel(), np.asarray(kscale[s]).ravel().view(ksc.dtype))
            # slots past the end of the last block are poisoned
            L = int(wl.seq_len[b])
            if L % 64:
                la, lsc, ke, ksc = _unpack_token(pool, kv, bt, L, wl)
                assert np.all(la == 0xFF) and np.all(ke == 0xFF)
        spare = [r for r in range(wl.num_blocks) if r not in used]
        assert len(spare) == wl.spare_blocks
        for r in spare:
            assert np.all(pool[r * kv.row_bytes:(r + 1) * kv.row_bytes] == 0xFF)


def test_block_tables_are_one_shuffled_pool():
    wl = synth.decode_config(4)
    bt = wl.block_table
    ids = bt[bt >= 0]
    assert len(np.unique(ids)) == len(ids)  # no block shared between sequences
    assert ids.max() < wl.num_blocks
    nb = (wl.seq_len + 63) // 64
    assert len(ids) == nb.sum()
    assert not np.array_equal(np.sort(ids), ids)  # shuffled


def test_footprint_table_of_the_page():
    # KV cache per token per GPU over 24 DSA layers: 24 x 576 (K3 FP8 latent) = 13,824;
    # 24 x (576 + 132) = 16,992; 24 x (352 + 68) = 10,080 with the page's NVFP4 latent size.
    assert 24 * 576 == 13824
    kv = sad.kv_layout(sad.IKEY_FP8, sad.LATENT_FP8, 1)
    key_bytes = (kv.ikey_scale_off - kv.ikey_off) // 64 + 4
    assert 24 * (576 + key_bytes) == 16992
    kv4 = sad.kv_layout(sad.IKEY_MXFP4, sad.LATENT_NVFP4, 1, 1.0)
    mx_bytes = (kv4.ikey_scale_off - kv4.ikey_off) // 64 + 4
    assert 24 * (352 + mx_bytes) == 10080
    # MXFP4 cuts index-key storage by 48.5% (page, Native MXFP4 indexer)
    assert round(100 * (key_bytes - mx_bytes) / key_bytes, 1) == 48.5
    # this build's NVFP4 latent: 576 E2M1 (288 B) + 36 E4M3 block scales = 324 B per token
    assert (kv4.latent_scale_off - kv4.latent_off) // 64 + 576 // 16 == 324
