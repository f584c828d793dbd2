"""The device status word: device data outside the contract (a block id outside the pool, a pool
row past the pool, more rows in a sequence than max_rows_per_seq) is detected where it is read,
recorded in the status word, and never read out of bounds.  Every case is in bounds by
construction: bad block ids become zero-length buffer records in the scorer and skipped tokens in
the attention."""
import numpy as np
import pytest
import torch

import sparse_attention_decode_amd as sad
import synth
import synth.device
from gpu_harness import check_workload, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def clean_status():
    sad.dsa_device_status(clear=True)
    yield
    sad.dsa_device_status(clear=True)


def _stage(wl, max_rows=None):
    kv = sad.kv_layout(wl.ikey_fmt, wl.lat_fmt, wl.num_blocks, wl.lat_tensor_scale)
    d = synth.device.stage(wl, kv.as_dict())
    mr = d["max_rows_per_seq"] if max_rows is None else max_rows
    batch = sad.DeviceBatch(d["block_table"], d["seq_row_start"], d["row_pos"], mr,
                            d["max_context"])
    return kv, d, batch, sad.DSALayer(kv, batch, wl.k, wl.softmax_scale)


def test_clean_run_leaves_status_zero():
    wl = synth.Workload("clean", 61, [3000, 700], [0, 1], [2999, 699])
    layer, _, _ = run_gpu(wl)
    assert sad.dsa_device_status() == 0
    check_workload(wl, layer)


def test_block_id_outside_pool_is_recorded_and_scored_zero():
    wl = synth.Workload("badblk", 62, [3000], [0], [2999])
    kv, d, batch, layer = _stage(wl)
    d["block_table"][0, 5] = wl.num_blocks + 3  # visible block 5 (tokens 320..383) off the pool
    layer.scores_step(d["pool"], d["q_idx"], d["w"])
    torch.cuda.synchronize()
    assert sad.dsa_device_status() == sad.DEVERR_BLOCK_ID
    assert torch.all(layer.scores[0, 320:384] == 0)
    # the attention's logical-index path meets the same entry when a selected token lies there
    layer.topk_step(phys=False)
    layer.idx[0, 0] = 330
    layer.attention_step(d["pool"], d["q"], use_phys=False)
    torch.cuda.synchronize()
    assert sad.dsa_device_status() & sad.DEVERR_BLOCK_ID
    assert torch.isfinite(layer.out.float()).all()


def test_pool_row_past_pool_is_recorded_and_skipped():
    wl = synth.Workload("badrow", 63, [3000], [0], [2999])
    kv, d, batch, layer = _stage(wl)
    layer.scores_step(d["pool"], d["q_idx"], d["w"])
    layer.topk_step(phys=True)
    torch.cuda.synchronize()
    assert sad.dsa_device_status() == 0
    layer.phys[0, 7] = wl.num_blocks * 64 + 1
    layer.attention_step(d["pool"], d["q"], use_phys=True)
    torch.cuda.synchronize()
    assert sad.dsa_device_status() == sad.DEVERR_POOL_ROW
    assert torch.isfinite(layer.out.float()).all()


def test_rows_beyond_max_rows_per_seq_poison_the_select():
    # two rows of one sequence declared as at most one per sequence: the second is never scored;
    # the select then reports count -1 for every row until the status word is cleared
    wl = synth.Workload("rows", 64, [3000, 1000], [0, 0, 1], [2998, 2999, 999])
    kv, d, batch, layer = _stage(wl, max_rows=1)
    layer.scores_step(d["pool"], d["q_idx"], d["w"])
    layer.topk_step()
    torch.cuda.synchronize()
    assert np.all(layer.count.cpu().numpy() == -1)
    assert torch.all(layer.idx == -1) and torch.all(layer.phys == -1)
    assert sad.dsa_device_status(clear=True) == sad.DEVERR_ROWS_PER_SEQ
    # once cleared, a run within the contract is exact again
    layer2, _, _ = run_gpu(wl)
    assert sad.dsa_device_status() == 0
    check_workload(wl, layer2)
