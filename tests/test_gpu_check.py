"""mla_check_metadata on the GPU: it counts exactly the out-of-range lengths
and the out-of-range page ids among the pages each sequence uses; ids in
unused table slots are ignored."""
import numpy as np
import pytest
import torch

from mla_latent_kv_29_amd import _lib as L
from mla_latent_kv_29_amd import inputs
from gpu_common import DEV

pytestmark = pytest.mark.gpu


def run(lengths, table, num_pages, dims=inputs.V3_DIMS):
    d = L.make_dims(dims)
    pages = torch.zeros((1, 64), dtype=torch.uint8, device=DEV)
    cache = L.cache_struct(pages, L.MLA_BF16, num_pages)
    bt = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(DEV)
    sl = torch.from_numpy(np.asarray(lengths, dtype=np.int32)).to(DEV)
    bad = torch.full((2,), -7, dtype=torch.int32, device=DEV)
    L.mla_check_metadata(d, cache, bt, table.shape[1], sl, len(lengths), bad)
    torch.cuda.synchronize()
    return bad.cpu().tolist()


def test_valid_ragged_shuffled_table_has_no_findings():
    lengths = inputs.seqlens(("uniform", 1, 32768), 128, 0, 2)
    table, pool = inputs.block_table(lengths, 64, "shuffled", 0, 2)
    assert run(lengths, table, pool) == [0, 0]


def test_bad_ids_in_used_pages_are_counted_and_unused_slots_ignored():
    lengths = np.array([130, 64, 1, 0], dtype=np.int64)   # pages used: 3, 1, 1, 0
    table, pool = inputs.block_table(lengths, 64, "inorder", 0, 0)
    table = np.array(table)
    mp = table.shape[1]
    assert mp == 3
    t = table.copy()
    t[0, 2] = pool           # last used page of sequence 0: one past the pool
    t[2, 0] = -1             # the only page of sequence 2
    t[1, 1] = 10 ** 6        # beyond sequence 1's one page: unused, ignored
    t[3, :] = -5             # the empty sequence uses no page
    assert run(lengths, t, pool) == [0, 2]


def test_out_of_range_lengths_are_counted():
    lengths = np.array([192, -3, 193, 5], dtype=np.int64)  # 3 pages of 64: 192 fits, 193 does not
    table = np.arange(12, dtype=np.int32).reshape(4, 3)
    assert run(lengths, table, 12) == [2, 0]
    table[2, 2] = 99  # the over-long sequence is checked over all of its table row
    assert run(lengths, table, 12) == [2, 1]


def test_empty_batch_writes_zeros():
    table = np.zeros((1, 2), dtype=np.int32)
    assert run(np.zeros(0, dtype=np.int64), table, 4) == [0, 0]
