"""GPU checks of mla_validate_paging: a valid workload's tables pass, and
lengths or page ids planted past the bounds (on the host, in the tables
handed over; the check only reads them) are counted and the first flagged
sequence reported.  Expected values come from the planted positions."""
import numpy as np
import pytest
import torch

import mla_latent_kv_32_amd as mla
import synth
from helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    mla.lib()


def check(seq_lens, block_table, max_len, num_blocks):
    bad = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    first = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    mla.mla_validate_paging(to_dev(np.asarray(seq_lens, np.int32)), to_dev(np.asarray(block_table, np.int32)),
                            max_len, num_blocks, bad, first)
    torch.cuda.synchronize()
    return int(bad.item()), int(first.item())


def test_valid_workloads_pass():
    for cfg in (1, 3):
        w = synth.workload(cfg)
        assert check(w["seq_lens"], w["block_table"], int(w["seq_lens"].max()), w["num_blocks"]) == (0, -1)
    w = synth.gaussian_workload(5, B=5, H=4, seq_lens=[0, 1, 64, 65, 700])
    assert check(w["seq_lens"], w["block_table"], 700, w["num_blocks"]) == (0, -1)


def test_planted_violations_are_counted():
    B, mb, nb = 40, 8, 64
    rng = np.random.default_rng(7)
    lens = rng.integers(0, mb * 64 + 1, B).astype(np.int32)
    table = rng.integers(0, nb, (B, mb)).astype(np.int32)
    max_len = int(lens.max())
    assert check(lens, table, max_len, nb) == (0, -1)
    # pages past a sequence's last page are never looked at
    t2 = table.copy()
    for b in range(B):
        t2[b, (lens[b] + 63) // 64:] = -7
    assert check(lens, t2, max_len, nb) == (0, -1)
    # planted: negative length (b=33), length past max_len (b=21), page id past
    # the pool (b=9, its last page in use), negative page id (b=17, first page)
    l3, t3 = lens.copy(), table.copy()
    l3[33] = -1
    l3[21] = max_len + 1
    l3[9], l3[17] = 130, 5
    t3[9, 2] = nb
    t3[17, 0] = -1
    assert check(l3, t3, max_len + 0, nb) == (4, 9)
    # length past the table row (max_blocks_per_seq * 64) with a large max_len
    l4 = lens.copy()
    l4[3] = mb * 64 + 1
    assert check(l4, table, mb * 64 + 100, nb) == (1, 3)


def test_many_sequences_and_pages():
    """More sequences than waves and more pages than lanes per sequence."""
    B, mb, nb = 300, 200, 5000
    rng = np.random.default_rng(8)
    lens = rng.integers(1, mb * 64 + 1, B).astype(np.int32)
    table = rng.integers(0, nb, (B, mb)).astype(np.int32)
    assert check(lens, table, mb * 64, nb) == (0, -1)
    bad_rows = [299, 150, 64, 65]
    for b in bad_rows:
        lens[b] = mb * 64
        table[b, mb - 1] = nb + 3       # the last page, lane 199 % 64 of the scan
    assert check(lens, table, mb * 64, nb) == (len(bad_rows), min(bad_rows))
