"""The decode entry point that allocates nothing (mla_decode_paged_noalloc)
against mla_decode_paged, through the C ABI: two calls in a row on the same
GPU, the second with a smaller input (the fixed scratch buffer then holds the
first call's partials), each equal bit for bit to the allocating call and
within the bf16 bound of the oracle on sampled heads; a request whose
partials exceed the buffer is refused before any launch."""
import numpy as np
import pytest
import torch

import mla_latent_kv_32_amd as mla
import oracle
import synth
from helpers import assert_close, bf16_tensor_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _inputs(w):
    return (to_dev_bf16(w["q_decode"]), to_dev_bf16(w["cache_full"]), to_dev(w["block_table"]),
            to_dev(w["seq_lens"]))


def _both(w, split):
    B, H = w["B"], w["H"]
    q, kv, bt, sl = _inputs(w)
    max_len = int(w["seq_lens"].max())
    outs = []
    for fn in (mla.mla_decode_paged_noalloc, mla.mla_decode_paged):
        o = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
        fn(q, kv, mla.KV_BF16, bt, sl, max_len, w["scale"], o, lse, split_tokens=split)
        outs.append((o, lse))
    torch.cuda.synchronize()
    return outs


def _check(w, outs, pairs):
    (o1, l1), (o2, l2) = outs
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    for b, heads in pairs:
        ref, _ = oracle.reference_decode(w, b, heads)
        assert_close(bf16_tensor_to_f64(o1[b, heads]), ref, what=f"noalloc o_latent b={b}")


def test_noalloc_decode_equals_allocating_decode_twice():
    assert torch.cuda.is_available()
    # first call: 32 sequences x 128 heads, up to 4096 tokens, planner's split (partials ~33 MB)
    lens = [4096 - 97 * i for i in range(32)]
    w1 = synth.gaussian_workload(900, B=32, H=128, seq_lens=lens)
    _check(w1, _both(w1, 0), [(0, [0, 127]), (31, [64])])
    # second call, smaller: 3 sequences x 16 heads in 256-token chunks
    w2 = synth.gaussian_workload(901, B=3, H=16, seq_lens=[5, 700, 1500])
    _check(w2, _both(w2, 256), [(b, list(range(16))) for b in range(3)])


def test_noalloc_refuses_requests_beyond_the_buffer():
    # 64 sequences x 128 heads x 128 chunks of 256 tokens: 1 GiB of partials
    B, H, max_len = 64, 128, 32768
    need = mla.mla_decode_workspace_bytes(B, H, max_len, 256)
    assert need > mla.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 64, 576), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, max_len // 64), dtype=torch.int32, device="cuda")
    sl = torch.zeros((B,), dtype=torch.int32, device="cuda")
    o = torch.zeros((B, H, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MLAError) as e:
        mla.mla_decode_paged_noalloc(q, kv, mla.KV_BF16, bt, sl, max_len, 0.07, o, split_tokens=256)
    assert e.value.status == -5
