"""GPU parity of mla_query_from_latent (the decode query from the low-rank
query latent: W_UQ, then W_UK on the nope part, RoPE on the rope part, one
launch) against the fp64 oracle, at the stated bf16 bound
|gpu - ref| <= 2e-3 + 2e-2 |ref|; the cache rows it appends are compared bit
for bit with those of mla_rope_append_cache."""
import numpy as np
import pytest
import torch

import mla_latent_kv_32_amd as mla
import oracle
import synth
from helpers import assert_close, bf16_tensor_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a ROCm device"
    mla.lib()


def run(w, seq_lens, append=None):
    B, H = w["c_q"].shape[0], np.asarray(w["w_uk"]).shape[0]
    q = torch.full((B, H, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    kw = {}
    if append is not None:
        kw = dict(kv_new=append["kv_new"], block_table=append["bt"], kv_cache=append["kv"], kv_dtype=append["dtype"])
    mla.mla_query_from_latent(to_dev_bf16(w["c_q"]), to_dev_bf16(w["w_uq"]), to_dev_bf16(w["w_uk"]),
                              to_dev(np.asarray(seq_lens, np.int32)), w["theta"], q, **kw)
    torch.cuda.synchronize()
    return q


def check(w, seq_lens, q):
    f = oracle.bf16_to_f64
    pos = np.maximum(np.asarray(seq_lens) - 1, 0)
    q_lat, q_rot = oracle.query_from_latent(f(w["c_q"]), f(w["w_uq"]), f(w["w_uk"]), pos, w["theta"])
    got = bf16_tensor_to_f64(q)
    assert_close(got[..., :512], q_lat, what="q_lat")
    assert_close(got[..., 512:], q_rot, what="q_rot")


def test_query_from_latent_full_size():
    """The DeepSeek-V3-shaped workload: c' and W_UQ of its 32 new tokens, all
    128 heads, every (sequence, head) pair."""
    w = synth.workload(2)
    q = run(w, w["seq_lens"])
    check(w, w["seq_lens"], q)


@pytest.mark.parametrize("B,H", [(1, 1), (45, 3), (64, 20), (130, 7)])
def test_query_from_latent_ragged(B, H):
    """Batch tiles of 64 with a ragged last tile, several head counts, empty
    and long sequences (positions up to 40000)."""
    w = synth.query_latent_inputs(1000 + B + H, B, H)
    sl = w["seq_lens"].copy()
    sl[0] = 0
    q = run(w, sl)
    check(w, sl, q)


@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_FP8])
def test_query_from_latent_appends_like_rope_append(kv_dtype):
    """With kv_new, the appended rows equal mla_rope_append_cache's bit for bit."""
    lens = [0, 1, 64, 65, 500, 8192, 3, 129, 4000]
    g = synth.gaussian_workload(1100 + kv_dtype, B=len(lens), H=5, seq_lens=lens, kv_dtype=kv_dtype)
    w = synth.query_latent_inputs(1101, len(lens), 5)
    w["w_uk"] = g["w_uk"]
    fp8 = kv_dtype == synth.KV_FP8
    dev = (lambda x: to_dev(x)) if fp8 else (lambda x: to_dev_bf16(x))
    kv1, kv2 = dev(g["cache_step"]), dev(g["cache_step"])
    bt, sl = to_dev(g["block_table"]), to_dev(g["seq_lens"])
    kvn = to_dev_bf16(g["kv_new"])
    q = run(w, g["seq_lens"], dict(kv_new=kvn, bt=bt, kv=kv1, dtype=kv_dtype))
    check(w, g["seq_lens"], q)
    q2 = torch.full((len(lens), 5, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    mla.mla_rope_append_cache(to_dev_bf16(g["q_pe"]), kvn, sl, bt, kv2, kv_dtype, g["theta"], q2)
    torch.cuda.synchronize()
    assert torch.equal(kv1.view(torch.uint8), kv2.view(torch.uint8))
