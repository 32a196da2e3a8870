"""The decode step replayed from a captured HIP graph gives, on every replay,
exactly what the same calls give when launched eagerly, with other eager work
(the same step on another query, which overwrites every output) and
synchronisations between the replays.  Covers the calls the benchmark
captures (the fused query side, the split decode, the fused combine) and the
single-call decodes (one chunk per sequence, and several new tokens per
sequence with their own workspace).
"""
import numpy as np
import pytest
import torch

import mla_latent_kv_32_amd as mla
import synth
from helpers import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    mla.lib()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _check_replays(run, outs):
    """run(k) launches the calls on input set k (0 or 1) into the tensors `outs`."""
    run(0)
    torch.cuda.synchronize()
    ref0 = [_bits(t).clone() for t in outs]
    run(1)
    torch.cuda.synchronize()
    ref1 = [_bits(t).clone() for t in outs]
    assert any(not torch.equal(a, b) for a, b in zip(ref0, ref1)), "the two input sets must differ"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(0)
    for r in range(REPLAYS):
        run(1)                                   # eager work between the replays
        torch.cuda.synchronize()
        for t, ref in zip(outs, ref1):
            assert torch.equal(_bits(t), ref), f"eager step after replay {r - 1}"
        g.replay()
        torch.cuda.synchronize()
        for k, (t, ref) in enumerate(zip(outs, ref0)):
            assert torch.equal(_bits(t), ref), f"replay {r}, output {k}"


def test_graph_replays_of_the_benchmark_step():
    w = synth.gaussian_workload(950, B=4, H=128, seq_lens=[1, 300, 1000, 2048])
    B, H = w["B"], w["H"]
    S = int(w["seq_lens"].max())
    alt = synth.gaussian_workload(951, B=4, H=128, seq_lens=[1, 300, 1000, 2048])
    q_nope = [to_dev_bf16(w["q_nope"]), to_dev_bf16(alt["q_nope"])]
    q_pe = [to_dev_bf16(w["q_pe"]), to_dev_bf16(alt["q_pe"])]
    w_uk, w_uv = to_dev_bf16(w["w_uk"]), to_dev_bf16(w["w_uv"])
    kv_new = to_dev_bf16(w["kv_new"])
    sl, bt = to_dev(w["seq_lens"]), to_dev(w["block_table"])
    cache = to_dev_bf16(w["cache_step"])
    split = mla.mla_decode_split_tokens(B, H, S)
    ws = torch.empty(mla.mla_decode_workspace_bytes(B, H, S, split), dtype=torch.uint8, device="cuda")
    q = torch.empty((B, H, 576), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((B, H, 128), dtype=torch.bfloat16, device="cuda")
    o_lat = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")

    def run(k):
        mla.mla_absorb_q_rope_append(q_nope[k], w_uk, q_pe[k], kv_new, sl, bt, cache, mla.KV_BF16, w["theta"], q)
        mla.mla_decode_partial(q, cache, mla.KV_BF16, bt, sl, S, w["scale"], ws, split_tokens=split)
        mla.mla_decode_combine_absorb_out(ws, sl, S, w_uv, o, o_latent=o_lat, lse=lse, split_tokens=split)

    _check_replays(run, [q, o, o_lat, lse])


@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_FP8])
def test_graph_replays_of_single_call_decodes(kv_dtype):
    lens = [0, 1, 65, 700, 1500]
    w = synth.gaussian_workload(960 + kv_dtype, B=len(lens), H=128, seq_lens=lens, kv_dtype=kv_dtype)
    B, H = w["B"], w["H"]
    S = int(max(lens))
    cache = to_dev_bf16(w["cache_full"]) if kv_dtype == synth.KV_BF16 else to_dev(w["cache_full"])
    sl, bt = to_dev(w["seq_lens"]), to_dev(w["block_table"])
    rng = np.random.default_rng(961)
    q = [to_dev_bf16(w["q_decode"]), to_dev_bf16(synth.f32_to_bf16_bits(
        rng.standard_normal(w["q_decode"].shape, dtype=np.float32)))]
    qm = [to_dev_bf16(synth.multi_token_query(962 + k, B, 3, H)) for k in range(2)]
    split = mla.mla_decode_split_tokens(B, 3 * H, S)
    ws = torch.empty(mla.mla_decode_workspace_bytes(B, 3 * H, S, split), dtype=torch.uint8, device="cuda")
    o1 = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
    l1 = torch.empty((B, H), dtype=torch.float32, device="cuda")
    o3 = torch.empty((B, 3, H, 512), dtype=torch.bfloat16, device="cuda")
    l3 = torch.empty((B, 3, H), dtype=torch.float32, device="cuda")

    def run(k):
        # one chunk per sequence: direct mode, no workspace
        mla.mla_decode_paged(q[k], cache, kv_dtype, bt, sl, S, w["scale"], o1, l1, split_tokens=2048)
        mla.mla_decode_paged_multi(qm[k], cache, kv_dtype, bt, sl, S, w["scale"], o3, l3, split_tokens=split,
                                   workspace=ws)

    _check_replays(run, [o1, l1, o3, l3])
