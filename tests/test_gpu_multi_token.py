"""GPU parity of the multi-token decode (q_len new tokens per sequence, causal
among themselves) against the fp64 oracle, and against single-token decodes
of the matching virtual sequences.

Tolerances are those of the single-token decode: |gpu - ref| <= 2e-3 +
2e-2 |ref| (bf16 cache) or 2e-3 + 6e-2 |ref| (fp8 cache).  The full-size
workload is held to that bound as stated; the synthetic ragged edge cases
(a few N(0,1) rows whose weighted sums can cancel to tiny values) add the
bf16 rounding of the softmax weights, 2^-8 sum_t p_t |c_t|.
"""
import numpy as np
import pytest
import torch

import mla_latent_kv_32_amd as mla
import oracle
import synth
from helpers import (BF16_ATOL, BF16_RTOL, FP8_ATOL, FP8_RTOL, assert_close, bf16_tensor_to_f64,
                     to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu

LSE_ATOL, LSE_RTOL = 1e-4, 1e-5
P_ROUNDING = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a ROCm device"
    mla.lib()


def _kv(w, pool=None):
    pool = w["cache_full"] if pool is None else pool
    return to_dev_bf16(pool) if w["kv_dtype"] == synth.KV_BF16 else to_dev(pool)


def run_multi(w, qm, split_tokens=0):
    B, q_len, H = qm.shape[:3]
    o = torch.full((B, q_len, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, q_len, H), float("nan"), dtype=torch.float32, device="cuda")
    max_len = int(np.max(w["seq_lens"])) if len(w["seq_lens"]) else 0
    mla.mla_decode_paged_multi(to_dev_bf16(qm), _kv(w), w["kv_dtype"], to_dev(w["block_table"]),
                               to_dev(w["seq_lens"]), max_len, w["scale"], o, lse, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return o, lse


def run_virtual(w, qm, split_tokens):
    """Single-token decodes of the B * q_len virtual sequences (b, j): length
    seq_lens[b] - q_len + j + 1 (clamped at 0), block-table row b."""
    B, q_len, H = qm.shape[:3]
    lens = np.maximum(0, w["seq_lens"][:, None] - q_len + 1 + np.arange(q_len)[None, :]).astype(np.int32)
    table = np.repeat(w["block_table"], q_len, axis=0)
    o = torch.full((B * q_len, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B * q_len, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_decode_paged(to_dev_bf16(qm.reshape(B * q_len, H, 576)), _kv(w), w["kv_dtype"], to_dev(table),
                         to_dev(lens.reshape(-1)), int(w["seq_lens"].max()), w["scale"], o, lse,
                         split_tokens=split_tokens)
    torch.cuda.synchronize()
    return o.view(B, q_len, H, 512), lse.view(B, q_len, H)


def check_multi(w, qm, o, lse, pairs, widen=True):
    """pairs: (b, heads); every query token j of the sequence is checked.
    widen=False holds o_latent to the stated bound with nothing added."""
    fp8 = w["kv_dtype"] == synth.KV_FP8
    tol = (FP8_ATOL, FP8_RTOL) if fp8 else (BF16_ATOL, BF16_RTOL)
    q_len = qm.shape[1]
    for b, heads in pairs:
        heads = list(heads)
        ref_o, ref_l = oracle.reference_decode_multi(w, qm, b, heads)
        S = int(w["seq_lens"][b])
        rows = oracle.gather_rows(w["cache_full"], w["block_table"], b, S)
        c, kr = oracle.rows_to_latent_rope(rows, fp8)
        got = bf16_tensor_to_f64(o[b][:, heads])
        got_l = lse[b][:, heads].cpu().numpy()
        for j in range(q_len):
            n = S - q_len + 1 + j
            if n <= 0:
                assert (got[j] == 0).all(), f"b={b} j={j}: a query that sees no row gives zeros"
                assert np.isneginf(got_l[j]).all(), f"b={b} j={j}: lse must be -inf"
                continue
            q = oracle.bf16_to_f64(qm[b, j])[heads]
            _, _, mag = oracle.decode_absorbed(q[:, :512], q[:, 512:], c[:n], kr[:n], w["scale"],
                                               with_magnitude=True)
            extra = P_ROUNDING * mag if widen else 0.0
            assert_close(got[j], ref_o[j], *tol, extra=extra, what=f"o_latent b={b} j={j} S={S}")
            lse_extra = 0.0
            if fp8:   # expansion to bf16 moves each score by at most scale 2^-9 sum |q||c|
                lse_extra = 1.01 * w["scale"] * 2.0 ** -9 * (np.abs(q[:, :512]) @ np.abs(c[:n]).T).max(axis=1)
            assert_close(got_l[j], ref_l[j], LSE_ATOL, LSE_RTOL, extra=lse_extra, what=f"lse b={b} j={j}")


LENS = [0, 1, 2, 3, 4, 31, 32, 33, 34, 63, 64, 65, 66, 97, 300, 513, 1000]


@pytest.mark.parametrize("H,q_len", [(16, 2), (16, 4), (8, 3), (128, 2), (40, 4), (2, 32), (8, 32)])
@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_FP8])
def test_multi_token_matches_oracle(H, q_len, kv_dtype):
    """Ragged lengths around block and chunk edges (and sequences shorter
    than q_len) with query rows on both decoders (q_len * H <= 64: two waves
    per SIMD; above: one wave per SIMD, 128 rows per workgroup), up to the
    largest q_len (32)."""
    w = synth.gaussian_workload(200 + H + 10 * q_len + kv_dtype, B=len(LENS), H=H, seq_lens=LENS,
                                kv_dtype=kv_dtype)
    qm = synth.multi_token_query(300 + H + q_len, len(LENS), q_len, H)
    heads = range(H) if H <= 40 else [0, 1, 31, 32, 77, 127]
    for split in [0, 64, 256]:
        o, lse = run_multi(w, qm, split_tokens=split)
        check_multi(w, qm, o, lse, [(b, heads) for b in range(len(LENS))])


# (H, q_len) pairs whose multi-token rows and single-token heads fall on the
# same decoder (q_len * H and H both <= 64, or both > 64)
@pytest.mark.parametrize("H,q_len,kv_dtype", [(16, 2, synth.KV_BF16), (128, 2, synth.KV_BF16),
                                              (128, 3, synth.KV_FP8), (16, 4, synth.KV_FP8),
                                              (32, 2, synth.KV_BF16)])
def test_multi_token_equals_virtual_sequences(H, q_len, kv_dtype):
    """Each query row's arithmetic is that of the single-token decode of its
    prefix: equal values (zeros of either sign) to mla_decode_paged on the
    virtual sequences, for the same chunking."""
    lens = [1, 2, 5, 33, 64, 65, 130, 700, 1025]
    w = synth.gaussian_workload(400 + H + q_len, B=len(lens), H=H, seq_lens=lens, kv_dtype=kv_dtype)
    qm = synth.multi_token_query(401 + H, len(lens), q_len, H)
    for split in [64, 256, 2048]:
        o1, l1 = run_multi(w, qm, split_tokens=split)
        o2, l2 = run_virtual(w, qm, split_tokens=split)
        assert torch.equal(o1.float(), o2.float()), f"split={split}"
        assert torch.equal(l1, l2), f"split={split}"


def test_multi_token_single_is_the_decode():
    w = synth.gaussian_workload(500, B=6, H=128, seq_lens=[0, 1, 64, 100, 1000, 3000])
    qm = w["q_decode"][:, None]
    for split in [0, 256]:
        o1, l1 = run_multi(w, qm, split_tokens=split)
        o2 = torch.full((6, 128, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        l2 = torch.full((6, 128), float("nan"), dtype=torch.float32, device="cuda")
        mla.mla_decode_paged(to_dev_bf16(w["q_decode"]), _kv(w), w["kv_dtype"], to_dev(w["block_table"]),
                             to_dev(w["seq_lens"]), 3000, w["scale"], o2, l2, split_tokens=split)
        torch.cuda.synchronize()
        assert torch.equal(o1[:, 0].view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1[:, 0], l2)


def test_multi_token_full_size():
    """Two new tokens per sequence on the 32 x 4096-token, 128-head workload
    in the planner's launch configuration: every head of both tokens of four
    sequences against the oracle at the stated bf16 bound (nothing added),
    and every row against the virtual-sequence decodes for the same chunking."""
    w = synth.workload(2)
    B, H = w["B"], w["H"]
    qm = synth.multi_token_query(600, B, 2, H)
    o, lse = run_multi(w, qm)
    assert not torch.isnan(o.float()).any().item()
    check_multi(w, qm, o, lse, [(b, range(H)) for b in (0, 9, 17, 31)], widen=False)
    split = mla.mla_decode_split_tokens(B, 2 * H, int(w["seq_lens"].max()))
    o2, l2 = run_virtual(w, qm, split_tokens=split)
    assert torch.equal(o.float(), o2.float()) and torch.equal(lse, l2)
