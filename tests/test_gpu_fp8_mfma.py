"""GPU parity of mla_decode_paged_fp8_mfma, the fp8-cache decode whose two
products run on fp8 MFMAs over the stored E4M3 codes, against the fp64
oracle (the cache dequantised exactly, code * group scale).

o_latent is held to the fp8-cache bound 2e-3 + 6e-2 |ref| with nothing
added, on every case.  lse: the query enters the scores as two E4M3 terms,
|q - (hi + lo)| <= 2^-8 |q| + 2^-17 max_j |q_j| per element (hi rounds q
scaled into [128, 256) to 4 significant bits, lo the remainder, each to
within half a unit or the subnormal step 2^-9 of the scaled value), the
codes and group scales enter exactly, and the products accumulate in fp32;
a score moves by at most scale * sum_j |dq_j| |c_tj| and lse by at most the
largest such move, on top of the fp32 tolerance of the other decode tests.

The weights enter the value product as two E4M3 terms as well, within 2^-8
of each weight (bf16 weights: 2^-9), so o_latent may move by up to
2^-8 sum_t p_t |c_t| beyond its own rounding.  Only the synthetic stress
case with group scales spread over a 64-fold range, whose large rows can
cancel to small outputs, adds that derived term (twice it, for margin).
"""
import numpy as np
import pytest
import torch

import mla_latent_kv_32_amd as mla
import oracle
import synth
from helpers import FP8_ATOL, FP8_RTOL, assert_close, bf16_tensor_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

LSE_ATOL, LSE_RTOL = 1e-4, 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a ROCm device"
    mla.lib()


def run(w, split_tokens=0, pool=None, table=None, fp8_mfma=True):
    B, H = w["B"], w["H"]
    q = to_dev_bf16(w["q_decode"])
    kv = to_dev(w["cache_full"] if pool is None else pool)
    bt = to_dev(w["block_table"] if table is None else table)
    sl = to_dev(w["seq_lens"])
    o = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    max_len = int(np.max(w["seq_lens"])) if len(w["seq_lens"]) else 0
    if fp8_mfma:
        mla.mla_decode_paged_fp8_mfma(q, kv, bt, sl, max_len, w["scale"], o, lse, split_tokens=split_tokens)
    else:
        mla.mla_decode_paged(q, kv, synth.KV_FP8, bt, sl, max_len, w["scale"], o, lse, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return o, lse


def lse_bound(w, b, heads, c):
    q = oracle.bf16_to_f64(w["q_decode"][b])[list(heads), :512]
    dq = 2.0 ** -8 * np.abs(q) + 2.0 ** -17 * np.abs(q).max(axis=1, keepdims=True)
    return 1.01 * w["scale"] * (dq @ np.abs(c).T).max(axis=1)


def check(w, o, lse, pairs, widen=False):
    for b, heads in pairs:
        heads = list(heads)
        S = int(w["seq_lens"][b])
        got = bf16_tensor_to_f64(o[b, heads])
        if S == 0:
            assert (got == 0).all(), f"b={b}: empty sequence must give zeros"
            assert torch.isneginf(lse[b, heads]).all().item()
            continue
        ref_o, ref_l, mag = oracle.reference_decode(w, b, heads, with_magnitude=True)
        extra = 2.0 ** -7 * mag if widen else 0.0
        assert_close(got, ref_o, FP8_ATOL, FP8_RTOL, extra=extra, what=f"o_latent b={b} S={S}")
        rows = oracle.gather_rows(w["cache_full"], w["block_table"], b, S)
        c, _ = oracle.rows_to_latent_rope(rows, kv_fp8=True)
        assert_close(lse[b, heads].cpu().numpy(), ref_l, LSE_ATOL, LSE_RTOL, extra=lse_bound(w, b, heads, c),
                     what=f"lse b={b}")


@pytest.mark.parametrize("H", [16, 40, 128, 200])
def test_fp8_mfma_ragged_lengths_and_heads(H):
    """Partial last pages, page-sized chunks, two head groups (200 heads, the
    second partly past H), every split size class; all heads at the stated
    bound."""
    lens = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 300, 1000, 2100]
    w = synth.gaussian_workload(170 + H, B=len(lens), H=H, seq_lens=lens, kv_dtype=synth.KV_FP8)
    for split in [0, 64, 256]:
        o, lse = run(w, split_tokens=split)
        check(w, o, lse, [(b, range(H)) for b in range(len(lens))])


def _scale_rope_pow2(w, picks):
    """Copy of w whose rows (b, token) have their bf16 rotary keys multiplied
    by 2^k exactly (exponent field + k on the nonzero entries): those rows'
    scores jump while their latent values stay as drawn."""
    pool = w["cache_full"].copy()
    for b, t, k in picks:
        row = pool[w["block_table"][b][t // 64], t % 64]
        kr = row[512:640].copy().view(np.uint16)
        nz = (kr & 0x7F80) != 0
        kr[nz] = kr[nz] + np.uint16(k << 7)
        row[512:640] = kr.view(np.uint8)
    return dict(w, cache_full=pool)


@pytest.mark.parametrize("H", [16, 128])
def test_fp8_mfma_running_max_jumps(H):
    """Late rows whose scores pass the running max by tens of log2 units
    (rotary keys scaled by up to 2^6): the value accumulators are rescaled
    and the weights of the other rows of such a block fall far below the
    block's largest."""
    lens = [700, 1500, 333]
    w = synth.gaussian_workload(150 + H, B=len(lens), H=H, seq_lens=lens, kv_dtype=synth.KV_FP8)
    w = _scale_rope_pow2(w, [(0, 300, 3), (0, 650, 5), (1, 40, 2), (1, 1200, 6), (2, 332, 4)])
    for split in [0, 256, 1024]:
        o, lse = run(w, split_tokens=split)
        check(w, o, lse, [(b, range(H)) for b in range(len(lens))])


def test_fp8_mfma_group_scale_spread():
    """Group scales spread over 2^-3 .. 2^3 times the drawn ones, per row and
    group: each block's per-group maximum E_g and the factors f_t,g vary
    over a 64-fold range within a block (held to the bound plus the
    weights' two-term rounding term)."""
    lens = [64, 129, 1000, 3000]
    w = synth.gaussian_workload(160, B=len(lens), H=128, seq_lens=lens, kv_dtype=synth.KV_FP8)
    pool = w["cache_full"].copy()
    rng = np.random.default_rng(161)
    sc = pool[..., 640:656].copy().view(np.float32)
    sc *= np.exp2(rng.integers(-3, 4, size=sc.shape)).astype(np.float32)
    pool[..., 640:656] = sc.view(np.uint8)
    w = dict(w, cache_full=pool)
    for split in [0, 512]:
        o, lse = run(w, split_tokens=split)
        check(w, o, lse, [(b, range(128)) for b in range(len(lens))], widen=True)


def test_fp8_mfma_ignores_rows_past_the_end():
    """Unwritten rows of a page filled with all-ones bytes (NaN codes and
    scales): the same bits as on the clean pool."""
    lens = [1, 33, 64, 65, 100, 511, 777]
    w = synth.gaussian_workload(190, B=len(lens), H=64, seq_lens=lens, kv_dtype=synth.KV_FP8)
    pool = w["cache_full"].copy()
    used = np.zeros(pool.shape[:2], bool)
    for b, S in enumerate(lens):
        for t in range(S):
            used[w["block_table"][b, t // 64], t % 64] = True
    pool[~used] = 0xFF
    for split in [0, 128]:
        o1, l1 = run(w, split_tokens=split)
        o2, l2 = run(w, split_tokens=split, pool=pool)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"split={split}"
        assert torch.equal(l1, l2)


def test_fp8_mfma_page_permutation_bit_identical():
    w = synth.gaussian_workload(191, B=5, H=128, seq_lens=[1, 200, 513, 1000, 2048], kv_dtype=synth.KV_FP8)
    o1, l1 = run(w, split_tokens=256)
    pool2, table2 = synth.permute_pages(w, 192)
    o2, l2 = run(w, split_tokens=256, pool=pool2, table=table2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_fp8_mfma_full_size():
    """Workload 4 (B=128, H=128, 8192 tokens, 688 MB of packed rows) in the
    planner's launch configuration: every head of 12 sequences spread over
    the batch at the fp8 bound, nothing added, and every output within that
    bound of the expanding decoder's."""
    w = synth.workload(4)
    o, lse = run(w)
    assert not torch.isnan(o.float()).any().item()
    check(w, o, lse, [(b, range(w["H"])) for b in (0, 1, 15, 31, 32, 63, 64, 77, 95, 100, 126, 127)])
    o2, _ = run(w, fp8_mfma=False)
    a, r = o.float(), o2.float()
    assert ((a - r).abs() <= 2 * (FP8_ATOL + FP8_RTOL * r.abs())).all().item()
