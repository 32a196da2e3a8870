"""GPU parity: every entry point of libmla.so against the fp64 oracle.

Inputs come from the seeded generators in synth/; expected values from
oracle/ only.  Floating-point outputs must satisfy |gpu - ref| <= 2e-3 +
2e-2 |ref| elementwise (bf16 cache) or 2e-3 + 6e-2 |ref| (fp8 cache);
copies, fp8 codes and scales are compared bit for bit.  At the full
DeepSeek-V3-shaped size the GPU runs the whole batch in the benchmark's
launch configuration and the oracle checks sampled (sequence, head) pairs.
"""
import math

import numpy as np
import pytest
import torch

import mla_latent_kv_32_amd as mla
import oracle
import synth
from helpers import (BF16_ATOL, BF16_RTOL, FP8_ATOL, FP8_RTOL, assert_close, bf16_tensor_to_f64,
                     to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu

# lse is formed from fp32 scores of exact bf16 products and unrounded fp32
# softmax weights: a few fp32 ulps of the 576-term dot products and of exp2.
LSE_ATOL, LSE_RTOL = 1e-4, 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a ROCm device"
    mla.lib()


def bf(t):
    return bf16_tensor_to_f64(t)


def nan_bf16(*shape):
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")


def run_decode(w, split_tokens=0, pool=None, table=None, with_lse=True):
    B, H = w["B"], w["H"]
    q = to_dev_bf16(w["q_decode"])
    pool = w["cache_full"] if pool is None else pool
    kv = to_dev_bf16(pool) if w["kv_dtype"] == synth.KV_BF16 else to_dev(pool)
    bt = to_dev(w["block_table"] if table is None else table)
    sl = to_dev(w["seq_lens"])
    o = nan_bf16(B, H, 512)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda") if with_lse else None
    max_len = int(np.max(w["seq_lens"])) if len(w["seq_lens"]) else 0
    mla.mla_decode_paged(q, kv, w["kv_dtype"], bt, sl, max_len, w["scale"], o, lse, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return o, lse


# Rounding the softmax weights P to bf16 for the P.V product perturbs each
# weight by at most 2^-9 relative, so o_latent may move by up to
# 2^-9 sum_t p_t |c_t| beyond the output's own rounding.  For the configured
# workloads this stays inside the stated bound; synthetic edge cases with a
# handful of O(1) rows can cancel to tiny outputs, and for them the bound is
# widened by this derived term (twice it, for margin).
P_ROUNDING = 2.0 ** -8


# fp8 cache: the kernel expands code * scale to bf16 before the score
# product, which moves latent value c_tj by at most 2^-9 |c_tj|.  A score
# then moves by at most scale * 2^-9 * sum_j |q_j| |c_tj|, and lse (a smooth
# maximum of the scores) by at most the largest such move over the tokens.
def fp8_lse_bound(w, b, heads):
    S = int(w["seq_lens"][b])
    rows = oracle.gather_rows(w["cache_full"], w["block_table"], b, S)
    c, _ = oracle.rows_to_latent_rope(rows, kv_fp8=True)
    q = oracle.bf16_to_f64(w["q_decode"][b])[list(heads), :512]
    return w["scale"] * 2.0 ** -9 * (np.abs(q) @ np.abs(c).T).max(axis=1)


def check_decode(w, o, lse, pairs, tol=None, p_rounding_term=False):
    """pairs: iterable of (b, heads).  The fp8 cache is held to the fp8 bound."""
    fp8 = w["kv_dtype"] == synth.KV_FP8
    if tol is None:
        tol = (FP8_ATOL, FP8_RTOL) if fp8 else (BF16_ATOL, BF16_RTOL)
    for b, heads in pairs:
        heads = list(heads)
        ref_o, ref_l, mag = oracle.reference_decode(w, b, heads, with_magnitude=True)
        got = bf(o[b, heads])
        S = int(w["seq_lens"][b])
        if S == 0:
            assert (got == 0).all(), f"b={b}: empty sequence must give zeros"
            if lse is not None:
                assert torch.isneginf(lse[b, heads]).all().item()
            continue
        extra = P_ROUNDING * mag if p_rounding_term else 0.0
        assert_close(got, ref_o, *tol, extra=extra, what=f"o_latent b={b} S={S}")
        if lse is not None:
            lse_extra = 1.01 * fp8_lse_bound(w, b, heads) if fp8 else 0.0
            assert_close(lse[b, heads].cpu().numpy(), ref_l, LSE_ATOL, LSE_RTOL, extra=lse_extra, what=f"lse b={b}")


# --------------------------------------------------------------------- K1
@pytest.mark.parametrize("cfg", [1, 2])
def test_absorb_q(cfg):
    w = synth.workload(cfg)
    B, H = w["B"], w["H"]
    q = nan_bf16(B, H, 576)
    mla.mla_absorb_q(to_dev_bf16(w["q_nope"]), to_dev_bf16(w["w_uk"]), q)
    torch.cuda.synchronize()
    ref = oracle.absorb_q(oracle.bf16_to_f64(w["q_nope"]), oracle.bf16_to_f64(w["w_uk"]))
    assert_close(bf(q[..., :512]), ref, what=f"q_lat cfg{cfg}")
    assert torch.isnan(q[..., 512:].float()).all().item(), "rotary columns must be left untouched"


def test_absorb_q_ragged_batch():
    B, H = 45, 3
    qn = synth.random_bf16(101, (B, H, 128))
    wk = synth.random_bf16(102, (H, 128, 512), 1 / math.sqrt(512))
    q = nan_bf16(B, H, 576)
    mla.mla_absorb_q(to_dev_bf16(qn), to_dev_bf16(wk), q)
    torch.cuda.synchronize()
    ref = oracle.absorb_q(oracle.bf16_to_f64(qn), oracle.bf16_to_f64(wk))
    assert_close(bf(q[..., :512]), ref, what="q_lat ragged")


# --------------------------------------------------------------------- K5
@pytest.mark.parametrize("B,H", [(32, 128), (8, 16), (45, 3)])
def test_absorb_out(B, H):
    ol = synth.random_bf16(201 + B, (B, H, 512), 0.05)
    wv = synth.random_bf16(202 + H, (H, 512, 128), 1 / math.sqrt(512))
    o = nan_bf16(B, H, 128)
    mla.mla_absorb_out(to_dev_bf16(ol), to_dev_bf16(wv), o)
    torch.cuda.synchronize()
    ref = oracle.absorb_out(oracle.bf16_to_f64(ol), oracle.bf16_to_f64(wv))
    assert_close(bf(o), ref, what=f"o B={B} H={H}")


# --------------------------------------------------------------------- K2
def _append_and_check(w):
    B, H = w["B"], w["H"]
    fp8 = w["kv_dtype"] == synth.KV_FP8
    pool0 = w["cache_step"]
    kv = to_dev(pool0) if fp8 else to_dev_bf16(pool0)
    q = nan_bf16(B, H, 576)
    mla.mla_rope_append_cache(to_dev_bf16(w["q_pe"]), to_dev_bf16(w["kv_new"]), to_dev(w["seq_lens"]),
                              to_dev(w["block_table"]), kv, w["kv_dtype"], w["theta"], q)
    torch.cuda.synchronize()
    got_q = bf(q[..., 512:])
    pool = kv.cpu().numpy() if fp8 else kv.cpu().view(torch.int16).numpy().view(np.uint16)
    touched = np.zeros(pool.shape[:2], bool)
    for b in range(B):
        S = int(w["seq_lens"][b])
        pos = max(S - 1, 0)
        ref_q = oracle.rope(oracle.bf16_to_f64(w["q_pe"][b]), pos, w["theta"])
        assert_close(got_q[b], ref_q, what=f"q_rot b={b}")
        if S == 0:
            continue
        page, slot = w["block_table"][b, pos // 64], pos % 64
        touched[page, slot] = True
        row = pool[page, slot]
        new = w["kv_new"][b]
        ref_kr = oracle.rope(oracle.bf16_to_f64(new[512:]), pos, w["theta"])
        if fp8:
            codes, scales = oracle.fp8_quantize_latent(new[:512])
            np.testing.assert_array_equal(row[:512], codes, err_msg=f"fp8 codes b={b}")
            np.testing.assert_array_equal(row[640:656].view(np.float32), scales, err_msg=f"fp8 scales b={b}")
            got_kr = oracle.bf16_to_f64(row[512:640].view(np.uint16))
        else:
            np.testing.assert_array_equal(row[:512], new[:512], err_msg=f"latent copy b={b}")
            got_kr = oracle.bf16_to_f64(row[512:])
        assert_close(got_kr, ref_kr, what=f"k_rot b={b}")
    np.testing.assert_array_equal(pool[~touched], pool0[~touched], err_msg="rows other than the appended ones changed")


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_rope_append_bf16(cfg):
    _append_and_check(synth.workload(cfg))


def test_rope_append_edge_positions():
    # empty slot, first token, page boundaries, long positions (angles in fp64)
    lens = [0, 1, 2, 63, 64, 65, 128, 4096, 32768, 100000]
    _append_and_check(synth.gaussian_workload(7, B=len(lens), H=5, seq_lens=lens))


def test_rope_append_fp8():
    lens = [0, 1, 64, 65, 500, 8192, 3, 129]
    w = synth.gaussian_workload(8, B=len(lens), H=4, seq_lens=lens, kv_dtype=synth.KV_FP8)
    # one all-zero latent group (scale 1, zero codes) and one with large values
    w = dict(w)
    kvn = w["kv_new"].copy()
    kvn[1, 128:256] = 0
    kvn[2, :128] = synth.f32_to_bf16_bits(np.linspace(-3000, 3000, 128, dtype=np.float32))
    w["kv_new"] = kvn
    _append_and_check(w)


def _fused_query_cases():
    lens45 = [0, 1, 2, 63, 64, 65, 100000] + [int(x) for x in np.arange(38) * 97 + 5]
    return [synth.workload(1), synth.workload(2),
            synth.gaussian_workload(60, B=45, H=3, seq_lens=lens45),
            synth.gaussian_workload(61, B=9, H=20, seq_lens=[0, 1, 64, 65, 500, 8192, 3, 129, 4000],
                                    kv_dtype=synth.KV_FP8)]


@pytest.mark.parametrize("case", range(4))
def test_absorb_q_rope_append_fused_equals_separate(case):
    """The one-launch query side gives exactly what mla_absorb_q + mla_rope_append_cache give."""
    w = _fused_query_cases()[case]
    B, H = w["B"], w["H"]
    key = "cache_step" if "cache_step" in w else "cache_full"
    pool = w[key]
    dev = (lambda x: to_dev_bf16(x)) if w["kv_dtype"] == synth.KV_BF16 else (lambda x: to_dev(x))
    sl, bt = to_dev(w["seq_lens"]), to_dev(w["block_table"])
    qn, wuk = to_dev_bf16(w["q_nope"]), to_dev_bf16(w["w_uk"])
    qpe, kvn = to_dev_bf16(w["q_pe"]), to_dev_bf16(w["kv_new"])
    q1, kv1 = nan_bf16(B, H, 576), dev(pool)
    mla.mla_absorb_q(qn, wuk, q1)
    mla.mla_rope_append_cache(qpe, kvn, sl, bt, kv1, w["kv_dtype"], w["theta"], q1)
    q2, kv2 = nan_bf16(B, H, 576), dev(pool)
    mla.mla_absorb_q_rope_append(qn, wuk, qpe, kvn, sl, bt, kv2, w["kv_dtype"], w["theta"], q2)
    torch.cuda.synchronize()
    assert torch.equal(q1.view(torch.int16), q2.view(torch.int16))
    assert torch.equal(kv1.view(torch.uint8), kv2.view(torch.uint8))


# --------------------------------------------------------------------- K3/K4
def test_decode_workload1_all_heads():
    w = synth.workload(1)
    for split in [0, 1024, 64, 320]:
        o, lse = run_decode(w, split_tokens=split)
        check_decode(w, o, lse, [(b, range(w["H"])) for b in range(w["B"])])


def test_decode_workload2_all_pairs():
    """The DeepSeek-V3-shaped decode (32 sequences x 4096 tokens, 128 heads) in
    the benchmark's launch configuration: every (sequence, head) pair against
    the oracle at the stated bf16 bound, nothing added to it."""
    w = synth.workload(2)
    o, lse = run_decode(w, split_tokens=0)
    assert torch.isfinite(o.float()).all().item() and torch.isfinite(lse).all().item()
    check_decode(w, o, lse, [(b, range(w["H"])) for b in range(w["B"])])


def test_decode_workload3_split256():
    w = synth.workload(3)
    o, lse = run_decode(w, split_tokens=256)
    check_decode(w, o, lse, [(b, [0, 5, 64, 127]) for b in range(w["B"])])


@pytest.mark.parametrize("H", [1, 16, 20, 32, 48, 64, 100, 128, 200, 256])
def test_decode_ragged_lengths_and_heads(H):
    """Every workgroup shape; above 128 heads, several 128-head groups per
    chunk (200: the second group partly past H, one wave of it entirely)."""
    lens = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 300, 1000]
    w = synth.gaussian_workload(30 + H, B=len(lens), H=H, seq_lens=lens)
    for split in [0, 64, 128]:
        o, lse = run_decode(w, split_tokens=split)
        check_decode(w, o, lse, [(b, range(H)) for b in range(len(lens))], p_rounding_term=True)


def _scale_rows_pow2(w, picks):
    """Copy of w whose cached rows (b, token) are multiplied by 2^k exactly
    (bf16 exponent field + k; the N(0,1) entries are normal numbers)."""
    pool = w["cache_full"].copy()
    for b, t, k in picks:
        row = pool[w["block_table"][b][t // 64], t % 64]
        nz = (row & 0x7F80) != 0
        row[nz] = row[nz] + np.uint16(k << 7)
    return dict(w, cache_full=pool)


@pytest.mark.parametrize("H", [16, 128])
def test_decode_running_max_jumps(H):
    """Late tokens whose scores exceed the running max by tens of log2 units:
    exercises the rescale of the value accumulators (lazy and forced)."""
    lens = [700, 1500, 333]
    w = synth.gaussian_workload(50 + H, B=len(lens), H=H, seq_lens=lens)
    w = _scale_rows_pow2(w, [(0, 300, 3), (0, 650, 5), (1, 40, 2), (1, 1200, 6), (2, 332, 4)])
    for split in [0, 256, 1024]:
        o, lse = run_decode(w, split_tokens=split)
        check_decode(w, o, lse, [(b, range(H)) for b in range(len(lens))], p_rounding_term=True)


def test_decode_without_lse_and_all_empty():
    w = synth.gaussian_workload(40, B=3, H=16, seq_lens=[0, 0, 0])
    o, _ = run_decode(w, with_lse=False)
    assert (o.float() == 0).all().item()


def test_decode_long_sequence_many_splits():
    w = synth.gaussian_workload(41, B=1, H=128, seq_lens=[140000])
    o, lse = run_decode(w, split_tokens=0)
    check_decode(w, o, lse, [(0, range(128))])


def test_decode_page_permutation_bit_identical():
    w = synth.gaussian_workload(42, B=6, H=128, seq_lens=[1, 200, 513, 1000, 64, 2048])
    o1, l1 = run_decode(w, split_tokens=256)
    pool2, table2 = synth.permute_pages(w, 43)
    o2, l2 = run_decode(w, split_tokens=256, pool=pool2, table=table2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_decode_partial_then_combine_equals_paged():
    w = synth.workload(3)
    B, H = w["B"], w["H"]
    max_len = int(w["seq_lens"].max())
    q = to_dev_bf16(w["q_decode"])
    kv, bt, sl = to_dev_bf16(w["cache_full"]), to_dev(w["block_table"]), to_dev(w["seq_lens"])
    ws = torch.full((mla.mla_decode_workspace_bytes(B, H, max_len, 512),), 0xFF, dtype=torch.uint8, device="cuda")
    mla.mla_decode_partial(q, kv, w["kv_dtype"], bt, sl, max_len, w["scale"], ws, split_tokens=512)
    o1 = nan_bf16(B, H, 512)
    l1 = torch.empty((B, H), dtype=torch.float32, device="cuda")
    mla.mla_decode_combine(ws, sl, max_len, o1, l1, split_tokens=512)
    o2, l2 = run_decode(w, split_tokens=512)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    # the partials themselves: chunk c of sequence b against the oracle on that token range
    rows = B * ((max_len + 511) // 512) * H
    o_part = bf(ws[:rows * 512 * 2].view(torch.bfloat16).view(B, -1, H, 512))
    off = ((rows * 512 * 2 + 255) // 256) * 256
    lse_part = ws[off:off + rows * 4].view(torch.float32).view(B, -1, H).cpu().numpy()
    for b in [0, 3]:
        S = int(w["seq_lens"][b])
        rows_b = oracle.gather_rows(w["cache_full"], w["block_table"], b, S)
        c, kr = oracle.rows_to_latent_rope(rows_b)
        qd = oracle.bf16_to_f64(w["q_decode"][b])
        for ch in [0, (S - 1) // 512]:
            t0, t1 = ch * 512, min(S, ch * 512 + 512)
            ro, rl = oracle.decode_absorbed(qd[:, :512], qd[:, 512:], c[t0:t1], kr[t0:t1], w["scale"])
            assert_close(o_part[b, ch], ro, 1e-5, 1e-2, extra=P_ROUNDING * np.abs(ro).max(), what=f"o_part b={b} c={ch}")
            assert_close(lse_part[b, ch], rl, LSE_ATOL, LSE_RTOL, what=f"lse_part b={b} c={ch}")


@pytest.mark.parametrize("H,lens,split", [
    (128, [4096] * 32, 512),                                   # one 32-row tile, every chunk full
    (16, [0, 1, 63, 64, 65, 700, 1500, 2048, 3000] * 4 + [17], 256),   # two tiles, ragged tail, empties
    (20, [5, 129, 4000], 64),                                  # many chunks, heads not a multiple of 16
    (128, [(37 * i) % 2600 for i in range(70)], 128),          # 5 tiles over 2 workgroups per head, 21 chunks
])
def test_combine_absorb_out_fused(H, lens, split):
    """One launch for merge + value absorption: bit-identical to mla_decode_combine
    followed by mla_absorb_out, and o within the bf16 bound of the oracle applied to
    the same partials (merged latent rounded to bf16, then W_UV)."""
    B = len(lens)
    w = synth.gaussian_workload(60 + H, B=B, H=H, seq_lens=lens)
    max_len = int(max(lens))
    q = to_dev_bf16(w["q_decode"])
    kv, bt, sl = to_dev_bf16(w["cache_full"]), to_dev(w["block_table"]), to_dev(w["seq_lens"])
    w_uv = to_dev_bf16(w["w_uv"])
    ws = torch.full((mla.mla_decode_workspace_bytes(B, H, max_len, split),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    mla.mla_decode_partial(q, kv, w["kv_dtype"], bt, sl, max_len, w["scale"], ws, split_tokens=split)
    o_lat1, l1, o1 = nan_bf16(B, H, 512), torch.empty((B, H), dtype=torch.float32, device="cuda"), nan_bf16(B, H, 128)
    mla.mla_decode_combine(ws, sl, max_len, o_lat1, l1, split_tokens=split)
    mla.mla_absorb_out(o_lat1, w_uv, o1)
    o_lat2, l2, o2 = nan_bf16(B, H, 512), torch.empty((B, H), dtype=torch.float32, device="cuda"), nan_bf16(B, H, 128)
    mla.mla_decode_combine_absorb_out(ws, sl, max_len, w_uv, o2, o_lat2, l2, split_tokens=split)
    o3 = nan_bf16(B, H, 128)
    mla.mla_decode_combine_absorb_out(ws, sl, max_len, w_uv, o3, split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(o_lat1.view(torch.int16), o_lat2.view(torch.int16))
    assert torch.equal(l1, l2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o2.view(torch.int16), o3.view(torch.int16))
    # oracle on the partials the GPU wrote
    n_splits = (max_len + split - 1) // split
    rows = B * n_splits * H
    o_part = bf(ws[:rows * 512 * 2].view(torch.bfloat16).view(B, n_splits, H, 512))
    off = ((rows * 512 * 2 + 255) // 256) * 256
    lse_part = ws[off:off + rows * 4].view(torch.float32).view(B, n_splits, H).cpu().numpy().astype(np.float64)
    w_uv64 = oracle.bf16_to_f64(w["w_uv"])
    got = bf(o2)
    for b in range(B):
        nv = (lens[b] + split - 1) // split
        if nv == 0:
            assert (got[b] == 0).all() and torch.isneginf(l2[b]).all().item()
            continue
        ref_lat, ref_l = oracle.combine_partials(o_part[b, :nv], lse_part[b, :nv])
        assert_close(bf(o_lat2[b]), ref_lat, what=f"merged o_latent b={b}")
        assert_close(l2[b].cpu().numpy(), ref_l, LSE_ATOL, LSE_RTOL, what=f"lse b={b}")
        ref_o = oracle.absorb_out(bf(o_lat2[b]), w_uv64)
        assert_close(got[b], ref_o, what=f"o b={b}")


# --------------------------------------------------------------------- fp8 cache
@pytest.mark.parametrize("H", [16, 64, 128, 200])
def test_decode_fp8_ragged_lengths_and_heads(H):
    """Packed E4M3 rows (656 bytes): every workgroup shape (2, 4, 8 waves),
    two head groups (200 heads), partial last blocks, page boundaries,
    several split sizes."""
    lens = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 300, 1000, 2100]
    w = synth.gaussian_workload(70 + H, B=len(lens), H=H, seq_lens=lens, kv_dtype=synth.KV_FP8)
    for split in [0, 64, 256]:
        o, lse = run_decode(w, split_tokens=split)
        check_decode(w, o, lse, [(b, range(H)) for b in range(len(lens))], p_rounding_term=True)


def test_decode_fp8_page_permutation_bit_identical():
    w = synth.gaussian_workload(80, B=5, H=128, seq_lens=[1, 200, 513, 1000, 2048], kv_dtype=synth.KV_FP8)
    o1, l1 = run_decode(w, split_tokens=256)
    pool2, table2 = synth.permute_pages(w, 81)
    o2, l2 = run_decode(w, split_tokens=256, pool=pool2, table=table2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_FP8])
def test_decode_ignores_rows_past_the_end(kv_dtype):
    """Rows of a page beyond a sequence's length (never written) may hold any
    bytes: fill them with all-ones (NaN in bf16, E4M3 and fp32) and expect
    the result of the clean pool bit for bit."""
    lens = [1, 33, 64, 65, 100, 511, 777]
    w = synth.gaussian_workload(90 + kv_dtype, B=len(lens), H=64, seq_lens=lens, kv_dtype=kv_dtype)
    pool = w["cache_full"].copy()
    used = np.zeros(pool.shape[:2], bool)
    for b, S in enumerate(lens):
        for t in range(S):
            used[w["block_table"][b, t // 64], t % 64] = True
    pool[~used] = np.iinfo(pool.dtype).max
    for split in [0, 128]:
        o1, l1 = run_decode(w, split_tokens=split)
        o2, l2 = run_decode(w, split_tokens=split, pool=pool)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"split={split}"
        assert torch.equal(l1, l2)


def test_decode_fp8_full_size():
    """Workload 4 (B=128, 8192 tokens, fp8 cache, 688 MB) in the planner's
    launch configuration: every head of 12 sequences spread over the batch
    against the oracle at the fp8 bound 2e-3 + 6e-2 |ref|, nothing added."""
    w = synth.workload(4)
    o, lse = run_decode(w, split_tokens=0)
    assert not torch.isnan(o.float()).any().item()
    check_decode(w, o, lse, [(b, range(w["H"])) for b in (0, 1, 15, 31, 32, 63, 64, 77, 95, 100, 126, 127)])


def test_decode_repeatable():
    w = synth.workload(1)
    o1, l1 = run_decode(w)
    o2, l2 = run_decode(w)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


# --------------------------------------------------------------------- whole step
def run_step(w):
    B, H = w["B"], w["H"]
    q = nan_bf16(B, H, 576)
    kv = to_dev_bf16(w["cache_step"])
    sl, bt = to_dev(w["seq_lens"]), to_dev(w["block_table"])
    o_lat = nan_bf16(B, H, 512)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    o = nan_bf16(B, H, 128)
    mla.mla_absorb_q(to_dev_bf16(w["q_nope"]), to_dev_bf16(w["w_uk"]), q)
    mla.mla_rope_append_cache(to_dev_bf16(w["q_pe"]), to_dev_bf16(w["kv_new"]), sl, bt, kv, w["kv_dtype"],
                              w["theta"], q)
    mla.mla_decode_paged(q, kv, w["kv_dtype"], bt, sl, int(w["seq_lens"].max()), w["scale"], o_lat, lse)
    mla.mla_absorb_out(o_lat, to_dev_bf16(w["w_uv"]), o)
    torch.cuda.synchronize()
    return q, o_lat, lse, o


@pytest.mark.parametrize("cfg,pairs", [
    (1, [(b, range(16)) for b in range(8)]),
    (2, [(0, range(128)), (17, [5, 64]), (31, range(128))]),
])
def test_full_step(cfg, pairs):
    w = synth.workload(cfg)
    q, o_lat, lse, o = run_step(w)
    for b, heads in pairs:
        heads = list(heads)
        r = oracle.reference_step(w, b, heads)
        assert_close(bf(q[b, heads, :512]), r["q_lat"], what=f"q_lat b={b}")
        assert_close(bf(q[b, heads, 512:]), r["q_rot"], what=f"q_rot b={b}")
        assert_close(bf(o_lat[b, heads]), r["o_lat"], what=f"o_latent b={b}")
        # q_lat and the appended rotary key are rounded to bf16 on the GPU
        # (2^-9 relative each), which moves every score by a few 1e-4 here: the
        # full step's lse is held to the bf16 absolute bound.
        assert_close(lse[b, heads].cpu().numpy(), r["lse"], BF16_ATOL, 0.0, what=f"lse b={b}")
        assert_close(bf(o[b, heads]), r["o"], what=f"o b={b}")
