"""GPU parity of the explicit-form prefill (mla_prefill) against the fp64
oracle: outputs within the bf16 bound |gpu - ref| <= 2e-3 + 2e-2 |ref|
(the 4 x 1024-token, 128-head shape exactly so; the ragged synthetic prompts
add 2^-8 sum_i p_i |V_i|, the bf16 rounding of the softmax weights and of
the materialised per-head values, 2^-9 each); the cache rows the
prompts leave: latent copies and fp8 codes/scales bit for bit, rotated keys
within the bf16 bound."""
import numpy as np
import pytest
import torch

import mla_latent_kv_32_amd as mla
import oracle
import synth
from helpers import assert_close, bf16_tensor_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
P_ROUNDING = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a ROCm device"
    mla.lib()


def run_prefill(w):
    T, H = w["T"], w["H"]
    fp8 = w["kv_dtype"] == synth.KV_FP8
    shape = (w["num_blocks"], 64, 656 if fp8 else 576)
    pool = torch.zeros(shape, dtype=torch.uint8 if fp8 else torch.bfloat16, device="cuda")
    o = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    mla.mla_prefill(to_dev_bf16(w["q_nope"]), to_dev_bf16(w["q_pe"]), to_dev_bf16(w["c"]), to_dev_bf16(w["k_pe"]),
                    to_dev_bf16(w["w_uk"]), to_dev_bf16(w["w_uv"]), to_dev(w["cu_seqlens"]), int(max(w["lens"])),
                    w["scale"], w["theta"], to_dev(w["block_table"]), pool, w["kv_dtype"], o)
    torch.cuda.synchronize()
    pool = pool.cpu().numpy() if fp8 else pool.cpu().view(torch.int16).numpy().view(np.uint16)
    return o, pool


def check_prefill(w, o, pool, pairs, rows_for=(), widen=True):
    fp8 = w["kv_dtype"] == synth.KV_FP8
    for b, heads in pairs:
        heads = list(heads)
        t0, t1 = int(w["cu_seqlens"][b]), int(w["cu_seqlens"][b + 1])
        if t1 == t0:
            continue
        ref, rows, mag = oracle.reference_prefill(w, b, heads, with_magnitude=True)
        got = bf16_tensor_to_f64(o[t0:t1][:, heads])
        assert_close(got, ref, extra=P_ROUNDING * mag if widen else 0.0, what=f"o prompt b={b} L={t1 - t0}")
        if b not in rows_for:
            continue
        for pos in range(t1 - t0):
            page, slot = w["block_table"][b, pos // 64], pos % 64
            row = pool[page, slot]
            c_bits = w["c"][t0 + pos]
            if fp8:
                codes, scales = oracle.fp8_quantize_latent(c_bits)
                np.testing.assert_array_equal(row[:512], codes, err_msg=f"fp8 codes b={b} pos={pos}")
                np.testing.assert_array_equal(row[640:656].view(np.float32), scales, err_msg=f"scales b={b}")
                got_kr = oracle.bf16_to_f64(row[512:640].view(np.uint16))
            else:
                np.testing.assert_array_equal(row[:512], c_bits, err_msg=f"latent copy b={b} pos={pos}")
                got_kr = oracle.bf16_to_f64(row[512:])
            assert_close(got_kr, rows[pos, 512:], what=f"k_rot b={b} pos={pos}")


@pytest.mark.parametrize("H", [5, 16, 128])
@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_FP8])
def test_prefill_matches_oracle(H, kv_dtype):
    """Ragged prompts around the 32-key blocks and 128-row query tiles,
    including a 1-token and an empty prompt; H = 5 leaves the up-projection's
    last pair of heads with one head."""
    lens = [1, 0, 31, 33, 128, 129, 300]
    w = synth.prefill_workload(700 + H + kv_dtype, H, lens, kv_dtype)
    o, pool = run_prefill(w)
    heads = range(H) if H <= 16 else [0, 1, 63, 127]
    check_prefill(w, o, pool, [(b, heads) for b in range(len(lens))], rows_for=range(len(lens)))


def test_prefill_rows_untouched_elsewhere():
    """Only the prompts' own (page, slot) rows are written."""
    lens = [5, 70, 64]
    w = synth.prefill_workload(710, 4, lens)
    o, pool = run_prefill(w)
    touched = np.zeros(pool.shape[:2], bool)
    for b, L in enumerate(lens):
        for pos in range(L):
            touched[w["block_table"][b, pos // 64], pos % 64] = True
    assert (pool[~touched] == 0).all()


def test_prefill_long_prompts_full_heads():
    """Four 1024-token prompts with DeepSeek-V3's 128 heads (the benchmark's
    prefill shape): every token of 16 heads of two prompts at the stated bf16
    bound, nothing added."""
    w = synth.prefill_workload(720, 128, [1024] * 4)
    o, pool = run_prefill(w)
    assert not torch.isnan(o.float()).any().item()
    check_prefill(w, o, pool, [(0, range(0, 128, 9)), (3, range(4, 128, 8))], widen=False)


def test_prefill_head_groups_with_a_partial_last_group():
    """100 heads over 4,072 keys: the up-projections take 6 heads per
    workgroup (16 token tiles, 17 head groups), so the last group holds 4
    heads, and the last token tile is ragged (4,072 = 15 x 256 + 232).
    Every token of heads on both sides of group boundaries and of the last
    group, in the first and the shortest prompt, at the stated bf16 bound."""
    w = synth.prefill_workload(750, 100, [1024, 1024, 1024, 1000])
    o, pool = run_prefill(w)
    assert not torch.isnan(o.float()).any().item()
    check_prefill(w, o, pool, [(0, [0, 5, 6, 95, 96, 99]), (3, [11, 12, 97])], widen=False)


def test_prefill_long_ragged_prompt():
    """One 4001-token prompt (126 key blocks, a ragged last query tile and
    page) beside a short one: every token of two heads against the oracle,
    and every cache row of the long prompt."""
    w = synth.prefill_workload(740, 8, [4001, 37])
    o, pool = run_prefill(w)
    assert not torch.isnan(o.float()).any().item()
    check_prefill(w, o, pool, [(0, [0, 7]), (1, [3])], rows_for=[0])


@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_FP8])
def test_decode_after_prefill(kv_dtype):
    """The rows a prefill leaves are the cache the decode reads: a decode
    query against each prompt's prefilled rows matches the oracle's decode
    over the oracle's rows for that prompt."""
    lens = [1, 40, 129, 300]
    H = 16
    w = synth.prefill_workload(730 + kv_dtype, H, lens, kv_dtype)
    o, pool = run_prefill(w)
    fp8 = kv_dtype == synth.KV_FP8
    q = synth.multi_token_query(731, len(lens), 1, H)[:, 0]
    sl = np.asarray(lens, np.int32)
    pool_dev = to_dev(pool) if fp8 else to_dev_bf16(pool)
    od = torch.full((len(lens), H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((len(lens), H), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_decode_paged(to_dev_bf16(q), pool_dev, kv_dtype, to_dev(w["block_table"]), to_dev(sl), max(lens),
                         w["scale"], od, lse, split_tokens=64)
    torch.cuda.synchronize()
    tol = (2e-3, 6e-2) if fp8 else (2e-3, 2e-2)
    for b, L in enumerate(lens):
        _, rows = oracle.reference_prefill(w, b, [0])
        if fp8:   # the cache holds the latent quantised to E4M3 per 128-wide group
            c = np.stack([(oracle.e4m3_to_f64(cd).reshape(4, 128) * sc.astype(np.float64)[:, None]).reshape(512)
                          for cd, sc in (oracle.fp8_quantize_latent(w["c"][int(w["cu_seqlens"][b]) + t])
                                         for t in range(L))])
        else:
            c = rows[:, :512]
        qb = oracle.bf16_to_f64(q[b])
        ref, ref_l, mag = oracle.decode_absorbed(qb[:, :512], qb[:, 512:], c, rows[:, 512:], w["scale"],
                                                 with_magnitude=True)
        assert_close(bf16_tensor_to_f64(od[b]), ref, *tol, extra=P_ROUNDING * mag, what=f"decode after prefill b={b}")
