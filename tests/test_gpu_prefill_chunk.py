"""GPU parity of mla_prefill_chunk, prompt chunks that continue a cached
prefix, against the fp64 oracle (prefill_chunk_explicit).

Each case draws whole prompts (synth.prefill_workload), writes the first
P_b rows of prompt b into the paged pool from the oracle's own rows (the
latent as drawn and RoPE(k_pe, t) rounded to bf16; fp8 pools through the
oracle's quantiser), then runs the remaining tokens as the chunk.  The
oracle sees the same prefix rows (fp8: code * group scale in fp64).

Tolerances are those of the prefill tests: |gpu - ref| <= 2e-3 + 2e-2 |ref|
(fp8 prefix rows: 2e-3 + 6e-2 |ref|), the ragged synthetic cases adding the
rounding of the half-precision weights and values, 2^-8 sum_i p_i |V_i|;
the 128-head case with a 1,900-token prefix holds the stated bound with
nothing added.  The chunk's cache rows: latent copies and fp8 codes/scales
bit for bit, rotated keys within the bf16 bound."""
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


def _prefix_rows(w, b, P):
    """Oracle rows of prompt b's first P tokens: (stored row bytes/bits, c, kr) in f64."""
    t0 = int(w["cu_seqlens"][b])
    c_bits = w["c"][t0:t0 + P]
    kr = oracle.rope(oracle.bf16_to_f64(w["k_pe"][t0:t0 + P]), np.arange(P, dtype=np.float64), w["theta"])
    kr_bits = synth.f32_to_bf16_bits(kr.astype(np.float32))
    if w["kv_dtype"] == synth.KV_FP8:
        codes, scales = oracle.fp8_quantize_latent(c_bits)
        stored = synth.pack_fp8_rows(codes, kr_bits, scales)
        c = (oracle.e4m3_to_f64(codes).reshape(P, 4, 128) * scales.astype(np.float64)[:, :, None]).reshape(P, 512)
    else:
        stored = np.concatenate([c_bits, kr_bits], 1)
        c = oracle.bf16_to_f64(c_bits)
    return stored, c, oracle.bf16_to_f64(kr_bits)


def make_case(seed, H, prefixes, chunks, kv_dtype):
    lens = [p + n for p, n in zip(prefixes, chunks)]
    w = synth.prefill_workload(seed, H, lens, kv_dtype)
    fp8 = kv_dtype == synth.KV_FP8
    pool = np.zeros((w["num_blocks"], 64, 656 if fp8 else 576), np.uint8 if fp8 else np.uint16)
    prefix = []
    for b, P in enumerate(prefixes):
        stored, c, kr = _prefix_rows(w, b, P)
        for t in range(P):
            pool[w["block_table"][b, t // 64], t % 64] = stored[t]
        prefix.append((c, kr))
    sel = np.concatenate([np.arange(int(w["cu_seqlens"][b]) + p, int(w["cu_seqlens"][b + 1]))
                          for b, p in enumerate(prefixes)]).astype(np.int64)
    chunk = {k: w[k][sel] for k in ("q_nope", "q_pe", "c", "k_pe")}
    chunk["cu"] = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    return w, pool, prefix, chunk


def run_chunk(w, pool, chunk, prefixes, chunks):
    fp8 = w["kv_dtype"] == synth.KV_FP8
    T, H = chunk["q_nope"].shape[:2]
    kv = to_dev(pool) if fp8 else to_dev_bf16(pool)
    o = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    total_keys = int(sum(prefixes) + sum(chunks))
    mla.mla_prefill_chunk(to_dev_bf16(chunk["q_nope"]), to_dev_bf16(chunk["q_pe"]), to_dev_bf16(chunk["c"]),
                          to_dev_bf16(chunk["k_pe"]), to_dev_bf16(w["w_uk"]), to_dev_bf16(w["w_uv"]),
                          to_dev(chunk["cu"]), to_dev(np.asarray(prefixes, np.int32)), int(max(chunks)), total_keys,
                          int(max(prefixes)), w["scale"], w["theta"], to_dev(w["block_table"]), kv,
                          w["kv_dtype"], o)
    torch.cuda.synchronize()
    out = kv.cpu().numpy() if fp8 else kv.cpu().view(torch.int16).numpy().view(np.uint16)
    return o, out


def check(w, o, pool_after, prefix, chunk, prefixes, heads_for, widen=True, rows=True):
    fp8 = w["kv_dtype"] == synth.KV_FP8
    tol = (2e-3, 6e-2) if fp8 else (2e-3, 2e-2)
    for b, P in enumerate(prefixes):
        t0, t1 = int(chunk["cu"][b]), int(chunk["cu"][b + 1])
        if t1 == t0:
            continue
        heads = list(heads_for(b))
        c_pre, kr_pre = prefix[b]
        ref, ref_rows, mag = oracle.prefill_chunk_explicit(
            oracle.bf16_to_f64(chunk["q_nope"][t0:t1])[:, heads], oracle.bf16_to_f64(chunk["q_pe"][t0:t1])[:, heads],
            oracle.bf16_to_f64(chunk["c"][t0:t1]), oracle.bf16_to_f64(chunk["k_pe"][t0:t1]), c_pre, kr_pre,
            oracle.bf16_to_f64(w["w_uk"])[heads], oracle.bf16_to_f64(w["w_uv"])[heads], w["scale"], w["theta"],
            with_magnitude=True)
        got = bf16_tensor_to_f64(o[t0:t1][:, heads])
        assert_close(got, ref, *tol, extra=P_ROUNDING * mag if widen else 0.0, what=f"o prompt b={b} P={P}")
        if not rows:
            continue
        for j in range(t1 - t0):
            pos = P + j
            row = pool_after[w["block_table"][b, pos // 64], pos % 64]
            c_bits = chunk["c"][t0 + j]
            if fp8:
                codes, scales = oracle.fp8_quantize_latent(c_bits)
                np.testing.assert_array_equal(row[:512], codes, err_msg=f"fp8 codes b={b} pos={pos}")
                np.testing.assert_array_equal(row[640:656].view(np.float32), scales, err_msg=f"scales b={b}")
                got_kr = oracle.bf16_to_f64(row[512:640].view(np.uint16))
            else:
                np.testing.assert_array_equal(row[:512], c_bits, err_msg=f"latent copy b={b} pos={pos}")
                got_kr = oracle.bf16_to_f64(row[512:])
            assert_close(got_kr, ref_rows[j, 512:], what=f"k_rot b={b} pos={pos}")


@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_FP8])
def test_prefill_chunk_matches_oracle(H, kv_dtype):
    """Prefixes around page and key-block edges (0, 1, 31, 64, 100, 300)
    with chunks of 1 .. 200 tokens, including an empty chunk."""
    prefixes = [0, 1, 31, 64, 100, 300, 5]
    chunks = [40, 33, 1, 129, 200, 64, 0]
    w, pool, prefix, chunk = make_case(900 + H + kv_dtype, H, prefixes, chunks, kv_dtype)
    o, pool_after = run_chunk(w, pool, chunk, prefixes, chunks)
    heads = (lambda b: range(H)) if H <= 16 else (lambda b: [0, 1, 63, 127])
    check(w, o, pool_after, prefix, chunk, prefixes, heads)


def test_prefill_chunk_long_prefix_full_heads():
    """128 heads, a 1,900-token prefix and a 300-token chunk beside a short
    one: every token of 16 heads at the stated bf16 bound, nothing added."""
    prefixes, chunks = [1900, 17], [300, 50]
    w, pool, prefix, chunk = make_case(930, 128, prefixes, chunks, synth.KV_BF16)
    o, pool_after = run_chunk(w, pool, chunk, prefixes, chunks)
    assert not torch.isnan(o.float()).any().item()
    check(w, o, pool_after, prefix, chunk, prefixes, lambda b: range(b, 128, 8), widen=False, rows=False)


@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_FP8])
def test_prefill_chunk_without_prefix_is_the_prefill(kv_dtype):
    """Every prefix empty: the same outputs and cache rows, bit for bit, as
    mla_prefill on the same prompts."""
    lens = [1, 40, 129, 300]
    w = synth.prefill_workload(940 + kv_dtype, 16, lens, kv_dtype)
    fp8 = kv_dtype == synth.KV_FP8
    shape = (w["num_blocks"], 64, 656 if fp8 else 576)
    args = [to_dev_bf16(w[k]) for k in ("q_nope", "q_pe", "c", "k_pe", "w_uk", "w_uv")]
    outs = []
    for chunked in (False, True):
        pool = torch.zeros(shape, dtype=torch.uint8 if fp8 else torch.bfloat16, device="cuda")
        o = torch.full((w["T"], 16, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        if chunked:
            mla.mla_prefill_chunk(*args, to_dev(w["cu_seqlens"]), to_dev(np.zeros(len(lens), np.int32)), max(lens),
                                  w["T"], 0, w["scale"], w["theta"], to_dev(w["block_table"]), pool, kv_dtype, o)
        else:
            mla.mla_prefill(*args, to_dev(w["cu_seqlens"]), max(lens), w["scale"], w["theta"],
                            to_dev(w["block_table"]), pool, kv_dtype, o)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).cpu(), pool.view(torch.uint8).cpu()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


def test_prefill_chunk_then_decode():
    """The rows a chunk leaves continue the prefix: a decode over the whole
    prompt (prefix + chunk rows) matches the oracle's decode over the oracle's
    rows."""
    prefixes, chunks = [70, 300], [60, 1]
    w, pool, prefix, chunk = make_case(950, 16, prefixes, chunks, synth.KV_BF16)
    o, pool_after = run_chunk(w, pool, chunk, prefixes, chunks)
    lens = [p + n for p, n in zip(prefixes, chunks)]
    q = synth.multi_token_query(951, len(lens), 1, 16)[:, 0]
    od = torch.full((len(lens), 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    mla.mla_decode_paged(to_dev_bf16(q), to_dev_bf16(pool_after), synth.KV_BF16, to_dev(w["block_table"]),
                         to_dev(np.asarray(lens, np.int32)), max(lens), w["scale"], od, None, split_tokens=64)
    torch.cuda.synchronize()
    for b, (P, n) in enumerate(zip(prefixes, chunks)):
        t0, t1 = int(chunk["cu"][b]), int(chunk["cu"][b + 1])
        _, rows = oracle.prefill_chunk_explicit(
            oracle.bf16_to_f64(chunk["q_nope"][t0:t1])[:, :1], oracle.bf16_to_f64(chunk["q_pe"][t0:t1])[:, :1],
            oracle.bf16_to_f64(chunk["c"][t0:t1]), oracle.bf16_to_f64(chunk["k_pe"][t0:t1]), prefix[b][0],
            prefix[b][1], oracle.bf16_to_f64(w["w_uk"])[:1], oracle.bf16_to_f64(w["w_uv"])[:1], w["scale"], w["theta"])
        c = np.concatenate([prefix[b][0], rows[:, :512]])
        kr = np.concatenate([prefix[b][1], rows[:, 512:]])
        qb = oracle.bf16_to_f64(q[b])
        ref, _, mag = oracle.decode_absorbed(qb[:, :512], qb[:, 512:], c, kr, w["scale"], with_magnitude=True)
        assert_close(bf16_tensor_to_f64(od[b]), ref, extra=P_ROUNDING * mag, what=f"decode after chunk b={b}")
