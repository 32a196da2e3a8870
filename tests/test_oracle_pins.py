"""Pins for the fp64 oracle: each check ties it to something other than itself.

Closed forms, brute-force evaluation, library routines (torch SDPA, torch's
float8_e4m3fn dtype) and the numbers the pages print.  A plausible mistake in
the oracle -- a dropped rotary part, a transposed weight, a wrong pair
convention, a missing scale, a wrong combine weight -- fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def _rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- RoPE (PIN-3)
def test_rope_pair_convention_closed_form():
    # d = 4, theta = 100: pair 0 turns at 1 rad/position, pair 1 at 100^(-1/2) = 0.1.
    for pos in [0.0, 1.0, 3.7, 1000.0]:
        e = np.eye(4)
        r = oracle.rope(e, pos, theta=100.0)
        c0, s0 = math.cos(pos), math.sin(pos)
        c1, s1 = math.cos(0.1 * pos), math.sin(0.1 * pos)
        np.testing.assert_allclose(r[0], [c0, s0, 0, 0], atol=1e-12)
        np.testing.assert_allclose(r[1], [-s0, c0, 0, 0], atol=1e-12)
        np.testing.assert_allclose(r[2], [0, 0, c1, s1], atol=1e-12)
        np.testing.assert_allclose(r[3], [0, 0, -s1, c1], atol=1e-12)


def test_rope_frequencies_d64():
    theta = 10000.0
    e = np.eye(64)[0::2]          # unit vectors on the first element of each pair
    r = oracle.rope(e, 1.0, theta)
    for i in range(32):
        w = theta ** (-2.0 * i / 64)
        assert abs(r[i, 2 * i] - math.cos(w)) < 1e-14
        assert abs(r[i, 2 * i + 1] - math.sin(w)) < 1e-14


def test_rope_identity_norm_and_relative_position():
    q, k = _rand(64), _rand(64)
    np.testing.assert_allclose(oracle.rope(q, 0.0), q, atol=0, rtol=0)
    for m in [0, 5, 4095, 32767]:
        assert abs(np.linalg.norm(oracle.rope(q, m)) - np.linalg.norm(q)) < 1e-12
    # <R_m q, R_n k> depends only on m - n (R_m R_n^T = R_{m-n}).
    for m, n, s in [(3, 1, 7), (4095, 10, 20000), (32768, 32760, -30000), (0, 9, 12345)]:
        a = oracle.rope(q, m) @ oracle.rope(k, n)
        b = oracle.rope(q, m + s) @ oracle.rope(k, n + s)
        assert abs(a - b) < 1e-10 * (1 + abs(a))


def test_rope_broadcast_positions():
    v = _rand(5, 8)
    pos = np.arange(5.0)
    r = oracle.rope(v, pos)
    for t in range(5):
        np.testing.assert_allclose(r[t], oracle.rope(v[t], float(t)), atol=1e-15)


# ----------------------------------------------------- brute-force attention
def _brute_decode(q_nope, q_rot, c, kr, w_uk, w_uv, scale):
    """Pure-Python loops over the explicit form; no numpy algebra."""
    H, dn = len(q_nope), len(q_nope[0])
    S, dc = len(c), len(c[0])
    dr, dv = len(kr[0]), len(w_uv[0][0])
    out, lses = [], []
    for h in range(H):
        scores = []
        for t in range(S):
            k = [sum(c[t][j] * w_uk[h][n][j] for j in range(dc)) for n in range(dn)]
            k += [kr[t][r] for r in range(dr)]
            q = list(q_nope[h]) + list(q_rot[h])
            scores.append(scale * sum(qa * ka for qa, ka in zip(q, k)))
        m = max(scores)
        ex = [math.exp(s - m) for s in scores]
        z = sum(ex)
        lses.append(m + math.log(z))
        o = [0.0] * dv
        for t in range(S):
            v = [sum(c[t][j] * w_uv[h][j][e] for j in range(dc)) for e in range(dv)]
            for e in range(dv):
                o[e] += ex[t] / z * v[e]
        out.append(o)
    return np.array(out), np.array(lses)


def test_decode_explicit_matches_brute_force():
    rng = np.random.default_rng(7)
    H, dn, dc, dr, dv, S = 3, 3, 5, 2, 4, 6
    q_nope, q_rot = _rand(H, dn, rng=rng), _rand(H, dr, rng=rng)
    c, kr = _rand(S, dc, rng=rng), _rand(S, dr, rng=rng)
    w_uk, w_uv = _rand(H, dn, dc, rng=rng), _rand(H, dc, dv, rng=rng)
    o, o_lat, lse = oracle.decode_explicit(q_nope, q_rot, c, kr, w_uk, w_uv, 0.37)
    ob, lb = _brute_decode(q_nope, q_rot, c, kr, w_uk, w_uv, 0.37)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-13)
    # o_lat is the latent-weighted sum with the same weights: o = o_lat W_UV.
    np.testing.assert_allclose(oracle.absorb_out(o_lat, w_uv), o, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------- absorption (PIN-1)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_absorbed_equals_explicit_random(seed):
    rng = np.random.default_rng(seed)
    H, dn, dc, dr, dv, S = 4, 6, 10, 4, 5, 17
    q_nope, q_rot = _rand(H, dn, rng=rng), _rand(H, dr, rng=rng)
    c, kr = _rand(S, dc, rng=rng), _rand(S, dr, rng=rng)
    w_uk, w_uv = _rand(H, dn, dc, rng=rng), _rand(H, dc, dv, rng=rng)
    scale = 1 / math.sqrt(dn + dr)
    o, o_lat_e, lse_e = oracle.decode_explicit(q_nope, q_rot, c, kr, w_uk, w_uv, scale)
    q_lat = oracle.absorb_q(q_nope, w_uk)
    o_lat, lse = oracle.decode_absorbed(q_lat, q_rot, c, kr, scale)
    np.testing.assert_allclose(o_lat, o_lat_e, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse_e, rtol=1e-12)
    np.testing.assert_allclose(oracle.absorb_out(o_lat, w_uv), o, rtol=1e-11, atol=1e-13)


def test_absorbed_equals_explicit_workload0():
    w = synth.workload(0)
    o, c, kr, q_nope, q_rot = oracle.prefill_mha_form(
        w["x"], w["w_dkv"], w["w_kr"], w["w_q"], w["w_uk"], w["w_uv"],
        w["d_nope"], w["d_r"], w["scale"], w["theta"])
    t = w["S"] - 1
    oe, _, _ = oracle.decode_explicit(q_nope[t], q_rot[t], c, kr, w["w_uk"], w["w_uv"], w["scale"])
    q_lat = oracle.absorb_q(q_nope[t], w["w_uk"])
    o_lat, _ = oracle.decode_absorbed(q_lat, q_rot[t], c, kr, w["scale"])
    oa = oracle.absorb_out(o_lat, w["w_uv"])
    np.testing.assert_allclose(oa, oe, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(oe, o[t], rtol=1e-11, atol=1e-13)


def test_rotary_part_is_not_dropped():
    # With the latent query zero, scores come from the rotary part alone: a
    # rotary key aligned with the query must dominate the softmax.
    S, dc, dr = 8, 6, 4
    c = np.eye(S, dc) if S <= dc else _rand(S, dc)
    kr = np.zeros((S, dr))
    kr[5] = [10, 0, 0, 0]
    q_lat, q_rot = np.zeros((1, dc)), np.array([[10.0, 0, 0, 0]])
    o_lat, _ = oracle.decode_absorbed(q_lat, q_rot, c, kr, 1.0)
    np.testing.assert_allclose(o_lat[0], c[5], atol=1e-30 + 1e-40)


def test_weighted_magnitude_bounds_output():
    rng = np.random.default_rng(21)
    c, kr = rng.standard_normal((40, 12)), rng.standard_normal((40, 4))
    q_lat, q_rot = rng.standard_normal((3, 12)), rng.standard_normal((3, 4))
    o, _, mag = oracle.decode_absorbed(q_lat, q_rot, c, kr, 0.3, with_magnitude=True)
    assert (np.abs(o) <= mag + 1e-15).all()
    o2, _, mag2 = oracle.decode_absorbed(q_lat, q_rot, np.abs(c), kr, 0.3, with_magnitude=True)
    np.testing.assert_allclose(o2, mag2, rtol=1e-14)


# ----------------------------------------------------------- softmax (PIN-4)
def test_softmax_rows_sum_to_one():
    s = _rand(7, 300) * 20
    p, lse = oracle.softmax_lse(s)
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    np.testing.assert_allclose(lse, np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1), rtol=1e-13)
    import scipy.special
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=1e-13)


# ------------------------------------------------------ closed forms (PIN-5)
def test_closed_forms():
    dc, dr, H = 12, 4, 3
    c, kr = _rand(9, dc), _rand(9, dr)
    q_lat, q_rot = _rand(H, dc), _rand(H, dr)
    # one visible token: weight 1 on it, lse equals its score
    o1, l1 = oracle.decode_absorbed(q_lat, q_rot, c[:1], kr[:1], 0.5)
    np.testing.assert_array_equal(o1, np.broadcast_to(c[0], o1.shape))
    np.testing.assert_allclose(l1, 0.5 * (q_lat @ c[0] + q_rot @ kr[0]), rtol=1e-14)
    # all rows equal: the output is that row; lse = score + log S
    ce, ke = np.repeat(c[:1], 9, 0), np.repeat(kr[:1], 9, 0)
    oe, le = oracle.decode_absorbed(q_lat, q_rot, ce, ke, 0.5)
    np.testing.assert_allclose(oe, np.broadcast_to(c[0], oe.shape), rtol=1e-14)
    np.testing.assert_allclose(le, 0.5 * (q_lat @ c[0] + q_rot @ kr[0]) + math.log(9), rtol=1e-14)
    # zero query (or zero scale): uniform weights -> mean of the latents
    oz, lz = oracle.decode_absorbed(np.zeros((H, dc)), np.zeros((H, dr)), c, kr, 0.5)
    np.testing.assert_allclose(oz, np.broadcast_to(c.mean(0), oz.shape), rtol=1e-13)
    np.testing.assert_allclose(lz, math.log(9), rtol=1e-14)
    # empty sequence
    o0, l0 = oracle.decode_absorbed(q_lat, q_rot, c[:0], kr[:0], 0.5)
    assert (o0 == 0).all() and np.isneginf(l0).all()


# ---------------------------------------------------- library routine (PIN-6)
def test_mqa_form_equals_torch_sdpa_fp64():
    rng = np.random.default_rng(3)
    H, S = 8, 200
    c, kr = rng.standard_normal((S, 512)), rng.standard_normal((S, 64))
    q = rng.standard_normal((H, 576)) * 0.05
    scale = 1 / math.sqrt(192)
    o_lat, _ = oracle.decode_absorbed(q[:, :512], q[:, 512:], c, kr, scale)
    tq = torch.from_numpy(q)[None, :, None, :]
    tk = torch.from_numpy(np.concatenate([c, kr], 1))[None, None].expand(1, H, S, 576)
    tv = torch.from_numpy(c)[None, None].expand(1, H, S, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)[0, :, 0].numpy()
    np.testing.assert_allclose(o_lat, ref, rtol=1e-11, atol=1e-14)


# --------------------------------------------------- split combine (PIN-7)
@pytest.mark.parametrize("cuts", [[256], [1, 2, 300], [64, 128, 192, 256, 320, 384, 448, 512]])
def test_split_combine_reproduces_unsplit(cuts):
    rng = np.random.default_rng(11)
    S, H = 530, 4
    c, kr = rng.standard_normal((S, 512)), rng.standard_normal((S, 64))
    q = rng.standard_normal((H, 576)) * 0.06
    full, lse = oracle.decode_absorbed(q[:, :512], q[:, 512:], c, kr, 0.07)
    bounds = [0] + cuts + [S, S]          # the last chunk is empty
    parts = [oracle.decode_absorbed(q[:, :512], q[:, 512:], c[a:b], kr[a:b], 0.07)
             for a, b in zip(bounds[:-1], bounds[1:])]
    o, l = oracle.combine_partials([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(o, full, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l, lse, rtol=1e-13)


def test_combine_all_empty():
    o, l = oracle.combine_partials(np.zeros((3, 2, 5)), np.full((3, 2), -np.inf))
    assert (o == 0).all() and np.isneginf(l).all()


# ---------------------------------------------------------- paging (PIN-8)
def test_page_permutation_and_contiguous_identity():
    rng = np.random.default_rng(5)
    S, blk = 200, 64
    rows = rng.standard_normal((S, 576))
    nb = (S + blk - 1) // blk
    contiguous = np.zeros((nb, blk, 576))
    contiguous.reshape(-1, 576)[:S] = rows
    perm = rng.permutation(nb + 3)[:nb]
    pool = np.full((nb + 3, blk, 576), np.nan)
    for j in range(nb):
        pool[perm[j], :min(blk, S - j * blk)] = rows[j * blk:(j + 1) * blk]
    g1 = oracle.gather_rows(contiguous, np.arange(nb)[None], 0, S, blk)
    g2 = oracle.gather_rows(pool, perm[None], 0, S, blk)
    np.testing.assert_array_equal(g1, rows)
    np.testing.assert_array_equal(g2, rows)


def test_token_order_invariance():
    rng = np.random.default_rng(6)
    c, kr = rng.standard_normal((77, 512)), rng.standard_normal((77, 64))
    q = rng.standard_normal((3, 576)) * 0.05
    p = rng.permutation(77)
    a, la = oracle.decode_absorbed(q[:, :512], q[:, 512:], c, kr, 0.07)
    b, lb = oracle.decode_absorbed(q[:, :512], q[:, 512:], c[p], kr[p], 0.07)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(la, lb, rtol=1e-13)


# ---------------------------------------------------------- prefix (PIN-9)
def test_prefill_rows_equal_absorbed_decode_of_prefix():
    w = synth.workload(0)
    o, c, kr, q_nope, q_rot = oracle.prefill_mha_form(
        w["x"], w["w_dkv"], w["w_kr"], w["w_q"], w["w_uk"], w["w_uv"],
        w["d_nope"], w["d_r"], w["scale"], w["theta"])
    for t in range(w["S"]):
        q_lat = oracle.absorb_q(q_nope[t], w["w_uk"])
        o_lat, _ = oracle.decode_absorbed(q_lat, q_rot[t], c[:t + 1], kr[:t + 1], w["scale"])
        np.testing.assert_allclose(oracle.absorb_out(o_lat, w["w_uv"]), o[t], rtol=1e-10, atol=1e-12)
    # position 0 attends only to itself: o_0 = c_0 W_UV
    np.testing.assert_allclose(o[0], oracle.absorb_out(np.broadcast_to(c[0], (4, 32)), w["w_uv"]), rtol=1e-12)


# -------------------------------------------------------------- fp8 (PIN-10)
def test_e4m3_decode_matches_format_and_torch():
    codes = np.arange(256, dtype=np.uint8)
    v = oracle.e4m3_to_f64(codes)
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x38] == 1.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(v[np.isfinite(v)], t[np.isfinite(v)])


def test_e4m3_encode_rne_and_saturation():
    enc = oracle.e4m3_encode
    assert enc(1.0) == 0x38
    assert enc(1.0625) == 0x38          # halfway 1 | 1.125 -> even mantissa (1.0)
    assert enc(1.1875) == 0x3A          # halfway 1.125 | 1.25 -> even mantissa (1.25)
    assert enc(449.0) == 0x7E and enc(1e9) == 0x7E and enc(-1e9) == 0xFE
    assert enc(2.0 ** -10) == 0x00      # halfway 0 | 2^-9 -> even (0)
    assert enc(1.5 * 2.0 ** -9) == 0x02  # halfway 2^-9 | 2^-8 -> even code 2
    finite = [c for c in range(256) if c not in (0x7F, 0xFF, 0x80)]
    back = enc(oracle.e4m3_to_f64(np.array(finite, np.uint8)))
    np.testing.assert_array_equal(back, np.array(finite, np.uint8))
    x = (np.random.default_rng(9).standard_normal(20000) * 100).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(enc(x.astype(np.float64)), ref)


def test_fp8_quantise_bounds():
    rng = np.random.default_rng(4)
    rows = synth.f32_to_bf16_bits(rng.standard_normal((50, 512)).astype(np.float32))
    codes, scales = oracle.fp8_quantize_latent(rows)
    x = oracle.bf16_to_f64(rows).reshape(50, 4, 128)
    deq = oracle.e4m3_to_f64(codes).reshape(50, 4, 128) * scales[..., None]
    bound = np.stack([oracle.quantise_roundtrip_bound(float(s), xg) for s, xg in
                      zip(scales.reshape(-1), x.reshape(-1, 128))]).reshape(x.shape)
    assert (np.abs(deq - x) <= bound * (1 + 1e-6) + 1e-30).all()
    # the group's largest magnitude maps to +-448
    amax_idx = np.abs(x).argmax(-1)
    top = np.take_along_axis(codes.reshape(50, 4, 128), amax_idx[..., None], -1)[..., 0]
    assert np.isin(top, [0x7E, 0xFE]).all()
    # zero group -> scale 1 and zero codes
    z_codes, z_scales = oracle.fp8_quantize_latent(np.zeros((1, 512), np.uint16))
    assert (z_codes == 0).all() and (z_scales == 1).all()


def test_fp8_row_decode_layout():
    codes = np.array([0x38] * 128 + [0xB8] * 128 + [0x40] * 128 + [0x00] * 128, np.uint8)[None]
    rope_bits = synth.f32_to_bf16_bits(np.arange(64, dtype=np.float32))[None]
    scales = np.array([[0.5, 2.0, 0.25, 8.0]], np.float32)
    rec = synth.pack_fp8_rows(codes, rope_bits, scales)
    assert rec.shape[1] == oracle.fp8_row_bytes() == 656
    c, r = oracle.fp8_row_decode(rec)
    np.testing.assert_array_equal(c[0, :128], 0.5)
    np.testing.assert_array_equal(c[0, 128:256], -2.0)
    np.testing.assert_array_equal(c[0, 256:384], 0.5)   # 2.0 * 0.25
    np.testing.assert_array_equal(c[0, 384:], 0.0)
    np.testing.assert_array_equal(r[0], np.arange(64))


# ------------------------------------------------ cache arithmetic (PIN-2)
def test_cache_arithmetic_matches_printed_numbers():
    g = json.load(open(os.path.join(GOLDEN, "cache_arithmetic.json")))
    v3 = g["deepseek_v3"]
    per = oracle.cache_elements_per_token("mla", 1, d_c=v3["kv_lora_rank"], d_r=v3["qk_rope_head_dim"])
    assert per == v3["mla_elements_per_layer"] == synth.ROW
    tot = oracle.cache_elements_per_token("mla", v3["layers"], d_c=512, d_r=64)
    assert tot == v3["mla_elements_all_layers"]
    assert 2 * tot == v3["mla_bytes_bf16_all_layers"]
    assert round(2 * tot / 1024, 1) == v3["mla_kib_bf16_all_layers_rounded_1dp"]
    mha1 = oracle.cache_elements_per_token("mha", 1, n_heads=128, d_h=128)
    mha = oracle.cache_elements_per_token("mha", 61, n_heads=128, d_h=128)
    assert mha1 == v3["mha_twin_elements_per_layer"] and mha == v3["mha_twin_elements_all_layers"]
    assert round(mha / tot, 1) == v3["mha_over_mla_ratio_rounded_1dp"]
    assert round(100 * (1 - tot / mha), 1) == v3["reduction_vs_mha_percent_rounded_1dp"]
    gqa1 = oracle.cache_elements_per_token("gqa", 1, n_groups=8, d_h=128)
    assert round(100 * (1 - per / gqa1), 1) == v3["reduction_vs_gqa8_percent_rounded_1dp"]
    q = g["qwen25_72b_gqa"]
    gq = oracle.cache_elements_per_token("gqa", q["layers"], n_groups=q["kv_heads"], d_h=q["d_h"])
    assert gq == q["gqa_elements_all_layers"] and 2 * gq == q["gqa_bytes_bf16_all_layers"]
    mh = oracle.cache_elements_per_token("mha", 80, n_heads=q["query_heads"], d_h=128)
    assert 2 * mh / 2 ** 20 == q["mha_mib_bf16_per_token"]
    assert 2 * oracle.cache_elements_per_token("mqa", 80, d_h=128) / 1024 == q["mqa_kib_bf16_per_token"]
    seq = g["sequence_128k_gib_bf16"]
    n = 128 * 1024
    assert 2 * mh * n / 2 ** 30 == seq["mha"] and 2 * gq * n / 2 ** 30 == seq["gqa8"]
    assert 2 * oracle.cache_elements_per_token("mqa", 80, d_h=128) * n / 2 ** 30 == seq["mqa"]
    assert round(2 * tot * n / 2 ** 30, 1) == seq["mla_v3_rounded_1dp"]
    cc = g["concurrency_32k_tokens_100gib"]
    assert 2 * gq * 32768 / 2 ** 30 == cc["gqa8_gib_per_seq"]
    assert round(2 * tot * 32768 / 2 ** 30, 2) == cc["mla_gib_per_seq_rounded_2dp"]
    assert int(100 * 2 ** 30 // (2 * gq * 32768)) == cc["gqa8_sequences"]
    assert int(100 * 2 ** 30 // (2 * tot * 32768)) == cc["mla_sequences"]
    # DeepSeek-V2: d_c = 4 d_h, d_r = d_h/2 -> 4.5 d_h per layer = 2.25 groups of 2 d_h
    assert oracle.cache_elements_per_token("mla", 1, d_c=4 * 128, d_r=64) / (2 * 128) == \
        g["deepseek_v2_equivalent_gqa_groups"]


# ----------------------------------------- whole-workload references (CPU)
def test_reference_step_consistent_forms_workload1():
    w = synth.workload(1)
    for b in [0, 5]:
        r = oracle.reference_step(w, b, heads=[0, 7, 15])
        S = int(w["seq_lens"][b])
        rows = oracle.gather_rows(w["cache_step"], w["block_table"], b, S - 1)
        c, kr = oracle.rows_to_latent_rope(rows)
        c = np.concatenate([c, r["new_c"][None]])
        kr = np.concatenate([kr, r["new_kr"][None]])
        o_lat, lse = oracle.decode_absorbed(r["q_lat"], r["q_rot"], c, kr, w["scale"])
        np.testing.assert_allclose(o_lat, r["o_lat"], rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(lse, r["lse"], rtol=1e-12)
        w_uv = oracle.bf16_to_f64(w["w_uv"])[[0, 7, 15]]
        np.testing.assert_allclose(oracle.absorb_out(o_lat, w_uv), r["o"], rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("S", [1, 2, 37, 64])
def test_decode_step_is_the_last_row_of_the_mha_prefill(S):
    """The step's composition, pinned to the MHA form from hidden states
    ([Su] MHA equation with i <= t; Part 2 decoupled RoPE): decoding token
    S - 1 of workload 0 -- prefix rows [c | RoPE(x W_KR, t)] for t < S - 1,
    the new token's latent, unrotated rope key and query projected from
    x[S - 1] -- reproduces row S - 1 of the causal MHA-form prefill.  A query
    or appended key rotated at any other position, or a new row left out of
    the softmax, fails this."""
    w = synth.workload(0)
    o, c, kr, _, _ = oracle.prefill_mha_form(
        w["x"], w["w_dkv"], w["w_kr"], w["w_q"], w["w_uk"], w["w_uv"], w["d_nope"], w["d_r"], w["scale"], w["theta"])
    x = np.asarray(w["x"], np.float64)[S - 1]
    q = (x @ np.asarray(w["w_q"], np.float64)).reshape(w["H"], -1)
    r = oracle.decode_step(q[:, :w["d_nope"]], q[:, w["d_nope"]:], x @ np.asarray(w["w_dkv"], np.float64),
                           x @ np.asarray(w["w_kr"], np.float64), c[:S - 1], kr[:S - 1], w["w_uk"], w["w_uv"],
                           w["scale"], w["theta"])
    np.testing.assert_allclose(r["o"], o[S - 1], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["new_kr"], kr[S - 1], rtol=1e-12, atol=1e-14)


def test_reference_step_passes_the_stored_prefix_and_new_token():
    """reference_step reads exactly the S_b - 1 prefix rows of the step cache
    (the slot of the new row holds poison) in logical order through the page
    table, and the new token from kv_new: equal to decode_step on rows
    gathered here one token at a time."""
    w = synth.gaussian_workload(3, B=3, H=4, seq_lens=[1, 70, 130])
    w_uk, w_uv = oracle.bf16_to_f64(w["w_uk"]), oracle.bf16_to_f64(w["w_uv"])
    for b in range(3):
        S = int(w["seq_lens"][b])
        rows = np.array([w["cache_step"][w["block_table"][b][t // 64], t % 64] for t in range(S - 1)],
                        dtype=np.uint16).reshape(S - 1, 576)
        vals = oracle.bf16_to_f64(rows)
        new = oracle.bf16_to_f64(w["kv_new"][b])
        ref = oracle.decode_step(oracle.bf16_to_f64(w["q_nope"][b]), oracle.bf16_to_f64(w["q_pe"][b]), new[:512],
                                 new[512:], vals[:, :512], vals[:, 512:], w_uk, w_uv, w["scale"], w["theta"])
        r = oracle.reference_step(w, b)
        for k in ("o", "o_lat", "lse", "q_rot", "new_kr", "q_lat"):
            np.testing.assert_array_equal(r[k], ref[k])


def test_reference_decode_empty_sequence():
    w = synth.gaussian_workload(1, B=3, H=2, seq_lens=[0, 1, 65])
    o, l = oracle.reference_decode(w, 0)
    assert (o == 0).all() and np.isneginf(l).all()
    o1, _ = oracle.reference_decode(w, 1)
    c, _ = oracle.rows_to_latent_rope(oracle.gather_rows(w["cache_full"], w["block_table"], 1, 1))
    np.testing.assert_array_equal(o1, np.broadcast_to(c[0], o1.shape))
    r = oracle.reference_step(w, 0)
    assert (r["o"] == 0).all() and np.isneginf(r["lse"]).all()


# ------------------------------------------------- multi-token decode (PIN-11)
def _brute_multi(q, c, kr, scale):
    """Tiny-case brute force: plain Python loops over the masked softmax."""
    q_len, H = len(q), len(q[0])
    S = len(c)
    o = [[None] * H for _ in range(q_len)]
    lse = [[None] * H for _ in range(q_len)]
    for j in range(q_len):
        last = S - q_len + j
        for h in range(H):
            qv = q[j][h]
            sc = []
            for t in range(S):
                if t > last:
                    continue
                dot = sum(qv[d] * c[t][d] for d in range(len(c[t])))
                dot += sum(qv[len(c[t]) + d] * kr[t][d] for d in range(len(kr[t])))
                sc.append((t, scale * dot))
            if not sc:
                o[j][h] = [0.0] * len(c[0])
                lse[j][h] = -math.inf
                continue
            z = sum(math.exp(v) for _, v in sc)
            o[j][h] = [sum(math.exp(v) / z * c[t][d] for t, v in sc) for d in range(len(c[0]))]
            lse[j][h] = math.log(z)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("S,q_len", [(6, 3), (3, 3), (2, 4), (1, 1), (9, 1)])
def test_multi_token_matches_brute_force(S, q_len):
    rng = np.random.default_rng(100 + 10 * S + q_len)
    H, dc, dr = 2, 5, 3
    c, kr = rng.standard_normal((S, dc)), rng.standard_normal((S, dr))
    q = rng.standard_normal((q_len, H, dc + dr))
    o, lse = oracle.decode_multi_token(q[..., :dc], q[..., dc:], c, kr, 0.6)
    ob, lb = _brute_multi(q.tolist(), c.tolist(), kr.tolist(), 0.6)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=1e-12)


def test_multi_token_each_query_is_a_prefix_decode():
    """Query j equals the single-token decode over rows 0 .. S - q_len + j."""
    rng = np.random.default_rng(7)
    S, q_len, H = 130, 5, 4
    c, kr = rng.standard_normal((S, 512)), rng.standard_normal((S, 64))
    q = rng.standard_normal((q_len, H, 576)) * 0.05
    o, lse = oracle.decode_multi_token(q[..., :512], q[..., 512:], c, kr, 0.09)
    for j in range(q_len):
        n = S - q_len + j + 1
        oj, lj = oracle.decode_absorbed(q[j, :, :512], q[j, :, 512:], c[:n], kr[:n], 0.09)
        np.testing.assert_allclose(o[j], oj, rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(lse[j], lj, rtol=1e-13)
    # the last query sees every row; the first does not see the last q_len - 1
    assert not np.allclose(o[0], oracle.decode_absorbed(q[0, :, :512], q[0, :, 512:], c, kr, 0.09)[0])


def test_multi_token_short_sequence_and_single_query():
    rng = np.random.default_rng(8)
    c, kr = rng.standard_normal((1, 512)), rng.standard_normal((1, 64))
    q = rng.standard_normal((3, 2, 576))
    o, lse = oracle.decode_multi_token(q[..., :512], q[..., 512:], c, kr, 0.1)
    # S = 1 < q_len: queries 0 and 1 see nothing; query 2 sees row 0 alone (weight 1)
    assert (o[:2] == 0).all() and np.isneginf(lse[:2]).all()
    np.testing.assert_allclose(o[2], np.broadcast_to(c[0], (2, 512)), rtol=1e-15)
    np.testing.assert_allclose(lse[2], 0.1 * (q[2, :, :512] @ c[0] + q[2, :, 512:] @ kr[0]), rtol=1e-12)
    # q_len = 1 is the decode of every row
    c, kr = rng.standard_normal((40, 512)), rng.standard_normal((40, 64))
    q = rng.standard_normal((1, 3, 576)) * 0.05
    o, lse = oracle.decode_multi_token(q[..., :512], q[..., 512:], c, kr, 0.2)
    o1, l1 = oracle.decode_absorbed(q[0, :, :512], q[0, :, 512:], c, kr, 0.2)
    np.testing.assert_allclose(o[0], o1, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse[0], l1, rtol=1e-13)


def test_reference_decode_multi_last_query_is_the_decode():
    w = synth.gaussian_workload(9, B=3, H=4, seq_lens=[70, 1, 200])
    qm = synth.multi_token_query(10, B=3, q_len=3, H=4)
    qm[:, -1] = w["q_decode"]
    for b in range(3):
        o, lse = oracle.reference_decode_multi(w, qm, b)
        od, ld = oracle.reference_decode(w, b)
        np.testing.assert_allclose(o[-1], od, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(lse[-1], ld, rtol=1e-13)
    o, lse = oracle.reference_decode_multi(w, qm, 1)
    assert (o[:2] == 0).all() and np.isneginf(lse[:2]).all()


# --------------------------------------------- explicit-form prefill (PIN-12)
def _tiny_prefill(rng, T, H, dn=6, dr=4, dc=10, dv=5):
    return (rng.standard_normal((T, H, dn)), rng.standard_normal((T, H, dr)), rng.standard_normal((T, dc)),
            rng.standard_normal((T, dr)), rng.standard_normal((H, dn, dc)) / 3, rng.standard_normal((H, dc, dv)) / 3)


def test_prefill_explicit_matches_brute_force():
    """Plain loops over the causal MHA definition with per-head K and V."""
    rng = np.random.default_rng(21)
    T, H = 7, 2
    qn, qp, c, kp, wuk, wuv = _tiny_prefill(rng, T, H)
    o, rows = oracle.prefill_explicit(qn, qp, c, kp, wuk, wuv, 0.4, theta=100.0)
    kr = oracle.rope(kp, np.arange(T, dtype=float), 100.0)
    qr = oracle.rope(qp, np.arange(T, dtype=float)[:, None], 100.0)
    for t in range(T):
        for h in range(H):
            q = list(qn[t, h]) + list(qr[t, h])
            sc = []
            for i in range(t + 1):
                k = [sum(c[i, m] * wuk[h, d, m] for m in range(c.shape[1])) for d in range(qn.shape[2])] + list(kr[i])
                sc.append(0.4 * sum(a * b for a, b in zip(q, k)))
            z = sum(math.exp(v) for v in sc)
            v_rows = [[sum(c[i, m] * wuv[h, m, e] for m in range(c.shape[1])) for e in range(wuv.shape[2])]
                      for i in range(t + 1)]
            want = [sum(math.exp(sc[i]) / z * v_rows[i][e] for i in range(t + 1)) for e in range(wuv.shape[2])]
            np.testing.assert_allclose(o[t, h], want, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(rows, np.concatenate([c, kr], 1), rtol=0, atol=0)


def test_prefill_rows_equal_absorbed_decode_of_each_prefix():
    """Token t of the prefill equals the absorbed decode of the prefix 0..t
    followed by the value up-projection (the absorption identity)."""
    rng = np.random.default_rng(22)
    T, H = 40, 3
    qn, qp, c, kp = (rng.standard_normal((T, H, 128)), rng.standard_normal((T, H, 64)),
                     rng.standard_normal((T, 512)), rng.standard_normal((T, 64)))
    wuk, wuv = rng.standard_normal((H, 128, 512)) / 22.6, rng.standard_normal((H, 512, 128)) / 22.6
    o, rows = oracle.prefill_explicit(qn, qp, c, kp, wuk, wuv, 1 / math.sqrt(192))
    q_rot = oracle.rope(qp, np.arange(T, dtype=float)[:, None])
    for t in [0, 1, 17, T - 1]:
        o_lat, _ = oracle.decode_absorbed(oracle.absorb_q(qn[t], wuk), q_rot[t], rows[:t + 1, :512],
                                          rows[:t + 1, 512:], 1 / math.sqrt(192))
        np.testing.assert_allclose(oracle.absorb_out(o_lat, wuv), o[t], rtol=1e-10, atol=1e-12)
    # token 0 sees only itself: o_0 = c_0 W_UV
    np.testing.assert_allclose(o[0], np.einsum("m,hme->he", c[0], wuv), rtol=1e-12)


def test_prefill_explicit_equals_mha_form_workload0():
    """From the projections of workload 0, the explicit prefill gives the
    MHA-form result computed from the hidden states."""
    w = synth.workload(0)
    o, c, kr, q_nope, q_rot = oracle.prefill_mha_form(
        w["x"], w["w_dkv"], w["w_kr"], w["w_q"], w["w_uk"], w["w_uv"], w["d_nope"], w["d_r"], w["scale"], w["theta"])
    x = np.asarray(w["x"], np.float64)
    q = (x @ np.asarray(w["w_q"], np.float64)).reshape(w["S"], w["H"], -1)
    o2, rows = oracle.prefill_explicit(q[..., :w["d_nope"]], q[..., w["d_nope"]:], c,
                                       x @ np.asarray(w["w_kr"], np.float64), w["w_uk"], w["w_uv"],
                                       w["scale"], w["theta"])
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(rows[:, w["d_c"]:], kr, rtol=1e-13, atol=1e-15)


# ------------------------------------------ chunked prefill over a cached prefix
def test_prefill_chunk_continues_the_whole_prompt():
    """A prompt cut at P: its first P cache rows as the prefix and the rest as
    the chunk give the whole prompt's outputs and rows for tokens P.. ."""
    rng = np.random.default_rng(31)
    T, H = 23, 2
    qn, qp, c, kp, wuk, wuv = _tiny_prefill(rng, T, H)
    o, rows = oracle.prefill_explicit(qn, qp, c, kp, wuk, wuv, 0.4, theta=100.0)
    for P in [0, 1, 7, 22]:
        oc, rc = oracle.prefill_chunk_explicit(qn[P:], qp[P:], c[P:], kp[P:], rows[:P, :10], rows[:P, 10:], wuk, wuv,
                                               0.4, theta=100.0)
        np.testing.assert_allclose(oc, o[P:], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(rc, rows[P:], rtol=1e-13, atol=1e-15)


def test_prefill_chunk_brute_force():
    """Loops over the definition with an arbitrary cached prefix: chunk token
    j sits at position P + j (its query and key rotated there) and sees the
    P prefix rows and chunk tokens 0..j."""
    rng = np.random.default_rng(32)
    P, n, H = 5, 4, 2
    qn, qp, c, kp, wuk, wuv = _tiny_prefill(rng, n, H)
    c_pre, kr_pre = rng.standard_normal((P, 10)), rng.standard_normal((P, 4))
    o, rows = oracle.prefill_chunk_explicit(qn, qp, c, kp, c_pre, kr_pre, wuk, wuv, 0.3, theta=50.0)

    def turn(v, pos):   # pairs (2i, 2i+1) turned by pos * 50^(-2i/d)
        d = len(v)
        out = []
        for i in range(d // 2):
            a = pos * 50.0 ** (-2.0 * i / d)
            out += [v[2 * i] * math.cos(a) - v[2 * i + 1] * math.sin(a), v[2 * i] * math.sin(a) + v[2 * i + 1] * math.cos(a)]
        return out
    keys_c = list(c_pre) + list(c)
    keys_r = [list(r) for r in kr_pre] + [turn(kp[j], P + j) for j in range(n)]
    for j in range(n):
        for h in range(H):
            q = list(qn[j, h]) + turn(qp[j, h], P + j)
            sc = []
            for i in range(P + j + 1):
                k = [sum(keys_c[i][m] * wuk[h, d, m] for m in range(10)) for d in range(6)] + keys_r[i]
                sc.append(0.3 * sum(a * b for a, b in zip(q, k)))
            z = sum(math.exp(v) for v in sc)
            want = [sum(math.exp(sc[i]) / z * sum(keys_c[i][m] * wuv[h, m, e] for m in range(10)) for i in range(P + j + 1))
                    for e in range(5)]
            np.testing.assert_allclose(o[j, h], want, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(rows[j], list(c[j]) + keys_r[P + j], rtol=1e-13, atol=1e-15)


def test_prefill_chunk_equals_mha_form_workload0():
    """Workload 0 cut at position 40: the prefix rows of the MHA form and the
    remaining tokens' projections reproduce the MHA form's last 24 outputs."""
    w = synth.workload(0)
    o, c, kr, q_nope, q_rot = oracle.prefill_mha_form(
        w["x"], w["w_dkv"], w["w_kr"], w["w_q"], w["w_uk"], w["w_uv"], w["d_nope"], w["d_r"], w["scale"], w["theta"])
    x = np.asarray(w["x"], np.float64)
    q = (x @ np.asarray(w["w_q"], np.float64)).reshape(w["S"], w["H"], -1)
    P = 40
    oc, rows = oracle.prefill_chunk_explicit(q[P:, :, :w["d_nope"]], q[P:, :, w["d_nope"]:], c[P:],
                                             (x @ np.asarray(w["w_kr"], np.float64))[P:], c[:P], kr[:P],
                                             w["w_uk"], w["w_uv"], w["scale"], w["theta"])
    np.testing.assert_allclose(oc, o[P:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(rows[:, w["d_c"]:], kr[P:], rtol=1e-13, atol=1e-15)


# ------------------------------------- query from its low-rank latent (NEXT-4)
def test_query_from_latent_brute_force():
    """Loops over the definition: q_h = c' W_UQ[:, head h's columns], the
    first d_nope entries times W_UK[h], the last d_r turned pair by pair."""
    rng = np.random.default_rng(21)
    B, dq, H, dn, dr, dc = 3, 5, 2, 3, 4, 6
    c_q = _rand(B, dq, rng=rng)
    w_uq = _rand(dq, H * (dn + dr), rng=rng)
    w_uk = _rand(H, dn, dc, rng=rng)
    pos = np.array([0, 7, 123])
    theta = 100.0
    q_lat, q_rot = oracle.query_from_latent(c_q, w_uq, w_uk, pos, theta, d_nope=dn)
    for b in range(B):
        for h in range(H):
            q = [sum(c_q[b][k] * w_uq[k][h * (dn + dr) + j] for k in range(dq)) for j in range(dn + dr)]
            lat = [sum(q[n] * w_uk[h][n][c] for n in range(dn)) for c in range(dc)]
            np.testing.assert_allclose(q_lat[b, h], lat, rtol=1e-12, atol=1e-13)
            for i in range(dr // 2):
                ang = pos[b] * theta ** (-2.0 * i / dr)
                x1, x2 = q[dn + 2 * i], q[dn + 2 * i + 1]
                assert abs(q_rot[b, h, 2 * i] - (x1 * math.cos(ang) - x2 * math.sin(ang))) < 1e-12
                assert abs(q_rot[b, h, 2 * i + 1] - (x1 * math.sin(ang) + x2 * math.cos(ang))) < 1e-12


def test_query_from_latent_equals_merged_product():
    """Sequential and merged orders reach the same q_lat in exact arithmetic
    ([Su] MLA additional notes): c' (W_UQ_nope W_UK) to 1e-12."""
    rng = np.random.default_rng(22)
    B, dq, H, dn, dr, dc = 4, 24, 3, 8, 4, 16
    c_q, w_uq, w_uk = _rand(B, dq, rng=rng), _rand(dq, H * (dn + dr), rng=rng), _rand(H, dn, dc, rng=rng)
    q_lat, _ = oracle.query_from_latent(c_q, w_uq, w_uk, 0, d_nope=dn)
    for h in range(H):
        merged = w_uq[:, h * (dn + dr):h * (dn + dr) + dn] @ w_uk[h]
        np.testing.assert_allclose(q_lat[:, h], c_q @ merged, rtol=1e-12, atol=1e-12)


# ------------------------------ merged vs sequential absorption (study)
def test_merged_and_sequential_query_absorption_precision():
    """[Su] MLA additional notes 1-2 weigh merging W_UQ W_UK^T into one matrix
    against applying the two projections in turn.  With bf16 operands and
    exactly accumulated products (what the MFMA path does), both land within
    the final bf16 rounding of q_lat of the exact product, and within a few
    percent of each other; the merged matrix costs d_q/d_n = 12x the weight
    bytes per head of W_UK (1536 x 512 vs 128 x 512) and 3x the FLOPs of the
    sequential pair, so the path keeps the sequential form."""
    rng = np.random.default_rng(11)
    B, dq, dn, dc, H = 64, 1536, 128, 512, 4

    def bf(x):
        return oracle.bf16_to_f64(synth.f32_to_bf16_bits(np.asarray(x, np.float64)))
    x = bf(rng.standard_normal((B, dq)))
    wuq = bf(rng.standard_normal((H, dq, dn)) / math.sqrt(dq))
    wuk = bf(rng.standard_normal((H, dn, dc)) / math.sqrt(dc))
    for h in range(H):
        exact = x @ wuq[h] @ wuk[h]
        seq = bf(bf(x @ wuq[h]) @ wuk[h])
        merged = bf(x @ bf(wuq[h] @ wuk[h]))
        e_seq = np.sqrt(((seq - exact) ** 2).sum() / (exact ** 2).sum())
        e_mer = np.sqrt(((merged - exact) ** 2).sum() / (exact ** 2).sum())
        assert e_seq < 2.0 ** -8 and e_mer < 2.0 ** -8
        assert abs(e_seq - e_mer) < 0.1 * max(e_seq, e_mer)
    # cost per token and head (multiply-adds): sequential d_q d_n + d_n d_c, merged d_q d_c
    assert (dq * dc) / (dq * dn + dn * dc) == 3.0
