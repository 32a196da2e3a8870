"""fp64 CPU oracle for MLA absorbed decode over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the library or its binding imports or
calls this module; only the test-suite, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the HIP path.

Every function computes the plain definition of what the method reaches, in
numpy float64, with library matmuls as the only building blocks and no
blocking or fusion beyond what the definitions state.  Inputs are the exact
values of the stored tensors (bf16 bit patterns, fp8 codes times their fp32
group scales), widened to float64.

Sources (cited by title and section):
  [Su]   "The Ultimate Tug-of-War Between Cache and Performance: From MHA, MQA,
         GQA to MLA" -- the MHA equation, the MLA Part 1 absorption identity,
         the Part 2 decoupled-RoPE equation, and the Part 3 MHA form
         (eq:mla-mha) and decoding-stage MQA form (eq:mla-mqa).
  [Riju] "Multi-Head Latent Attention vs GQA vs MQA: KV-Cache Compression
         Explained" -- "A latent KV projection in PyTorch" (the RoPE pair
         convention, non-absorbed module, absorbed decode sketch, the
         equivalence test),
         "Worked numbers from real configs", "Interaction with quantisation
         and paging".
  [DL0107] "DL0107 Multi-head Latent Attention MLA" -- the cache holds the
         latent and the decoupled RoPE key in rotated form.

Readings where the pages are silent (each is listed with its reason in the
design notes): interleaved RoPE pairs; the decode query sits at position
S-1 and attends to itself; softmax scale 1/sqrt(d_nope + d_rope) on the sum of
the latent and rotary score parts; empty sequence -> zero output and
lse = -inf; several new tokens decoded together see the cache causally (query
j of q_len at position S-q_len+j sees rows 0..S-q_len+j); fp8 = OCP E4M3 (max 448) with one fp32 scale per 128-wide group,
scale = amax/448 in fp32 and codes by round-to-nearest-even after an fp32
division.

Parity pins: every function here is pinned by a test under tests/ against a
closed form, a brute-force evaluation, a library routine or a number printed
on the pages.  The fp8 scale formula is pinned only by internal consistency
(parity unpinned against the pages, which give no quantiser).
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64

# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(F64)


def e4m3_to_f64(codes) -> np.ndarray:
    """OCP E4M3 (e4m3fn) byte codes -> float64.

    Layout s.eeee.mmm, exponent bias 7; e == 0 encodes subnormals m/8 * 2^-6;
    S.1111.111 is NaN; there is no infinity, so the largest finite value is
    1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = s * mag
    return np.where((e == 15) & (m == 7), np.nan, val).astype(F64)


_E4M3_POS = e4m3_to_f64(np.arange(0, 127, dtype=np.uint8))   # codes 0..126, ascending
E4M3_MAX = 448.0


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code to each value (ties to the even code), saturating at +-448.

    Implemented as a nearest-neighbour search over the table of the 127
    non-negative finite values, so it shares nothing with a bit-twiddling
    encoder.
    """
    x = np.asarray(x, dtype=F64)
    if np.isnan(x).any():
        raise ValueError("NaN has no saturating e4m3 encoding here")
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_hi = _E4M3_POS[hi] - a
    d_lo = a - _E4M3_POS[lo]
    take_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(take_lo, lo, hi).astype(np.uint8)
    neg = (x < 0) & (code != 0)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def fp8_quantize_latent(c_bits, group=128):
    """Quantise bf16 latent rows [..., 512] into e4m3 codes and fp32 group scales.

    Per row and per group of `group` values: scale = amax / 448 computed as an
    IEEE float32 division (1 when amax == 0); code = round-to-nearest-even of
    float32(c / scale), saturated to +-448.  Both divisions are float32, as the
    GPU computes them, so the integer codes are decided in the same precision.
    """
    c = np.asarray(bf16_to_f64(c_bits), dtype=np.float32)      # exact widening
    shp = c.shape
    g = c.reshape(shp[:-1] + (shp[-1] // group, group))
    amax = np.abs(g).max(axis=-1)
    scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    q = (g / scale[..., None]).astype(np.float32)
    codes = e4m3_encode(q.astype(F64)).reshape(shp)
    return codes, scale


def fp8_row_decode(rec):
    """Packed fp8 cache records [..., 656] bytes -> (latent [...,512], rope [...,64]) float64."""
    rec = np.asarray(rec, dtype=np.uint8)
    codes = rec[..., :512]
    rope_bits = np.ascontiguousarray(rec[..., 512:640]).view(np.uint16)
    scales = np.ascontiguousarray(rec[..., 640:656]).view(np.float32).astype(F64)
    c = e4m3_to_f64(codes).reshape(codes.shape[:-1] + (4, 128)) * scales[..., None]
    return c.reshape(codes.shape), bf16_to_f64(rope_bits)


# --------------------------------------------------------------------------
# rotary position embedding  ([Su] Part 2, the rotation R_m)
# --------------------------------------------------------------------------


def rope(v, pos, theta=10000.0) -> np.ndarray:
    """Apply R_pos to v: the block-diagonal rotation of [Su] Part 2.

    Block i of R_m acts on the interleaved pair (v[2i], v[2i+1]) and turns it
    by the angle m * w_i, w_i = theta^(-2i/d).  Written here in complex form:
    the pair is z_i = v[2i] + 1j v[2i+1], R_m multiplies it by the unit phasor
    e^(1j m w_i), and the real and imaginary parts go back to slots 2i and
    2i+1.  R_m R_n^T = R_(m-n) holds because the phasors multiply.

    v: [..., d] (d even); pos: scalar or array broadcastable to v[..., 0].
    """
    v = np.asarray(v, dtype=F64)
    d = v.shape[-1]
    half = d // 2
    omega = np.power(F64(theta), -2.0 * np.arange(half, dtype=F64) / d)
    pairs = v.reshape(v.shape[:-1] + (half, 2))
    z = pairs[..., 0] + 1j * pairs[..., 1]
    phasor = np.exp(1j * (np.asarray(pos, dtype=F64)[..., None] * omega))
    w = z * phasor
    return np.stack([w.real, w.imag], axis=-1).reshape(w.shape[:-1] + (d,))


# --------------------------------------------------------------------------
# absorption ([Su] MLA Part 1 identity and eq:mla-mqa)
# --------------------------------------------------------------------------


def absorb_q(q_nope, w_uk) -> np.ndarray:
    """q_lat[..., h, :] = q_nope[..., h, :] W_UK[h]   (W_UK: [H, d_nope, d_c]).

    The query side of the absorbed score: q^(s) k_i^(s)T = (x W_q^(s)) W_k^(s)T c_i^T
    evaluated in the sequential order ([Su], MLA additional notes 1-2).
    """
    q = np.asarray(q_nope, dtype=F64)
    w = np.asarray(w_uk, dtype=F64)
    return np.einsum("...hn,hnc->...hc", q, w)


def query_from_latent(c_q, w_uq, w_uk, pos, theta=10000.0, d_nope=128):
    """Absorbed decode query from the low-rank query latent, sequential order.

    [Su] Part 3 (queries pass through their own low-rank latent c'_i) and MLA
    additional notes 1-2 (the up-projection and W_UK are applied one after the
    other, never merged); [Riju] "Query compression is separate".  For each
    head h, with W_UQ's output split head-major into [nope | rope] (the
    layout reading of the configs):
        q_h   = c_q W_UQ[:, h (d_nope + d_r) : (h + 1) (d_nope + d_r)]
        q_lat = q_h[:d_nope] W_UK[h]            (absorb_q)
        q_rot = RoPE(q_h[d_nope:], pos)         (rope, the query's position)
    c_q [B, d_q], w_uq [d_q, H (d_nope + d_r)], w_uk [H, d_nope, d_c],
    pos [B] (or scalar).  Returns (q_lat [B, H, d_c], q_rot [B, H, d_r]).
    """
    c_q = np.asarray(c_q, F64)
    w_uq = np.asarray(w_uq, F64)
    w_uk = np.asarray(w_uk, F64)
    H = w_uk.shape[0]
    q = (c_q @ w_uq).reshape(c_q.shape[0], H, -1)
    q_lat = absorb_q(q[..., :d_nope], w_uk)
    q_rot = rope(q[..., d_nope:], np.asarray(pos, F64).reshape(-1, 1), theta)
    return q_lat, q_rot


def absorb_out(o_lat, w_uv) -> np.ndarray:
    """o[..., h, :] = o_lat[..., h, :] W_UV[h]   (W_UV: [H, d_c, d_v]); [Su] eq:mla-mqa first line."""
    o = np.asarray(o_lat, dtype=F64)
    w = np.asarray(w_uv, dtype=F64)
    return np.einsum("...hc,hcv->...hv", o, w)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------


def softmax_lse(s):
    """Row softmax of scores s [..., S] and its log-sum-exp; empty rows give (zeros, -inf).

    [Su] MHA equation: weights exp(q k^T) / sum_i exp(q k^T), evaluated with the
    row maximum subtracted.
    """
    s = np.asarray(s, dtype=F64)
    if s.shape[-1] == 0:
        return np.zeros(s.shape, F64), np.full(s.shape[:-1], -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[..., 0]


def decode_explicit(q_nope, q_rot, c, kr, w_uk, w_uv, scale, heads=None):
    """One decode step of one sequence with per-head K and V rebuilt explicitly.

    q_nope [H, d_nope], q_rot [H, d_r] (already rotated at the query position),
    c [S, d_c] latents and kr [S, d_r] rotated shared keys of the S visible
    tokens, W_UK [H, d_nope, d_c], W_UV [H, d_c, d_v].

    For each head h ([Su] Part 2 decoupled-RoPE equation / eq:mla-mha;
    [Riju] non-absorbed module):
        K_h = [c W_UK[h]^T | kr],  V_h = c W_UV[h]
        s   = scale * [q_nope[h] | q_rot[h]] . K_h^T
        p   = softmax(s),  o[h] = p V_h
    Also returns o_lat[h] = p c (the latent-weighted sum the absorbed form
    produces, from the same p) and lse[h].
    """
    c = np.asarray(c, F64)
    kr = np.asarray(kr, F64)
    H = np.asarray(q_nope).shape[0]
    heads = range(H) if heads is None else heads
    o, o_lat, lse = [], [], []
    for h in heads:
        k_h = np.concatenate([c @ np.asarray(w_uk[h], F64).T, kr], axis=1)
        v_h = c @ np.asarray(w_uv[h], F64)
        qh = np.concatenate([np.asarray(q_nope[h], F64), np.asarray(q_rot[h], F64)])
        p, l = softmax_lse(scale * (k_h @ qh))
        o.append(p @ v_h if len(p) else np.zeros(v_h.shape[1]))
        o_lat.append(p @ c if len(p) else np.zeros(c.shape[1]))
        lse.append(l)
    return np.array(o), np.array(o_lat), np.array(lse)


def decode_absorbed(q_lat, q_rot, c, kr, scale, with_magnitude=False):
    """The decoding-stage MQA form ([Su] eq:mla-mqa; [Riju] absorbed decode sketch).

    q_lat [H, d_c], q_rot [H, d_r]; every head scores the shared key [c | kr]:
        s = scale * (q_lat . c^T + q_rot . kr^T),  o_lat = softmax(s) c.
    with_magnitude also returns sum_t p_t |c_t|, the scale against which a
    relative perturbation of the weights p moves o_lat (used to state
    tolerances; it is not part of the method).
    """
    c = np.asarray(c, F64)
    kr = np.asarray(kr, F64)
    s = scale * (np.asarray(q_lat, F64) @ c.T + np.asarray(q_rot, F64) @ kr.T)
    p, lse = softmax_lse(s)
    empty = np.zeros((s.shape[0], c.shape[1]))
    o_lat = p @ c if c.shape[0] else empty
    if with_magnitude:
        return o_lat, lse, (p @ np.abs(c) if c.shape[0] else empty)
    return o_lat, lse


def decode_multi_token(q_lat, q_rot, c, kr, scale):
    """Decode of q_len new tokens of one sequence against its whole cache.

    [Riju] "Interaction with quantisation and paging": speculative decoding
    and multi-token prediction heads use the latent cache like any other
    decode; read here as the causal rule of decoder attention ([Su] MHA
    equation with the decoder's causal mask): the new tokens are the last
    q_len of the S cached rows, and query j (position S - q_len + j) sees the
    rows t <= S - q_len + j.
        q_lat [q_len, H, d_c], q_rot [q_len, H, d_r]; c [S, d_c], kr [S, d_r]
        s[j,h,t] = scale * (q_lat[j,h] . c_t + q_rot[j,h] . kr_t)  (visible t)
        o_lat[j,h] = sum_t softmax(s[j,h])_t c_t,  lse[j,h] = log sum_t e^s
    A query that sees no row (S - q_len + j < 0) gives zeros and lse = -inf.
    Written with an explicit visibility mask over all S rows.
    """
    q_lat = np.asarray(q_lat, F64)
    q_rot = np.asarray(q_rot, F64)
    c = np.asarray(c, F64)
    kr = np.asarray(kr, F64)
    q_len, H = q_lat.shape[:2]
    S = c.shape[0]
    s = scale * (q_lat.reshape(q_len * H, -1) @ c.T + q_rot.reshape(q_len * H, -1) @ kr.T)
    s = s.reshape(q_len, H, S)
    last = S - q_len + np.arange(q_len)                     # last visible row of query j
    visible = np.arange(S)[None, :] <= last[:, None]        # [q_len, S]
    vis = np.broadcast_to(visible[:, None, :], s.shape)
    any_vis = vis.any(axis=-1)
    m = np.where(any_vis, np.where(vis, s, -np.inf).max(axis=-1, initial=-np.inf), 0.0)
    e = np.where(vis, np.exp(np.where(vis, s, 0.0) - m[..., None]), 0.0)
    z = e.sum(axis=-1)
    zs = np.where(any_vis, z, 1.0)
    o_lat = (e / zs[..., None]).reshape(q_len * H, S) @ c if S else np.zeros((q_len * H, c.shape[1]))
    o_lat = np.where(any_vis[..., None], o_lat.reshape(q_len, H, -1), 0.0)
    lse = np.where(any_vis, m + np.log(zs), -np.inf)
    return o_lat, lse


def combine_partials(o_parts, lse_parts):
    """Merge attention over disjoint token chunks from (o_c, lse_c) pairs.

    o = sum_c w_c o_c / sum_c w_c with w_c = exp(lse_c - L), L = max_c lse_c;
    lse = L + log sum_c w_c.  Chunks with lse = -inf carry weight 0; if all are
    empty the result is (0, -inf).  This is the softmax definition regrouped
    over a partition of the tokens.
    """
    o_parts = np.asarray(o_parts, F64)
    lse_parts = np.asarray(lse_parts, F64)
    L = lse_parts.max(axis=0)
    finite = np.isfinite(L)
    Ls = np.where(finite, L, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - Ls), 0.0)
    z = w.sum(axis=0)
    zs = np.where(z > 0, z, 1.0)
    o = (w[..., None] * o_parts).sum(axis=0) / zs[..., None]
    lse = np.where(finite, Ls + np.log(zs), -np.inf)
    return np.where(finite[..., None], o, 0.0), lse


# --------------------------------------------------------------------------
# paged cache access ([Riju] "Interaction with quantisation and paging")
# --------------------------------------------------------------------------


def gather_rows(pool, block_table, b, n_tokens, block_size=64):
    """Logical rows 0..n_tokens-1 of sequence b from a paged pool [N_blk, block, ...].

    block_table[b][j] is the physical page holding tokens [j*block, (j+1)*block).
    """
    idx = np.arange(n_tokens)
    pages = np.asarray(block_table)[b, idx // block_size]
    return np.asarray(pool)[pages, idx % block_size]


def rows_to_latent_rope(rows, kv_fp8=False, d_c=512):
    """Stored rows -> (c [S,d_c], kr [S,d_r]) as float64."""
    if kv_fp8:
        return fp8_row_decode(rows)
    r = bf16_to_f64(rows)
    return r[:, :d_c], r[:, d_c:]


# --------------------------------------------------------------------------
# whole-step references over a synthetic workload
# --------------------------------------------------------------------------


def reference_decode(inp, b, heads=None, with_magnitude=False):
    """Decode-only reference for sequence b: the stored cache and query as given.

    Q = inp["q_decode"] [B,H,576] (latent query | rotated query), all S_b rows of
    inp["cache_full"] attended.  Returns (o_lat [h,512], lse [h]) and, with
    with_magnitude, sum_t p_t |c_t| as a third item.
    """
    S = int(inp["seq_lens"][b])
    fp8 = inp["kv_dtype"] == 1
    rows = gather_rows(inp["cache_full"], inp["block_table"], b, S, inp["block_size"])
    c, kr = rows_to_latent_rope(rows, fp8)
    q = bf16_to_f64(inp["q_decode"][b])
    heads = list(range(q.shape[0])) if heads is None else list(heads)
    return decode_absorbed(q[heads, :512], q[heads, 512:], c, kr, inp["scale"], with_magnitude)


def reference_decode_multi(inp, q_multi, b, heads=None):
    """Multi-token decode reference for sequence b: queries q_multi [B, q_len, H, 576]
    (bf16 bits) against all S_b rows of inp["cache_full"] (decode_multi_token).
    Returns (o_lat [q_len, h, 512], lse [q_len, h])."""
    S = int(inp["seq_lens"][b])
    fp8 = inp["kv_dtype"] == 1
    rows = gather_rows(inp["cache_full"], inp["block_table"], b, S, inp["block_size"])
    c, kr = rows_to_latent_rope(rows, fp8)
    q = bf16_to_f64(np.asarray(q_multi)[b])
    heads = list(range(q.shape[1])) if heads is None else list(heads)
    q = q[:, heads]
    return decode_multi_token(q[..., :512], q[..., 512:], c, kr, inp["scale"])


def decode_step(q_nope, q_pe, new_c, new_k_pe, c_prefix, kr_prefix, w_uk, w_uv, scale, theta=10000.0,
                heads=None):
    """One decode step of one sequence from values (explicit K/V form).

    The sequence holds S = len(c_prefix) + 1 tokens after the step; the new
    token is the last, at position S - 1 ([Su] MHA equation: token t attends
    to i <= t, itself included; [Riju] absorbed decode sketch: the new latent
    and rotated key are appended before attending).  Its key row is
    [new_c | RoPE(new_k_pe, S - 1)] and its query [q_nope | RoPE(q_pe, S - 1)];
    prefix row t (rotated at position t when it was cached) is
    [c_prefix[t] | kr_prefix[t]].
        q_nope [H, d_nope], q_pe [H, d_r] (unrotated), new_c [d_c],
        new_k_pe [d_r] (unrotated), c_prefix [S-1, d_c], kr_prefix [S-1, d_r]
    Returns a dict with q_rot, new_kr, q_lat, o_lat, lse and o for the heads.
    """
    c_prefix = np.asarray(c_prefix, F64)
    pos = c_prefix.shape[0]
    H = np.asarray(q_nope).shape[0]
    heads = list(range(H)) if heads is None else list(heads)
    q_nope = np.asarray(q_nope, F64)
    q_rot = rope(np.asarray(q_pe, F64), pos, theta)
    new_kr = rope(np.asarray(new_k_pe, F64), pos, theta)
    c = np.concatenate([c_prefix, np.asarray(new_c, F64)[None]], 0)
    kr = np.concatenate([np.asarray(kr_prefix, F64).reshape(pos, new_kr.shape[0]), new_kr[None]], 0)
    o, o_lat, lse = decode_explicit(q_nope, q_rot, c, kr, w_uk, w_uv, scale, heads)
    w_uk_h = np.asarray(w_uk, F64)[heads]
    return dict(q_rot=q_rot[heads], new_kr=new_kr, q_lat=absorb_q(q_nope[heads], w_uk_h),
                o_lat=o_lat, lse=lse, o=o)


def reference_step(inp, b, heads=None):
    """Full decode step for sequence b from the stored step inputs.

    Decodes the storage formats and runs decode_step on sequence b's S_b - 1
    cached prefix rows (inp["cache_step"]) and its new token inp["kv_new"][b]
    (fp8 caches: the new latent quantised and dequantised by this module's
    quantiser, as the append stores it).  Returns decode_step's dict plus
    new_c (and new_codes / new_scales for fp8).  S_b = 0 is an empty slot:
    zero outputs and lse = -inf, the query rotated at position 0.
    """
    S = int(inp["seq_lens"][b])
    H = inp["H"]
    heads = list(range(H)) if heads is None else list(heads)
    fp8 = inp["kv_dtype"] == 1
    theta = inp["theta"]
    new = inp["kv_new"][b]
    out = {}
    if fp8:
        codes, scales = fp8_quantize_latent(new[:512])
        out["new_codes"], out["new_scales"] = codes, scales
        new_c = (e4m3_to_f64(codes).reshape(4, 128) * scales.astype(F64)[:, None]).reshape(512)
    else:
        new_c = bf16_to_f64(new[:512])
    out["new_c"] = new_c
    q_nope = bf16_to_f64(inp["q_nope"][b])
    q_pe = bf16_to_f64(inp["q_pe"][b])
    w_uk = bf16_to_f64(inp["w_uk"])
    if S == 0:
        n = len(heads)
        out.update(q_rot=rope(q_pe[heads], 0, theta), new_kr=rope(bf16_to_f64(new[512:]), 0, theta),
                   q_lat=absorb_q(q_nope[heads], w_uk[heads]),
                   o_lat=np.zeros((n, 512)), lse=np.full(n, -np.inf), o=np.zeros((n, 128)))
        return out
    rows = gather_rows(inp["cache_step"], inp["block_table"], b, S - 1, inp["block_size"])
    c, kr = rows_to_latent_rope(rows, fp8)
    out.update(decode_step(q_nope, q_pe, new_c, bf16_to_f64(new[512:]), c, kr, w_uk, bf16_to_f64(inp["w_uv"]),
                           inp["scale"], theta, heads))
    return out


# --------------------------------------------------------------------------
# MHA-form prefill (tiny fp32 workload): [Su] eq:mla-mha without the query
# latent, i.e. the Part 2 equation; [Riju] non-absorbed module with is_causal
# --------------------------------------------------------------------------


def prefill_mha_form(x, w_dkv, w_kr, w_q, w_uk, w_uv, d_nope, d_r, scale, theta=10000.0):
    """Causal attention over all positions of x [S, d] in the explicit (MHA) form.

    c_t = x_t W_DKV, kr_t = RoPE(x_t W_KR, t), q_t^(h) = [x_t W_Q^(h)_nope |
    RoPE(x_t W_Q^(h)_rope, t)], K^(h) = [c W_UK[h]^T | kr], V^(h) = c W_UV[h];
    o_t^(h) = sum_{i<=t} softmax_i(scale q_t^(h) . K_i^(h)) V_i^(h).
    Returns (o [S,H,d_v], c [S,d_c], kr [S,d_r], q_nope [S,H,d_nope], q_rot [S,H,d_r]).
    """
    x = np.asarray(x, F64)
    S = x.shape[0]
    H = np.asarray(w_uk).shape[0]
    pos = np.arange(S, dtype=F64)
    c = x @ np.asarray(w_dkv, F64)
    kr = rope(x @ np.asarray(w_kr, F64), pos, theta)
    q = (x @ np.asarray(w_q, F64)).reshape(S, H, d_nope + d_r)
    q_nope = q[..., :d_nope]
    q_rot = rope(q[..., d_nope:], pos[:, None], theta)
    o = np.zeros((S, H, np.asarray(w_uv).shape[2]))
    for h in range(H):
        k_h = np.concatenate([c @ np.asarray(w_uk[h], F64).T, kr], 1)
        v_h = c @ np.asarray(w_uv[h], F64)
        q_h = np.concatenate([q_nope[:, h], q_rot[:, h]], 1)
        s = scale * (q_h @ k_h.T)
        s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
        p, _ = softmax_lse(s)
        o[:, h] = p @ v_h
    return o, c, kr, q_nope, q_rot


def prefill_explicit(q_nope, q_pe, c, k_pe, w_uk, w_uv, scale, theta=10000.0, with_magnitude=False):
    """Causal prefill of one prompt of T tokens in the explicit (MHA) form, from its
    projected inputs.

    [Su] Part 3 MHA form (eq:mla-mha) with the Part 2 decoupled RoPE; [Riju]
    non-absorbed module.  Token t sits at position t.  q_nope [T,H,d_nope],
    q_pe [T,H,d_r] and k_pe [T,d_r] unrotated, c [T,d_c], W_UK [H,d_nope,d_c],
    W_UV [H,d_c,d_v]:
        K^(h) = [c W_UK[h]^T | RoPE(k_pe)],  V^(h) = c W_UV[h],
        Q^(h) = [q_nope[:,h] | RoPE(q_pe[:,h])]
        o_t^(h) = sum_{i<=t} softmax_i(scale Q_t^(h) . K_i^(h)) V_i^(h)
    Returns (o [T,H,d_v], rows [T, d_c + d_r]) where rows are the latent-cache
    rows [c_t | RoPE(k_pe_t, t)] the prompt leaves behind; with_magnitude also
    returns sum_i p_i |V_i| [T,H,d_v], the scale against which a relative
    perturbation of the weights or values moves o (for stating tolerances;
    not part of the method).
    """
    q_nope = np.asarray(q_nope, F64)
    c = np.asarray(c, F64)
    T, H = q_nope.shape[:2]
    pos = np.arange(T, dtype=F64)
    kr = rope(np.asarray(k_pe, F64), pos, theta)
    q_rot = rope(np.asarray(q_pe, F64), pos[:, None], theta)
    causal = np.tril(np.ones((T, T), bool))
    o = np.zeros((T, H, np.asarray(w_uv).shape[2]))
    mag = np.zeros_like(o)
    for h in range(H):
        k_h = np.concatenate([c @ np.asarray(w_uk[h], F64).T, kr], 1)
        v_h = c @ np.asarray(w_uv[h], F64)
        q_h = np.concatenate([q_nope[:, h], q_rot[:, h]], 1)
        p, _ = softmax_lse(np.where(causal, scale * (q_h @ k_h.T), -np.inf))
        o[:, h] = p @ v_h
        if with_magnitude:
            mag[:, h] = p @ np.abs(v_h)
    rows = np.concatenate([c, kr], 1)
    return (o, rows, mag) if with_magnitude else (o, rows)


def prefill_chunk_explicit(q_nope, q_pe, c, k_pe, c_prefix, kr_prefix, w_uk, w_uv, scale, theta=10000.0,
                           with_magnitude=False):
    """A prompt chunk that continues a cached prefix, in the explicit (MHA) form.

    [Su] Part 3 MHA form (eq:mla-mha) and the causal MHA equation (query t
    attends to keys i <= t); [Riju] "Prefill versus decode" (the prefill and
    the decode share one cache).  The prefix's P rows are already cached:
    c_prefix [P, d_c] and kr_prefix [P, d_r], the latter rotated at positions
    0..P-1.  Chunk token j (q_nope [n,H,d_nope], q_pe [n,H,d_r], c [n,d_c],
    k_pe [n,d_r], unrotated) sits at position P + j and attends to the keys at
    positions 0..P + j:
        K^(h) = [[c_prefix; c] W_UK[h]^T | [kr_prefix; RoPE(k_pe, P + j)]]
        V^(h) = [c_prefix; c] W_UV[h]
        o_j^(h) = sum_{i <= P+j} softmax_i(scale [q_nope | RoPE(q_pe, P+j)]_j . K_i^(h)) V_i^(h)
    Returns (o [n,H,d_v], rows [n, d_c + d_r]) with the chunk's cache rows
    [c_j | RoPE(k_pe_j, P + j)]; with_magnitude also returns sum_i p_i |V_i|.
    """
    q_nope = np.asarray(q_nope, F64)
    c = np.asarray(c, F64)
    c_prefix = np.asarray(c_prefix, F64).reshape(-1, c.shape[1])
    P = c_prefix.shape[0]
    n, H = q_nope.shape[:2]
    pos = P + np.arange(n, dtype=F64)
    kr = rope(np.asarray(k_pe, F64), pos, theta)
    q_rot = rope(np.asarray(q_pe, F64), pos[:, None], theta)
    c_all = np.concatenate([c_prefix, c], 0)
    kr_all = np.concatenate([np.asarray(kr_prefix, F64).reshape(P, kr.shape[1]), kr], 0)
    # key i is visible to chunk token j while i <= P + j
    visible = np.arange(P + n)[None, :] <= (P + np.arange(n))[:, None]
    o = np.zeros((n, H, np.asarray(w_uv).shape[2]))
    mag = np.zeros_like(o)
    for h in range(H):
        k_h = np.concatenate([c_all @ np.asarray(w_uk[h], F64).T, kr_all], 1)
        v_h = c_all @ np.asarray(w_uv[h], F64)
        q_h = np.concatenate([q_nope[:, h], q_rot[:, h]], 1)
        p, _ = softmax_lse(np.where(visible, scale * (q_h @ k_h.T), -np.inf))
        o[:, h] = p @ v_h
        if with_magnitude:
            mag[:, h] = p @ np.abs(v_h)
    rows = np.concatenate([c, kr], 1)
    return (o, rows, mag) if with_magnitude else (o, rows)


def reference_prefill(inp, b, heads=None, with_magnitude=False):
    """Prefill reference for prompt b of a batch from synth.prefill_workload:
    (o [T_b, h, d_v], rows [T_b, d_c + d_r][, magnitude]) by prefill_explicit
    on its tokens."""
    t0, t1 = int(inp["cu_seqlens"][b]), int(inp["cu_seqlens"][b + 1])
    H = np.asarray(inp["q_nope"]).shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    return prefill_explicit(bf16_to_f64(inp["q_nope"][t0:t1])[:, heads], bf16_to_f64(inp["q_pe"][t0:t1])[:, heads],
                            bf16_to_f64(inp["c"][t0:t1]), bf16_to_f64(inp["k_pe"][t0:t1]),
                            bf16_to_f64(inp["w_uk"])[heads], bf16_to_f64(inp["w_uv"])[heads],
                            inp["scale"], inp["theta"], with_magnitude)


# --------------------------------------------------------------------------
# cache-size arithmetic ([Riju] "The Cache Arithmetic", "Worked numbers")
# --------------------------------------------------------------------------


def cache_elements_per_token(kind, layers=1, n_heads=0, d_h=0, n_groups=0, d_c=0, d_r=0):
    """Cached scalars per token: MHA 2 n_h d_h, MQA 2 d_h, GQA 2 n_g d_h, MLA d_c + d_r (per layer)."""
    per_layer = {
        "mha": 2 * n_heads * d_h,
        "mqa": 2 * d_h,
        "gqa": 2 * n_groups * d_h,
        "mla": d_c + d_r,
    }[kind]
    return per_layer * layers


def fp8_row_bytes(d_c=512, d_r=64, group=128):
    """Bytes of one packed fp8 cache record: codes + bf16 rotary key + fp32 group scales."""
    return d_c + 2 * d_r + 4 * (d_c // group)


def quantise_roundtrip_bound(scale, x):
    """Half the e4m3 spacing at |x|/scale, times scale: the rounding bound of one value."""
    a = np.minimum(np.abs(np.asarray(x, F64)) / scale, E4M3_MAX)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="right"), 1, 126)
    return 0.5 * (_E4M3_POS[hi] - _E4M3_POS[hi - 1]) * scale


def sdpa_scale(d_nope, d_r):
    """Softmax scale 1/sqrt(d_nope + d_rope) ([Riju] absorbed decode sketch)."""
    return 1.0 / math.sqrt(d_nope + d_r)
