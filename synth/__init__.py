"""Seeded synthetic inputs for MLA absorbed decode over a paged latent cache.

This module is shared by the tests, the smoke check and the benchmark.  It
draws random tensors and lays them out in the storage formats the decode path
consumes; it performs no step of the decode path itself (no rotary embedding,
no absorption, no attention, no fp8 quantiser).  Values the method would
compute are either drawn from their distribution directly or come from the
hidden-state projections that sit *before* the decode path (the down- and
up-projections of the MLA layer), which are part of how the inputs are made.

Workloads (the sizes the pages' DeepSeek-V2/V3 geometry fixes: d_c = 512
latent, d_r = 64 rotary key, d_nope = d_v = 128, 128 heads; see
"Multi-Head Latent Attention vs GQA vs MQA", "Worked numbers from real
configs"):

  0  tiny fp32 self-check: B=1, H=4, d=64, d_c=32, d_r=8, d_nope=d_v=16,
     64 tokens, contiguous cache (hidden states and weights only).
  1  bf16, B=8, H=16, d=2048, 1024 tokens per sequence, paged (64-token
     pages, random page permutation), cache rows from projected hidden states.
  2  bf16, DeepSeek-V3 shaped: B=32, H=128, d=7168, query latent 1536,
     4096 tokens per sequence, paged, rows from projected hidden states.
  3  bf16, B=4, H=128, lengths uniform in [1024, 32768], paged and scattered,
     entries drawn N(0,1); split into 256-token chunks.
  4  fp8 e4m3 latent (one fp32 scale per token per 128-wide group) with a
     bf16 rotary part: B=128, H=128, 8192 tokens per sequence.

Storage conventions (all row-major):
  bf16 tensors are returned as uint16 bit patterns (round-to-nearest-even
  from float32); fp8 rows are packed 656-byte records
  [512 e4m3 codes | 64 bf16 rotary values | 4 fp32 group scales].
"""
from __future__ import annotations

import functools
import math

import numpy as np

D_C = 512
D_R = 64
D_NOPE = 128
D_V = 128
ROW = D_C + D_R              # 576 values per cached token
BLOCK = 64                   # tokens per cache page
FP8_ROW_BYTES = D_C + 2 * D_R + 16   # 656
ROPE_THETA = 10000.0

KV_BF16 = 0
KV_FP8 = 1

# Marker written into cache slots that the append step must fill; 0xFFFF is a
# bf16 NaN and 0xFF an e4m3 NaN, so an unwritten slot poisons any result.
POISON_BF16 = np.uint16(0xFFFF)
POISON_BYTE = np.uint8(0xFF)


# --------------------------------------------------------------------------
# storage-format helpers
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("bf16 conversion expects finite values")
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


# --------------------------------------------------------------------------
# paging
# --------------------------------------------------------------------------
def page_layout(rng, seq_lens, block=BLOCK, spare_pages=0):
    """Assign each sequence's logical pages to a random permutation of physical pages.

    Returns (block_table [B, max_blocks] int32, num_blocks).  Table entries past
    a sequence's last page are 0 (a valid page id that must be ignored).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    nblk = (seq_lens + block - 1) // block
    max_blocks = max(1, int(nblk.max()) if len(nblk) else 1)
    total = int(nblk.sum()) + spare_pages
    perm = rng.permutation(max(total, 1)).astype(np.int32)
    table = np.zeros((len(seq_lens), max_blocks), dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[off:off + n]
        off += int(n)
    return table, max(total, 1)


def scatter_rows(rows_per_seq, seq_lens, table, num_blocks, row_shape, dtype,
                 block=BLOCK, fill=0):
    """Place per-sequence token rows into a paged pool [num_blocks, block, *row_shape]."""
    pool = np.full((num_blocks, block) + tuple(row_shape), fill, dtype=dtype)
    for b, rows in enumerate(rows_per_seq):
        n = int(seq_lens[b])
        for j in range((n + block - 1) // block):
            t0, t1 = j * block, min(n, (j + 1) * block)
            pool[table[b, j], :t1 - t0] = rows[t0:t1]
    return pool


# --------------------------------------------------------------------------
# fp8 stored rows (drawn directly: codes and scales are random stored data)
# --------------------------------------------------------------------------
def draw_e4m3_codes(rng, shape) -> np.ndarray:
    """Random e4m3 byte codes shaped like a per-group-scaled Gaussian.

    A group scaled so that its largest magnitude maps near the top of the e4m3
    range puts most values within a few binades below it; the exponent field is
    drawn around 13 (values 64..120) with a spread of about 1.5 binades, the
    mantissa uniformly, the sign with probability 1/2.  NaN codes (S.1111.111)
    are never produced.
    """
    e = np.clip(np.rint(13 + 1.5 * rng.standard_normal(shape)), 0, 15).astype(np.uint8)
    m = rng.integers(0, 8, size=shape, dtype=np.uint8)
    m = np.where((e == 15) & (m == 7), np.uint8(6), m)
    s = rng.integers(0, 2, size=shape, dtype=np.uint8)
    return (s << 7) | (e << 3) | m


def pack_fp8_rows(codes, rope_bits, scales) -> np.ndarray:
    """Pack [N,512] codes, [N,64] bf16 bits and [N,4] fp32 scales into [N,656] bytes."""
    n = codes.shape[0]
    out = np.empty((n, FP8_ROW_BYTES), dtype=np.uint8)
    out[:, :D_C] = codes
    out[:, D_C:D_C + 2 * D_R] = np.ascontiguousarray(rope_bits, np.uint16).view(np.uint8).reshape(n, 2 * D_R)
    out[:, D_C + 2 * D_R:] = np.ascontiguousarray(scales, np.float32).view(np.uint8).reshape(n, 16)
    return out


# --------------------------------------------------------------------------
# workload builders
# --------------------------------------------------------------------------
def tiny_config0(seed=0):
    """Workload 0: fp32 hidden states and weights for the oracle's own checks."""
    rng = np.random.default_rng(seed)
    d, H, d_c, d_r, d_n, d_v, S = 64, 4, 32, 8, 16, 16, 64
    x = _normal(rng, (S, d))
    w_dkv = _normal(rng, (d, d_c), 1 / math.sqrt(d))
    w_kr = _normal(rng, (d, d_r), 1 / math.sqrt(d))
    w_q = _normal(rng, (d, H * (d_n + d_r)), 1 / math.sqrt(d))
    w_uk = _normal(rng, (H, d_n, d_c), 1 / math.sqrt(d_c))
    w_uv = _normal(rng, (H, d_c, d_v), 1 / math.sqrt(d_c))
    return dict(x=x, w_dkv=w_dkv, w_kr=w_kr, w_q=w_q, w_uk=w_uk, w_uv=w_uv,
                H=H, d_c=d_c, d_r=d_r, d_nope=d_n, d_v=d_v, S=S,
                theta=ROPE_THETA, scale=1 / math.sqrt(d_n + d_r))


def _finish(rng, B, H, seq_lens, rows_prefix, rows_new, q_nope, q_pe, w_uk, w_uv,
            kv_dtype, spare_pages=0, draw_decode_q=True):
    """Shared tail of every builder: pages, pools and the decode-only query."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    table, nblocks = page_layout(rng, seq_lens, spare_pages=spare_pages)
    out = dict(B=B, H=H, seq_lens=seq_lens, block_table=table, num_blocks=nblocks,
               block_size=BLOCK, kv_dtype=kv_dtype, theta=ROPE_THETA,
               scale=1 / math.sqrt(D_NOPE + D_R),
               q_nope=q_nope, q_pe=q_pe, w_uk=w_uk, w_uv=w_uv)
    if kv_dtype == KV_BF16:
        full = [np.concatenate([p, n[None]], 0) if int(L) > 0 else p[:0]
                for p, n, L in zip(rows_prefix, rows_new, seq_lens)]
        out["kv_new"] = np.stack(rows_new)
        out["cache_full"] = scatter_rows(full, seq_lens, table, nblocks, (ROW,), np.uint16)
        step = [f.copy() for f in full]
        for f in step:
            if len(f):
                f[-1] = POISON_BF16
        out["cache_step"] = scatter_rows(step, seq_lens, table, nblocks, (ROW,), np.uint16)
    else:
        # rows_prefix / rows_new carry packed 656-byte records for the stored
        # rows and bf16 [576] rows for the token to append.
        full = [np.concatenate([p, r[None]], 0) if int(L) > 0 else p[:0]
                for p, r, L in zip(rows_prefix["stored"], rows_prefix["stored_last"], seq_lens)]
        out["kv_new"] = np.stack(rows_new)
        out["cache_full"] = scatter_rows(full, seq_lens, table, nblocks, (FP8_ROW_BYTES,), np.uint8)
        step = [f.copy() for f in full]
        for f in step:
            if len(f):
                f[-1] = POISON_BYTE
        out["cache_step"] = scatter_rows(step, seq_lens, table, nblocks, (FP8_ROW_BYTES,), np.uint8)
    if draw_decode_q:
        # Decode-only query [B,H,576]: the absorbed latent part has variance
        # d_nope/d_c times that of q_nope (unit-variance weights scaled by
        # 1/fan_in), the rotary part unit variance.
        q_lat = _normal(rng, (B, H, D_C), math.sqrt(D_NOPE / D_C))
        q_rot = _normal(rng, (B, H, D_R))
        out["q_decode"] = f32_to_bf16_bits(np.concatenate([q_lat, q_rot], -1))
    return out


def _projected_workload(seed, B, H, d, S, q_latent_dim=None):
    """Workloads 1 and 2: rows and queries from projected random hidden states.

    Draw order: W_DKV, W_KR, (W_Q) or (W_DQ, W_UQ), W_UK, W_UV, then one block
    of hidden states x[b] of shape [S, d] per sequence, then the page
    permutation and the decode-only query.  Row t of sequence b is
    [x[b,t] W_DKV | x[b,t] W_KR] rounded to bf16; the query comes from the
    hidden state at position S-1, the same one that yields the appended row.
    Prefix rows store the projected rotary key as-is: a rotated Gaussian
    vector has the same law as the unrotated one, so stored rows are drawn
    from the law of cached (rotated) keys without rotating them here.
    """
    rng = np.random.default_rng(seed)
    f = 1 / math.sqrt(d)
    w_kv = np.concatenate([_normal(rng, (d, D_C), f), _normal(rng, (d, D_R), f)], 1)
    if q_latent_dim is None:
        w_q = _normal(rng, (d, H * (D_NOPE + D_R)), f)
    else:
        w_dq = _normal(rng, (d, q_latent_dim), f)
        w_uq = _normal(rng, (q_latent_dim, H * (D_NOPE + D_R)), 1 / math.sqrt(q_latent_dim))
    w_uk = f32_to_bf16_bits(_normal(rng, (H, D_NOPE, D_C), 1 / math.sqrt(D_C)))
    w_uv = f32_to_bf16_bits(_normal(rng, (H, D_C, D_V), 1 / math.sqrt(D_C)))
    prefix, new, qs, cqs = [], [], [], []
    for b in range(B):
        x = _normal(rng, (S, d))
        rows = f32_to_bf16_bits(x @ w_kv)
        prefix.append(rows[:-1])
        new.append(rows[-1])
        xq = x[-1:]
        if q_latent_dim is None:
            q = xq @ w_q
        else:
            cq = xq @ w_dq
            cqs.append(cq[0])
            q = cq @ w_uq
        qs.append(q.reshape(H, D_NOPE + D_R))
        del x
    q = np.stack(qs)
    q_nope = f32_to_bf16_bits(q[..., :D_NOPE])
    q_pe = f32_to_bf16_bits(q[..., D_NOPE:])
    out = _finish(rng, B, H, [S] * B, prefix, new, q_nope, q_pe, w_uk, w_uv, KV_BF16)
    if q_latent_dim is not None:
        # the query latent c' = x W_DQ of the new token and W_UQ, rounded to
        # bf16, for the path that starts from the query latent
        out["c_q"] = f32_to_bf16_bits(np.stack(cqs))
        out["w_uq"] = f32_to_bf16_bits(w_uq)
    return out


def gaussian_workload(seed, B, H, seq_lens, kv_dtype=KV_BF16, spare_pages=0):
    """Entries drawn N(0,1) directly (workloads 3 and 4, and every edge case).

    Draw order: W_UK, W_UV, q_nope, q_pe, new-token rows, then per sequence its
    stored prefix rows, then the page permutation and the decode-only query.
    For fp8 caches the stored rows are random e4m3 codes (see draw_e4m3_codes)
    with group scales uniform in [2.5, 3.5]/448 and a N(0,1) bf16 rotary part.
    """
    rng = np.random.default_rng(seed)
    seq_lens = [int(s) for s in seq_lens]
    w_uk = f32_to_bf16_bits(_normal(rng, (H, D_NOPE, D_C), 1 / math.sqrt(D_C)))
    w_uv = f32_to_bf16_bits(_normal(rng, (H, D_C, D_V), 1 / math.sqrt(D_C)))
    q_nope = f32_to_bf16_bits(_normal(rng, (B, H, D_NOPE)))
    q_pe = f32_to_bf16_bits(_normal(rng, (B, H, D_R)))
    new = list(f32_to_bf16_bits(_normal(rng, (B, ROW))))
    if kv_dtype == KV_BF16:
        prefix = [f32_to_bf16_bits(_normal(rng, (max(S - 1, 0), ROW))) for S in seq_lens]
        return _finish(rng, B, H, seq_lens, prefix, new, q_nope, q_pe, w_uk, w_uv,
                       kv_dtype, spare_pages)
    stored, stored_last = [], []
    for S in seq_lens:
        n = max(S, 1)
        codes = draw_e4m3_codes(rng, (n, D_C))
        scales = (rng.uniform(2.5, 3.5, size=(n, 4)) / 448.0).astype(np.float32)
        rope = f32_to_bf16_bits(_normal(rng, (n, D_R)))
        rec = pack_fp8_rows(codes, rope, scales)
        stored.append(rec[:max(S - 1, 0)])
        stored_last.append(rec[n - 1])
    rows = dict(stored=stored, stored_last=stored_last)
    return _finish(rng, B, H, seq_lens, rows, new, q_nope, q_pe, w_uk, w_uv,
                   kv_dtype, spare_pages)


@functools.lru_cache(maxsize=4)
def workload(cfg: int, seed: int | None = None):
    """The numbered workloads; seed defaults to the workload number."""
    seed = cfg if seed is None else seed
    if cfg == 0:
        return tiny_config0(seed)
    if cfg == 1:
        return _projected_workload(seed, B=8, H=16, d=2048, S=1024)
    if cfg == 2:
        return _projected_workload(seed, B=32, H=128, d=7168, S=4096, q_latent_dim=1536)
    if cfg == 3:
        rng = np.random.default_rng(seed + 1000)
        lens = rng.integers(1024, 32768, size=4, endpoint=True)
        return gaussian_workload(seed, B=4, H=128, seq_lens=lens)
    if cfg == 4:
        return gaussian_workload(seed, B=128, H=128, seq_lens=[8192] * 128, kv_dtype=KV_FP8)
    raise ValueError(f"unknown workload {cfg}")


def multi_token_query(seed, B, q_len, H):
    """Queries of q_len new tokens per sequence [B, q_len, H, 576] (bf16 bits),
    drawn like the decode-only query: latent part N(0, d_nope/d_c), rotary
    part N(0, 1)."""
    rng = np.random.default_rng(seed)
    q_lat = _normal(rng, (B, q_len, H, D_C), math.sqrt(D_NOPE / D_C))
    q_rot = _normal(rng, (B, q_len, H, D_R))
    return f32_to_bf16_bits(np.concatenate([q_lat, q_rot], -1))


def prefill_workload(seed, H, lens, kv_dtype=KV_BF16):
    """Prompts of the given lengths for the explicit-form prefill, packed
    token-major (cu_seqlens offsets): q_nope [T, H, 128], q_pe [T, H, 64],
    c [T, 512], k_pe [T, 64] drawn N(0, 1) (c W_UK^T then has unit variance,
    like the decode workloads' keys), W_UK / W_UV N(0, 1/d_c) as elsewhere,
    and a page layout for the cache rows the prompts leave (64-token pages in
    a seeded permutation)."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in lens]
    T = int(sum(lens))
    w_uk = f32_to_bf16_bits(_normal(rng, (H, D_NOPE, D_C), 1 / math.sqrt(D_C)))
    w_uv = f32_to_bf16_bits(_normal(rng, (H, D_C, D_V), 1 / math.sqrt(D_C)))
    q_nope = f32_to_bf16_bits(_normal(rng, (T, H, D_NOPE)))
    q_pe = f32_to_bf16_bits(_normal(rng, (T, H, D_R)))
    c = f32_to_bf16_bits(_normal(rng, (T, D_C)))
    k_pe = f32_to_bf16_bits(_normal(rng, (T, D_R)))
    table, nblocks = page_layout(rng, np.asarray(lens, np.int32))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return dict(B=len(lens), H=H, lens=np.asarray(lens, np.int32), cu_seqlens=cu, T=T,
                q_nope=q_nope, q_pe=q_pe, c=c, k_pe=k_pe, w_uk=w_uk, w_uv=w_uv,
                block_table=table, num_blocks=nblocks, block_size=BLOCK, kv_dtype=kv_dtype,
                theta=ROPE_THETA, scale=1 / math.sqrt(D_NOPE + D_R))


def query_latent_inputs(seed, B, H, d_q=1536):
    """Query latent c' [B, d_q] ~ N(0, 1) and W_UQ [d_q, H (d_nope + d_r)] ~
    N(0, 1/d_q) (the 1/fan_in law of the configs), W_UK as in every builder,
    sequence lengths U{0..40000}, all rounded to bf16: the inputs of the path
    that starts from the query latent, at any batch and head count."""
    rng = np.random.default_rng(seed)
    c_q = f32_to_bf16_bits(_normal(rng, (B, d_q)))
    w_uq = f32_to_bf16_bits(_normal(rng, (d_q, H * (D_NOPE + D_R)), 1 / math.sqrt(d_q)))
    w_uk = f32_to_bf16_bits(_normal(rng, (H, D_NOPE, D_C), 1 / math.sqrt(D_C)))
    seq_lens = rng.integers(0, 40000, size=B, endpoint=True).astype(np.int32)
    return dict(B=B, H=H, c_q=c_q, w_uq=w_uq, w_uk=w_uk, seq_lens=seq_lens, theta=ROPE_THETA)


def random_bf16(seed, shape, std=1.0):
    """Plain N(0, std^2) draw rounded to bf16 bits (stand-alone operands for single-kernel tests)."""
    return f32_to_bf16_bits(_normal(np.random.default_rng(seed), shape, std))


def permute_pages(inp, seed):
    """Same logical cache, different physical placement: returns (pool, block_table) for key
    'cache_full' with every page moved to a new random id (plus the unchanged contents)."""
    rng = np.random.default_rng(seed)
    pool = inp["cache_full"]
    perm = rng.permutation(pool.shape[0])
    new_pool = np.empty_like(pool)
    new_pool[perm] = pool
    return new_pool, perm[inp["block_table"]].astype(np.int32)


SPLIT_TOKENS = {3: 256}
