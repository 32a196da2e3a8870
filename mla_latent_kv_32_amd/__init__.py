"""MI355X (gfx950) MLA absorbed decode over a paged 576-wide latent cache.

Thin ctypes binding over libmla.so (declared in include/mla.h).  The functions
carry the C names and only marshal arguments: shapes are read from the torch
tensors, pointers and the current HIP stream are passed through, and every
step of the computation runs in the library's kernels.  There is no fallback:
if libmla.so is missing or fails to load, every call raises.

torch is used for device memory and streams only.  It is imported before the
library is loaded so that both share torch's HIP runtime.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "MLAError", "KV_BF16", "KV_FP8_E4M3", "D_C", "D_R", "D_NOPE", "D_V", "BLOCK_SIZE",
    "FP8_ROW_BYTES", "library_path", "lib", "abi_version",
    "mla_absorb_q", "mla_rope_append_cache", "mla_decode_paged", "mla_absorb_out",
    "mla_decode_workspace_bytes", "mla_decode_split_tokens", "mla_decode_partial", "mla_decode_combine",
    "mla_decode_combine_absorb_out", "mla_absorb_q_rope_append", "mla_decode_paged_multi", "MAX_Q_LEN",
    "mla_prefill", "mla_prefill_workspace_bytes", "mla_decode_paged_noalloc", "NOALLOC_SCRATCH_BYTES",
    "mla_query_from_latent", "D_Q", "mla_decode_paged_fp8_mfma", "mla_prefill_chunk",
    "mla_prefill_chunk_workspace_bytes",
]

KV_BF16 = 0
KV_FP8_E4M3 = 1
D_C, D_R, D_NOPE, D_V, BLOCK_SIZE = 512, 64, 128, 128, 64
D_Q = 1536
FP8_ROW_BYTES = 656
MAX_Q_LEN = 32
NOALLOC_SCRATCH_BYTES = 72 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported size or format",
           -3: "workspace too small", -4: "kernel launch failed",
           -5: "request exceeds the fixed scratch buffer"}


class MLAError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed with status {status} ({_STATUS.get(status, 'unknown')})")
        self.status = status


def library_path() -> str:
    return os.environ.get("MLA_LIBRARY", os.path.join(_HERE, "libmla.so"))


def lib():
    """Load libmla.so once; raises if it is absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() or "
                           "python -m mla_latent_kv_32_amd.build")
    L = ctypes.CDLL(path)
    vp, i32p, c_int, c_float, c_size = (ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_float, ctypes.c_size_t)
    L.mla_status_string.argtypes = [c_int]
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_abi_version.argtypes = []
    L.mla_abi_version.restype = c_int
    L.mla_absorb_q.argtypes = [vp, vp, vp, c_int, c_int, c_int, c_int, c_int, vp]
    L.mla_absorb_q.restype = c_int
    L.mla_rope_append_cache.argtypes = [vp, vp, i32p, i32p, c_int, vp, c_int, c_int, c_int, c_float,
                                        vp, c_int, c_int, c_int, c_int, vp]
    L.mla_rope_append_cache.restype = c_int
    L.mla_absorb_q_rope_append.argtypes = [vp, vp, vp, vp, i32p, i32p, c_int, vp, c_int, c_int, c_int, c_float,
                                           vp, c_int, c_int, c_int, c_int, c_int, vp]
    L.mla_absorb_q_rope_append.restype = c_int
    L.mla_query_from_latent.argtypes = [vp, vp, vp, vp, i32p, i32p, c_int, vp, c_int, c_int, c_int, c_float,
                                        vp, c_int, c_int, c_int, c_int, c_int, c_int, vp]
    L.mla_query_from_latent.restype = c_int
    L.mla_decode_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int]
    L.mla_decode_workspace_bytes.restype = c_size
    L.mla_decode_split_tokens.argtypes = [c_int, c_int, c_int]
    L.mla_decode_split_tokens.restype = c_int
    L.mla_validate_paging.argtypes = [i32p, i32p, c_int, c_int, c_int, c_int, c_int, i32p, i32p, vp]
    L.mla_validate_paging.restype = c_int
    L.mla_decode_paged.argtypes = [vp, vp, c_int, i32p, c_int, i32p, c_int, c_int, c_int, c_float, c_int,
                                   vp, c_size, vp, vp, c_int, c_int, vp]
    L.mla_decode_paged.restype = c_int
    L.mla_decode_paged_fp8_mfma.argtypes = L.mla_decode_paged.argtypes
    L.mla_decode_paged_fp8_mfma.restype = c_int
    L.mla_decode_paged_noalloc.argtypes = [vp, vp, c_int, i32p, c_int, i32p, c_int, c_int, c_int, c_float, c_int,
                                           vp, vp, c_int, c_int, vp]
    L.mla_decode_paged_noalloc.restype = c_int
    L.mla_decode_paged_multi.argtypes = [vp, vp, c_int, i32p, c_int, i32p, c_int, c_int, c_int, c_float, c_int,
                                         vp, c_size, vp, vp, c_int, c_int, c_int, vp]
    L.mla_decode_paged_multi.restype = c_int
    L.mla_prefill_workspace_bytes.argtypes = [c_int, c_int]
    L.mla_prefill_workspace_bytes.restype = c_size
    L.mla_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32p, c_int, c_int, c_int, c_int, c_float, c_float,
                              i32p, c_int, vp, c_int, c_int, c_int, vp, vp, c_size, vp]
    L.mla_prefill.restype = c_int
    L.mla_prefill_chunk_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int]
    L.mla_prefill_chunk_workspace_bytes.restype = c_size
    L.mla_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, vp, i32p, i32p, c_int, c_int, c_int, c_int, c_int, c_int,
                                    c_float, c_float, i32p, c_int, vp, c_int, c_int, c_int, vp, vp, c_size, vp]
    L.mla_prefill_chunk.restype = c_int
    L.mla_decode_partial.argtypes = [vp, vp, c_int, i32p, c_int, i32p, c_int, c_int, c_int, c_float, c_int,
                                     vp, c_size, c_int, c_int, vp]
    L.mla_decode_partial.restype = c_int
    L.mla_decode_combine.argtypes = [vp, c_size, i32p, c_int, c_int, vp, vp, c_int, c_int, vp]
    L.mla_decode_combine.restype = c_int
    L.mla_absorb_out.argtypes = [vp, vp, vp, c_int, c_int, c_int, c_int, vp]
    L.mla_absorb_out.restype = c_int
    L.mla_decode_combine_absorb_out.argtypes = [vp, c_size, i32p, c_int, c_int, vp, vp, vp, vp, c_int, c_int,
                                                c_int, c_int, vp]
    L.mla_decode_combine_absorb_out.restype = c_int
    _LIB = L
    return L


def abi_version() -> int:
    return lib().mla_abi_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != 0:
        raise MLAError(fn, status)


def _dense(t, name, dtype=None):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def mla_absorb_q(q_nope, w_uk, q, stream=None):
    """q[:, :, :512] = q_nope . W_UK (per head).  q_nope [B,H,128], w_uk [H,128,512], q [B,H,576]; bf16."""
    B, H, dn = q_nope.shape
    for t, n in ((q_nope, "q_nope"), (w_uk, "w_uk"), (q, "q")):
        _dense(t, n, torch.bfloat16)
    _check("mla_absorb_q", lib().mla_absorb_q(_ptr(q_nope), _ptr(w_uk), _ptr(q), B, H, dn,
                                              w_uk.shape[2], q.shape[2] - w_uk.shape[2], _stream(stream)))


def mla_rope_append_cache(q_pe, kv_new, seq_lens, block_table, kv_cache, kv_dtype, rope_theta, q,
                          stream=None):
    """Rotate q_pe into q[:, :, 512:] and append [c | RoPE(k_R)] at position seq_lens-1 of each sequence."""
    B, H, dr = q_pe.shape
    _dense(q_pe, "q_pe", torch.bfloat16)
    _dense(kv_new, "kv_new", torch.bfloat16)
    _dense(q, "q", torch.bfloat16)
    _dense(seq_lens, "seq_lens", torch.int32)
    _dense(block_table, "block_table", torch.int32)
    _dense(kv_cache, "kv_cache")
    _check("mla_rope_append_cache", lib().mla_rope_append_cache(
        _ptr(q_pe), _ptr(kv_new), _ptr(seq_lens), _ptr(block_table), block_table.shape[1],
        _ptr(kv_cache), int(kv_dtype), kv_cache.shape[0], kv_cache.shape[1], float(rope_theta),
        _ptr(q), B, H, kv_new.shape[1] - dr, dr, _stream(stream)))


def mla_absorb_q_rope_append(q_nope, w_uk, q_pe, kv_new, seq_lens, block_table, kv_cache, kv_dtype, rope_theta, q,
                             stream=None):
    """mla_absorb_q then mla_rope_append_cache in one launch (bit-identical results)."""
    B, H, dn = q_nope.shape
    dr = q_pe.shape[2]
    for t, n in ((q_nope, "q_nope"), (w_uk, "w_uk"), (q_pe, "q_pe"), (kv_new, "kv_new"), (q, "q")):
        _dense(t, n, torch.bfloat16)
    _dense(seq_lens, "seq_lens", torch.int32)
    _dense(block_table, "block_table", torch.int32)
    _dense(kv_cache, "kv_cache")
    _check("mla_absorb_q_rope_append", lib().mla_absorb_q_rope_append(
        _ptr(q_nope), _ptr(w_uk), _ptr(q_pe), _ptr(kv_new), _ptr(seq_lens), _ptr(block_table), block_table.shape[1],
        _ptr(kv_cache), int(kv_dtype), kv_cache.shape[0], kv_cache.shape[1], float(rope_theta),
        _ptr(q), B, H, dn, w_uk.shape[2], dr, _stream(stream)))



def mla_query_from_latent(c_q, w_uq, w_uk, seq_lens, rope_theta, q, kv_new=None, block_table=None, kv_cache=None,
                          kv_dtype=KV_BF16, stream=None):
    """q[:, :, 0:512] = bf16(c_q W_UQ_nope) . W_UK and q[:, :, 512:] = RoPE(c_q W_UQ_rope) at
    seq_lens - 1, in one launch; with kv_new, the new tokens' cache rows as mla_rope_append_cache.

    c_q [B, 1536] bf16; w_uq [1536, H*192] bf16 (per head [nope 128 | rope 64]); w_uk [H,128,512];
    q [B,H,576] bf16 output."""
    B, dq = c_q.shape
    H = w_uk.shape[0]
    for t, n in ((c_q, "c_q"), (w_uq, "w_uq"), (w_uk, "w_uk"), (q, "q")):
        _dense(t, n, torch.bfloat16)
    _dense(seq_lens, "seq_lens", torch.int32)
    if kv_new is not None:
        _dense(kv_new, "kv_new", torch.bfloat16)
        _dense(block_table, "block_table", torch.int32)
        _dense(kv_cache, "kv_cache")
    _check("mla_query_from_latent", lib().mla_query_from_latent(
        _ptr(c_q), _ptr(w_uq), _ptr(w_uk), _ptr(kv_new), _ptr(seq_lens), _ptr(block_table),
        block_table.shape[1] if block_table is not None else 0, _ptr(kv_cache), int(kv_dtype),
        kv_cache.shape[0] if kv_cache is not None else 0, kv_cache.shape[1] if kv_cache is not None else 0,
        float(rope_theta), _ptr(q), B, H, dq, w_uk.shape[1], w_uk.shape[2], q.shape[2] - w_uk.shape[2],
        _stream(stream)))

def mla_decode_workspace_bytes(B, H, max_seq_len, split_tokens=0) -> int:
    return int(lib().mla_decode_workspace_bytes(B, H, max_seq_len, split_tokens))


def mla_decode_split_tokens(B, H, max_seq_len) -> int:
    return int(lib().mla_decode_split_tokens(B, H, max_seq_len))


def mla_validate_paging(seq_lens, block_table, max_seq_len, num_blocks, bad, first_bad=None, stream=None):
    """Flag sequences whose length or pages in use break the bounds the other calls trust:
    bad (int32 [1] on the device) receives the count, first_bad (int32 [1] or None) the
    smallest flagged sequence or -1.  Asynchronous; read the results after synchronising."""
    _dense(seq_lens, "seq_lens", torch.int32)
    _dense(block_table, "block_table", torch.int32)
    _dense(bad, "bad", torch.int32)
    if first_bad is not None:
        _dense(first_bad, "first_bad", torch.int32)
    B = seq_lens.shape[0]
    _check("mla_validate_paging", lib().mla_validate_paging(
        _ptr(seq_lens), _ptr(block_table), block_table.shape[1], int(max_seq_len), int(num_blocks), BLOCK_SIZE,
        B, _ptr(bad), _ptr(first_bad), _stream(stream)))


def mla_decode_paged(q, kv_cache, kv_dtype, block_table, seq_lens, max_seq_len, softmax_scale, o_latent,
                     lse=None, split_tokens=0, workspace=None, stream=None):
    """o_latent = softmax(scale q . rows^T) rows[:, :512] over each sequence's paged rows.

    q [B,H,576] bf16; kv_cache [num_blocks, 64, 576] bf16 (or [num_blocks, 64, 656] uint8 for
    fp8); block_table [B, max_blocks] int32; seq_lens [B] int32; o_latent [B,H,512] bf16;
    lse [B,H] float32 or None.  A workspace of mla_decode_workspace_bytes(...) bytes is
    allocated with torch when not given.
    """
    B, H, _ = q.shape
    _dense(q, "q", torch.bfloat16)
    _dense(o_latent, "o_latent", torch.bfloat16)
    _dense(kv_cache, "kv_cache")
    _dense(block_table, "block_table", torch.int32)
    _dense(seq_lens, "seq_lens", torch.int32)
    if lse is not None:
        _dense(lse, "lse", torch.float32)
    sp = split_tokens or mla_decode_split_tokens(B, H, max_seq_len)
    need = mla_decode_workspace_bytes(B, H, max_seq_len, split_tokens) if max_seq_len > sp else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_decode_paged", lib().mla_decode_paged(
        _ptr(q), _ptr(kv_cache), int(kv_dtype), _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
        int(max_seq_len), kv_cache.shape[0], kv_cache.shape[1], float(softmax_scale), int(split_tokens),
        _ptr(workspace), ws_bytes, _ptr(o_latent), _ptr(lse), B, H, _stream(stream)))


def mla_decode_paged_fp8_mfma(q, kv_cache, block_table, seq_lens, max_seq_len, softmax_scale, o_latent,
                              lse=None, split_tokens=0, workspace=None, stream=None):
    """mla_decode_paged over an fp8 cache ([num_blocks, 64, 656] uint8) with both
    products on fp8 MFMAs over the stored codes (two-term E4M3 query and weights)."""
    B, H, _ = q.shape
    _dense(q, "q", torch.bfloat16)
    _dense(o_latent, "o_latent", torch.bfloat16)
    _dense(kv_cache, "kv_cache")
    _dense(block_table, "block_table", torch.int32)
    _dense(seq_lens, "seq_lens", torch.int32)
    if lse is not None:
        _dense(lse, "lse", torch.float32)
    sp = split_tokens or mla_decode_split_tokens(B, H, max_seq_len)
    need = mla_decode_workspace_bytes(B, H, max_seq_len, split_tokens) if max_seq_len > sp else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_decode_paged_fp8_mfma", lib().mla_decode_paged_fp8_mfma(
        _ptr(q), _ptr(kv_cache), KV_FP8_E4M3, _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
        int(max_seq_len), kv_cache.shape[0], kv_cache.shape[1], float(softmax_scale), int(split_tokens),
        _ptr(workspace), ws_bytes, _ptr(o_latent), _ptr(lse), B, H, _stream(stream)))


def mla_decode_paged_noalloc(q, kv_cache, kv_dtype, block_table, seq_lens, max_seq_len, softmax_scale, o_latent,
                             lse=None, split_tokens=0, stream=None):
    """mla_decode_paged with the split-KV partials in the library's fixed device
    scratch buffer (NOALLOC_SCRATCH_BYTES per GPU): nothing is allocated, here
    or in the library.  Calls that overlap on one GPU race on that buffer."""
    B, H, _ = q.shape
    _dense(q, "q", torch.bfloat16)
    _dense(o_latent, "o_latent", torch.bfloat16)
    _dense(kv_cache, "kv_cache")
    _dense(block_table, "block_table", torch.int32)
    _dense(seq_lens, "seq_lens", torch.int32)
    if lse is not None:
        _dense(lse, "lse", torch.float32)
    _check("mla_decode_paged_noalloc", lib().mla_decode_paged_noalloc(
        _ptr(q), _ptr(kv_cache), int(kv_dtype), _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
        int(max_seq_len), kv_cache.shape[0], kv_cache.shape[1], float(softmax_scale), int(split_tokens),
        _ptr(o_latent), _ptr(lse), B, H, _stream(stream)))


def mla_decode_paged_multi(q, kv_cache, kv_dtype, block_table, seq_lens, max_seq_len, softmax_scale, o_latent,
                           lse=None, split_tokens=0, workspace=None, stream=None):
    """Decode of q_len new tokens per sequence (causal among them) in one pass over the cache.

    q [B,q_len,H,576] bf16; o_latent [B,q_len,H,512] bf16; lse [B,q_len,H] float32 or None;
    the other arguments as for mla_decode_paged.  Split and workspace are sized for
    q_len * H query rows; a workspace is allocated with torch when not given.
    """
    B, q_len, H, _ = q.shape
    _dense(q, "q", torch.bfloat16)
    _dense(o_latent, "o_latent", torch.bfloat16)
    _dense(kv_cache, "kv_cache")
    _dense(block_table, "block_table", torch.int32)
    _dense(seq_lens, "seq_lens", torch.int32)
    if lse is not None:
        _dense(lse, "lse", torch.float32)
    rows = q_len * H
    sp = split_tokens or mla_decode_split_tokens(B, rows, max_seq_len)
    need = mla_decode_workspace_bytes(B, rows, max_seq_len, split_tokens) if max_seq_len > sp else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_decode_paged_multi", lib().mla_decode_paged_multi(
        _ptr(q), _ptr(kv_cache), int(kv_dtype), _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
        int(max_seq_len), kv_cache.shape[0], kv_cache.shape[1], float(softmax_scale), int(split_tokens),
        _ptr(workspace), ws_bytes, _ptr(o_latent), _ptr(lse), B, H, q_len, _stream(stream)))


def mla_prefill_workspace_bytes(total_tokens, H) -> int:
    return int(lib().mla_prefill_workspace_bytes(total_tokens, H))


def mla_prefill(q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, cu_seqlens, max_seqlen, softmax_scale, rope_theta,
                block_table, kv_cache, kv_dtype, o, workspace=None, stream=None):
    """Causal prefill of packed prompts in the explicit form; also writes their cache rows.

    q_nope [T,H,128], q_pe [T,H,64], c_kv [T,512], k_pe [T,64], w_uk [H,128,512], w_uv [H,512,128]
    (bf16); cu_seqlens [B+1] int32; block_table [B, max_blocks] int32; kv_cache as for
    mla_rope_append_cache; o [T,H,128] bf16.  A workspace of mla_prefill_workspace_bytes(T, H)
    bytes is allocated with torch when not given.
    """
    T, H, _ = q_nope.shape
    for t, n in ((q_nope, "q_nope"), (q_pe, "q_pe"), (c_kv, "c_kv"), (k_pe, "k_pe"), (w_uk, "w_uk"),
                 (w_uv, "w_uv"), (o, "o")):
        _dense(t, n, torch.bfloat16)
    _dense(cu_seqlens, "cu_seqlens", torch.int32)
    _dense(block_table, "block_table", torch.int32)
    _dense(kv_cache, "kv_cache")
    B = cu_seqlens.shape[0] - 1
    if workspace is None and T > 0:
        workspace = torch.empty(mla_prefill_workspace_bytes(T, H), dtype=torch.uint8, device=q_nope.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_prefill", lib().mla_prefill(
        _ptr(q_nope), _ptr(q_pe), _ptr(c_kv), _ptr(k_pe), _ptr(w_uk), _ptr(w_uv), _ptr(cu_seqlens), B, T,
        int(max_seqlen), H, float(softmax_scale), float(rope_theta), _ptr(block_table), block_table.shape[1],
        _ptr(kv_cache), int(kv_dtype), kv_cache.shape[0], kv_cache.shape[1], _ptr(o), _ptr(workspace), ws_bytes,
        _stream(stream)))


def mla_prefill_chunk_workspace_bytes(total_tokens, total_keys, B, H) -> int:
    return int(lib().mla_prefill_chunk_workspace_bytes(total_tokens, total_keys, B, H))


def mla_prefill_chunk(q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, cu_seqlens, prefix_lens, max_seqlen, total_keys,
                      max_prefix, softmax_scale, rope_theta, block_table, kv_cache, kv_dtype, o, workspace=None,
                      stream=None):
    """Prompt chunks that continue cached prefixes (prefix_lens [B] int32 rows already cached):
    chunk token j of prompt b at position prefix_lens[b] + j, attending to the cached rows
    and to the chunk's tokens up to itself; writes the chunk's cache rows.  Shapes as for
    mla_prefill; total_keys = sum_b (prefix_lens[b] + chunk length b) and max_prefix are
    host values.  A workspace of mla_prefill_chunk_workspace_bytes(...) bytes is allocated
    with torch when not given."""
    T, H, _ = q_nope.shape
    for t, n in ((q_nope, "q_nope"), (q_pe, "q_pe"), (c_kv, "c_kv"), (k_pe, "k_pe"), (w_uk, "w_uk"),
                 (w_uv, "w_uv"), (o, "o")):
        _dense(t, n, torch.bfloat16)
    _dense(cu_seqlens, "cu_seqlens", torch.int32)
    _dense(prefix_lens, "prefix_lens", torch.int32)
    _dense(block_table, "block_table", torch.int32)
    _dense(kv_cache, "kv_cache")
    B = cu_seqlens.shape[0] - 1
    if workspace is None and T > 0:
        workspace = torch.empty(mla_prefill_chunk_workspace_bytes(T, total_keys, B, H), dtype=torch.uint8,
                                device=q_nope.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_prefill_chunk", lib().mla_prefill_chunk(
        _ptr(q_nope), _ptr(q_pe), _ptr(c_kv), _ptr(k_pe), _ptr(w_uk), _ptr(w_uv), _ptr(cu_seqlens),
        _ptr(prefix_lens), B, T, int(max_seqlen), int(total_keys), int(max_prefix), H, float(softmax_scale),
        float(rope_theta), _ptr(block_table), block_table.shape[1], _ptr(kv_cache), int(kv_dtype),
        kv_cache.shape[0], kv_cache.shape[1], _ptr(o), _ptr(workspace), ws_bytes, _stream(stream)))


def mla_decode_partial(q, kv_cache, kv_dtype, block_table, seq_lens, max_seq_len, softmax_scale, workspace,
                       split_tokens=0, stream=None):
    """Per-chunk (o_part, lse_part) into `workspace` (layout in include/mla.h)."""
    B, H, _ = q.shape
    _dense(q, "q", torch.bfloat16)
    _dense(kv_cache, "kv_cache")
    _dense(block_table, "block_table", torch.int32)
    _dense(seq_lens, "seq_lens", torch.int32)
    _dense(workspace, "workspace")
    _check("mla_decode_partial", lib().mla_decode_partial(
        _ptr(q), _ptr(kv_cache), int(kv_dtype), _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
        int(max_seq_len), kv_cache.shape[0], kv_cache.shape[1], float(softmax_scale), int(split_tokens),
        _ptr(workspace), workspace.numel() * workspace.element_size(), B, H, _stream(stream)))


def mla_decode_combine(workspace, seq_lens, max_seq_len, o_latent, lse=None, split_tokens=0, stream=None):
    """Log-sum-exp merge of the workspace partials into o_latent [B,H,512] bf16 (and lse)."""
    B, H, _ = o_latent.shape
    _dense(workspace, "workspace")
    _dense(seq_lens, "seq_lens", torch.int32)
    _dense(o_latent, "o_latent", torch.bfloat16)
    if lse is not None:
        _dense(lse, "lse", torch.float32)
    _check("mla_decode_combine", lib().mla_decode_combine(
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(seq_lens), int(max_seq_len),
        int(split_tokens), _ptr(o_latent), _ptr(lse), B, H, _stream(stream)))


def mla_absorb_out(o_latent, w_uv, o, stream=None):
    """o = o_latent . W_UV (per head).  o_latent [B,H,512], w_uv [H,512,128], o [B,H,128]; bf16."""
    B, H, dc = o_latent.shape
    for t, n in ((o_latent, "o_latent"), (w_uv, "w_uv"), (o, "o")):
        _dense(t, n, torch.bfloat16)
    _check("mla_absorb_out", lib().mla_absorb_out(_ptr(o_latent), _ptr(w_uv), _ptr(o), B, H, dc,
                                                  w_uv.shape[2], _stream(stream)))


def mla_decode_combine_absorb_out(workspace, seq_lens, max_seq_len, w_uv, o, o_latent=None, lse=None,
                                  split_tokens=0, stream=None):
    """Merge the workspace partials and apply W_UV in one launch: o [B,H,128] bf16
    (optionally also o_latent [B,H,512] bf16 and lse [B,H] fp32)."""
    B, H, dv = o.shape
    _dense(workspace, "workspace")
    _dense(seq_lens, "seq_lens", torch.int32)
    _dense(w_uv, "w_uv", torch.bfloat16)
    _dense(o, "o", torch.bfloat16)
    if o_latent is not None:
        _dense(o_latent, "o_latent", torch.bfloat16)
    if lse is not None:
        _dense(lse, "lse", torch.float32)
    _check("mla_decode_combine_absorb_out", lib().mla_decode_combine_absorb_out(
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(seq_lens), int(max_seq_len),
        int(split_tokens), _ptr(w_uv), _ptr(o), _ptr(o_latent), _ptr(lse), B, H, w_uv.shape[1], dv,
        _stream(stream)))
