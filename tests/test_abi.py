"""Host-side checks of the C ABI: the library loads, exports every declared
entry point, reports status strings, sizes workspaces and rejects invalid
arguments before launching anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

import mla_latent_kv_32_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

needs_lib = pytest.mark.skipif(not os.path.exists(mla.library_path()),
                               reason="libmla.so not built (run __graft_entry__.build())")

FAKE = 0x10000          # aligned, never dereferenced: every call below fails validation first
NULL = None


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*\s*|int\s+|size_t\s+)(mla_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_calls():
    syms = declared_symbols()
    for name in ["mla_absorb_q", "mla_rope_append_cache", "mla_decode_paged", "mla_absorb_out"]:
        assert name in syms
    assert "mla_decode_workspace_bytes" in syms and "mla_status_string" in syms


@needs_lib
def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(mla.library_path())
    for name in declared_symbols():
        assert hasattr(L, name), f"{name} declared in mla.h but not exported"


@needs_lib
def test_abi_version_and_status_strings():
    L = mla.lib()
    assert L.mla_abi_version() == 1
    assert L.mla_status_string(0) == b"ok"
    assert L.mla_status_string(-1) == b"invalid argument"
    assert L.mla_status_string(-2) == b"unsupported size or format"
    assert L.mla_status_string(-3) == b"workspace too small"
    assert L.mla_status_string(-4) == b"kernel launch failed"
    assert L.mla_status_string(7) == b"unknown status"


@needs_lib
def test_workspace_sizing():
    L = mla.lib()
    # one chunk per sequence: room for one partial per (b, h)
    rows1 = 32 * 128
    assert L.mla_decode_workspace_bytes(32, 128, 4096, 4096) == \
        ((rows1 * 512 * 2 + 255) // 256) * 256 + ((rows1 * 4 + 255) // 256) * 256
    assert L.mla_decode_workspace_bytes(32, 128, 0, 0) == 0
    # 256-token chunks over 4096 tokens: 16 partial (o, lse) rows per (b, h)
    rows = 32 * 16 * 128
    want = ((rows * 512 * 2 + 255) // 256) * 256 + ((rows * 4 + 255) // 256) * 256
    assert L.mla_decode_workspace_bytes(32, 128, 4096, 256) == want
    # invalid sizes report 0
    assert L.mla_decode_workspace_bytes(0, 128, 4096, 0) == 0
    assert L.mla_decode_workspace_bytes(32, 128, 4096, 100) == 0
    # the planner picks a multiple of 64 no smaller than 256 (or the whole sequence)
    for B, H, S in [(32, 128, 4096), (4, 128, 32768), (8, 16, 1024), (128, 128, 8192), (1, 1, 1)]:
        sp = L.mla_decode_split_tokens(B, H, S)
        assert sp % 64 == 0 and sp >= min(256, ((S + 63) // 64) * 64)


@needs_lib
def test_validation_rejects_before_launch():
    L = mla.lib()
    # absorb_q: null pointer, misaligned pointer, unsupported widths
    assert L.mla_absorb_q(NULL, FAKE, FAKE, 1, 1, 128, 512, 64, NULL) == -1
    assert L.mla_absorb_q(FAKE + 2, FAKE, FAKE, 1, 1, 128, 512, 64, NULL) == -1
    assert L.mla_absorb_q(FAKE, FAKE, FAKE, 0, 1, 128, 512, 64, NULL) == -1
    assert L.mla_absorb_q(FAKE, FAKE, FAKE, 1, 1, 64, 512, 64, NULL) == -2
    assert L.mla_absorb_q(FAKE, FAKE, FAKE, 1, 1, 128, 256, 64, NULL) == -2
    # absorb_out
    assert L.mla_absorb_out(FAKE, NULL, FAKE, 1, 1, 512, 128, NULL) == -1
    assert L.mla_absorb_out(FAKE, FAKE, FAKE, 1, 1, 512, 64, NULL) == -2
    # rope/append: bad theta, bad dtype, unsupported block size
    args = [FAKE, FAKE, FAKE, FAKE, 4, FAKE]
    assert L.mla_rope_append_cache(*args, 0, 8, 64, ctypes.c_float(0.0), FAKE, 1, 1, 512, 64, NULL) == -1
    assert L.mla_rope_append_cache(*args, 5, 8, 64, ctypes.c_float(1e4), FAKE, 1, 1, 512, 64, NULL) == -1
    assert L.mla_rope_append_cache(*args, 0, 8, 32, ctypes.c_float(1e4), FAKE, 1, 1, 512, 64, NULL) == -2
    # decode: bad split, block size, max_seq_len beyond capacity, workspace too small
    dec = L.mla_decode_paged

    def call(split=0, ws=NULL, ws_bytes=0, max_seq=256, mbps=4, block=64, kv=0, lse=NULL, scale=0.07):
        return dec(FAKE, FAKE, kv, FAKE, mbps, FAKE, max_seq, 16, block, ctypes.c_float(scale), split,
                   ws, ws_bytes, FAKE, lse, 2, 128, NULL)
    assert call(split=100) == -1
    assert call(split=-64) == -1
    assert call(block=32) == -2
    assert call(max_seq=257) == -1
    assert call(kv=3) == -1
    assert call(lse=FAKE + 4) == -1
    assert call(scale=float("inf")) == -1
    assert call(split=64, ws=NULL) == -3
    assert call(split=64, ws=FAKE, ws_bytes=1024) == -3
    assert call(split=262144, max_seq=256) == -2
    # partial/combine
    part = L.mla_decode_partial
    assert part(FAKE, FAKE, 0, FAKE, 4, FAKE, 0, 16, 64, ctypes.c_float(0.07), 64, FAKE, 1 << 20, 2, 128,
                NULL) == -1   # max_seq_len 0
    assert part(FAKE, FAKE, 0, FAKE, 4, FAKE, 256, 16, 64, ctypes.c_float(0.07), 64, FAKE, 1024, 2, 128,
                NULL) == -3
    comb = L.mla_decode_combine
    assert comb(NULL, 0, FAKE, 256, 64, FAKE, NULL, 2, 128, NULL) == -1
    assert comb(FAKE, 16, FAKE, 256, 64, FAKE, NULL, 2, 128, NULL) == -3
    assert comb(FAKE, 1 << 30, FAKE, 256, 96, FAKE, NULL, 2, 128, NULL) == -1
    fused = L.mla_decode_combine_absorb_out
    assert fused(NULL, 0, FAKE, 256, 64, FAKE, FAKE, NULL, NULL, 2, 128, 512, 128, NULL) == -1
    assert fused(FAKE, 1 << 30, FAKE, 256, 64, FAKE, FAKE + 2, NULL, NULL, 2, 128, 512, 128, NULL) == -1
    assert fused(FAKE, 16, FAKE, 256, 64, FAKE, FAKE, NULL, NULL, 2, 128, 512, 128, NULL) == -3
    assert fused(FAKE, 1 << 30, FAKE, 256, 64, FAKE, FAKE, NULL, NULL, 2, 128, 256, 128, NULL) == -2
    assert fused(FAKE, 1 << 30, FAKE, 256, 64, FAKE, FAKE, NULL, NULL, 2, 70000, 512, 128, NULL) == -2


def test_fused_query_call_validates_like_its_parts():
    L = mla.lib()
    q = L.mla_absorb_q_rope_append

    def call(qn=FAKE, wuk=FAKE, qpe=FAKE, kvn=FAKE, sl=FAKE, bt=FAKE, mb=4, kv=FAKE, dt=0, nb=16, bs=64,
             theta=10000.0, qo=FAKE, B=2, H=128, dn=128, dc=512, dr=64):
        return q(qn, wuk, qpe, kvn, sl, bt, mb, kv, dt, nb, bs, ctypes.c_float(theta), qo, B, H, dn, dc, dr, NULL)

    assert call(qn=NULL) == -1
    assert call(wuk=FAKE + 2) == -1
    assert call(qpe=NULL) == -1
    assert call(dt=7) == -1
    assert call(theta=0.0) == -1
    assert call(B=0) == -1
    assert call(dn=64) == -2
    assert call(dc=256) == -2
    assert call(bs=32) == -2


@needs_lib
def test_fp8_mfma_call_validates():
    L = mla.lib()
    dec = L.mla_decode_paged_fp8_mfma

    def call(kv=1, split=0, ws=NULL, ws_bytes=0, max_seq=256, block=64):
        return dec(FAKE, FAKE, kv, FAKE, 4, FAKE, max_seq, 16, block, ctypes.c_float(0.07), split,
                   ws, ws_bytes, FAKE, NULL, 2, 128, NULL)
    assert call(kv=0, split=256) == -2        # a bf16 cache: the call is for the fp8 cache only
    assert call(kv=5) == -1
    assert call(split=100) == -1
    assert call(block=32) == -2
    assert call(max_seq=257) == -1
    assert call(split=64, ws=FAKE, ws_bytes=1024) == -3


@needs_lib
def test_prefill_chunk_call_validates():
    L = mla.lib()
    f = L.mla_prefill_chunk

    def call(B=2, T=8, max_len=4, total_keys=20, max_prefix=6, bs=64, dt=0, theta=10000.0, mbps=4, ws=NULL, wsb=0,
             prefix=FAKE):
        return f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, prefix, B, T, max_len, total_keys, max_prefix, 16,
                 ctypes.c_float(0.07), ctypes.c_float(theta), FAKE, mbps, FAKE, dt, 16, bs, FAKE, ws, wsb, NULL)
    assert call(prefix=NULL) == -1
    assert call(prefix=FAKE + 4) == -1
    assert call(total_keys=7) == -1          # fewer keys than chunk tokens
    assert call(max_prefix=-1) == -1
    assert call(max_prefix=257) == -1        # a prefix beyond the block-table row
    assert call(max_len=257, T=300, total_keys=400) == -1
    assert call(dt=3) == -1
    assert call(theta=0.0) == -1
    assert call(bs=32) == -2
    assert call() == -3                      # no workspace
    need = L.mla_prefill_chunk_workspace_bytes(8, 20, 2, 16)
    assert need > L.mla_prefill_workspace_bytes(8, 16)
    assert call(ws=FAKE, wsb=need - 256) == -3
    assert L.mla_prefill_chunk_workspace_bytes(8, 7, 2, 16) == 0


@needs_lib
def test_multi_token_call_validates():
    L = mla.lib()
    dec = L.mla_decode_paged_multi

    def call(q_len=2, H=16, split=0, ws=NULL, ws_bytes=0, max_seq=256, block=64):
        return dec(FAKE, FAKE, 0, FAKE, 4, FAKE, max_seq, 16, block, ctypes.c_float(0.07), split,
                   ws, ws_bytes, FAKE, NULL, 2, H, q_len, NULL)
    assert call(q_len=0) == -1
    assert call(q_len=-3) == -1
    assert call(q_len=mla.MAX_Q_LEN + 1) == -2
    assert call(H=0) == -1
    assert call(split=100) == -1
    assert call(block=32) == -2
    assert call(max_seq=257) == -1
    # the workspace is sized for q_len * H query rows
    need = L.mla_decode_workspace_bytes(2, 2 * 16, 256, 64)
    assert need == L.mla_decode_workspace_bytes(2, 32, 256, 64) > L.mla_decode_workspace_bytes(2, 16, 256, 64)
    assert call(split=64, ws=FAKE, ws_bytes=need - 256) == -3


@needs_lib
def test_prefill_call_validates():
    L = mla.lib()
    pre = L.mla_prefill

    def call(qn=FAKE, B=2, T=100, max_len=64, H=16, scale=0.07, theta=10000.0, mb=1, dt=0, bs=64, ws=FAKE,
             ws_bytes=1 << 40):
        return pre(qn, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, T, max_len, H, ctypes.c_float(scale),
                   ctypes.c_float(theta), FAKE, mb, FAKE, dt, 16, bs, FAKE, ws, ws_bytes, NULL)
    assert call(qn=NULL) == -1
    assert call(qn=FAKE + 2) == -1
    assert call(B=0) == -1
    assert call(scale=float("nan")) == -1
    assert call(theta=0.0) == -1
    assert call(dt=5) == -1
    assert call(bs=32) == -2
    assert call(max_len=65) == -1            # beyond one page of block table
    assert call(ws=NULL) == -3
    assert call(ws_bytes=L.mla_prefill_workspace_bytes(100, 16) - 1) == -3
    assert call(T=0) == 0                    # nothing to do, nothing launched
    assert L.mla_prefill_workspace_bytes(0, 16) == 0
    assert L.mla_prefill_workspace_bytes(100, 16) >= 100 * 16 * (64 + 2 * 128) * 2 + 100 * 64 * 2


@needs_lib
def test_paging_check_validates():
    L = mla.lib()

    def call(sl=FAKE, bt=FAKE, mb=4, max_len=256, nb=10, bs=64, B=2, bad=FAKE, first=FAKE):
        return L.mla_validate_paging(sl, bt, mb, max_len, nb, bs, B, bad, first, NULL)

    assert call(sl=NULL) == -1
    assert call(bt=NULL) == -1
    assert call(bad=NULL) == -1
    assert call(B=0) == -1
    assert call(mb=0) == -1
    assert call(max_len=-1) == -1
    assert call(nb=0) == -1
    assert call(bs=32) == -2


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mla, "_LIB", None)
    monkeypatch.setenv("MLA_LIBRARY", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        mla.lib()
