"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, sizes workspaces, and rejects invalid arguments before enqueueing
anything (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import flash_attention_kv_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fakv.h")

EINVAL, EUNSUP = 1, 2


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", src, flags=re.M)) - {"if"})


def test_header_symbols_exported():
    names = header_functions()
    assert set(names) == set(F.SIGNATURES), (names, sorted(F.SIGNATURES))
    L = ctypes.CDLL(F.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_tile_rows():
    L = F.lib()
    assert L.fakv_abi_version() == 102
    # jagged bf16 tiles: 8 waves of 32 rows, split over the query heads that
    # share a KV tile
    assert F.query_tile_rows(32, 8, 128) == 64      # 4 query heads share a KV tile
    assert F.query_tile_rows(32, 32, 256) == 256
    assert F.query_tile_rows(6, 3, 64) == 128
    assert F.query_tile_rows(4, 4, 128, F.F32) == 128
    assert F.query_tile_rows(3, 2, 128) == 0


def test_workspace_sizes():
    assert F.ring_attn_workspace_bytes(8192, 8192, 32, 8, 128, 8, 1, 1, 0, F.BF16) == 0
    # fp32 dense: a call of 1 query tile is split over its KV range -- the 4
    # chunks of 128 keys cut into 4 parts of 32 each: 16 partial triplets of
    # (d + 2) fp32 per row -- while 128 tiles or more need no workspace
    assert F.ring_attn_workspace_bytes(128, 512, 1, 1, 64, 4, 0, 1, 0, F.F32) == \
        16 * 128 * 64 * 4 + 2 * 16 * 128 * 4
    assert F.ring_attn_workspace_bytes(2048, 2048, 8, 8, 64, 4, 1, 1, 0, F.F32) == 0
    n = F.ring_attn_workspace_bytes(1240379, 1240379, 4, 4, 128, 1, 1, 1152, 1, F.BF16)
    cap = 1240379 // 128 + 1152
    assert n >= 256 + 32 * cap
    ws = F.splitkv_decode_workspace_bytes(8, 64, 128, 64)
    parts = 8 * 64 * 64
    assert ws >= parts * 128 * 4 + 2 * parts * 4


def _ring(**kw):
    a = dict(q=16, k=16, v=16, o=16, T_q=8, S_kv=8, h_q=4, h_kv=2, d=128, C=1, causal=0,
             seq_offsets=None, n_seqs=1, dtype=F.BF16, ws=None, wsb=0)
    a.update(kw)
    return F.lib().ring_attn_fwd(a["q"], a["k"], a["v"], a["o"], a["T_q"], a["S_kv"], a["h_q"],
                                 a["h_kv"], a["d"], a["C"], a["causal"], a["seq_offsets"],
                                 a["n_seqs"], a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=None), EINVAL, "non-null"),
    (dict(k=24), EINVAL, "aligned"),
    (dict(h_q=3, h_kv=2), EINVAL, "multiple"),
    (dict(h_kv=0), EINVAL, ">= 1"),
    (dict(d=96), EUNSUP, "not supported"),
    (dict(dtype=7), EINVAL, "dtype"),
    (dict(C=0), EINVAL, "C must"),
    (dict(S_kv=10, C=4), EINVAL, "multiple of C"),
    (dict(causal=1, T_q=8, S_kv=16), EINVAL, "T_q == S_kv"),
    (dict(n_seqs=0), EINVAL, "n_seqs"),
    (dict(T_q=-1), EINVAL, ">= 0"),
    (dict(S_kv=0), EINVAL, "undefined"),
    (dict(seq_offsets=16, n_seqs=2, T_q=8, S_kv=8), EINVAL, "workspace"),
    (dict(seq_offsets=16, n_seqs=2, T_q=8, S_kv=9), EINVAL, "T_q == S_kv"),
    (dict(seq_offsets=18, n_seqs=2), EINVAL, "4-byte"),
])
def test_ring_attn_fwd_rejects(kw, code, msg):
    assert _ring(**kw) == code
    assert msg in F.lib().fakv_last_error().decode()


def test_valid_empty_call_enqueues_nothing():
    # T_q == 0 is valid and returns before any HIP call
    assert _ring(T_q=0, S_kv=0) == 0 and F.lib().fakv_last_error() == b""
    # nothing is read or written, so the data pointers may be NULL
    assert _ring(q=None, k=None, v=None, o=None, T_q=0, S_kv=0) == 0
    # a jagged batch of empty sequences: the workspace size is 0 and none is needed
    assert F.ring_attn_workspace_bytes(0, 0, 4, 2, 128, 1, 1, 3, 1, F.BF16) == 0
    assert _ring(q=None, k=None, v=None, o=None, T_q=0, S_kv=0, seq_offsets=16, n_seqs=3) == 0
    assert F.lib().attn_partial(None, None, None, None, None, None, 0, 64, 4, 2, 128, 0, 0, 1, 1,
                                F.BF16, None) == 0
    # with rows to compute, NULL data pointers are still refused
    assert _ring(q=None, T_q=8, S_kv=8) == EINVAL


def test_other_entry_points_reject():
    L = F.lib()
    assert L.attn_partial(16, 16, 16, 16, None, 16, 4, 4, 2, 1, 64, 0, 0, 0, 0, 1, None) == EINVAL
    assert b"non-null" in L.fakv_last_error()
    assert L.attn_partial(16, 16, 16, 16, 16, 16, 4, 4, 2, 1, 48, 0, 0, 0, 0, 1, None) == EUNSUP
    assert L.lse_merge(16, 16, 16, 0, 4, 64, 16, None, 1, None) == EINVAL
    assert L.lse_merge(16, 16, 16, 2, 4, 32, 16, None, 1, None) == EUNSUP
    ws = F.splitkv_decode_workspace_bytes(2, 8, 128, 4)
    assert L.splitkv_decode(16, 16, 16, 16, 2, 8, 1, 128, 64, 4, F.F32, 16, ws, None) == EUNSUP
    assert L.splitkv_decode(16, 16, 16, 16, 2, 8, 1, 128, 64, 65, F.BF16, 16, ws, None) == EINVAL
    assert L.splitkv_decode(16, 16, 16, 16, 2, 64, 1, 128, 64, 4, F.BF16, 16, 10**9, None) == EUNSUP
    assert L.splitkv_decode(16, 16, 16, 16, 2, 8, 1, 128, 64, 4, F.BF16, 16, ws - 1, None) == EINVAL
    assert L.fakv_jagged_worklist(16, 2, 100, 32, 16, 16, 4, None) == EINVAL
    assert b"capacity" in L.fakv_last_error()


def test_attn_partial_empty_chunk_accepts_null_kv():
    """An empty KV chunk reads no key, so k and v may be NULL (torch gives an
    empty tensor a null data pointer): merging it into a running state is a
    valid call that enqueues nothing; q must still be given."""
    L = F.lib()
    assert L.attn_partial(16, None, None, 16, 16, 16, 4, 0, 2, 1, 64, 0, 0, 1, 1, F.BF16, None) == 0
    assert L.attn_partial(None, None, None, 16, 16, 16, 4, 0, 2, 1, 64, 0, 0, 1, 1, F.BF16, None) == EINVAL
    assert L.attn_partial(16, None, 16, 16, 16, 16, 4, 4, 2, 1, 64, 0, 0, 1, 1, F.BF16, None) == EINVAL


def test_attn_partial_rejects_positions_beyond_32_bit_range():
    """Query and key positions are compared in 32-bit arithmetic on the device:
    positions beyond 2^29 (or a chunk reaching past it) are refused on the
    host, before any HIP call."""
    L = F.lib()
    lim = 1 << 29
    for qp, kp, T, S in ((lim, 0, 4, 4), (0, lim - 2, 4, 4), (-lim - 1, 0, 4, 4), (0, -lim - 5, 4, 4),
                         (2**31 - 1, -2**31, 4, 4)):
        assert L.attn_partial(16, 16, 16, 16, 16, 16, T, S, 2, 1, 64, qp, kp, 1, 0, F.BF16, None) == EINVAL, (qp, kp)
        assert "positions" in F.lib().fakv_last_error().decode()
    # the limits themselves are accepted by the checks (the call then needs a GPU, so only
    # the refusal above is exercised here)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import flash_attention_kv_amd._binding as B
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        B.lib()


def test_window_entry_rejects():
    L = F.lib()
    # sliding window: window >= 1, and the ring_attn_fwd checks apply
    assert L.ring_attn_fwd_window(16, 16, 16, 16, 8, 8, 4, 2, 128, 1, 0, None, 1, F.BF16, None, 0, None) == EINVAL
    assert b"window" in L.fakv_last_error()
    assert L.ring_attn_fwd_window(16, 16, 16, 16, 8, 16, 4, 2, 128, 1, 4, None, 1, F.BF16, None, 0, None) == EINVAL
    assert b"T_q == S_kv" in L.fakv_last_error()
    assert L.ring_attn_fwd_window(16, 16, 16, 16, 0, 0, 4, 2, 128, 1, 4, None, 1, F.BF16, None, 0, None) == 0


def test_kv_span_limit():
    # one sequence's K (or V) span must stay below 2 GiB (the buffer resources
    # that bound every tile load are 31-bit); 65535 keys x 64 heads x d = 256
    # is the largest such span, one key more is refused before any HIP call
    L = F.lib()
    assert _ring(T_q=0, S_kv=65535, h_q=64, h_kv=64, d=256) == 0
    assert _ring(T_q=0, S_kv=65536, h_q=64, h_kv=64, d=256) == EUNSUP
    assert b"2 GiB" in L.fakv_last_error()
    assert L.attn_partial(16, 16, 16, 16, 16, 16, 8, 65536, 64, 64, 256, 0, 0, 0, 0, F.BF16, None) == EUNSUP
    assert b"2 GiB" in L.fakv_last_error()
    ws = F.splitkv_decode_workspace_bytes(1, 64, 256, 64)
    assert L.splitkv_decode(16, 16, 16, 16, 1, 64, 64, 256, 65536, 64, F.BF16, 16, ws, None) == EUNSUP
    assert b"2 GiB" in L.fakv_last_error()


def test_noalloc_decode_rejects_before_any_hip_call():
    """splitkv_decode_noalloc applies splitkv_decode's checks and refuses a
    call whose partial triplets would not fit the library's scratch, all on
    the host (no device is touched)."""
    L = F.lib()
    assert L.splitkv_decode_noalloc(16, 16, 16, 16, 2, 8, 1, 128, 64, 4, F.F32, None) == EUNSUP
    assert L.splitkv_decode_noalloc(16, 16, 16, 16, 2, 8, 1, 128, 64, 65, F.BF16, None) == EINVAL
    assert L.splitkv_decode_noalloc(None, 16, 16, 16, 2, 8, 1, 128, 64, 4, F.BF16, None) == EINVAL
    # the decode workload's partials (17 MB) fit; 64 more chunks do not
    assert F.splitkv_decode_workspace_bytes(8, 64, 128, 64) <= F.DECODE_SCRATCH_BYTES
    assert F.splitkv_decode_workspace_bytes(8, 64, 128, 128) > F.DECODE_SCRATCH_BYTES
    assert L.splitkv_decode_noalloc(16, 16, 16, 16, 8, 64, 8, 128, 131072, 128, F.BF16, None) == EINVAL
    assert b"scratch" in L.fakv_last_error()
    header = open(HEADER).read()
    assert "#define FAKV_DECODE_SCRATCH_BYTES (32u << 20)" in header
    assert F.DECODE_SCRATCH_BYTES == 32 << 20
