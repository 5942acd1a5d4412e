"""ctypes binding of libfakv.so (the C ABI in include/fakv.h).

Argument marshalling only: each wrapper checks torch dtypes, devices, shapes
and contiguity, allocates the outputs (PyTorch is the allocator), passes raw
device pointers plus torch's current HIP stream, and raises on a non-zero
status.  Every step of the computation runs in the library's HIP kernels;
there is no fallback of any kind.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfakv.so")

F32, BF16 = 0, 1
STATUS = {0: "FAKV_OK", 1: "FAKV_EINVAL", 2: "FAKV_EUNSUPPORTED", 3: "FAKV_EDEVICE"}

# name -> (restype, argtypes); mirrors include/fakv.h
_P, _I, _SZ, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = {
    "attn_partial": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    "lse_merge": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _I, _P]),
    "ring_attn_fwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _I, _I, _P, _SZ, _P]),
    "ring_attn_fwd_window": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _I, _I, _P, _SZ, _P]),
    "ring_attn_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "splitkv_decode": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _SZ, _P]),
    "splitkv_decode_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "splitkv_decode_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "fakv_jagged_worklist": (_I, [_P, _I, _I, _I, _P, _P, _SZ, _P]),
    "fakv_query_tile_rows": (_I, [_I, _I, _I, _I]),
    "fakv_last_error": (ctypes.c_char_p, []),
    "fakv_abi_version": (_I, []),
}

_lib = None


class FakvError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with {STATUS.get(status, status)}: {msg}")
        self.status = status


def lib():
    """The loaded library.  Raises if it has not been built: the product path
    has no substitute for it."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m flash_attention_kv_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise FakvError(fn, status, lib().fakv_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(*ts: torch.Tensor):
    idx = ts[0].get_device()          # -1 for host tensors
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a HIP device")
        if t.get_device() != idx:
            raise ValueError("tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return ts[0].device


def _out_like(out: Optional[torch.Tensor], ref: torch.Tensor) -> torch.Tensor:
    """The caller's output tensor, checked to be exactly like ref (device,
    dtype, shape, contiguity), or a new one."""
    if out is None:
        return torch.empty_like(ref)
    _dev(ref, out)
    if out.dtype != ref.dtype or out.shape != ref.shape:
        raise ValueError(f"out must be {ref.dtype} {tuple(ref.shape)}, got {out.dtype} {tuple(out.shape)}")
    return out


def _ptr(t: Optional[torch.Tensor]):
    # a plain int: the c_void_p argtypes convert it (None is NULL)
    return None if t is None else t.data_ptr()


# torch's current HIP stream of a device as a raw handle.  The raw-stream query
# skips building a torch.cuda.Stream object per call (about 1.7 us on the
# host); where this torch build lacks it, the public API gives the same handle.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


_SAME_DEVICE = contextlib.nullcontext()


def _on(dev):
    """The tensors' device made current for the call (the C ABI enqueues on the
    current HIP device); no device switch when it already is current."""
    cur = torch.cuda.current_device()
    if dev.index is None or dev.index == cur:
        return _SAME_DEVICE
    return torch.cuda.device(dev.index)


def _stream(dev) -> int:
    if _raw_stream is not None:
        return _raw_stream(dev.index if dev.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(dev).cuda_stream


def query_tile_rows(h_q: int, h_kv: int, d: int, dtype: int = BF16) -> int:
    return lib().fakv_query_tile_rows(h_q, h_kv, d, dtype)


@functools.lru_cache(maxsize=256)
def _ring_ws_bytes(T_q, S_kv, h_q, h_kv, d, C, causal, n_seqs, jagged, dtype) -> int:
    return lib().ring_attn_workspace_bytes(T_q, S_kv, h_q, h_kv, d, C, causal, n_seqs, jagged, dtype)


def ring_attn_workspace_bytes(T_q, S_kv, h_q, h_kv, d, C, causal, n_seqs, jagged, dtype) -> int:
    # a pure function of its integer arguments: cached per shape
    return _ring_ws_bytes(int(T_q), int(S_kv), int(h_q), int(h_kv), int(d), int(C), int(causal),
                          int(n_seqs), int(jagged), int(dtype))


def splitkv_decode_workspace_bytes(B, h_q, d, n_chunks) -> int:
    return lib().splitkv_decode_workspace_bytes(B, h_q, d, n_chunks)


def ring_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, C: int = 1,
                  causal: bool = False, seq_offsets: Optional[torch.Tensor] = None,
                  n_seqs: int = 1, workspace: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, window: Optional[int] = None) -> torch.Tensor:
    """Prefill attention.  q (n_seqs*T_q, h_q, d), k/v (n_seqs*S_kv, h_kv, d);
    jagged when ``seq_offsets`` (int32, n_seqs+1, on the device) is given.
    ``window`` W (causal only): query i sees keys i - W < j <= i
    (``ring_attn_fwd_window``)."""
    dev = _dev(q, k, v)
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be (tokens, h_q, d) and k, v (tokens, h_kv, d)")
    Tt, h_q, d = q.shape
    St, h_kv, dk = k.shape
    if v.shape != k.shape or dk != d:
        raise ValueError("shape mismatch between q, k and v")
    if seq_offsets is not None:
        _dev(seq_offsets)
        if seq_offsets.dtype != torch.int32 or seq_offsets.dim() != 1:
            raise TypeError("seq_offsets must be a 1-D int32 tensor")
        n_seqs = seq_offsets.numel() - 1
        T_q, S_kv = Tt, St
    else:
        if Tt % n_seqs or St % n_seqs:
            raise ValueError("token counts must divide by n_seqs")
        T_q, S_kv = Tt // n_seqs, St // n_seqs
    o = _out_like(out, q)
    need = ring_attn_workspace_bytes(T_q, S_kv, h_q, h_kv, d, C, causal, n_seqs,
                                     seq_offsets is not None, dt)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif need:
        _dev(q, workspace)
    if window is None:
        with _on(dev):
            st = lib().ring_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), T_q, S_kv, h_q, h_kv, d, C,
                                     int(causal), _ptr(seq_offsets), n_seqs, dt,
                                     _ptr(workspace) if need else None, need, _stream(dev))
        _check("ring_attn_fwd", st)
    else:
        if not causal:
            raise ValueError("a sliding window needs causal=True")
        with _on(dev):
            st = lib().ring_attn_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), T_q, S_kv, h_q, h_kv, d, C,
                                            int(window), _ptr(seq_offsets), n_seqs, dt,
                                            _ptr(workspace) if need else None, need, _stream(dev))
        _check("ring_attn_fwd_window", st)
    return o


def attn_partial(q, k, v, *, q_pos0: int = 0, k_pos0: int = 0, causal: bool = False,
                 state: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Partial triplet (m, l, O) of q (T, h_q, d) against one KV chunk
    (n, h_kv, d); with ``state`` = (m, l, O) it is merged into that state in
    place and the same tensors are returned."""
    dev = _dev(q, k, v)
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be (T, h_q, d) and k, v (n, h_kv, d)")
    T, h_q, d = q.shape
    n, h_kv, dk = k.shape
    if v.shape != k.shape or dk != d:
        raise ValueError("shape mismatch between q, k and v")
    if state is None:
        m = torch.empty((T, h_q), dtype=torch.float32, device=dev)
        l = torch.empty((T, h_q), dtype=torch.float32, device=dev)
        o = torch.empty((T, h_q, d), dtype=torch.float32, device=dev)
        acc = 0
    else:
        m, l, o = state
        _dev(m, l, o)
        if any(t.dtype != torch.float32 for t in (m, l, o)):
            raise TypeError("state tensors must be float32")
        if m.shape != (T, h_q) or l.shape != (T, h_q) or o.shape != (T, h_q, d):
            raise ValueError("state shapes must be (T, h_q), (T, h_q), (T, h_q, d)")
        acc = 1
    with _on(dev):
        st = lib().attn_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(l), _ptr(o), T, n, h_q, h_kv,
                                d, q_pos0, k_pos0, int(causal), acc, dt, _stream(dev))
    _check("attn_partial", st)
    return m, l, o


def lse_merge(m_parts, l_parts, o_parts, *, out_dtype=torch.bfloat16, return_lse: bool = False):
    """Merge n triplets per row: m/l (n, rows), O (n, rows, d) -> O / l (rows, d)."""
    dev = _dev(m_parts, l_parts, o_parts)
    if any(t.dtype != torch.float32 for t in (m_parts, l_parts, o_parts)):
        raise TypeError("m_parts, l_parts and o_parts must be float32")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"out_dtype must be torch.bfloat16 or torch.float32, got {out_dtype}")
    if o_parts.dim() != 3:
        raise ValueError("o_parts must be (n_parts, rows, d)")
    n, rows, d = o_parts.shape
    if m_parts.shape != (n, rows) or l_parts.shape != (n, rows):
        raise ValueError("m_parts and l_parts must be (n_parts, rows)")
    out = torch.empty((rows, d), dtype=out_dtype, device=dev)
    lse = torch.empty(rows, dtype=torch.float32, device=dev) if return_lse else None
    with _on(dev):
        st = lib().lse_merge(_ptr(m_parts), _ptr(l_parts), _ptr(o_parts), n, rows, d, _ptr(out),
                             _ptr(lse), BF16 if out_dtype == torch.bfloat16 else F32, _stream(dev))
    _check("lse_merge", st)
    return (out, lse) if return_lse else out


def splitkv_decode(q, k, v, *, n_chunks: int, workspace: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None):
    """One decode step: q (B, h_q, d), K/V cache (B, S, h_kv, d) -> o (B, h_q, d)."""
    dev = _dev(q, k, v)
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be (B, h_q, d) and k, v (B, S, h_kv, d)")
    B, h_q, d = q.shape
    Bk, S, h_kv, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k and v")
    o = _out_like(out, q)
    need = splitkv_decode_workspace_bytes(B, h_q, d, n_chunks)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _dev(q, workspace)
    with _on(dev):
        st = lib().splitkv_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, h_q, h_kv, d, S, n_chunks, dt,
                                  _ptr(workspace), need, _stream(dev))
    _check("splitkv_decode", st)
    return o


# bytes of the per-device scratch splitkv_decode_noalloc uses (FAKV_DECODE_SCRATCH_BYTES)
DECODE_SCRATCH_BYTES = 32 << 20


def splitkv_decode_noalloc(q, k, v, *, n_chunks: int, out: torch.Tensor):
    """splitkv_decode with the library's own per-device scratch for the
    partial triplets: no workspace, and the caller passes the output, so the
    call allocates nothing.  Calls that may overlap on one device race on
    that scratch (serialise them, e.g. on one stream)."""
    dev = _dev(q, k, v)
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be (B, h_q, d) and k, v (B, S, h_kv, d)")
    B, h_q, d = q.shape
    Bk, S, h_kv, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k and v")
    o = _out_like(out, q)
    with _on(dev):
        st = lib().splitkv_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, h_q, h_kv, d, S, n_chunks, dt,
                                          _stream(dev))
    _check("splitkv_decode_noalloc", st)
    return o


def jagged_worklist(seq_offsets: torch.Tensor, total_tokens: int, BQ: int):
    """Device-built worklist: (records int32 (capacity, 8), count int32 (1,))."""
    dev = _dev(seq_offsets)
    n_seqs = seq_offsets.numel() - 1
    cap = total_tokens // BQ + n_seqs
    items = torch.zeros((max(cap, 1), 8), dtype=torch.int32, device=dev)
    n_items = torch.zeros(1, dtype=torch.int32, device=dev)
    with _on(dev):
        st = lib().fakv_jagged_worklist(_ptr(seq_offsets), n_seqs, total_tokens, BQ, _ptr(items),
                                        _ptr(n_items), cap, _stream(dev))
    _check("fakv_jagged_worklist", st)
    return items, n_items
