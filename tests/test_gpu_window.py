"""GPU parity of the causal sliding window (ring_attn_fwd_window): query i
sees keys i - W < j <= i.  Against the fp64 oracle on the same inputs, over
head dims, GQA groupings, ring chunk counts, ragged lengths, jagged batches
and fp32; plus what must hold bit for bit: W = 1 returns V, W >= the
sequence length is plain causal attention, and skipping the tiles below the
window (dependent lower bound, whole-chunk skip) equals masking them."""
import numpy as np
import pytest
import torch

import flash_attention_kv_amd as F
import oracle
from tests._gpu import check, host
from workloads import randn, seq_offsets_from_lengths

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _qkv(T, h_q, h_kv, d, dtype, seed):
    q, k, v = randn([(T, h_q, d), (T, h_kv, d), (T, h_kv, d)], seed, dtype)
    return q, k, v


CASES = [
    # T, h_q, h_kv, d, C, n_seqs, W
    (300, 8, 2, 128, 2, 1, 64),
    (513, 4, 1, 128, 1, 1, 100),
    (256, 32, 8, 128, 8, 1, 17),
    (300, 6, 3, 64, 3, 1, 129),
    (200, 2, 2, 256, 4, 1, 40),
    (192, 4, 4, 128, 1, 3, 33),
    (129, 2, 1, 64, 1, 2, 1000),
    (640, 4, 2, 128, 4, 1, 1),
]


@pytest.mark.parametrize("T,h_q,h_kv,d,C,n_seqs,W", CASES)
def test_window_bf16(T, h_q, h_kv, d, C, n_seqs, W):
    q, k, v = _qkv(n_seqs * T, h_q, h_kv, d, "bf16", T + W + d)
    o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=C, causal=True, n_seqs=n_seqs, window=W)
    torch.cuda.synchronize()
    ref = oracle.attention_ref(q, k, v, causal=True, n_seqs=n_seqs, window=W)
    check(host(o), ref, "bf16", f"window T={T} h={h_q}/{h_kv} d={d} C={C} W={W}")


def test_window_f32():
    T, W = 300, 33
    q, k, v = _qkv(T, 2, 1, 64, "f32", 3)
    o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=2, causal=True, window=W)
    torch.cuda.synchronize()
    check(host(o), oracle.attention_ref(q, k, v, causal=True, window=W), "f32", "window f32")


@pytest.mark.parametrize("W", [1, 50, 700])
def test_window_jagged(W):
    lens = [300, 1, 77, 0, 200, 1025]
    T = sum(lens)
    q, k, v = _qkv(T, 4, 4, 128, "bf16", 7 + W)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, window=W,
                        seq_offsets=torch.from_numpy(offs).to(DEV))
    torch.cuda.synchronize()
    check(host(o), oracle.attention_ref(q, k, v, causal=True, seq_offsets=offs, window=W), "bf16",
          f"window jagged W={W}")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_window_one_returns_v(d):
    T, h_q, h_kv = 200, 4, 2
    q, k, v = (x.to(DEV) for x in _qkv(T, h_q, h_kv, d, "bf16", d))
    o = F.ring_attn_fwd(q, k, v, C=2, causal=True, window=1)
    torch.cuda.synchronize()
    assert torch.equal(o, v.repeat_interleave(h_q // h_kv, dim=1))


@pytest.mark.parametrize("d,C", [(128, 4), (256, 1)])
def test_window_covering_sequence_is_causal_bitwise(d, C):
    T = 256
    q, k, v = (x.to(DEV) for x in _qkv(T, 8, 2, d, "bf16", 11))
    a = F.ring_attn_fwd(q, k, v, C=C, causal=True)
    b = F.ring_attn_fwd(q, k, v, C=C, causal=True, window=T)
    c = F.ring_attn_fwd(q, k, v, C=C, causal=True, window=10 * T)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("d,heads,C,W", [(128, (8, 2), 2, 70), (64, (2, 2), 1, 5), (256, (4, 4), 3, 97)])
def test_window_pruning_equals_masking_bitwise(d, heads, C, W, monkeypatch):
    h_q, h_kv = heads
    T = 384
    q, k, v = (x.to(DEV) for x in _qkv(T, h_q, h_kv, d, "bf16", d + C + W))
    a = F.ring_attn_fwd(q, k, v, C=C, causal=True, window=W)
    monkeypatch.setenv("FAKV_NO_PRUNE", "1")
    b = F.ring_attn_fwd(q, k, v, C=C, causal=True, window=W)
    monkeypatch.delenv("FAKV_NO_PRUNE")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("jagged", [False, True])
def test_window_beyond_any_sequence_is_causal(jagged):
    """A window far longer than any sequence (2^31 - 1 keys) admits every
    causal key: plain causal attention (the window bounds are computed in
    32 bits on the device, so such a window must not wrap them)."""
    h_q, h_kv, d = 4, 2, 128
    if jagged:
        lens = [300, 1, 0, 129]
        offs = seq_offsets_from_lengths(lens)
        N = int(offs[-1])
        q, k, v = randn([(N, h_q, d), (N, h_kv, d), (N, h_kv, d)], 71, "bf16")
        o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, window=2**31 - 1,
                            seq_offsets=torch.from_numpy(offs).to(DEV))
        ref = oracle.attention_ref(q, k, v, causal=True, seq_offsets=offs)
    else:
        T = 300
        q, k, v = randn([(T, h_q, d), (T, h_kv, d), (T, h_kv, d)], 72, "bf16")
        o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=2, causal=True, window=2**31 - 1)
        ref = oracle.attention_ref(q, k, v, causal=True)
    torch.cuda.synchronize()
    check(host(o), ref, "bf16", f"window 2^31-1 jagged={jagged}")
