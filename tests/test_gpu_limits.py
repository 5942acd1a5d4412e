"""The largest inputs the boundary accepts.

Every K/V load goes through a buffer resource that spans one sequence's keys
of one KV head, so a sequence's K (or V) span -- keys x h_kv x d x 2 bytes --
must stay below 2 GiB; the library rejects anything larger (checked on the
CPU in test_abi.py).  Here the span is one key short of that bound (65535
keys x 64 heads x d = 256: 2,147,450,880 bytes), so tile offsets reach the top
of the 31-bit range, and sampled rows are compared with the oracle."""
import numpy as np
import pytest
import torch

import flash_attention_kv_amd as F
import oracle
from tests._gpu import check, host
from workloads import Workload, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
S_MAX, H, D = 65535, 64, 256          # 65535 * 64 * 256 * 2 < 2^31 <= 65536 * 64 * 256 * 2


def test_prefill_largest_kv_span():
    w = Workload("kv_span_limit", "prefill", "bf16", h_q=H, h_kv=H, d=D, seed=41,
                 T_q=64, S_kv=S_MAX, C=1, causal=False)
    q, k, v, _ = make_prefill_inputs(w, device=DEV)
    assert k.numel() * 2 == S_MAX * H * D * 2 and k.numel() * 2 < 2 ** 31
    o = F.ring_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    hs = [0, 31, H - 1]                       # heads checked (the oracle sees only these)
    qs, ks, vs = q[:, hs].cpu(), k[:, hs].cpu(), v[:, hs].cpu()
    toks = np.array([0, 1, 31, 32, 62, 63])
    heads = np.array([0, 1, 2, 0, 1, 2])
    ref = oracle.attention_rows_ref(qs, ks, vs, toks, heads)
    got = host(o[:, hs])[toks, heads]
    check(got, ref, "bf16", "prefill at the largest K/V span")


def test_decode_largest_kv_span():
    w = Workload("kv_span_limit_decode", "decode", "bf16", h_q=H, h_kv=H, d=D, seed=42,
                 B=1, S_cache=S_MAX, n_chunks=64)
    q, k, v = make_decode_inputs(w, device=DEV)
    o = F.splitkv_decode(q, k, v, n_chunks=w.n_chunks)
    torch.cuda.synchronize()
    hs = [0, 40, H - 1]
    # one query token per (sequence, head): the decode rows are prefill rows
    # of a single query against the whole cache
    qs = q[0, hs].cpu().reshape(1, len(hs), D)
    ks, vs = k[0, :, hs].cpu(), v[0, :, hs].cpu()
    ref = oracle.attention_rows_ref(qs, ks, vs, np.zeros(3, int), np.arange(3))
    got = host(o[0, hs])
    check(got, ref, "bf16", "decode at the largest K/V span")
