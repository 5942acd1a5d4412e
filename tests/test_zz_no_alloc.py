"""splitkv_decode_noalloc against splitkv_decode on the GPU: the entry point
that keeps its partial triplets in the library's own per-device scratch must
give the result of the workspace entry point on the same inputs, call after
call, including a second call on a smaller input (the scratch keeps the
first call's triplets; every triplet the second call reads it also writes)."""
import pytest
import torch

import flash_attention_kv_amd as F
import oracle
from tests._gpu import check, host
from workloads import randn

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _decode_pair(B, h_q, h_kv, d, S, n_chunks, seed):
    q, k, v = (t.to(DEV) for t in randn([(B, h_q, d), (B, S, h_kv, d), (B, S, h_kv, d)], seed, "bf16"))
    ref_out = F.splitkv_decode(q, k, v, n_chunks=n_chunks)
    out = torch.full_like(q, 7.0)
    got = F.splitkv_decode_noalloc(q, k, v, n_chunks=n_chunks, out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    return (q, k, v), ref_out, out


def test_noalloc_decode_matches_workspace_entry_twice():
    # first call: many chunks and heads (fills a large part of the scratch)
    (q, k, v), ref1, got1 = _decode_pair(4, 64, 8, 128, 20000, 64, 11)
    assert torch.equal(got1, ref1)
    # second call, smaller: fewer chunks, rows and a different head dim
    (q2, k2, v2), ref2, got2 = _decode_pair(2, 8, 2, 64, 700, 5, 12)
    assert torch.equal(got2, ref2)
    check(host(got2), oracle.splitkv_decode_ref(q2.cpu(), k2.cpu(), v2.cpu(), 5), "bf16", "noalloc decode (small)")
    # the first input again after the smaller one: still equal
    got3 = F.splitkv_decode_noalloc(q, k, v, n_chunks=64, out=torch.empty_like(q))
    torch.cuda.synchronize()
    assert torch.equal(got3, ref1)


def test_noalloc_decode_at_decode_workload_size():
    """The decode workload's shape (B = 8, 64/8 heads, d = 128, 64 chunks) with
    a shorter cache: its 17 MB of partials fit the 32 MiB scratch."""
    (q, k, v), ref, got = _decode_pair(8, 64, 8, 128, 8192, 64, 13)
    assert torch.equal(got, ref)


def test_noalloc_decode_refuses_oversize():
    q, k, v = (t.to(DEV) for t in randn([(8, 64, 128), (8, 256, 8, 128), (8, 256, 8, 128)], 14, "bf16"))
    out = torch.full_like(q, 7.0)
    with pytest.raises(F.FakvError, match="scratch"):
        F.splitkv_decode_noalloc(q, k, v, n_chunks=256, out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
