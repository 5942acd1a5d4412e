"""GPU tests of argument handling: offsets whose differences wrap are refused
on the device, the binding refuses mismatched dtypes and shapes before it
enqueues anything, and lse_merge gives an all-empty row a defined result."""
import numpy as np
import pytest
import torch

import flash_attention_kv_amd as F
from workloads import randn

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# Offsets whose pairwise int32 differences are all non-negative only because
# one of them wraps: 1610612736 -> -1610612736 is a decreasing pair.
WRAPPING = [0, 1610612736, -1610612736, 0, 100]


def test_worklist_refuses_wrapping_offsets():
    offs = torch.tensor(WRAPPING, dtype=torch.int32, device=DEV)
    items, n = F.jagged_worklist(offs, 100, 64)
    torch.cuda.synchronize()
    assert int(n.item()) == 0


def test_worklist_refuses_out_of_range_offsets():
    for offs in ([0, -5, 100], [0, 150, 100], [0, 2147483647, 100]):
        items, n = F.jagged_worklist(torch.tensor(offs, dtype=torch.int32, device=DEV), 100, 32)
        torch.cuda.synchronize()
        assert int(n.item()) == 0, offs


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ring_wrapping_offsets_leave_output_untouched(dtype):
    N = 100
    q, k, v = (t.to(DEV) for t in randn([(N, 2, 64), (N, 1, 64), (N, 1, 64)], 3, dtype))
    o = torch.full(q.shape, 7.0, dtype=q.dtype, device=DEV)
    F.ring_attn_fwd(q, k, v, causal=True, seq_offsets=torch.tensor(WRAPPING, dtype=torch.int32, device=DEV),
                    out=o)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())


def _launches():
    """A refused call enqueued nothing: the stream drains without error."""
    torch.cuda.synchronize()


def test_lse_merge_refuses_dtypes():
    n, rows, d = 2, 3, 64
    m = torch.zeros(n, rows, device=DEV)
    l = torch.ones(n, rows, device=DEV)
    o = torch.zeros(n, rows, d, device=DEV)
    with pytest.raises(TypeError):
        F.lse_merge(m, l, o, out_dtype=torch.float16)
    with pytest.raises(TypeError):
        F.lse_merge(m, l, o.to(torch.bfloat16))
    with pytest.raises(TypeError):
        F.lse_merge(m.to(torch.bfloat16), l, o)
    with pytest.raises(TypeError):
        F.lse_merge(m, l.double(), o)
    _launches()


def test_attn_partial_refuses_mismatches():
    q, k, v = (t.to(DEV) for t in randn([(32, 4, 128), (16, 2, 128), (16, 2, 128)], 4, "bf16"))
    with pytest.raises(ValueError):
        F.attn_partial(q, k[..., :64].contiguous(), v[..., :64].contiguous())   # head dim of k
    with pytest.raises(ValueError):
        F.attn_partial(q, k, v[:8].contiguous())                                 # v rows
    with pytest.raises(TypeError):
        F.attn_partial(q, k.float(), v.float())                                   # k/v dtype
    with pytest.raises(TypeError):
        F.attn_partial(q, k, v.float())
    _launches()


def test_splitkv_decode_refuses_mismatched_dtypes():
    q, k, v = (t.to(DEV) for t in randn([(2, 4, 128), (2, 64, 2, 128), (2, 64, 2, 128)], 5, "bf16"))
    o = torch.full(q.shape, 7.0, dtype=q.dtype, device=DEV)
    with pytest.raises(TypeError):
        F.splitkv_decode(q, k.float(), v, n_chunks=2, out=o)
    with pytest.raises(TypeError):
        F.splitkv_decode(q, k, v.float(), n_chunks=2, out=o)
    _launches()
    assert bool((o == 7.0).all())


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_lse_merge_all_empty_row(out):
    """Rows whose parts are all the identity (-inf, 0, 0) merge to the
    identity: the output row is zero and its lse -inf.  Other rows merge as
    usual."""
    n, rows, d = 5, 4, 128
    rng = np.random.default_rng(9)
    m = rng.normal(size=(n, rows)) * 2
    l = rng.uniform(0.5, 3.0, size=(n, rows))
    O = rng.normal(size=(n, rows, d))
    m[:, 1] = -np.inf
    l[:, 1] = 0.0
    O[:, 1] = 0.0
    mt, lt, Ot = (torch.tensor(x, dtype=torch.float32, device=DEV) for x in (m, l, O))
    got, lse = F.lse_merge(mt, lt, Ot, out_dtype=out, return_lse=True)
    torch.cuda.synchronize()
    g = got.float().cpu().numpy()
    assert np.all(g[1] == 0.0)
    assert np.isneginf(float(lse[1]))
    others = [0, 2, 3]
    assert np.all(np.isfinite(g[others])) and torch.isfinite(lse[others]).all()
