"""GPU tests of the bf16 prefill kernels' LDS staging of Q rows (whole-row
loads into LDS, read back into the MFMA operand layout) and of output rows
(written to LDS in the accumulator layout, stored as whole rows), on every
instance the dispatch picks: dense d = 128 on 8 waves with 128-key tiles
(4 or 1 query heads per workgroup), dense d = 128 with a window and d = 64
on 4 waves, d = 256 (output staged, Q in registers), and the persistent
jagged instances.  Row counts leave a wave's 32 rows wholly, partly or not at
all inside the tile, so the rows the buffer resources read as zero and the
stores skipped past the tile's end are both exercised; everything is checked
against the oracle's definition of attention ("_gqa_prefill_long.py": the
final O / l of the ring; "[pallas] Support dependent Tile.end bounds in
Pallas": causal and sliding-window bounds)."""
import numpy as np
import pytest
import torch

import flash_attention_kv_amd as F
import oracle
from tests._gpu import check, host
from workloads import randn, seq_offsets_from_lengths

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (h_q, h_kv, d, window) -> the kernel instance the dispatch picks
INSTANCES = [(8, 2, 128, None),   # 4 query heads per 8-wave workgroup, 128-key tiles
             (4, 4, 128, None),   # 1 query head per 8-wave workgroup (256 rows)
             (8, 2, 128, 40),     # sliding window: 4 waves, 64-key tiles
             (4, 2, 64, None),    # d = 64: 4 waves
             (2, 2, 256, None)]   # d = 256: output staged, Q rows in registers


@pytest.mark.parametrize("h_q,h_kv,d,window", INSTANCES)
@pytest.mark.parametrize("T", [1, 17, 33, 95, 161])
def test_dense_ragged_rows(h_q, h_kv, d, window, T):
    causal = window is not None or T % 2 == 1
    q, k, v = randn([(T, h_q, d), (T, h_kv, d), (T, h_kv, d)], 500 + T + d + h_q, "bf16")
    o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=1, causal=causal, window=window)
    torch.cuda.synchronize()
    ref = oracle.attention_ref(q, k, v, causal=causal, window=window)
    check(host(o), ref, "bf16", f"T={T} heads {h_q}/{h_kv} d={d} window={window}")


@pytest.mark.parametrize("T", [1, 33, 95])
@pytest.mark.parametrize("h_q,h_kv,d", [(8, 2, 128), (4, 2, 64)])
def test_partial_ragged_rows(T, h_q, h_kv, d):
    """attn_partial writes and then accumulates fp32 triplets; its Q rows go
    through the same LDS staging."""
    S = 96
    q, k, v = randn([(T, h_q, d), (2 * S, h_kv, d), (2 * S, h_kv, d)], 700 + T + d, "bf16")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    st, ref = None, None
    for c in (1, 0):
        st = F.attn_partial(qd, kd[c * S:(c + 1) * S].contiguous(), vd[c * S:(c + 1) * S].contiguous(),
                            q_pos0=S, k_pos0=c * S, causal=True, state=st)
        ref = oracle.attn_partial_ref(q, k[c * S:(c + 1) * S], v[c * S:(c + 1) * S], q_pos0=S,
                                      k_pos0=c * S, causal=True, state=ref)
    torch.cuda.synchronize()
    m, l, o = (host(x) for x in st)
    fin = np.isfinite(ref.m)
    assert np.array_equal(np.isfinite(m), fin)
    np.testing.assert_allclose(m[fin], ref.m[fin], atol=1e-4, rtol=0)
    np.testing.assert_allclose(l[fin], ref.l[fin], rtol=2e-2)
    check(o[fin] / l[fin][:, None], ref.O[fin] / ref.l[fin][:, None], "bf16", f"partial T={T} d={d}",
          out_bf16=False)


@pytest.mark.parametrize("d,heads", [(128, (4, 4)), (128, (8, 2)), (64, (4, 4)), (64, (8, 8))])
def test_jagged_ragged_rows(d, heads):
    """Sequences whose lengths put the item's last rows anywhere in a wave's
    32, one-row and empty sequences included, and enough items per
    workgroup that the staged Q rows of one item follow another's output."""
    h_q, h_kv = heads
    lens = [1, 31, 33, 255, 257, 513, 0, 64, 97, 700, 2, 129, 383, 1000]
    offs = seq_offsets_from_lengths(lens)
    N = int(offs[-1])
    q, k, v = randn([(N, h_q, d), (N, h_kv, d), (N, h_kv, d)], 900 + d + h_q, "bf16")
    o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=1, causal=True,
                        seq_offsets=torch.from_numpy(offs).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.attention_ref(q, k, v, causal=True, seq_offsets=offs)
    check(host(o), ref, "bf16", f"jagged ragged d={d} heads {heads}")
