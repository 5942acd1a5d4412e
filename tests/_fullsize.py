"""Full-output parity at the benchmark sizes: the fp64 oracle evaluated on
every (sequence, query head) block of a workload, the blocks spread over a
thread pool (NumPy releases the GIL in its ufuncs and BLAS calls; BLAS itself
is held to one thread per worker so the pool does not oversubscribe the
cores), each block compared with the GPU output as soon as it is computed.
Each block is one call of oracle.attention_ref on that sequence's rows of one
query head against the KV head oracle.kv_head_of assigns it -- the
definition, unchanged, evaluated independently per block."""
from __future__ import annotations

import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from oracle._util import segments
from tests._gpu import BF16_ATOL, BF16_FROB, F32_ATOL, errors


def workers() -> int:
    # at most 16: the CPU share of one GPU on the test machines
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _pool_map(fn, jobs):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), ThreadPoolExecutor(workers()) as ex:
        return list(ex.map(fn, jobs))


def prefill_blocks(q, k, v, *, causal, n_seqs=1, seq_offsets=None, window=None):
    """(q0, q1, k0, k1, h, kv_head) for every non-empty (sequence, query head)."""
    T, h_q, _ = q.shape
    S, h_kv, _ = k.shape
    out = []
    for (q0, q1, k0, k1) in segments(T, S, n_seqs, seq_offsets):
        if q1 > q0:
            out += [(q0, q1, k0, k1, h, oracle.kv_head_of(h, h_q, h_kv)) for h in range(h_q)]
    return out


def compare_prefill(got: torch.Tensor, q, k, v, *, causal, n_seqs=1, seq_offsets=None, window=None,
                    out_bf16=True, keep_ref=False):
    """Compare the whole GPU output got (tokens, h_q, d), on the host, with the
    oracle.  Returns a stats dict (and the fp64 reference when keep_ref)."""
    t0 = time.perf_counter()
    ref_all = np.empty(tuple(got.shape), dtype=np.float64) if keep_ref else None

    def one(b):
        q0, q1, k0, k1, h, kvh = b
        ref = oracle.attention_ref(q[q0:q1, h:h + 1], k[k0:k1, kvh:kvh + 1], v[k0:k1, kvh:kvh + 1],
                                   causal=causal, window=window)[:, 0]
        g = got[q0:q1, h].to(torch.float64).numpy()
        if ref_all is not None:
            ref_all[q0:q1, h] = ref
        return errors(g, ref, out_bf16), bool(np.isfinite(g).all())

    res = _pool_map(one, prefill_blocks(q, k, v, causal=causal, n_seqs=n_seqs, seq_offsets=seq_offsets,
                                        window=window))
    st = summarize(res, time.perf_counter() - t0)
    return (st, ref_all) if keep_ref else st


def compare_decode(got: torch.Tensor, q, k, v):
    """Decode: got (B, h_q, d); q (B, h_q, d); K/V (B, S, h_kv, d).  One block
    per (sequence, query head): one query row against the whole cache."""
    t0 = time.perf_counter()
    B, h_q, _ = q.shape
    h_kv = k.shape[2]

    def one(b_h):
        b, h = b_h
        kvh = oracle.kv_head_of(h, h_q, h_kv)
        ref = oracle.attention_ref(q[b:b + 1, h:h + 1], k[b, :, kvh:kvh + 1], v[b, :, kvh:kvh + 1])[0, 0]
        g = got[b, h].to(torch.float64).numpy()
        return errors(g, ref, True), bool(np.isfinite(g).all())

    return summarize(_pool_map(one, [(b, h) for b in range(B) for h in range(h_q)]), time.perf_counter() - t0)


def compare_to_ref(got: torch.Tensor, ref: np.ndarray, out_bf16: bool):
    g = got.to(torch.float64).numpy()
    return summarize([(errors(g, ref, out_bf16), bool(np.isfinite(g).all()))], 0.0)


def summarize(res, seconds):
    mx = max(r[0][0] for r in res)
    excess = max(r[0][1] for r in res)
    se = sum(r[0][2] for r in res)
    sr = sum(r[0][3] for r in res)
    return {"max_abs": mx, "max_abs_beyond_rounding": excess, "frob_rel": float(np.sqrt(se / max(sr, 1e-300))),
            "finite": all(r[1] for r in res), "blocks": len(res), "oracle_s": round(seconds, 1),
            "workers": workers()}


def assert_bar(st, dtype: str, tag: str):
    print(f"{tag}: max abs {st['max_abs']:.3e} (beyond output rounding {st['max_abs_beyond_rounding']:.3e}), "
          f"frob rel {st['frob_rel']:.3e}, {st['blocks']} blocks, oracle {st['oracle_s']} s on "
          f"{st['workers']} threads", flush=True)
    assert st["finite"], f"{tag}: non-finite output"
    if dtype == "f32":
        assert st["max_abs"] <= F32_ATOL, f"{tag}: {st}"
    else:
        assert st["max_abs_beyond_rounding"] <= BF16_ATOL and st["frob_rel"] <= BF16_FROB, f"{tag}: {st}"
