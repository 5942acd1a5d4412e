"""The C ABI from plain C: flash_attention_kv_amd/examples/abi_consumer (built
with the library, no Python inside) runs a causal GQA ring prefill and a
split-KV decode step through include/fakv.h and dumps inputs and outputs.
The Python binding, given the same inputs, must produce the same bits, and
both must match the fp64 oracle."""
import os
import subprocess

import numpy as np
import pytest
import torch

import flash_attention_kv_amd as F
import oracle
from tests._gpu import check, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "flash_attention_kv_amd", "examples", "abi_consumer")


def _bf16(raw: bytes, off: int, shape):
    n = int(np.prod(shape))
    a = np.frombuffer(raw, dtype=np.int16, count=n, offset=off).copy()
    return torch.from_numpy(a).view(torch.bfloat16).reshape(shape), off + 2 * n


def test_plain_c_caller_matches_binding_and_oracle(tmp_path):
    if not os.path.exists(EXE):
        pytest.skip("abi_consumer is not built (__graft_entry__.build() links it with the library)")
    path = tmp_path / "abi.bin"
    r = subprocess.run([EXE, str(path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    raw = path.read_bytes()
    T, h_q, h_kv, d, C, B, S, n_chunks = (int(x) for x in np.frombuffer(raw, dtype=np.int32, count=8))
    off = 32
    q, off = _bf16(raw, off, (T, h_q, d))
    k, off = _bf16(raw, off, (T, h_kv, d))
    v, off = _bf16(raw, off, (T, h_kv, d))
    dq, off = _bf16(raw, off, (B, h_q, d))
    dk, off = _bf16(raw, off, (B, S, h_kv, d))
    dv, off = _bf16(raw, off, (B, S, h_kv, d))
    o_c, off = _bf16(raw, off, (T, h_q, d))
    do_c, off = _bf16(raw, off, (B, h_q, d))
    assert off == len(raw)

    o_py = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=C, causal=True)
    do_py = F.splitkv_decode(dq.to(DEV), dk.to(DEV), dv.to(DEV), n_chunks=n_chunks)
    torch.cuda.synchronize()
    assert torch.equal(o_py.cpu(), o_c), "prefill: C and Python callers differ"
    assert torch.equal(do_py.cpu(), do_c), "decode: C and Python callers differ"
    check(host(o_c), oracle.ring_ref(q, k, v, C, causal=True), "bf16", "C caller, prefill")
    check(host(do_c), oracle.splitkv_decode_ref(dq, dk, dv, n_chunks), "bf16", "C caller, decode")
