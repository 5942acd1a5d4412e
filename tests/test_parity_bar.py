"""The parity bar's bf16 rounding allowance (host logic, no GPU): every fp32
value lies within half_ulp_bf16(g) of the bf16 value g it rounds to, and the
allowance is exactly half the spacing of bf16 values at g."""
import numpy as np
import torch

from tests._gpu import errors, half_ulp_bf16


def test_half_ulp_covers_rounding():
    x = torch.randn(200000, generator=torch.Generator().manual_seed(0)) * torch.logspace(-3, 3, 200000)
    g = x.to(torch.bfloat16).to(torch.float64).numpy()
    xd = x.to(torch.float64).numpy()
    assert np.all(np.abs(xd - g) <= half_ulp_bf16(g))


def test_half_ulp_values():
    g = np.array([1.0, 1.5, -1.0, 2.0, 3.0, 0.75, 0.0, 4.0, -7.5])
    assert list(half_ulp_bf16(g)) == [2 ** -8, 2 ** -8, 2 ** -8, 2 ** -7, 2 ** -7, 2 ** -9, 0.0, 2 ** -6, 2 ** -6]
    # the next bf16 value above g is g + 2 half ulps
    for v in (1.0, 3.0, 0.75, 4.0):
        t = torch.tensor([v], dtype=torch.bfloat16)
        nxt = torch.nextafter(t.float(), torch.tensor([10.0])).to(torch.bfloat16)   # rounds to g
        assert float(nxt) == v
        up = (t.view(torch.int16) + 1).view(torch.bfloat16)
        assert float(up) - v == 2 * half_ulp_bf16(np.array([v]))[0]


def test_errors_beyond_rounding():
    got = np.array([1.0, 2.0])
    ref = np.array([1.0 + 2 ** -8, 2.0 - 0.01])
    mx, excess, se, sr = errors(got, ref, True)
    assert abs(mx - 0.01) < 1e-15 and abs(excess - (0.01 - 2 ** -7)) < 1e-15
    assert errors(got, ref, False)[1] == mx
