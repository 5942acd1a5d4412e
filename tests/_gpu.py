"""Helpers of the GPU parity tests: tolerance checks and host copies."""
import numpy as np
import torch

# Tolerances of the parity bar: fp32 max |err| <= 1e-5; bf16 inputs with fp32
# accumulation: max |err| <= 1.5e-2 and Frobenius-relative err <= 2e-2.
# Where the output itself is stored in bf16, the bar applies to the value the
# kernel computed before it rounded it to bf16: an output g stands for every
# fp32 value within half a bf16 ulp of g, so the error checked is
# |g - ref| - half_ulp(g) (the distance from ref to g's rounding interval,
# at most 2^-9 |g| short of it at a power of two).  The raw max |g - ref| is
# reported beside it.
F32_ATOL = 1e-5
BF16_ATOL = 1.5e-2
BF16_FROB = 2e-2


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def half_ulp_bf16(g) -> np.ndarray:
    """Half the spacing of bf16 values at each (bf16-representable) g: for
    2^e <= |g| < 2^(e+1) the spacing is 2^(e-7) (8 significant bits); 0 at 0."""
    g = np.asarray(g, dtype=np.float64)
    _, ex = np.frexp(g)                 # |g| = f 2^ex, 0.5 <= f < 1, so e = ex - 1
    return np.where(g == 0.0, 0.0, np.ldexp(1.0, ex - 9))


def errors(got, ref, out_bf16: bool):
    """(raw max |err|, max |err| beyond the output rounding, sum err^2, sum ref^2)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0, 0.0, 0.0, 0.0
    err = np.abs(got - ref)
    excess = err - half_ulp_bf16(got) if out_bf16 else err
    return float(err.max()), float(excess.max()), float(np.square(got - ref).sum()), float(np.square(ref).sum())


def check(got, ref, dtype: str, tag: str = "", out_bf16: bool = None):
    """out_bf16: whether `got` was stored in bf16 (default: dtype == "bf16")."""
    if out_bf16 is None:
        out_bf16 = dtype == "bf16"
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (tag, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
    mx, excess, se, sr = errors(got, ref, out_bf16)
    if dtype == "f32":
        assert mx <= F32_ATOL, f"{tag}: max abs err {mx:.3e} > {F32_ATOL}"
    else:
        frob = float(np.sqrt(se) / max(np.sqrt(sr), 1e-30))
        assert excess <= BF16_ATOL and frob <= BF16_FROB, \
            f"{tag}: max abs {mx:.3e} (beyond output rounding {excess:.3e}), frob rel {frob:.3e}"
    return mx
