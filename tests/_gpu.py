"""Helpers of the GPU parity tests: tolerance checks and host copies."""
import numpy as np
import torch

# Tolerances of the parity bar: fp32 max |err| <= 1e-5; bf16 inputs with fp32
# accumulation: max |err| <= 1.5e-2 and Frobenius-relative err <= 2e-2.
# A bf16 *output* cannot represent the exact result closer than half an ulp
# (up to 2^-8 |x|), which alone exceeds 1.5e-2 once |x| >= 4; that
# representation error is allowed on top of the absolute bound.
F32_ATOL = 1e-5
BF16_ATOL = 1.5e-2
BF16_FROB = 2e-2
BF16_HALF_ULP = 2.0 ** -8


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def check(got, ref, dtype: str, tag: str = "", out_bf16: bool = None):
    """out_bf16: whether `got` was stored in bf16 (default: dtype == "bf16")."""
    if out_bf16 is None:
        out_bf16 = dtype == "bf16"
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (tag, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    if dtype == "f32":
        assert mx <= F32_ATOL, f"{tag}: max abs err {mx:.3e} > {F32_ATOL}"
    else:
        frob = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
        excess = float((err - (BF16_HALF_ULP * np.abs(ref) if out_bf16 else 0.0)).max()) if err.size else 0.0
        assert excess <= BF16_ATOL and frob <= BF16_FROB, \
            f"{tag}: max abs {mx:.3e} (beyond output rounding {excess:.3e}), frob rel {frob:.3e}"
    return mx
