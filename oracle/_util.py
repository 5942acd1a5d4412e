"""Conversion of inputs to float64 NumPy arrays (test infrastructure only)."""
import numpy as np


def f64(x) -> np.ndarray:
    """Exact upcast to float64.  torch tensors (fp32 or bf16) are widened on the
    host first; every bf16 and fp32 value is representable in float64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def segments(T_q: int, S_kv: int, n_seqs: int, seq_offsets):
    """(q_begin, q_end, k_begin, k_end) of every sequence in a packed batch.

    Dense batch: ``n_seqs`` sequences of T_q / n_seqs queries and S_kv / n_seqs
    keys.  Jagged batch: query and key ranges both come from the prefix offsets
    (self-attention)."""
    if seq_offsets is not None:
        o = np.asarray(seq_offsets, dtype=np.int64)
        return [(int(o[b]), int(o[b + 1]), int(o[b]), int(o[b + 1])) for b in range(len(o) - 1)]
    if T_q % n_seqs or S_kv % n_seqs:
        raise ValueError("dense batch: token counts must divide by n_seqs")
    tq, sk = T_q // n_seqs, S_kv // n_seqs
    return [(b * tq, (b + 1) * tq, b * sk, (b + 1) * sk) for b in range(n_seqs)]
