"""RMSNorm between MoE layers (test infrastructure only).

The pages give no normalisation; the 40-layer stack workload puts a
pre-norm RMSNorm with eps 1e-6 and unit scale between layers:

    xn = bf16( x / sqrt(mean(x^2) + eps) * gamma )

Pinned by tests/test_oracle_pins.py against torch.nn.functional.rms_norm in
float64 and by the identity that a normalised row has root-mean-square 1.
"""
import numpy as np

from . import bf16


def rmsnorm(x_bits, eps: float = 1e-6, gamma=None):
    x = bf16.to_f64(x_bits)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)[None, :]
    return bf16.from_f64(y)
