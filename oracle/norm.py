"""Gated RMSNorm on the recurrence output, fp64.

Source: model card "Agnes-3.0-Flash Preview", 架构 table, delta-rule row (a
gated RMS-norm follows the recurrence).  The pages give no formula.

Reading: per head row of ``dim`` values, normalise first, then apply the
per-channel weight and the SiLU of the gate:
    y = o / sqrt(mean(o^2) + eps) * w * z / (1 + exp(-z)),
with one weight vector [dim] shared by all heads.
"""
import numpy as np

from .inputs import as_f64


def gated_rmsnorm(o, z, w, eps=1e-6):
    """o, z: [..., dim]; w: [dim]. Returns y [..., dim] in fp64."""
    o = as_f64(o)
    z = as_f64(z)
    w = as_f64(w)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * r * w * (z / (1.0 + np.exp(-z)))
