"""One quantized decode step (float64), uniform and dual-axis modes.

STEPQuant Sec. 3 (Eq. 4) and appendix A: the stored state S_hat_{t-1} is
reconstructed, the gated delta update runs in floating point,

    X_t = A_t S_hat_{t-1} + B_t,

the head output is read from X_t *before* quantization (appendix A: the
output is read from X_t before Q_t(X_t) is stored),

    y_t = X_t^T q_t,

and Q_t(X_t) is what gets stored.  Sec. 4.4 fuses reconstruction, the delta
update and the readout; appendix F.1 runs the fit and packed writeback after
the readout.
"""
from __future__ import annotations

import numpy as np

from . import quantizers as Q
from .recurrence import delta_update, readout, retained


def uniform_step(state: dict, inp: dict, bits: int, dvec: np.ndarray) -> dict:
    """state: z [..., d_k, d_v], s [..., d_k]; inp: q, k, v, beta (float64).
    Returns y, X and the new state (with the unrounded decision values)."""
    S_hat = Q.dequant_uniform(state["z"], state["s"])
    X = delta_update(retained(S_hat, dvec), inp["k"], inp["v"], inp["beta"])
    y = readout(X, inp["q"])
    new = Q.quantize_uniform(X, bits)
    return {"y": y, "X": X, "S_hat": S_hat, "new": new}


def step_step(state: dict, inp: dict, w: np.ndarray, row_bits: np.ndarray,
              dvec: np.ndarray) -> dict:
    """state: z, r, c, h (pivot values); w [..., d_k]; row_bits [..., d_k]."""
    S_hat = Q.dequant_step(state["z"], state["r"], state["c"], row_bits, state["h"])
    X = delta_update(retained(S_hat, dvec), inp["k"], inp["v"], inp["beta"])
    y = readout(X, inp["q"])
    new = Q.quantize_step(X, w, row_bits)
    return {"y": y, "X": X, "S_hat": S_hat, "new": new}
