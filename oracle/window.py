"""Per-window decode variant (float64), GDN scalar gate.

LeapQuant notes Sec. 2.3 (Eq. 4, appendix Eq. 9): a window keeps a fixed
boundary state S_hat_0 and the records (alpha_j, k~_j, u_j) of its tokens, with
the cumulative decay Gamma_{a:b} = alpha_b ... alpha_a (identity when a > b):

    S_l = Gamma_{1:l} S_hat_0 + sum_{j=1..l} Gamma_{j+1:l} k~_j u_j^T,
    S_l^T x = S_hat_0^T Gamma_{1:l} x + sum_j u_j (k~_j . Gamma_{j+1:l} x).

For GDN the write vector is k~ = beta k and the read vector is alpha k (the
notes' Table 4), so the corrected value of token i is
u_i = v_i - S_{i-1}^T (alpha_i k_i); the token's output is o_i = S_i^T q_i
(Sec. 2.1 Eq. 1).  The per-token loop of Sec. 2.6 computes u_i, appends the
record, emits o_i and rebuilds the dense state when the window holds p
records; the rebuilt state is re-encoded with the smoothed INT8 quantizer
(Sec. 2.5, appendix B.3) and the window restarts.  Compensator tokens
(Sec. 2.4) are not part of this variant.

Storage precision follows the layout: records and the boundary scales are
float32, so u_i and beta_i k_i are rounded to float32 when recorded and every
later use reads the rounded value.
"""
from __future__ import annotations

from typing import List

import numpy as np

from . import quantizers as Q
from .numerics import fp32


def new_window_state(S_init: np.ndarray, p: int) -> dict:
    """Boundary encoding of an initial state, empty window."""
    d_k, d_v = S_init.shape[-2:]
    enc = Q.quantize_window(S_init)
    return {"Z": enc["Z"], "C": enc["C"], "B": enc["B"], "ell": 0,
            "alpha": np.zeros(p), "kt": np.zeros((p, d_k)), "u": np.zeros((p, d_v)),
            "pre_z": enc["pre_z"]}


def _gamma(alphas: np.ndarray, a: int, b: int) -> float:
    """Gamma_{a:b} = prod_{m=a..b} alpha_m over 1-based record indices."""
    if a > b:
        return 1.0
    return float(np.prod(alphas[a - 1:b]))


def window_readout(S0: np.ndarray, alphas, kt, u, n: int, x: np.ndarray) -> np.ndarray:
    """S_n^T x from the boundary state and the first n records."""
    out = S0.T @ (_gamma(alphas, 1, n) * x)
    for j in range(1, n + 1):
        out = out + u[j - 1] * float(kt[j - 1] @ (_gamma(alphas, j + 1, n) * x))
    return out


def window_dense(S0: np.ndarray, alphas, kt, u, n: int) -> np.ndarray:
    """S_n = Gamma_{1:n} S_hat_0 + sum_j Gamma_{j+1:n} k~_j u_j^T."""
    S = _gamma(alphas, 1, n) * S0
    for j in range(1, n + 1):
        S = S + _gamma(alphas, j + 1, n) * np.outer(kt[j - 1], u[j - 1])
    return S


def window_step(st: dict, q, k, v, beta: float, alpha: float, p: int) -> dict:
    """One token on one (slot, head) window state.  Returns the output o_i,
    the record written and the new state (a fresh dict)."""
    ell = int(st["ell"])
    i = ell + 1
    S0 = Q.dequant_window(st["Z"], st["C"], st["B"])
    alphas = st["alpha"].copy()
    kt = st["kt"].copy()
    u = st["u"].copy()
    alphas[i - 1] = alpha
    prev = window_readout(S0, alphas, kt, u, i - 1, alpha * k)
    u_i = fp32(v - prev)
    kt[i - 1] = fp32(beta * k)
    u[i - 1] = u_i
    o = window_readout(S0, alphas, kt, u, i, q)
    new = dict(st, alpha=alphas, kt=kt, u=u, ell=i)
    flushed = None
    if i == p:
        flushed = Q.quantize_window(window_dense(S0, alphas, kt, u, p))
        new.update(Z=flushed["Z"], C=flushed["C"], B=flushed["B"], ell=0,
                   pre_z=flushed["pre_z"])
    return {"o": o, "u": u_i, "kt": kt[i - 1], "state": new, "flushed": flushed,
            "S0": S0}


def window_flush(st: dict, p: int) -> dict:
    """Rebuild and re-encode a window holding 0 < l < p records (no-op at l = 0)."""
    ell = int(st["ell"])
    if ell == 0:
        return dict(st)
    S0 = Q.dequant_window(st["Z"], st["C"], st["B"])
    enc = Q.quantize_window(window_dense(S0, st["alpha"], st["kt"], st["u"], ell))
    return dict(st, Z=enc["Z"], C=enc["C"], B=enc["B"], ell=0, pre_z=enc["pre_z"])


def window_state_dense(st: dict) -> np.ndarray:
    S0 = Q.dequant_window(st["Z"], st["C"], st["B"])
    return window_dense(S0, st["alpha"], st["kt"], st["u"], int(st["ell"]))


def window_run(S_init: np.ndarray, inputs: List[dict], p: int) -> List[dict]:
    st = new_window_state(S_init, p)
    outs = []
    for inp in inputs:
        r = window_step(st, inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], p)
        outs.append(r)
        st = r["state"]
    return outs
