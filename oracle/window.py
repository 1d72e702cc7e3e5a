"""Per-window decode variant (float64), GDN scalar gate.

LeapQuant notes Sec. 2.3 (Eq. 4, appendix Eq. 9): a window keeps a fixed
boundary state S_hat_0 and the records (alpha_j, k~_j, u_j) of its tokens, with
the cumulative decay Gamma_{a:b} = alpha_b ... alpha_a (identity when a > b):

    S_l = Gamma_{1:l} S_hat_0 + sum_{j=1..l} Gamma_{j+1:l} k~_j u_j^T,
    S_l^T x = S_hat_0^T Gamma_{1:l} x + sum_j u_j (k~_j . Gamma_{j+1:l} x).

For GDN the write vector is k~ = beta k and the read vector is alpha k (the
notes' Table 4), so the corrected value of token i is
u_i = v_i - S_{i-1}^T (alpha_i k_i) and the token's output is o_i = S_i^T q_i
(Sec. 2.1 Eq. 1).  The oracle forms the window's dense state from the
expansion and reads u_i and o_i from it; once p records are held the dense
state is re-encoded with the smoothed INT8 quantizer (Sec. 2.5, appendix
B.3) as the next boundary.  The expansion's read form (Eq. 10,
window_readout) is what the kernel evaluates; a pin checks it against the
dense form.

Compensator tokens (Sec. 2.4, Eqs. 5-7 and 10), rank r > 0: the boundary is
S_hat_0 = C dequant(R_hat) + K~c U~c^T with r FP16 factor pairs (k~c_h, u~c_h).
They enter a window with identity decay and then decay with the boundary, so

    S_l = Gamma_{1:l} (C dequant(R_hat) + K~c U~c^T) + sum_j Gamma_{j+1:l} k~_j u_j^T,
    S_l^T x = dequant(R_hat)^T C Gamma_{1:l} x + U~c (K~c^T Gamma_{1:l} x)
              + sum_j u_j (k~_j . Gamma_{j+1:l} x).

At a rebuild the old factors are part of S_p; a new rank-r fit by power
iteration replaces them and only the residual R = S_p - K~c U~c^T is smoothed
and quantized.  The pages fix the objective (the Frobenius-optimal rank-r
outer-product sum), that it is reached by power iteration rather than an
exact decomposition, the rank and the FP16 storage; the rest is this
oracle's reading (``lowrank_fit``): the r pairs are fitted one after another,
each from the residual left by the ones before, with a fixed number of
iterations started from that pair's previous value u~c_h (a freshly packed
state starts from the all-ones vector), and each pair is rounded to FP16
before it is taken out of the residual, so the stored factors are exactly
what was removed.

Storage precision follows the layout: records and the boundary scales are
float32, so u_i and beta_i k_i are rounded to float32 when recorded and every
later use reads the rounded value; compensator factors are binary16.
"""
from __future__ import annotations

from typing import List

import numpy as np

from . import quantizers as Q
from .numerics import FP16_MAX, fp16, fp32


def fp16_value(x) -> np.ndarray:
    """Binary16 round-to-nearest-even of a signed value, saturating at the
    largest finite binary16 magnitude (compensator factors)."""
    return fp16(np.clip(np.asarray(x, dtype=np.float64), -FP16_MAX, FP16_MAX))


def lowrank_fit(M: np.ndarray, rank: int, iters: int, init=None, exact: bool = False,
                adopt=None):
    """Rank-`rank` outer-product fit of M by power iteration (Sec. 2.4, Eqs. 5-6).

    Pair h is fitted to the residual left by pairs 0..h-1: starting from
    b = init[h] (the all-ones vector when init is None or init[h] is zero),
    `iters` times a = M b / |M b|, b = M^T a; then with sigma = |b| the pair is
    k~ = sqrt(sigma) a, u~ = b / sqrt(sigma), so k~ u~^T = a (M^T a)^T is the
    best rank-one fit along a.  A start with M b = 0 (M = 0 in particular)
    gives a zero pair.  Unless `exact`, the pair is rounded to FP16 before it
    is subtracted.  `adopt(h, k, u)` (teacher-forced parity) receives the
    unrounded pair and returns the FP16 pair that is subtracted and stored.
    Returns (K [rank, d_k], U [rank, d_v], residual)."""
    Rm = np.array(M, dtype=np.float64, copy=True)
    d_k, d_v = Rm.shape
    K = np.zeros((rank, d_k))
    U = np.zeros((rank, d_v))
    for h in range(rank):
        if init is not None and np.any(np.asarray(init[h]) != 0):
            b = np.asarray(init[h], dtype=np.float64)
        else:
            b = np.ones(d_v)
        a = None
        for _ in range(iters):
            a = Rm @ b
            na = float(np.sqrt(a @ a))
            if na == 0.0:
                a = None
                break
            a = a / na
            b = Rm.T @ a
        k = np.zeros(d_k)
        u = np.zeros(d_v)
        if a is not None:
            sigma = float(np.sqrt(b @ b))
            if sigma > 0.0:
                sq = np.sqrt(sigma)
                k, u = sq * a, b / sq
        if adopt is not None and not exact:
            k, u = adopt(h, k, u)
        elif not exact:
            k, u = fp16_value(k), fp16_value(u)
        K[h], U[h] = k, u
        Rm = Rm - np.outer(k, u)
    return K, U, Rm


def encode_boundary(S: np.ndarray, rank: int = 0, iters: int = 4, init=None,
                    exact: bool = False, adopt=None) -> dict:
    """Boundary of a dense state: compensator fit (rank > 0), then the
    smoothed INT8 encoding of the residual (identity when `exact`)."""
    d_k, d_v = S.shape
    if rank > 0:
        Kc, Uc, Rm = lowrank_fit(S, rank, iters, init, exact, adopt)
    else:
        Kc, Uc, Rm = np.zeros((0, d_k)), np.zeros((0, d_v)), np.asarray(S, dtype=np.float64)
    if exact:
        return {"S0": Rm.copy(), "Kc": Kc, "Uc": Uc}
    enc = Q.quantize_window(Rm)
    return {"Z": enc["Z"], "C": enc["C"], "B": enc["B"], "pre_z": enc["pre_z"],
            "Kc": Kc, "Uc": Uc, "R": Rm}


def boundary_residual(st: dict) -> np.ndarray:
    """C dequant(R_hat) (or the exact residual of an `exact` state)."""
    if "S0" in st:
        return st["S0"]
    return Q.dequant_window(st["Z"], st["C"], st["B"])


def new_window_state(S_init: np.ndarray, p: int, rank: int = 0, iters: int = 4,
                     exact: bool = False) -> dict:
    """Boundary encoding of an initial state, empty window (a pack starts the
    compensator fit from the all-ones vector)."""
    d_k, d_v = S_init.shape[-2:]
    enc = encode_boundary(S_init, rank, iters, None, exact)
    st = {k: v for k, v in enc.items() if k != "R"}
    st.update(ell=0, alpha=np.zeros(p), kt=np.zeros((p, d_k)), u=np.zeros((p, d_v)))
    return st


def _gamma(alphas: np.ndarray, a: int, b: int) -> float:
    """Gamma_{a:b} = prod_{m=a..b} alpha_m over 1-based record indices."""
    if a > b:
        return 1.0
    return float(np.prod(alphas[a - 1:b]))


def _comp(Kc, Uc):
    if Kc is None or len(Kc) == 0:
        return None
    return np.asarray(Kc, dtype=np.float64), np.asarray(Uc, dtype=np.float64)


def window_readout(S0: np.ndarray, alphas, kt, u, n: int, x: np.ndarray,
                   Kc=None, Uc=None) -> np.ndarray:
    """S_n^T x from the boundary residual S0, the compensators and the first
    n records (Eq. 10)."""
    gx = _gamma(alphas, 1, n) * x
    out = S0.T @ gx
    c = _comp(Kc, Uc)
    if c is not None:
        out = out + c[1].T @ (c[0] @ gx)
    for j in range(1, n + 1):
        out = out + u[j - 1] * float(kt[j - 1] @ (_gamma(alphas, j + 1, n) * x))
    return out


def window_dense(S0: np.ndarray, alphas, kt, u, n: int, Kc=None, Uc=None) -> np.ndarray:
    """S_n = Gamma_{1:n} (S0 + K~c U~c^T) + sum_j Gamma_{j+1:n} k~_j u_j^T (Eq. 7)."""
    base = np.asarray(S0, dtype=np.float64)
    c = _comp(Kc, Uc)
    if c is not None:
        base = base + c[0].T @ c[1]
    S = _gamma(alphas, 1, n) * base
    for j in range(1, n + 1):
        S = S + _gamma(alphas, j + 1, n) * np.outer(kt[j - 1], u[j - 1])
    return S


def close_window(st: dict, iters: int = 4, exact: bool = False, adopt=None):
    """Rebuild and re-encode: the window's records are folded into its dense
    state S_l (Eq. 7, window_state_dense), which becomes the next boundary
    (compensator fit from the current pairs u~c, then the smoothed INT8
    encoding of the residual, Sec. 2.4-2.5); the window restarts empty.
    Returns (new state, the encoding with its residual "R")."""
    Kc = st.get("Kc")
    rank = 0 if Kc is None else len(Kc)
    enc = encode_boundary(window_state_dense(st), rank, iters, st.get("Uc"), exact, adopt)
    new = dict(st, ell=0)
    new.update({kk: vv for kk, vv in enc.items() if kk != "R"})
    return new, enc


def window_step(st: dict, q, k, v, beta: float, alpha: float, p: int, iters: int = 4,
                exact: bool = False, adopt=None) -> dict:
    """One token on one (slot, head) window state.

    The window holds l records and its dense state is S_l (Eq. 7).  Token
    i = l + 1 follows the gated delta rule (Sec. 2.1, Eq. 1) with the GDN
    read vector alpha_i k_i and write vector beta_i k_i (Table 4):
      u_i = v_i - S_l^T (alpha_i k_i)           the corrected value,
      S_i = alpha_i S_l + (beta_i k_i) u_i^T    one more record in Eq. 4,
      o_i = S_i^T q_i                           the token's output,
    and the record (alpha_i, beta_i k_i, u_i) is kept (float32 unless
    `exact`).  When the window holds p records it is closed (close_window).
    The compensator rank is that of st["Kc"] (absent or empty: none).
    Returns the output, the record and the new state (a fresh dict)."""
    ell = int(st["ell"])
    i = ell + 1
    rnd = (lambda x: np.asarray(x, dtype=np.float64)) if exact else fp32
    u_i = rnd(v - window_state_dense(st).T @ (alpha * k))
    kt_i = rnd(beta * k)
    alphas, kt, u = st["alpha"].copy(), st["kt"].copy(), st["u"].copy()
    alphas[i - 1], kt[i - 1], u[i - 1] = alpha, kt_i, u_i
    new = dict(st, alpha=alphas, kt=kt, u=u, ell=i)
    o = window_state_dense(new).T @ q
    flushed = None
    if i == p:
        new, flushed = close_window(new, iters, exact, adopt)
    return {"o": o, "u": u_i, "kt": kt_i, "state": new, "flushed": flushed,
            "S0": boundary_residual(st)}


def window_flush(st: dict, p: int, iters: int = 4, exact: bool = False, adopt=None) -> dict:
    """Close a window holding 0 < l < p records early (no-op at l = 0)."""
    if int(st["ell"]) == 0:
        return dict(st)
    return close_window(st, iters, exact, adopt)[0]


def window_state_dense(st: dict) -> np.ndarray:
    return window_dense(boundary_residual(st), st["alpha"], st["kt"], st["u"], int(st["ell"]),
                        st.get("Kc"), st.get("Uc"))


def window_run(S_init: np.ndarray, inputs: List[dict], p: int, rank: int = 0, iters: int = 4,
               exact: bool = False) -> List[dict]:
    st = new_window_state(S_init, p, rank, iters, exact)
    outs = []
    for inp in inputs:
        r = window_step(st, inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], p, iters,
                        exact)
        outs.append(r)
        st = r["state"]
    return outs
