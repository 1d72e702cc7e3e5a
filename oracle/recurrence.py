"""Gated delta rule in float64 (the unquantised recurrence).

STEPQuant, Sec. 3 (Eq. 1): for one head, with retention gate D_t (GDN:
alpha_t I; KDA: diag(d_t)) and write strength beta_t in [0, 1],

    S_t = D_t S_{t-1} + beta_t k_t (v_t - (D_t S_{t-1})^T k_t)^T,
    y_t = S_t^T q_t.

The key retrieves k_t^T D_t S_{t-1} from the *retained* state.  The same
update in affine-transport form (STEPQuant Eq. 2; the Korean summary of
STEPQuant states A_t explicitly) is S_t = A_t S_{t-1} + B_t with
A_t = (I - beta_t k_t k_t^T) D_t and B_t = beta_t k_t v_t^T.

Every function accepts leading batch axes: states are [..., d_k, d_v], key
and query [..., d_k], value [..., d_v], beta [...], and the retention gate is
given as a per-key-row vector ``dvec`` [..., d_k] (a GDN gate alpha is the
vector alpha * 1).
"""
from __future__ import annotations

import numpy as np


def gate_vector(gate, kind: str, d_k: int) -> np.ndarray:
    """Per-key-row retention vector: GDN broadcasts its scalar gate."""
    g = np.asarray(gate, dtype=np.float64)
    if kind == "gdn":
        return np.repeat(g[..., None], d_k, axis=-1)
    return g


def retained(S: np.ndarray, dvec: np.ndarray) -> np.ndarray:
    """D_t S_{t-1}: row i of the state scaled by the retention of key row i."""
    return dvec[..., :, None] * S


def delta_update(Sd: np.ndarray, k: np.ndarray, v: np.ndarray, beta) -> np.ndarray:
    """X = S' + beta k (v - S'^T k)^T applied to a retained state S'."""
    beta = np.asarray(beta, dtype=np.float64)
    delta = np.einsum("...ij,...i->...j", Sd, k)
    return Sd + beta[..., None, None] * k[..., :, None] * (v - delta)[..., None, :]


def readout(X: np.ndarray, q: np.ndarray) -> np.ndarray:
    """y = X^T q."""
    return np.einsum("...ij,...i->...j", X, q)


def dense_step(S, q, k, v, beta, dvec):
    """One unquantised step: returns (S_t, y_t)."""
    X = delta_update(retained(S, dvec), k, v, beta)
    return X, readout(X, q)


def transition(k: np.ndarray, beta, dvec: np.ndarray) -> np.ndarray:
    """A_t = (I - beta_t k_t k_t^T) D_t  [..., d_k, d_k]."""
    beta = np.asarray(beta, dtype=np.float64)
    d_k = k.shape[-1]
    P = np.eye(d_k) - beta[..., None, None] * k[..., :, None] * k[..., None, :]
    return P * dvec[..., None, :]


def write_term(k: np.ndarray, v: np.ndarray, beta) -> np.ndarray:
    """B_t = beta_t k_t v_t^T."""
    beta = np.asarray(beta, dtype=np.float64)
    return beta[..., None, None] * k[..., :, None] * v[..., None, :]


def transported_query(q: np.ndarray, k: np.ndarray, beta, dvec: np.ndarray) -> np.ndarray:
    """g_t = A_t^T q_t = D_t (q_t - beta_t k_t (k_t . q_t)) (STEPQuant Sec. 4.1;
    D_t is diagonal so A_t^T = D_t (I - beta k k^T))."""
    beta = np.asarray(beta, dtype=np.float64)
    kq = np.einsum("...i,...i->...", k, q)
    return dvec * (q - beta[..., None] * k * kq[..., None])
