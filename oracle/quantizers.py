"""State quantizers of the oracle (float64).

Three encodings, each written as the steps the pages give:

1. Uniform symmetric rowwise quantizer (STEPQuant baseline, Sec. 5.1 and
   appendix B.5): one FP16 scale per key row, s_i = absmax_i / q_b clamped to
   [2^-14, 65504], codes = nearest integer of X / s in [-q_b, q_b].

2. Key-row-aware dual-axis quantizer (STEPQuant Sec. 4.3 and appendix C; the
   Korean summary of STEPQuant gives the explicit formulas):
   X_hat_ij = r_i c_j z_ij / q_{b_i}, with
     m_i  = mean_j |X_ij|                    (row magnitude),
     r_i  = fp16(m_i^{1/2} w_i^{-1/2})        (row scale with impact factor w_i),
     c0_j = fp16(max_i |X_ij| / r_i)          (initial column scale),
     z_ij = clamp(rne(q_b X_ij / (r_i c0_j)), +-q_b),
     c_j  = fp16(N_j / D_j) minimising sum_ij w_i^2 (X_ij - r_i c_j z_ij/q_b)^2
            with the codes held fixed ("fixed-code column-scale update"):
            N_j = sum_i w_i^2 r_i zt_ij X_ij,  D_j = sum_i w_i^2 r_i^2 zt_ij^2,
            zt = z / q_b; c_j = c0_j when D_j = 0.
   Units kept as FP16 pivots (a whole GDN head, or KDA key rows; STEPQuant
   Sec. 4 "sparse FP16 pivots") store fp16(X) and take no part in r, c.
   The codebook is normalised by q_b ("fixed by precision and consumes no
   metadata", appendix D), so rows of different widths share one c.

3. Smoothed per-column INT8 quantizer of the window boundary (LeapQuant
   notes Sec. 2.5, Eq. 7 and appendix B.3): c_a = max(sqrt(mean_j |S_aj|),
   c_floor) per key row, T = C^{-1} S, B_j = max_a |T_aj|,
   Z = clamp(rne(127 T / B), +-127); dequant = C (Z/127) B.  C and B are
   stored as float32.

Each quantizer is split into its stages so that the parity comparator in the
tests can evaluate them one decision at a time.
"""
from __future__ import annotations

import numpy as np

from .numerics import PIVOT_BITS, fp16, fp16_scale, fp32, qmax, rne

WINDOW_CODE_MAX = 127.0
WINDOW_C_FLOOR = 1e-6


# ----------------------------------------------------------------- uniform
def uniform_scale(X: np.ndarray, bits: int):
    """(unrounded, stored) row scales: absmax / q_b, then FP16 with clamp."""
    pre = np.max(np.abs(X), axis=-1) / qmax(bits)
    return pre, fp16_scale(pre)


def uniform_codes(X: np.ndarray, s: np.ndarray, bits: int):
    """(unrounded, stored) codes: nearest integer of X / s_i, clamped."""
    q = qmax(bits)
    pre = X / s[..., :, None]
    return pre, np.clip(rne(pre), -q, q)


def quantize_uniform(X: np.ndarray, bits: int) -> dict:
    pre_s, s = uniform_scale(X, bits)
    pre_z, z = uniform_codes(X, s, bits)
    return {"z": z, "s": s, "pre_s": pre_s, "pre_z": pre_z}


def dequant_uniform(z: np.ndarray, s: np.ndarray) -> np.ndarray:
    return s[..., :, None] * z


# ------------------------------------------------------------ dual-axis STEP
def _rows(row_bits: np.ndarray):
    row_bits = np.asarray(row_bits)
    piv = row_bits == PIVOT_BITS
    qb = np.where(piv, 1.0, qmax(np.where(piv, 2, row_bits)))
    return piv, qb


def step_row_scales(X: np.ndarray, w: np.ndarray, row_bits: np.ndarray):
    """m_i = mean_j |X_ij|, r_i = fp16(sqrt(m_i / w_i)); pivot rows get 0."""
    piv, _ = _rows(row_bits)
    m = np.mean(np.abs(X), axis=-1)
    pre = np.sqrt(m / w)
    r = np.where(piv, 0.0, fp16_scale(pre))
    return pre, r


def step_col_init(X: np.ndarray, r: np.ndarray, row_bits: np.ndarray):
    """c0_j = fp16(max over quantized rows of |X_ij| / r_i) (0 if no such row)."""
    piv, _ = _rows(row_bits)
    safe_r = np.where(piv, 1.0, r)
    ratio = np.where(piv[..., :, None], 0.0, np.abs(X) / safe_r[..., :, None])
    pre = np.max(ratio, axis=-2)
    return pre, fp16_scale(pre)


def step_codes(X: np.ndarray, r: np.ndarray, c0: np.ndarray, row_bits: np.ndarray):
    """z_ij = clamp(rne(q_b X_ij / (r_i c0_j)), +-q_b); 0 on pivot rows."""
    piv, qb = _rows(row_bits)
    safe_r = np.where(piv, 1.0, r)
    pre = qb[..., :, None] * X / (safe_r[..., :, None] * c0[..., None, :])
    pre = np.where(piv[..., :, None], 0.0, pre)
    z = np.clip(rne(pre), -qb[..., :, None], qb[..., :, None])
    return pre, z


def step_col_refit(X, w, r, z, c0, row_bits):
    """Weighted least-squares column scale with the codes fixed."""
    piv, qb = _rows(row_bits)
    keep = ~piv
    zt = z / qb[..., :, None]
    w2 = np.where(keep, w * w, 0.0)
    N = np.einsum("...i,...ij->...j", w2 * r, zt * X)
    D = np.einsum("...i,...ij->...j", w2 * r * r, zt * zt)
    pre = np.where(D > 0, N / np.where(D > 0, D, 1.0), 0.0)
    c = np.where(D > 0, fp16_scale(pre), c0)
    return N, D, pre, c


def step_pivots(X: np.ndarray, row_bits: np.ndarray) -> np.ndarray:
    """FP16 pivot values (round to nearest even, no clamp); 0 elsewhere."""
    piv, _ = _rows(row_bits)
    return np.where(piv[..., :, None], fp16(X), 0.0)


def quantize_step(X: np.ndarray, w: np.ndarray, row_bits: np.ndarray) -> dict:
    """Dual-axis quantization of head tiles X [..., d_k, d_v] with impact
    factors w [..., d_k] and per-row widths row_bits [..., d_k] (16 = pivot)."""
    row_bits = np.broadcast_to(np.asarray(row_bits), X.shape[:-1])
    pre_r, r = step_row_scales(X, w, row_bits)
    pre_c0, c0 = step_col_init(X, r, row_bits)
    pre_z, z = step_codes(X, r, c0, row_bits)
    N, D, pre_c, c = step_col_refit(X, w, r, z, c0, row_bits)
    h = step_pivots(X, row_bits)
    return {"z": z, "r": r, "c": c, "h": h, "c0": c0, "pre_r": pre_r,
            "pre_c0": pre_c0, "pre_z": pre_z, "pre_c": pre_c, "N": N, "D": D}


def dequant_step(z, r, c, row_bits, h) -> np.ndarray:
    """X_hat_ij = r_i c_j z_ij / q_{b_i}; pivot rows return their FP16 value."""
    row_bits = np.broadcast_to(np.asarray(row_bits), z.shape[:-1])
    piv, qb = _rows(row_bits)
    xq = r[..., :, None] * c[..., None, :] * (z / qb[..., :, None])
    return np.where(piv[..., :, None], h, xq)


# ------------------------------------------------------ smoothed INT8 window
def window_row_smoothing(S: np.ndarray, c_floor: float = WINDOW_C_FLOOR) -> np.ndarray:
    """C_a = fp32(max(sqrt(mean_j |S_aj|), c_floor))."""
    return fp32(np.maximum(np.sqrt(np.mean(np.abs(S), axis=-1)), c_floor))


def window_col_scales(S: np.ndarray, C: np.ndarray):
    """T = C^{-1} S and B_j = fp32(max_a |T_aj|)."""
    T = S / C[..., :, None]
    return T, fp32(np.max(np.abs(T), axis=-2))


def window_codes(T: np.ndarray, B: np.ndarray):
    """(unrounded, stored) codes: rne(127 T / B_j) clamped; column 0 if B_j=0."""
    safe_B = np.where(B > 0, B, 1.0)
    pre = np.where(B[..., None, :] > 0, WINDOW_CODE_MAX * T / safe_B[..., None, :], 0.0)
    return pre, np.clip(rne(pre), -WINDOW_CODE_MAX, WINDOW_CODE_MAX)


def quantize_window(S: np.ndarray, c_floor: float = WINDOW_C_FLOOR) -> dict:
    C = window_row_smoothing(S, c_floor)
    T, B = window_col_scales(S, C)
    pre_z, Z = window_codes(T, B)
    return {"Z": Z, "C": C, "B": B, "pre_z": pre_z}


def dequant_window(Z: np.ndarray, C: np.ndarray, B: np.ndarray) -> np.ndarray:
    """S_hat_0 = diag(C) (Z / 127) diag(B)."""
    return C[..., :, None] * (Z / WINDOW_CODE_MAX) * B[..., None, :]
