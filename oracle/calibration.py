"""Offline calibration (float64): statistics, impact factors, pivots, bits.

STEPQuant "Lifetime-aware Bit Allocation" (Sec. 4, Eqs. 6-8; the Korean
summary of STEPQuant restates the formulas):

* unit u = a whole head (GDN) or one key row (KDA); n_u its element count;
* mean log retention l_u = E_cal[log r_{t,u}] with r = alpha_t (GDN) or
  d_{t,i} (KDA); half-life tau_u = ln2 / (-l_u) (appendix B.5);
* lifetime weight L_u = sum_{j=0}^{H-1} exp(2 j l_u) over a horizon of H
  updates;
* minimise sum_u L_u d_u(b_u) subject to sum_u n_u b_u <= b_bar sum_u n_u,
  b_u drawn from the candidate widths; the highest-risk units are kept as
  FP16 pivots and charged as eight-bit units ("residual integer budget
  b_bar N - 8 N_piv", appendix D).

Row impact (STEPQuant Sec. 4.1 and appendix C): omega_i = E_cal[g_{t,i}^2]
with g_t = A_t^T q_t, relaxed with gamma = 0.25 and normalised to geometric
mean 1 within each head (Korean summary); w_i proportional to omega_i^{1/8}
(appendix B), i.e. w = (omega / geomean(omega))^{gamma / 2}.

Readings the pages leave open (each one is listed in the design notes):
the distortion d_u(b) is the mean, over reference-trajectory snapshots, of
the squared error of the dual-axis quantizer at uniform width b without
pivots; pivots are the ceil(rho U) units with the largest L_u d_u(b_max);
the allocation is the greedy that repeatedly takes the affordable upgrade to
the next candidate width with the largest L_u (d_u(b) - d_u(b+)) / (n_u
(b+ - b)); ties go to the lower unit index.  The d_u(b) estimator and the
greedy are "parity unpinned" beyond self-consistency and brute force.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Sequence

import numpy as np

from . import quantizers as Q
from .recurrence import dense_step, gate_vector, transported_query

PIVOT_BITS = 16


def lifetime_weight(ell, horizon: int) -> np.ndarray:
    """L_u = sum_{j=0}^{H-1} exp(2 j l_u), summed term by term."""
    ell = np.asarray(ell, dtype=np.float64)
    j = np.arange(horizon, dtype=np.float64)
    return np.exp(2.0 * j * ell[..., None]).sum(-1)


def impact_factors(omega: np.ndarray, gamma: float = 0.25, floor_rel: float = 1e-12
                   ) -> np.ndarray:
    """w [H, d_k] from omega [H, d_k]: relative floor, geometric-mean
    normalisation per head, exponent gamma / 2."""
    om = np.maximum(omega, floor_rel * omega.max(axis=-1, keepdims=True))
    gm = np.exp(np.mean(np.log(om), axis=-1, keepdims=True))
    return (om / gm) ** (gamma / 2.0)


def select_pivots(score: np.ndarray, n_piv: int) -> np.ndarray:
    """Indices of the n_piv largest scores; equal scores favour lower index."""
    order = sorted(range(len(score)), key=lambda u: (-score[u], u))
    return np.array(sorted(order[:n_piv]), dtype=np.int64)


def greedy_allocate(L: np.ndarray, dist: np.ndarray, n_u: np.ndarray,
                    cand: Sequence[int], nominal: float, pivots: np.ndarray
                    ) -> np.ndarray:
    """Per-unit widths (PIVOT_BITS for pivots) under the budget
    b_bar sum n_u - 8 sum_{pivots} n_u for the non-pivot units."""
    cand = list(cand)
    U = len(L)
    is_piv = np.zeros(U, dtype=bool)
    is_piv[pivots] = True
    level = np.zeros(U, dtype=np.int64)          # index into cand
    budget = nominal * float(n_u.sum()) - 8.0 * float(n_u[is_piv].sum())
    used = float(sum(n_u[u] * cand[0] for u in range(U) if not is_piv[u]))
    if used > budget + 1e-9:
        raise ValueError("bit budget below the smallest candidate width")
    cand_arr = np.array(cand + [cand[-1]], dtype=np.float64)
    dist_ext = np.concatenate([dist, dist[:, -1:]], axis=1)
    units = np.arange(U)
    while True:
        # every unit's next upgrade: its cost and lifetime-weighted gain per bit
        can_up = (~is_piv) & (level + 1 < len(cand))
        cost = n_u * (cand_arr[level + 1] - cand_arr[level])
        affordable = can_up & (used + cost <= budget + 1e-9)
        if not affordable.any():
            break
        gain = L * (dist_ext[units, level] - dist_ext[units, level + 1]) / np.where(
            cost > 0, cost, 1.0)
        gain = np.where(affordable, gain, -np.inf)
        best = int(np.argmax(gain))              # first maximum = lowest index
        used += float(cost[best])
        level[best] += 1
    bits = np.array([cand[lv] for lv in level], dtype=np.int64)
    bits[is_piv] = PIVOT_BITS
    return bits


def allocate(kind: str, heads: int, d_k: int, d_v: int, ell: np.ndarray,
             dist: np.ndarray, omega: np.ndarray, cand: Sequence[int], nominal: float,
             pivot_frac: float, gamma: float = 0.25, horizon: int = 2048,
             floor_rel: float = 1e-12) -> Dict[str, np.ndarray]:
    """Calibration artefacts from statistics.  ell [U], dist [U, n_cand],
    omega [heads, d_k].  Returns unit bits [U], pivots, w [heads, d_k]."""
    U = heads if kind == "gdn" else heads * d_k
    n_u = np.full(U, d_k * d_v if kind == "gdn" else d_v, dtype=np.int64)
    L = lifetime_weight(ell, horizon)
    n_piv = int(math.ceil(pivot_frac * U - 1e-12))
    pivots = select_pivots(L * dist[:, -1], n_piv)
    bits = greedy_allocate(L, dist, n_u, cand, nominal, pivots)
    w = impact_factors(omega, gamma, floor_rel)
    return {"bits": bits, "pivots": pivots, "w": w, "L": L, "n_u": n_u}


def collect_stats(kind: str, heads: int, d_k: int, d_v: int, steps: int,
                  inputs_at: Callable[[int], dict], cand: Sequence[int],
                  snapshot_start: int = 128, snapshot_every: int = 16,
                  gamma: float = 0.25, floor_rel: float = 1e-12) -> Dict[str, np.ndarray]:
    """Statistics over a calibration stream (batch axis = sequences), from
    S = 0 with the unquantised recurrence.  Pass 1: l_u and omega; pass 2:
    d_u(b) on snapshots after steps snapshot_start + k * snapshot_every,
    using the impact factors of pass 1."""
    log_sum = None
    om_sum = np.zeros((heads, d_k))
    count = 0
    for t in range(steps):
        inp = {k: np.asarray(v, dtype=np.float64) for k, v in inputs_at(t).items()}
        dvec = gate_vector(inp["gate"], kind, d_k)
        lg = np.log(inp["gate"])                       # [n, H] or [n, H, d_k]
        log_sum = lg.sum(0) if log_sum is None else log_sum + lg.sum(0)
        g = transported_query(inp["q"], inp["k"], inp["beta"], dvec)
        om_sum += (g * g).sum(0)
        count += g.shape[0]
    ell = (log_sum / count).reshape(-1)
    omega = om_sum / count
    w = impact_factors(omega, gamma, floor_rel)

    U = heads if kind == "gdn" else heads * d_k
    dist = np.zeros((U, len(cand)))
    n_snap = 0
    S = None
    for t in range(steps):
        inp = {k: np.asarray(v, dtype=np.float64) for k, v in inputs_at(t).items()}
        dvec = gate_vector(inp["gate"], kind, d_k)
        if S is None:
            S = np.zeros(inp["q"].shape[:2] + (d_k, d_v))
        S, _ = dense_step(S, inp["q"], inp["k"], inp["v"], inp["beta"], dvec)
        done = t + 1
        if done > snapshot_start and (done - snapshot_start) % snapshot_every == 0:
            n_snap += 1
            for ci, b in enumerate(cand):
                enc = Q.quantize_step(S, w[None], np.full(S.shape[:-1], b))
                E = Q.dequant_step(enc["z"], enc["r"], enc["c"], np.full(S.shape[:-1], b),
                                   enc["h"]) - S
                e2 = (E * E).sum(-1)                     # [n, H, d_k]
                per = e2.sum(-1) if kind == "gdn" else e2
                dist[:, ci] += per.mean(0).reshape(-1)
    dist /= max(n_snap, 1)
    return {"ell": ell, "omega": omega, "dist": dist, "w": w, "snapshots": n_snap}
