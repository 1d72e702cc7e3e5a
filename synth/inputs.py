"""Seeded input generators for the five decode workloads.

Every array is produced by ``numpy.random.default_rng`` (PCG64) keyed by
``[seed, stream, step]`` so that any single decode step can be regenerated on
its own, on any machine, bit for bit.  Arrays are float32 (the precision the
kernels consume); the oracle reads the same float32 values and widens them to
float64 exactly.

Distributions (one "token" of one (slot, head) tile):

* key and query: standard Gaussian vectors scaled to unit L2 norm;
* value: standard Gaussian;
* write strength beta: logistic sigmoid of a standard Gaussian;
* GDN retention: a per-head constant alpha = exp(-ln2 / half_life);
* KDA retention: per key row d = exp(-softplus(mu + N(0, 1))) where mu is
  solved so that the mean log retention gives the row's target half-life
  (half-life = ln2 / (-E[log d]), the definition used by STEPQuant's lifetime
  statistic, appendix B.5).

The KDA workload also applies fixed per-head log-normal gains to key channels
(before the L2 normalisation) and to value channels, which gives the state the
strong row and column magnitude contrasts STEPQuant reports (Sec. 4.2 and
appendix B: maximum-to-median RMS contrast 10.3x over key rows and 19.4x over
value columns).  Both spreads are 1.21, chosen once on this seeded stream:
the 128-step warm-up states then have a median contrast of 10.3x over key
rows and 19.4x over value columns (row RMS sqrt(mean_j S_ij^2), column RMS
alike, median by linear interpolation, over 4 slots x 32 heads).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

# random-number streams (second key word)
_STREAM_DECODE = 0
_STREAM_WARMUP = 1
_STREAM_CALIB = 2
_STREAM_STATIC = 3


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "gdn" (scalar gate per head) or "kda" (gate per key row)
    mode: str            # "uniform" | "step" | "window" | "dense" (fp32 state, no codec)
    batch: int           # live requests per decode step
    n_slots: int         # slots in the state pool
    heads: int
    d_k: int
    d_v: int
    steps: int           # decode steps of the workload
    seed: int
    bits: int = 8                       # uniform mode code width
    nominal_bits: float = 6.0           # STEP budget (bits per state value)
    cand_bits: Tuple[int, ...] = (4, 6, 8)
    pivot_frac: float = 0.0
    window: int = 16                    # window length p (window mode)
    comp_rank: int = 0                  # window mode: compensator pairs per head
    power_iters: int = 4                # window mode: power iterations per pair
    half_life: float = 64.0             # constant GDN half-life (tokens)
    half_life_range: Optional[Tuple[float, float]] = None  # log-uniform range
    warmup_steps: int = 128
    calib_steps: int = 2048
    calib_seqs: int = 32                # STEPQuant Sec. 5.1: 32 segments of 2048 tokens
    calib_snapshot_every: int = 16
    calib_snapshot_start: int = 128
    calib_horizon: int = 2048
    gamma: float = 0.25
    key_gain_sigma: float = 0.0         # log-normal gain spread on key channels
    value_gain_sigma: float = 0.0       # log-normal gain spread on value channels
    calib: Optional[str] = None         # workload whose calibration statistics give the plan

    @property
    def tiles(self) -> int:
        return self.batch * self.heads


WORKLOADS: Dict[str, Workload] = {
    # batch 1, 1 head, d=64, uniform symmetric INT8 with one scale per key row
    "tiny_gdn_int8": Workload(
        name="tiny_gdn_int8", kind="gdn", mode="uniform", batch=1, n_slots=1, heads=1,
        d_k=64, d_v=64, steps=256, seed=0, bits=8, half_life=64.0),
    # batch 64, 16 heads, mixed {4,6,8} per head at nominal 6 bits, 2% FP16 pivot heads
    "gdn_mid_step6": Workload(
        name="gdn_mid_step6", kind="gdn", mode="step", batch=64, n_slots=64, heads=16,
        d_k=128, d_v=128, steps=1024, seed=1, nominal_bits=6.0, cand_bits=(4, 6, 8),
        pivot_frac=0.02, half_life_range=(1.0, 4096.0)),
    # batch 256, 32 heads, KDA with per-key-row {4,6,8} at nominal 6 bits, 1.4% FP16 rows
    "kda_step6": Workload(
        name="kda_step6", kind="kda", mode="step", batch=256, n_slots=256, heads=32,
        d_k=128, d_v=128, steps=512, seed=2, nominal_bits=6.0, cand_bits=(4, 6, 8),
        pivot_frac=0.014, half_life_range=(1.0, 8192.0),
        key_gain_sigma=1.21, value_gain_sigma=1.21),
    # batch 512 drawn from a 1024-slot pool, 48 heads, nominal 4 bits with FP16 pivots
    "gdn_pool_step4": Workload(
        name="gdn_pool_step4", kind="gdn", mode="step", batch=512, n_slots=1024, heads=48,
        d_k=128, d_v=128, steps=256, seed=3, nominal_bits=4.0, cand_bits=(2, 4, 6, 8),
        pivot_frac=0.0139, half_life=64.0),
    # the pool workload's shape with the fp32 state kept dense (no codec): the
    # same-hardware denominator of the packed path's speed-up
    "gdn_pool_fp32": Workload(
        name="gdn_pool_fp32", kind="gdn", mode="dense", batch=512, n_slots=1024, heads=48,
        d_k=128, d_v=128, steps=256, seed=3, half_life=64.0),
    # the pool workload's shape with uniform rowwise INT4 (absmax, one FP16 scale per key row)
    "gdn_pool_int4": Workload(
        name="gdn_pool_int4", kind="gdn", mode="uniform", batch=512, n_slots=1024, heads=48,
        d_k=128, d_v=128, steps=256, seed=3, bits=4, half_life=64.0),
    # the mid workload's heads and 6-bit plan at batch 512 (the pages' 6-bit, batch-512 setting),
    # and the same shape with the fp32 state kept dense: a same-hardware 6-bit speed-up
    "gdn_b512_step6": Workload(
        name="gdn_b512_step6", kind="gdn", mode="step", batch=512, n_slots=512, heads=16,
        d_k=128, d_v=128, steps=256, seed=1, nominal_bits=6.0, cand_bits=(4, 6, 8),
        pivot_frac=0.02, half_life_range=(1.0, 4096.0), calib="gdn_mid_step6"),
    "gdn_b512_fp32": Workload(
        name="gdn_b512_fp32", kind="gdn", mode="dense", batch=512, n_slots=512, heads=16,
        d_k=128, d_v=128, steps=256, seed=1, half_life_range=(1.0, 4096.0)),
    # the KDA workload's shape, inputs and gates with the fp32 state kept dense:
    # the same-hardware denominator of the packed KDA step
    "kda_fp32": Workload(
        name="kda_fp32", kind="kda", mode="dense", batch=256, n_slots=256, heads=32,
        d_k=128, d_v=128, steps=512, seed=2, half_life_range=(1.0, 8192.0),
        key_gain_sigma=1.21, value_gain_sigma=1.21),
    # the window workloads' shape and inputs with the fp32 state kept dense
    "gdn_window_fp32": Workload(
        name="gdn_window_fp32", kind="gdn", mode="dense", batch=256, n_slots=256, heads=32,
        d_k=128, d_v=128, steps=1024, seed=4, half_life=64.0),
    # per-window variant: INT8 boundary + FP32 records, p = 16
    "gdn_window16": Workload(
        name="gdn_window16", kind="gdn", mode="window", batch=256, n_slots=256, heads=32,
        d_k=128, d_v=128, steps=1024, seed=4, window=16, half_life=64.0),
    # the same with r = 4 FP16 compensator pairs per head, 4 power iterations
    "gdn_window16_r4": Workload(
        name="gdn_window16_r4", kind="gdn", mode="window", batch=256, n_slots=256, heads=32,
        d_k=128, d_v=128, steps=1024, seed=4, window=16, half_life=64.0, comp_rank=4,
        power_iters=4),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (smaller test sizes)."""
    return dataclasses.replace(WORKLOADS[name], **overrides)


def _rng(seed: int, stream: int, step: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream), int(step)])


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _solve_mu_for_half_life(tau: np.ndarray) -> np.ndarray:
    """mu such that E[softplus(mu + Z)] = ln2 / tau, Z ~ N(0, 1).

    64-node probabilists' Gauss-Hermite quadrature for the expectation and
    bisection on mu (the expectation is increasing in mu)."""
    nodes, weights = np.polynomial.hermite_e.hermegauss(64)
    weights = weights / math.sqrt(2.0 * math.pi)
    target = math.log(2.0) / np.asarray(tau, dtype=np.float64)
    lo = np.full(target.shape, -60.0)
    hi = np.full(target.shape, 20.0)
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        val = (_softplus(mid[..., None] + nodes) * weights).sum(-1)
        too_big = val > target
        hi = np.where(too_big, mid, hi)
        lo = np.where(too_big, lo, mid)
    return 0.5 * (lo + hi)


def gate_params(w: Workload) -> Dict[str, np.ndarray]:
    """Static per-head / per-row gate and gain parameters of a workload."""
    rng = _rng(w.seed, _STREAM_STATIC, 0)
    out: Dict[str, np.ndarray] = {}
    if w.kind == "gdn":
        if w.half_life_range is None:
            tau = np.full(w.heads, float(w.half_life))
        else:
            lo, hi = w.half_life_range
            tau = np.exp(rng.uniform(math.log(lo), math.log(hi), size=w.heads))
        out["half_life"] = tau
        out["alpha"] = np.exp(-math.log(2.0) / tau).astype(np.float32)
    else:
        lo, hi = w.half_life_range or (w.half_life, w.half_life)
        tau = np.exp(rng.uniform(math.log(lo), math.log(hi), size=(w.heads, w.d_k)))
        out["half_life"] = tau
        out["mu"] = _solve_mu_for_half_life(tau)
    gk = np.exp(w.key_gain_sigma * rng.standard_normal((w.heads, w.d_k)))
    gv = np.exp(w.value_gain_sigma * rng.standard_normal((w.heads, w.d_v)))
    out["key_gain"] = gk
    out["value_gain"] = gv
    return out


def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _draw(w: Workload, rng: np.random.Generator, batch: int,
          params: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    H, dk, dv = w.heads, w.d_k, w.d_v
    q = _unit(rng.standard_normal((batch, H, dk)))
    k = _unit(params["key_gain"] * rng.standard_normal((batch, H, dk)))
    v = params["value_gain"] * rng.standard_normal((batch, H, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((batch, H))))
    if w.kind == "gdn":
        gate = np.broadcast_to(params["alpha"], (batch, H)).astype(np.float32)
    else:
        z = rng.standard_normal((batch, H, dk))
        gate = np.exp(-_softplus(params["mu"] + z)).astype(np.float32)
    return {
        "q": q.astype(np.float32),
        "k": k.astype(np.float32),
        "v": v.astype(np.float32),
        "beta": beta.astype(np.float32),
        "gate": np.ascontiguousarray(gate),
    }


def step_inputs(w: Workload, t: int, params: Optional[Dict[str, np.ndarray]] = None
                ) -> Dict[str, np.ndarray]:
    """Inputs of decode step ``t`` for the whole live batch: q, k [B,H,d_k],
    v [B,H,d_v], beta [B,H], gate [B,H] (GDN) or [B,H,d_k] (KDA)."""
    params = params if params is not None else gate_params(w)
    return _draw(w, _rng(w.seed, _STREAM_DECODE, t), w.batch, params)


def warmup_inputs(w: Workload, t: int, params: Optional[Dict[str, np.ndarray]] = None
                  ) -> Dict[str, np.ndarray]:
    """Inputs of warm-up step ``t`` (the unquantised steps that build the
    initial state); same distributions, independent stream."""
    params = params if params is not None else gate_params(w)
    return _draw(w, _rng(w.seed, _STREAM_WARMUP, t), w.batch, params)


def calib_inputs(w: Workload, t: int, params: Optional[Dict[str, np.ndarray]] = None
                 ) -> Dict[str, np.ndarray]:
    """Inputs of calibration step ``t`` for ``calib_seqs`` sequences (the
    batch axis holds the calibration sequences)."""
    params = params if params is not None else gate_params(w)
    return _draw(w, _rng(w.seed + 1000, _STREAM_CALIB, t), w.calib_seqs, params)


def slot_ids(w: Workload) -> np.ndarray:
    """Distinct pool slots of the live batch (a seeded permutation when the
    pool is larger than the batch)."""
    if w.n_slots == w.batch:
        return np.arange(w.batch, dtype=np.int32)
    rng = _rng(w.seed, _STREAM_STATIC, 1)
    return rng.permutation(w.n_slots)[: w.batch].astype(np.int32)
