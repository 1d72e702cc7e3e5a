"""Pins of the oracle's calibration-statistics collector (oracle.calibration.collect_stats).

STEPQuant Sec. 4 (Eqs. 6-8) and Sec. 4.1 define what the collector averages
over a calibration stream: the mean log retention l_u of each allocation unit
(a GDN head, a KDA key row), the row-impact score omega_i = E[g_{t,i}^2] with
g_t = A_t^T q_t, and the distortion d_u(b) of the dual-axis quantizer on
reference-trajectory snapshots (STEPQuant Sec. 5.1 fixes the 2048-token
calibration segment; snapshots every 16 steps after step 128 are this
implementation's reading of the estimator).  The streams below are built so
that each statistic has a closed form, or is recomputed by explicit loops
that share nothing with the collector's vectorised code.
"""
import math

import numpy as np
import pytest

from oracle import calibration as C
from oracle import quantizers as Q


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def stream(rng, kind, n, heads, d_k, d_v, steps, gate_fn, qk="random"):
    """Inputs of a calibration stream, drawn once (so a statistic can be
    recomputed from the same arrays)."""
    out = []
    for t in range(steps):
        q = unit(rng.standard_normal((n, heads, d_k)))
        if qk == "orth":      # k orthogonal to q: A_t^T q_t = D_t q_t
            k = rng.standard_normal((n, heads, d_k))
            k = unit(k - (k * q).sum(-1, keepdims=True) * q)
        elif qk == "same":    # k = q: A_t^T q_t = (1 - beta_t) D_t q_t
            k = q.copy()
        else:
            k = unit(rng.standard_normal((n, heads, d_k)))
        out.append({"q": q, "k": k, "v": rng.standard_normal((n, heads, d_v)),
                    "beta": 1.0 / (1.0 + np.exp(-rng.standard_normal((n, heads)))),
                    "gate": gate_fn(t)})
    return out


def collect(kind, heads, d_k, d_v, inputs, cand=(4, 6), **kw):
    return C.collect_stats(kind, heads, d_k, d_v, len(inputs), lambda t: inputs[t], cand, **kw)


def test_ell_is_log_alpha_for_constant_gdn_gate(rng):
    """A constant per-head GDN retention alpha_h gives l_h = log alpha_h exactly
    (STEPQuant Eq. 6: l_u is the mean log retention of the unit)."""
    alpha = np.array([0.5, 0.9, 0.999])
    inp = stream(rng, "gdn", 2, 3, 4, 4, 24, lambda t: np.broadcast_to(alpha, (2, 3)).copy())
    st = collect("gdn", 3, 4, 4, inp, snapshot_start=8, snapshot_every=8)
    np.testing.assert_allclose(st["ell"], np.log(alpha), rtol=0, atol=1e-15)
    # the half-life of a head (ln2 / -l_u) is the one the gate was built from
    np.testing.assert_allclose(math.log(2.0) / -st["ell"], math.log(2.0) / -np.log(alpha), rtol=1e-12)


def test_ell_is_per_row_mean_log_for_kda(rng):
    """KDA units are key rows: with row i's retention alternating between a_i
    and b_i on sequence 0 and between a_i^2 and b_i^2 on sequence 1, the mean
    log retention is 3/4 (log a_i + log b_i)."""
    heads, d_k = 2, 4
    a = rng.uniform(0.3, 0.99, size=(heads, d_k))
    b = rng.uniform(0.3, 0.99, size=(heads, d_k))

    def gate(t):
        g = a if t % 2 == 0 else b
        return np.stack([g, g * g])
    inp = stream(rng, "kda", 2, heads, d_k, 3, 20, gate)
    st = collect("kda", heads, d_k, 3, inp, snapshot_start=4, snapshot_every=8)
    want = 0.75 * (np.log(a) + np.log(b))
    np.testing.assert_allclose(st["ell"], want.reshape(-1), rtol=1e-13, atol=0)
    assert st["ell"].shape == (heads * d_k,)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_omega_when_query_is_orthogonal_to_key(rng, kind):
    """With k_t . q_t = 0 the delta transition leaves the query alone, so
    g_t = A_t^T q_t = D_t q_t and omega_i = mean_t d_{t,i}^2 q_{t,i}^2
    (STEPQuant Sec. 4.1; A_t^T = D_t (I - beta_t k_t k_t^T) because D_t is
    diagonal)."""
    n, heads, d_k = 3, 2, 5
    if kind == "gdn":
        gates = [rng.uniform(0.5, 1.0, size=(n, heads)) for _ in range(16)]
        dv = [np.repeat(g[..., None], d_k, axis=-1) for g in gates]
    else:
        gates = [rng.uniform(0.2, 1.0, size=(n, heads, d_k)) for _ in range(16)]
        dv = gates
    inp = stream(rng, kind, n, heads, d_k, 3, 16, lambda t: gates[t], qk="orth")
    st = collect(kind, heads, d_k, 3, inp, snapshot_start=4, snapshot_every=4)
    want = np.mean([(dv[t] * inp[t]["q"]) ** 2 for t in range(16)], axis=(0, 1))
    np.testing.assert_allclose(st["omega"], want, rtol=1e-13)


def test_omega_when_query_equals_key(rng):
    """With k_t = q_t (unit norm) the transported query is (1 - beta_t) D_t q_t,
    so omega_i = mean_t (1 - beta_t)^2 d_{t,i}^2 q_{t,i}^2.  A sign slip in the
    delta term (1 + beta) or the gate applied before the projection would fail."""
    n, heads, d_k = 2, 2, 6
    gates = [rng.uniform(0.2, 1.0, size=(n, heads, d_k)) for _ in range(12)]
    inp = stream(rng, "kda", n, heads, d_k, 3, 12, lambda t: gates[t], qk="same")
    st = collect("kda", heads, d_k, 3, inp, snapshot_start=4, snapshot_every=4)
    want = np.mean([((1.0 - inp[t]["beta"])[..., None] * gates[t] * inp[t]["q"]) ** 2
                    for t in range(12)], axis=(0, 1))
    np.testing.assert_allclose(st["omega"], want, rtol=1e-12)


def test_snapshot_schedule():
    """2048 calibration steps with snapshots every 16 steps after step 128 give
    (2048 - 128) / 16 = 120 snapshots; a 40-step stream with snapshots every 16
    after step 8 takes them after steps 24 and 40."""
    def zero_stream(steps, d=2):
        z = {"q": np.full((1, 1, d), 1.0 / math.sqrt(d)), "k": np.full((1, 1, d), 1.0 / math.sqrt(d)),
             "v": np.zeros((1, 1, d)), "beta": np.full((1, 1), 0.5), "gate": np.full((1, 1), 0.9)}
        return [z] * steps
    st = collect("gdn", 1, 2, 2, zero_stream(2048), cand=(4,), snapshot_start=128, snapshot_every=16)
    assert st["snapshots"] == 120
    st = collect("gdn", 1, 2, 2, zero_stream(40), cand=(4,), snapshot_start=8, snapshot_every=16)
    assert st["snapshots"] == 2


def test_distortion_zero_on_grid_states():
    """A state whose entries all sit on the quantizer's grid has zero
    distortion at every width.  Stream: q = (1,1,1,1)/2 and k = (1,-1,1,-1)/2
    (orthogonal, so every row has the same impact and w = 1), alpha = 1, and a
    single write beta = 1 of v = 8 (1,-1,-1,1); afterwards beta = 0.  The state
    is then k v^T with entries +-4: row scale 2, column scale 2, codes +-q_b,
    reconstruction exact."""
    q = np.array([1.0, 1.0, 1.0, 1.0]) / 2.0
    k = np.array([1.0, -1.0, 1.0, -1.0]) / 2.0
    v = 8.0 * np.array([1.0, -1.0, -1.0, 1.0])
    inp = [{"q": q[None, None], "k": k[None, None], "v": v[None, None],
            "beta": np.full((1, 1), 1.0 if t == 0 else 0.0), "gate": np.ones((1, 1))}
           for t in range(64)]
    st = collect("gdn", 1, 4, 4, inp, cand=(2, 4, 6, 8), snapshot_start=16, snapshot_every=16)
    assert st["snapshots"] == 3
    np.testing.assert_array_equal(st["dist"], np.zeros((1, 4)))
    # entries +-1.48 instead (0.37 v): the row scale FP16(sqrt(1.48)) times the
    # column scale no longer lands on 1.48, so the same stream now has a
    # nonzero distortion, which shows the zero above is not vacuous
    inp2 = [dict(x, v=x["v"] * 0.37) for x in inp]
    st2 = collect("gdn", 1, 4, 4, inp2, cand=(2,), snapshot_start=16, snapshot_every=16)
    assert st2["dist"][0, 0] > 0.0


def _explicit_states(inp, kind, d_k, d_v, snap_after):
    """Reference states by scalar loops (S' = D S, delta_j = sum_i k_i S'_ij,
    S_ij = S'_ij + beta k_i (v_j - delta_j)), recorded after the given steps."""
    n, heads = inp[0]["q"].shape[:2]
    S = [[[[0.0] * d_v for _ in range(d_k)] for _ in range(heads)] for _ in range(n)]
    snaps = []
    for t, x in enumerate(inp):
        for s in range(n):
            for h in range(heads):
                d = ([float(x["gate"][s, h])] * d_k if kind == "gdn"
                     else [float(x["gate"][s, h, i]) for i in range(d_k)])
                M = S[s][h]
                for i in range(d_k):
                    for j in range(d_v):
                        M[i][j] *= d[i]
                for j in range(d_v):
                    delta = sum(x["k"][s, h, i] * M[i][j] for i in range(d_k))
                    e = x["v"][s, h, j] - delta
                    for i in range(d_k):
                        M[i][j] += x["beta"][s, h] * x["k"][s, h, i] * e
        if t + 1 in snap_after:
            snaps.append(np.array(S))
    return snaps


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_distortion_matches_explicit_loops(rng, kind):
    """d_u(b) = mean over sequences and snapshots of the unit's summed squared
    reconstruction error (a whole head for GDN, one key row for KDA), with the
    impact factors from the stream's own omega.  Recomputed here with scalar
    loops over the states, the snapshot steps and the error sums."""
    n, heads, d_k, d_v, steps = 2, 2, 4, 4, 48
    if kind == "gdn":
        gates = [rng.uniform(0.7, 1.0, size=(n, heads)) for _ in range(steps)]
    else:
        gates = [rng.uniform(0.5, 1.0, size=(n, heads, d_k)) for _ in range(steps)]
    inp = stream(rng, kind, n, heads, d_k, d_v, steps, lambda t: gates[t])
    cand = (2, 4, 8)
    st = collect(kind, heads, d_k, d_v, inp, cand=cand, snapshot_start=8, snapshot_every=16)
    assert st["snapshots"] == 2
    snaps = _explicit_states(inp, kind, d_k, d_v, {24, 40})
    w = C.impact_factors(st["omega"])
    U = heads if kind == "gdn" else heads * d_k
    want = np.zeros((U, len(cand)))
    for ci, b in enumerate(cand):
        for S in snaps:
            for s in range(n):
                for h in range(heads):
                    X = S[s, h]
                    enc = Q.quantize_step(X, w[h], np.full(d_k, b))
                    Xh = Q.dequant_step(enc["z"], enc["r"], enc["c"], np.full(d_k, b), enc["h"])
                    for i in range(d_k):
                        e2 = sum((Xh[i, j] - X[i, j]) ** 2 for j in range(d_v))
                        u = h if kind == "gdn" else h * d_k + i
                        want[u, ci] += e2 / (n * len(snaps))
    np.testing.assert_allclose(st["dist"], want, rtol=1e-9, atol=0)
    assert np.all(want[:, 0] > want[:, -1]) and np.all(want > 0)
