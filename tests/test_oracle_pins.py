"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage it checks.  None of them retypes an oracle
formula: they use identities between independently written code paths
(transport form vs. delta update, windowed expansion vs. step recurrence),
inequalities, special cases, numbers the pages print (tests/golden) and brute
force on tiny inputs (explicit loops, exhaustive code search, exhaustive
allocation search, numerical minimisation).
"""
import itertools
import math

import numpy as np
import pytest
from scipy.optimize import minimize_scalar

from conftest import golden
from oracle import calibration as C
from oracle import layout as L
from oracle import numerics as N
from oracle import quantizers as Q
from oracle import recurrence as R
from oracle import step as ST
from oracle import window as W


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def draw(rng, d_k, d_v, kind="gdn"):
    inp = {"q": unit(rng.standard_normal(d_k)), "k": unit(rng.standard_normal(d_k)),
           "v": rng.standard_normal(d_v), "beta": float(1 / (1 + np.exp(-rng.standard_normal())))}
    dvec = (np.full(d_k, rng.uniform(0.8, 1.0)) if kind == "gdn"
            else rng.uniform(0.3, 1.0, size=d_k))
    return inp, dvec


# --------------------------------------------------------------- P1 / P2 / P3
@pytest.mark.parametrize("mode,kind", [("uniform", "gdn"), ("step", "gdn"), ("step", "kda")])
def test_prop1_error_recursion(rng, mode, kind):
    """STEPQuant Proposition 1: E_t = A_t E_{t-1} + eps_t when the reference
    and the quantized path share keys, values, queries and gates."""
    d_k, d_v = 16, 12
    w = np.exp(0.3 * rng.standard_normal(d_k))
    row_bits = rng.choice([4, 6, 8], size=d_k) if kind == "kda" else np.full(d_k, 6)
    S_ref = rng.standard_normal((d_k, d_v))
    if mode == "uniform":
        enc = Q.quantize_uniform(S_ref, 6)
        state = {"z": enc["z"], "s": enc["s"]}
        S_hat = Q.dequant_uniform(enc["z"], enc["s"])
    else:
        enc = Q.quantize_step(S_ref, w, row_bits)
        state = {k: enc[k] for k in ("z", "r", "c", "h")}
        S_hat = Q.dequant_step(enc["z"], enc["r"], enc["c"], row_bits, enc["h"])
    E_prev = S_hat - S_ref
    for _ in range(40):
        inp, dvec = draw(rng, d_k, d_v, kind)
        A = R.transition(inp["k"], inp["beta"], dvec)
        S_ref = A @ S_ref + R.write_term(inp["k"], inp["v"], inp["beta"])
        if mode == "uniform":
            res = ST.uniform_step(state, inp, 6, dvec)
            state = {"z": res["new"]["z"], "s": res["new"]["s"]}
            S_hat = Q.dequant_uniform(state["z"], state["s"])
        else:
            res = ST.step_step(state, inp, w, row_bits, dvec)
            state = {k: res["new"][k] for k in ("z", "r", "c", "h")}
            S_hat = Q.dequant_step(state["z"], state["r"], state["c"], row_bits, state["h"])
        eps = S_hat - res["X"]
        E = S_hat - S_ref
        resid = E - (A @ E_prev + eps)
        assert np.linalg.norm(resid) <= 1e-12 * (1.0 + np.linalg.norm(E))
        E_prev = E


def test_transport_form_matches_delta_update(rng):
    """STEPQuant Eq. (1) and Eq. (2) describe the same update."""
    for kind in ("gdn", "kda"):
        inp, dvec = draw(rng, 9, 7, kind)
        S = rng.standard_normal((9, 7))
        X, y = R.dense_step(S, inp["q"], inp["k"], inp["v"], inp["beta"], dvec)
        A = R.transition(inp["k"], inp["beta"], dvec)
        np.testing.assert_allclose(X, A @ S + R.write_term(inp["k"], inp["v"], inp["beta"]),
                                   rtol=0, atol=1e-13)
        np.testing.assert_allclose(y, X.T @ inp["q"], rtol=0, atol=1e-13)


def test_prop1_contraction(rng):
    """STEPQuant Proposition 1 (and its Korean summary): ||k|| <= 1,
    beta in [0, 1], 0 <= D <= I imply ||A_t||_2 <= ||D_t||_2 <= 1."""
    d = 24
    cases = []
    for _ in range(300):
        k = unit(rng.standard_normal(d)) * rng.uniform(0.0, 1.0) ** 0.25
        cases.append((k, rng.uniform(0, 1), rng.uniform(0, 1, size=d)))
    k1 = unit(rng.standard_normal(d))
    cases += [(k1, 0.0, np.ones(d)), (k1, 1.0, np.ones(d)), (k1, 1.0, rng.uniform(0, 1, d)),
              (k1, 0.5, np.full(d, 0.999)), (np.zeros(d), 1.0, np.ones(d))]
    for k, beta, dvec in cases:
        A = R.transition(k, beta, dvec)
        nA = np.linalg.norm(A, 2)
        nD = np.max(np.abs(dvec))
        assert nA <= nD + 1e-12 and nD <= 1.0 + 1e-15


def test_eq19_directional_contraction(rng):
    """STEPQuant Eq. (19): with P = I - beta k k^T,
    P^T P = I - beta (2 - beta ||k||^2) k k^T (also for ||k|| != 1)."""
    d = 10
    for _ in range(20):
        k = rng.standard_normal(d) * rng.uniform(0.1, 1.5)
        beta = rng.uniform(0, 1)
        P = R.transition(k, beta, np.ones(d))
        rhs = np.eye(d) - beta * (2 - beta * (k @ k)) * np.outer(k, k)
        np.testing.assert_allclose(P.T @ P, rhs, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ P4 / P5
@pytest.mark.parametrize("mode", ["uniform", "step"])
def test_beta_zero_is_pure_decay(rng, mode):
    """beta = 0 removes the delta write (LeapQuant notes Sec. 2.1: without the
    delta rule beta = 0): X = D S_hat and y = X^T q."""
    d_k, d_v = 8, 8
    S = rng.standard_normal((d_k, d_v))
    inp, dvec = draw(rng, d_k, d_v, "kda")
    inp["beta"] = 0.0
    w = np.ones(d_k)
    if mode == "uniform":
        e = Q.quantize_uniform(S, 8)
        res = ST.uniform_step({"z": e["z"], "s": e["s"]}, inp, 8, dvec)
    else:
        e = Q.quantize_step(S, w, np.full(d_k, 8))
        res = ST.step_step({k: e[k] for k in ("z", "r", "c", "h")}, inp, w, np.full(d_k, 8), dvec)
    np.testing.assert_allclose(res["X"], dvec[:, None] * res["S_hat"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(res["y"], (dvec[:, None] * res["S_hat"]).T @ inp["q"],
                               rtol=0, atol=1e-14)


@pytest.mark.parametrize("mode", ["dense", "uniform", "step"])
def test_associative_recall(rng, mode):
    """beta = 1, ||k|| = 1 and q = k read back exactly the written value:
    k^T (I - k k^T) = 0, so y = X^T k = v whatever the state and gate
    (gated delta rule, STEPQuant Sec. 3; readout from X, appendix A)."""
    d_k, d_v = 12, 10
    for _ in range(5):
        inp, dvec = draw(rng, d_k, d_v, "kda")
        inp["beta"] = 1.0
        inp["q"] = inp["k"].copy()
        S = rng.standard_normal((d_k, d_v)) * 3
        if mode == "dense":
            _, y = R.dense_step(S, inp["q"], inp["k"], inp["v"], 1.0, dvec)
        elif mode == "uniform":
            e = Q.quantize_uniform(S, 4)
            y = ST.uniform_step({"z": e["z"], "s": e["s"]}, inp, 4, dvec)["y"]
        else:
            rb = np.full(d_k, 4)
            e = Q.quantize_step(S, np.ones(d_k), rb)
            y = ST.step_step({k: e[k] for k in ("z", "r", "c", "h")}, inp, np.ones(d_k), rb,
                             dvec)["y"]
        np.testing.assert_allclose(y, inp["v"], rtol=0, atol=1e-12)


# ------------------------------------------------------------------------ P6
def test_row_impact_identity(rng):
    """STEPQuant appendix B: a unit-Frobenius perturbation E_i confined to key
    row i changes the next readout by E_i^T g with ||E_i^T g||^2 = g_i^2,
    g = A^T q.  The readout change is measured by running the recurrence twice."""
    d_k, d_v = 10, 7
    for kind in ("gdn", "kda"):
        inp, dvec = draw(rng, d_k, d_v, kind)
        g = R.transported_query(inp["q"], inp["k"], inp["beta"], dvec)
        A = R.transition(inp["k"], inp["beta"], dvec)
        np.testing.assert_allclose(g, A.T @ inp["q"], rtol=0, atol=1e-14)
        S = rng.standard_normal((d_k, d_v))
        _, y0 = R.dense_step(S, inp["q"], inp["k"], inp["v"], inp["beta"], dvec)
        for i in range(d_k):
            E = np.zeros((d_k, d_v))
            E[i] = unit(rng.standard_normal(d_v))
            _, y1 = R.dense_step(S + E, inp["q"], inp["k"], inp["v"], inp["beta"], dvec)
            assert abs(np.sum((y1 - y0) ** 2) - g[i] ** 2) <= 1e-12


def test_gdn_gate_cancels_in_impact_factors(rng):
    """STEPQuant appendix B: all channels of a GDN head share one scalar gate,
    so the gate scales omega uniformly and cancels in w."""
    d_k = 16
    n = 200
    q = unit(rng.standard_normal((n, d_k)))
    k = unit(rng.standard_normal((n, d_k)))
    beta = rng.uniform(0, 1, n)
    om1 = (R.transported_query(q, k, beta, np.ones((n, d_k))) ** 2).mean(0)
    om2 = (R.transported_query(q, k, beta, np.full((n, d_k), 0.7)) ** 2).mean(0)
    np.testing.assert_allclose(om2, 0.49 * om1, rtol=1e-13)
    np.testing.assert_allclose(C.impact_factors(om2[None]), C.impact_factors(om1[None]),
                               rtol=1e-12)


# ------------------------------------------------------------------------ P7
def _tiles(rng):
    yield rng.standard_normal((4, 4))
    yield rng.standard_normal((4, 6)) * np.exp(rng.standard_normal((4, 1))) \
        * np.exp(rng.standard_normal((1, 6)))
    t = rng.standard_normal((4, 4))
    t[2] = 0.0
    yield t


@pytest.mark.parametrize("bits", [2, 4, 6, 8])
def test_uniform_codes_brute_force(rng, bits):
    """Appendix B.5 (symmetric rowwise baseline): every stored code is the
    nearest grid point s_i z in [-q_b, q_b] (exhaustive search; exact ties
    take the even code), s_i = fp16(absmax_i / q_b)."""
    q = 2 ** (bits - 1) - 1
    for X in _tiles(rng):
        enc = Q.quantize_uniform(X, bits)
        for i in range(X.shape[0]):
            amax = max(abs(x) for x in X[i])
            assert enc["s"][i] == float(np.float16(min(max(amax / q, 2 ** -14), 65504.0)))
            for j in range(X.shape[1]):
                best = min(range(-q, q + 1),
                           key=lambda z: (abs(X[i, j] - enc["s"][i] * z), z % 2))
                assert enc["z"][i, j] == best


@pytest.mark.parametrize("bits", [2, 4, 6, 8])
def test_dual_axis_brute_force(rng, bits):
    """STEPQuant Sec. 4.3 / appendix C on 4x4 and 4x6 tiles, by explicit
    loops: m_i is the row's mean |X|, r_i = fp16(sqrt(m_i / w_i)),
    c0_j = fp16(max_i |X_ij| / r_i), each code is the nearest grid point
    r_i c0_j z / q_b (exhaustive search), and c_j is the w^2-weighted least
    squares scale with the codes fixed (numerical minimisation)."""
    q = 2 ** (bits - 1) - 1
    for X in _tiles(rng):
        n_r, n_c = X.shape
        w = np.exp(0.5 * rng.standard_normal(n_r))
        enc = Q.quantize_step(X, w, np.full(n_r, bits))
        for i in range(n_r):
            m = sum(abs(X[i, j]) for j in range(n_c)) / n_c
            r = float(np.float16(min(max(math.sqrt(m / w[i]), 2 ** -14), 65504.0)))
            assert enc["r"][i] == r
        for j in range(n_c):
            cmax = max(abs(X[i, j]) / enc["r"][i] for i in range(n_r))
            assert enc["c0"][j] == float(np.float16(min(max(cmax, 2 ** -14), 65504.0)))
            for i in range(n_r):
                s = enc["r"][i] * enc["c0"][j] / q
                best = min(range(-q, q + 1), key=lambda z: (abs(X[i, j] - s * z), z % 2))
                assert enc["z"][i, j] == best

            def sse(c, j=j):
                return sum(w[i] ** 2 * (X[i, j] - enc["r"][i] * c * enc["z"][i, j] / q) ** 2
                           for i in range(n_r))
            if any(enc["z"][:, j] != 0):
                opt = minimize_scalar(sse, bounds=(0.0, 4 * enc["c0"][j] + 1), method="bounded",
                                      options={"xatol": 1e-13})
                assert abs(opt.x - enc["pre_c"][j]) <= 1e-6 * enc["pre_c"][j]
                # P16: the refit never does worse than the initial scale
                assert sse(enc["pre_c"][j]) <= sse(enc["c0"][j]) + 1e-15
                assert enc["c"][j] == float(np.float16(min(max(enc["pre_c"][j], 2 ** -14), 65504.)))
            else:
                assert enc["c"][j] == enc["c0"][j]


def test_dual_axis_reconstruction_grid(rng):
    """X_hat = r_i c_j z_ij / q_b (STEPQuant Sec. 4.3, codebook normalised by
    q_b): reconstructed with c0 every element lies within half a grid step of
    X; reconstructed with the refit c it matches an explicit loop."""
    for bits in (2, 4, 6, 8):
        q = 2 ** (bits - 1) - 1
        X = rng.standard_normal((5, 7)) * np.exp(rng.standard_normal((1, 7)))
        w = np.exp(0.4 * rng.standard_normal(5))
        rb = np.full(5, bits)
        enc = Q.quantize_step(X, w, rb)
        rec0 = Q.dequant_step(enc["z"], enc["r"], enc["c0"], rb, enc["h"])
        rec = Q.dequant_step(enc["z"], enc["r"], enc["c"], rb, enc["h"])
        for i in range(5):
            for j in range(7):
                step = enc["r"][i] * enc["c0"][j] / q
                assert abs(rec0[i, j] - X[i, j]) <= 0.5 * step * (1 + 1e-9) + 1e-300
                assert abs(rec[i, j] - enc["r"][i] * enc["c"][j] * enc["z"][i, j] / q) <= 1e-15 * abs(rec[i, j])


def test_impact_factor_exponent(rng):
    """STEPQuant appendix B: w_i proportional to omega_i^{1/8}; the Korean
    summary: normalised to geometric mean 1 within the head."""
    om = np.exp(rng.uniform(-6, 6, (3, 16)))
    w = C.impact_factors(om, gamma=0.25)
    for h in range(3):
        np.testing.assert_allclose(np.exp(np.mean(np.log(w[h]))), 1.0, rtol=1e-12)
        for i in range(16):
            np.testing.assert_allclose((w[h, i] / w[h, 0]) ** 8, om[h, i] / om[h, 0], rtol=1e-9)


def test_window_quantizer_brute_force(rng):
    """LeapQuant notes Sec. 2.5 (Eq. 7) and appendix B.3, by explicit loops:
    c_a = max(sqrt(mean_j |S_aj|), floor), T = S / c_a, B_j = max_a |T_aj|,
    each code is the nearest grid point of T on the grid B_j z / 127, and the
    reconstruction C (Z/127) B stays within half a grid step of S."""
    S = rng.standard_normal((5, 6)) * np.exp(rng.standard_normal((5, 1)))
    S[:, 4] = 0.0
    enc = Q.quantize_window(S)
    rec = Q.dequant_window(enc["Z"], enc["C"], enc["B"])
    for a in range(5):
        c = max(math.sqrt(sum(abs(S[a, j]) for j in range(6)) / 6), 1e-6)
        assert enc["C"][a] == float(np.float32(c))
    for j in range(6):
        bj = max(abs(S[a, j] / enc["C"][a]) for a in range(5))
        assert enc["B"][j] == float(np.float32(bj))
        for a in range(5):
            t = S[a, j] / enc["C"][a]
            if enc["B"][j] == 0:
                assert enc["Z"][a, j] == 0
                continue
            best = min(range(-127, 128),
                       key=lambda z: (abs(t - enc["B"][j] * z / 127), z % 2))
            assert enc["Z"][a, j] == best
            assert abs(rec[a, j] - S[a, j]) <= 0.5 * enc["C"][a] * enc["B"][j] / 127 * (1 + 1e-9)


def test_dual_axis_pivot_rows_and_scaling(rng):
    """FP16 pivot units (STEPQuant Sec. 4) store fp16(X) and take no part in
    the scales; scaling X by 4 doubles r and c exactly and keeps the codes."""
    X = rng.standard_normal((8, 8))
    X[3] *= 50.0                       # an outlier row kept as pivot
    w = np.ones(8)
    rb = np.full(8, 4)
    rb[3] = 16
    enc = Q.quantize_step(X, w, rb)
    np.testing.assert_array_equal(enc["h"][3], N.fp16(X[3]))
    assert enc["r"][3] == 0 and np.all(enc["z"][3] == 0)
    keep = np.arange(8) != 3
    enc_drop = Q.quantize_step(X[keep], w[keep], rb[keep])
    np.testing.assert_array_equal(enc["c"], enc_drop["c"])
    np.testing.assert_array_equal(enc["z"][keep], enc_drop["z"])
    Y = rng.standard_normal((6, 6))
    e1 = Q.quantize_step(Y, np.ones(6), np.full(6, 6))
    e4 = Q.quantize_step(4 * Y, np.ones(6), np.full(6, 6))
    np.testing.assert_array_equal(e4["z"], e1["z"])
    np.testing.assert_array_equal(e4["r"], 2 * e1["r"])
    np.testing.assert_array_equal(e4["c"], 2 * e1["c"])


def test_int6_baseline_description():
    """STEPQuant appendix B.5: absmax/31 scale in FP16 clamped to
    [2^-14, 65504], nearest-integer codes in [-31, 31]."""
    g = golden("int6_baseline.json")
    X = np.array([[1e-9, -2e-9, 0.0, 5e-10],
                  [3.1, -0.05, 1.55, 0.0],
                  [1e7, -3e6, 2.0, 0.0]])
    enc = Q.quantize_uniform(X, g["bits"])
    assert enc["s"][0] == g["scale_min"] and np.all(enc["z"][0] == 0)
    assert enc["s"][1] == float(np.float16(3.1 / 31))
    assert enc["s"][2] == g["scale_max"]
    assert enc["z"].max() == g["code_max"] and enc["z"].min() == -g["code_max"]
    assert np.all(np.abs(enc["z"]) <= g["code_max"])


# ------------------------------------------------------------------------ P9
def test_qwen_six_bit_byte_count(rng):
    """STEPQuant appendix D / F.1: 2304 heads at 128x128, nominal six bits,
    32 FP16 pivot heads -> 29,999,104 B per request in the serving layout
    (no pivot scale slots) and 30,015,488 B with the analytic scale slots."""
    g = golden("state_bytes.json")
    U, d = g["qwen_heads"], g["qwen_d"]
    L_u = C.lifetime_weight(-rng.uniform(1e-4, 0.5, U), 2048)
    base = rng.uniform(0.5, 2.0, U)
    dist = np.stack([base * 16.0, base * 4.0, base * 1.0], axis=1)   # convex in b
    alloc = C.allocate("gdn", U, d, d, np.log(rng.uniform(0.5, 0.999, U)), dist,
                       np.ones((U, d)), (4, 6, 8), g["qwen_nominal_bits"],
                       g["qwen_pivot_heads"] / U)
    assert (alloc["bits"] == 16).sum() == g["qwen_pivot_heads"]
    desc = {"mode": "step", "kind": "gdn", "heads": U, "d_k": d, "d_v": d,
            "head_bits": alloc["bits"]}
    serving = sum(L.head_fields(desc, h)["used"] for h in range(U))
    assert serving == g["qwen_serving_bytes_per_request"]
    assert serving + 2 * d * 2 * g["qwen_pivot_heads"] == g["qwen_analytic_bytes_per_request"]
    assert U * d * d * 4 == g["qwen_fp32_bytes_per_request"]
    assert round(U * d * d * 4 / serving, 2) == g["qwen_compression_ratio"]


@pytest.mark.parametrize("nominal,cand", [(6, (4, 6, 8)), (4, (2, 4, 6, 8))])
def test_kda_compact_count(nominal, cand):
    """STEPQuant appendix D: KDA row-level allocation, one shared FP16 column
    vector and one FP16 row vector per head, 512 FP16 pivot rows charged as
    eight-bit rows -> 6.30 / 4.30 bits per value, 7.875 / 5.375 MiB."""
    g = golden("state_bytes.json")
    H, d, n_piv = g["kda_heads"], g["kda_d"], g["kda_pivot_rows"]
    U = H * d
    budget = nominal * U - 8 * n_piv           # row-bits for the integer rows
    rows = U - n_piv
    # fill the budget exactly with the two widths around the nominal one
    hi = nominal
    lo = cand[cand.index(nominal) - 1]
    n_lo = (hi * rows - budget) // (hi - lo)
    bits = np.full(U, hi)
    bits[:n_lo] = lo
    bits[-n_piv:] = 16
    desc = {"mode": "step", "kind": "kda", "heads": H, "d_k": d, "d_v": d,
            "row_bits": bits.reshape(H, d)}
    total = sum(L.head_fields(desc, h)["used"] for h in range(H))
    assert round(8 * total / (U * d), 2) == g["kda_bits_per_value"][str(nominal)]
    assert total / 2 ** 20 == g["kda_mib_per_request"][str(nominal)]


def test_window_boundary_bytes():
    """LeapQuant notes Sec. 4.5: 1 + 2r(d_k+d_v)/(d_k d_v) + 4(d_k+d_v)/(d_k d_v)
    bytes per element (1.1875 at r = 4; 1.0625 with no compensators, the
    layout here) and a p = 16 FP16 record buffer of 8,224 bytes (FP32 here:
    twice that)."""
    g = golden("window_bytes.json")
    d_k, d_v, p = g["d_k"], g["d_v"], g["p"]
    f = L.head_fields({"mode": "window", "heads": 1, "d_k": d_k, "d_v": d_v, "p": p}, 0)
    base = (f["K"] - f["Z"]) / (d_k * d_v)
    assert base == g["boundary_bytes_per_element_r0"]
    records = (f["used"] - f["K"]) + 4 * p            # K~ and U arrays plus alpha[p]
    assert records == 2 * g["record_buffer_bytes_fp16"]
    # with r = 4 compensator pairs stored in the head (FP16 K~c, U~c)
    f4 = L.head_fields({"mode": "window", "heads": 1, "d_k": d_k, "d_v": d_v, "p": p,
                        "rank": 4}, 0)
    boundary4 = (f4["K"] - f4["Z"]) + (f4["used"] - f4["Kc"])
    assert boundary4 / (d_k * d_v) == g["boundary_bytes_per_element_r4"]
    assert f4["Kc"] - f4["K"] == records - 4 * p


# ------------------------------------------------- compensator tokens (N2)
def _spectral(rng, d_k, d_v, s):
    """A matrix with the given singular values (distinct) and its factors."""
    Uo, _ = np.linalg.qr(rng.standard_normal((d_k, d_k)))
    Vo, _ = np.linalg.qr(rng.standard_normal((d_v, d_v)))
    n = len(s)
    return (Uo[:, :n] * s) @ Vo[:, :n].T, Uo[:, :n], Vo[:, :n]


def test_lowrank_rank1_limit_is_top_singular_pair(rng):
    """Sec. 2.4, Eq. 5: with many iterations the rank-one power fit reaches the
    Frobenius-optimal rank-one term sigma_1 u_1 v_1^T (Eckart-Young), split
    evenly between the two factors."""
    s = np.array([9.0, 4.0, 2.5, 1.0, 0.3])
    M, Uo, Vo = _spectral(rng, 24, 17, s)
    K, U, Rm = W.lowrank_fit(M, 1, 300, exact=True)
    np.testing.assert_allclose(np.outer(K[0], U[0]), s[0] * np.outer(Uo[:, 0], Vo[:, 0]),
                               rtol=0, atol=1e-12 * s[0])
    assert abs(np.linalg.norm(K[0]) - np.sqrt(s[0])) < 1e-12
    assert abs(np.linalg.norm(U[0]) - np.sqrt(s[0])) < 1e-12
    assert abs(np.linalg.norm(Rm) ** 2 - np.sum(s[1:] ** 2)) < 1e-10


def test_lowrank_rank_r_is_truncated_decomposition(rng):
    """Sec. 2.4, Eq. 6: r pairs fitted one after another on the residual reach
    the best rank-r approximation (the truncated singular decomposition) and
    leave the energy of the remaining directions."""
    s = np.array([12.0, 7.0, 4.0, 2.0, 0.9, 0.4, 0.1])
    M, Uo, Vo = _spectral(rng, 20, 30, s)
    K, U, Rm = W.lowrank_fit(M, 4, 400, exact=True)
    best = (Uo[:, :4] * s[:4]) @ Vo[:, :4].T
    np.testing.assert_allclose(K.T @ U, best, rtol=0, atol=1e-10 * s[0])
    np.testing.assert_allclose(Rm, M - best, rtol=0, atol=1e-10 * s[0])


def test_lowrank_exact_on_rank1_and_zero(rng):
    """A rank-one matrix is fitted exactly after one iteration from any start
    not orthogonal to its row vector; a zero matrix gives zero pairs."""
    a, b = rng.standard_normal(9), rng.standard_normal(6)
    K, U, Rm = W.lowrank_fit(np.outer(a, b), 2, 1, exact=True)
    np.testing.assert_allclose(np.outer(K[0], U[0]), np.outer(a, b), rtol=0, atol=1e-13)
    assert np.abs(Rm).max() < 1e-13
    assert np.abs(np.outer(K[1], U[1])).max() < 1e-13  # only rounding noise left to fit
    K, U, Rm = W.lowrank_fit(np.zeros((5, 7)), 3, 4)
    assert not np.any(K) and not np.any(U) and not np.any(Rm)


def test_lowrank_start_vector_is_used(rng):
    """The fit starts from init[h]: started at the exact top right singular
    vector, one iteration already gives the top pair (from the all-ones start
    it does not)."""
    s = np.array([5.0, 4.5, 1.0])
    M, Uo, Vo = _spectral(rng, 10, 8, s)
    K, U, _ = W.lowrank_fit(M, 1, 1, init=Vo[:, :1].T, exact=True)
    np.testing.assert_allclose(np.outer(K[0], U[0]), s[0] * np.outer(Uo[:, 0], Vo[:, 0]),
                               rtol=0, atol=1e-12)
    K1, U1, _ = W.lowrank_fit(M, 1, 1, exact=True)
    assert np.abs(np.outer(K1[0], U1[0]) - s[0] * np.outer(Uo[:, 0], Vo[:, 0])).max() > 1e-3


def test_lowrank_stored_pairs_are_what_was_removed(rng):
    """Rounded to FP16, the stored pairs are exactly the terms taken out of the
    residual: residual + sum_h k~c_h u~c_h^T reproduces the input."""
    M = rng.standard_normal((16, 12)) * 3.0
    K, U, Rm = W.lowrank_fit(M, 3, 4)
    np.testing.assert_array_equal(K, K.astype(np.float16).astype(np.float64))
    np.testing.assert_array_equal(U, U.astype(np.float16).astype(np.float64))
    np.testing.assert_allclose(Rm + K.T @ U, M, rtol=0, atol=1e-13)


def test_compensated_window_exact_with_identity_quantizer(rng):
    """Sec. 2.4-2.5, Eqs. 7 and 10: with an identity boundary quantizer and
    unrounded records and factors, the compensated window path (readouts,
    rebuilds, refits across three windows) reproduces the step recurrence."""
    d_k, d_v, p, r = 10, 7, 4, 2
    S = rng.standard_normal((d_k, d_v))
    st = W.new_window_state(S, p, r, 3, exact=True)
    np.testing.assert_allclose(W.window_state_dense(st), S, rtol=0, atol=1e-12)
    assert np.abs(st["Kc"]).max() > 0
    for t in range(3 * p):
        inp, dvec = draw(rng, d_k, d_v, "gdn")
        res = W.window_step(st, inp["q"], inp["k"], inp["v"], inp["beta"], dvec[0], p, 3,
                            exact=True)
        S, y = R.dense_step(S, inp["q"], inp["k"], inp["v"], inp["beta"], dvec)
        np.testing.assert_allclose(res["o"], y, rtol=0, atol=1e-11)
        st = res["state"]
        np.testing.assert_allclose(W.window_state_dense(st), S, rtol=0, atol=1e-11)
    assert st["ell"] == 0


@pytest.mark.parametrize("rank", [0, 2])
def test_window_flush_keeps_the_state_and_restarts(rng, rank):
    """LeapQuant notes Sec. 2.6: closing a window early folds its records into
    the boundary.  With an identity quantizer the dense state is unchanged
    (Eq. 7 before, boundary plus pairs after) and the window is empty; at
    l = 0 the flush is a no-op; the next tokens still follow the step
    recurrence."""
    d_k, d_v, p = 9, 6, 8
    S = rng.standard_normal((d_k, d_v))
    st = W.new_window_state(S, p, rank, 3, exact=True)
    assert W.window_flush(st, p, 3, exact=True)["ell"] == 0
    for t in range(3):
        inp, dvec = draw(rng, d_k, d_v, "gdn")
        st = W.window_step(st, inp["q"], inp["k"], inp["v"], inp["beta"], dvec[0], p, 3,
                           exact=True)["state"]
        S, _ = R.dense_step(S, inp["q"], inp["k"], inp["v"], inp["beta"], dvec)
    assert st["ell"] == 3
    fl = W.window_flush(st, p, 3, exact=True)
    assert fl["ell"] == 0
    np.testing.assert_allclose(W.window_state_dense(fl), S, rtol=0, atol=1e-12)
    np.testing.assert_allclose(W.boundary_residual(fl) + (fl["Kc"].T @ fl["Uc"] if rank else 0.0),
                               S, rtol=0, atol=1e-12)
    inp, dvec = draw(rng, d_k, d_v, "gdn")
    res = W.window_step(fl, inp["q"], inp["k"], inp["v"], inp["beta"], dvec[0], p, 3, exact=True)
    S, y = R.dense_step(S, inp["q"], inp["k"], inp["v"], inp["beta"], dvec)
    np.testing.assert_allclose(res["o"], y, rtol=0, atol=1e-11)


def test_compensated_readout_matches_dense(rng):
    """Eq. 10 term by term: boundary residual, compensators decaying with the
    boundary, records with their own decay, equals (S_l)^T x of Eq. 7."""
    d_k, d_v, p, r = 9, 11, 6, 3
    S0 = rng.standard_normal((d_k, d_v))
    Kc, Uc = rng.standard_normal((r, d_k)), rng.standard_normal((r, d_v))
    alphas = rng.uniform(0.5, 1.0, p)
    kt, u = rng.standard_normal((p, d_k)), rng.standard_normal((p, d_v))
    x = rng.standard_normal(d_k)
    for n in range(p + 1):
        np.testing.assert_allclose(W.window_readout(S0, alphas, kt, u, n, x, Kc, Uc),
                                   W.window_dense(S0, alphas, kt, u, n, Kc, Uc).T @ x,
                                   rtol=0, atol=1e-12)
    g = np.prod(alphas[:2])
    manual = g * (S0 + Kc.T @ Uc) + alphas[1] * np.outer(kt[0], u[0]) + np.outer(kt[1], u[1])
    np.testing.assert_allclose(W.window_dense(S0, alphas, kt, u, 2, Kc, Uc), manual,
                               rtol=0, atol=1e-12)


# ----------------------------------------------------------------- P10-P13
def test_window_expansion_is_exact(rng):
    """LeapQuant notes Sec. 2.3 (Eq. 4, appendix Eq. 9): the windowed state
    and readout equal the step-by-step recurrence (unrounded records)."""
    d_k, d_v, p = 12, 9, 16
    S0 = rng.standard_normal((d_k, d_v))
    alphas, kt, u = np.zeros(p), np.zeros((p, d_k)), np.zeros((p, d_v))
    S = S0.copy()
    for i in range(1, p + 1):
        inp, dvec = draw(rng, d_k, d_v, "gdn")
        a = dvec[0]
        alphas[i - 1] = a
        prev = W.window_readout(S0, alphas, kt, u, i - 1, a * inp["k"])
        u[i - 1] = inp["v"] - prev
        kt[i - 1] = inp["beta"] * inp["k"]
        S, y = R.dense_step(S, inp["q"], inp["k"], inp["v"], inp["beta"], dvec)
        o = W.window_readout(S0, alphas, kt, u, i, inp["q"])
        np.testing.assert_allclose(o, y, rtol=0, atol=1e-12)
        np.testing.assert_allclose(W.window_dense(S0, alphas, kt, u, i), S, rtol=0, atol=1e-12)


def test_window_p1_is_per_step_smoothed_quantization(rng):
    """With p = 1 every token rebuilds the boundary: the window path equals
    per-step quantization with the smoothed INT8 quantizer."""
    d_k, d_v = 16, 16
    st = W.new_window_state(rng.standard_normal((d_k, d_v)), 1)
    for _ in range(6):
        inp, dvec = draw(rng, d_k, d_v, "gdn")
        S_hat = Q.dequant_window(st["Z"], st["C"], st["B"])
        X, y = R.dense_step(S_hat, inp["q"], inp["k"], inp["v"], inp["beta"], dvec)
        res = W.window_step(st, inp["q"], inp["k"], inp["v"], inp["beta"], dvec[0], 1)
        np.testing.assert_allclose(res["o"], y, rtol=1e-6, atol=1e-6)
        enc = Q.quantize_window(X)
        tie = np.abs(np.abs(enc["pre_z"] - np.floor(enc["pre_z"])) - 0.5) < 1e-3
        diff = res["state"]["Z"] != enc["Z"]
        assert np.all(~diff | tie)
        np.testing.assert_allclose(res["state"]["C"], enc["C"], rtol=1e-6)
        st = res["state"]


def test_smoothed_dequant_identity(rng):
    """LeapQuant notes appendix B.3: [C dequant(R)]^T Gamma x =
    B (Z^T / 127) C Gamma x (C on key rows, B on value columns)."""
    S = rng.standard_normal((10, 6)) * np.exp(rng.standard_normal((10, 1)))
    enc = Q.quantize_window(S)
    x = rng.standard_normal(10)
    gam = 0.83
    lhs = Q.dequant_window(enc["Z"], enc["C"], enc["B"]).T @ (gam * x)
    rhs = enc["B"] * ((enc["Z"].T / 127.0) @ (enc["C"] * gam * x))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-13, atol=1e-14)
    assert np.all(np.abs(enc["Z"]) <= 127) and np.all(np.abs(enc["Z"]).max(0) == 127)


def test_delayed_rounding_example():
    """LeapQuant notes Sec. 2.2: start 10, add 0.1 per token, step-1 rounding:
    per-step rounding stays at 10 (error 1.6), a 16-token window reaches 12
    (error 0.4)."""
    g = golden("delayed_rounding.json")
    n = g["tokens"]
    s = g["initial"]
    for _ in range(n):
        s = float(N.rne((s + g["increment"]) / g["step"]) * g["step"])
    assert s == g["per_step_result"]
    exact = g["initial"] + n * g["increment"]
    assert abs(abs(s - exact) - g["per_step_abs_error"]) < 1e-12
    dense = W.window_dense(np.array([[g["initial"]]]), np.ones(n), np.ones((n, 1)),
                           np.full((n, 1), g["increment"]), n)
    wres = float(N.rne(dense[0, 0] / g["step"]) * g["step"])
    assert wres == g["window_result"]
    assert abs(abs(wres - exact) - g["window_abs_error"]) < 1e-12


# ----------------------------------------------------------------- P14-P15
def test_lifetime_weight_closed_form():
    """STEPQuant Eq. 7: L_u = sum_{j<H} exp(2 j l_u) = (1 - e^{2Hl})/(1 - e^{2l});
    L = H when l = 0; the half-life of alpha = exp(-ln2/64) is 64 tokens."""
    H = 2048
    for ell in (-1e-4, -0.01, -0.3, -2.0):
        closed = (1 - math.exp(2 * H * ell)) / (1 - math.exp(2 * ell))
        assert abs(C.lifetime_weight(np.array([ell]), H)[0] - closed) <= 1e-10 * closed
    assert C.lifetime_weight(np.array([0.0]), H)[0] == H
    g = golden("halflife.json")
    ell = math.log(math.exp(-math.log(2) / g["half_life"]))
    assert abs(math.log(2) / -ell - g["half_life"]) < 1e-9


def test_greedy_matches_brute_force(rng):
    """Lifetime-aware allocation (STEPQuant Eq. 8) on tiny instances: with equal
    unit sizes and convex distortions the greedy reaches the exhaustive optimum
    of sum L_u d_u(b_u) under the budget."""
    cand = (4, 6, 8)
    for trial in range(25):
        U = int(rng.integers(2, 8))
        n_u = np.full(U, 16)
        L_u = rng.uniform(0.5, 20.0, U)
        a = rng.uniform(0.2, 3.0, U)
        dist = np.stack([a * 2.0 ** (-(b - 4) * rng.uniform(0.8, 1.2)) for b in cand], axis=1)
        nominal = float(rng.choice([4.5, 5.0, 6.0, 7.0, 7.5]))
        bits = C.greedy_allocate(L_u, dist, n_u, cand, nominal, np.array([], dtype=np.int64))
        budget = nominal * n_u.sum()
        best = math.inf
        for combo in itertools.product(range(3), repeat=U):
            if sum(n_u[u] * cand[c] for u, c in enumerate(combo)) <= budget:
                best = min(best, sum(L_u[u] * dist[u, c] for u, c in enumerate(combo)))
        got = sum(L_u[u] * dist[u, cand.index(b)] for u, b in enumerate(bits))
        assert sum(n_u * bits) <= budget
        assert got <= best * (1 + 1e-12)


def test_pivots_and_budget_charge(rng):
    """Pivots are the highest-risk units and are charged as eight-bit units
    (STEPQuant appendix D): the non-pivot units share b_bar N - 8 N_piv."""
    U = 12
    n_u = np.full(U, 64)
    L_u = rng.uniform(1, 5, U)
    dist = np.stack([np.full(U, 4.0), np.full(U, 2.0), np.full(U, 1.0)], 1) * rng.uniform(
        0.5, 2, (U, 1))
    score = L_u * dist[:, -1]
    piv = C.select_pivots(score, 2)
    assert set(piv) == set(np.argsort(-score)[:2])
    bits = C.greedy_allocate(L_u, dist, n_u, (4, 6, 8), 6.0, piv)
    assert np.all(bits[piv] == 16)
    nonpiv = np.setdiff1d(np.arange(U), piv)
    assert (n_u[nonpiv] * bits[nonpiv]).sum() <= 6.0 * n_u.sum() - 8 * n_u[piv].sum()
    with pytest.raises(ValueError):
        C.greedy_allocate(L_u, dist, n_u, (4, 6, 8), 3.0, piv)


# ------------------------------------------------------------------- layout
def test_layout_hand_computed_bytes():
    """Bit order of the layout on a hand-worked row (two's complement fields,
    little-endian bit stream)."""
    z = np.array([-7, 1, 0, 3, 7, -1, -3, 2])
    assert L.pack_code_row(z, 4) == bytes([0x19, 0x30, 0xF7, 0x2D])
    assert L.pack_code_row(np.array([1, -1, 0, -1]), 2) == bytes([0xCD])
    assert L.pack_code_row(np.array([31, -31, 5, -1]), 6) == bytes([0x5F, 0x58, 0xFC])
    assert L.pack_code_row(np.array([-127, 127, 0, -2]), 8) == bytes([0x81, 0x7F, 0x00, 0xFE])
    for b in (2, 4, 6, 8):
        qb = 2 ** (b - 1) - 1
        zz = np.arange(-qb, qb + 1)
        zz = np.resize(zz, 16 * ((len(zz) + 15) // 16))
        assert np.array_equal(L.unpack_code_row(L.pack_code_row(zz, b), b, len(zz)), zz)


def test_layout_blocked_positions():
    """Column-pair blocked order on a hand-worked 64 x 4 tile at 4 bits: element
    (row 32 rb + m, col 2 p + c) is value n = 2 m + c of chunk (rb, p); piece q
    of that chunk sits at byte (rb * 2 * 2 + q * 2 + p) * 16."""
    z = np.zeros((64, 4))
    z[0, 0] = 3          # rb 0, p 0, n 0  -> piece 0 of chunk (0,0), low nibble of byte 0
    z[0, 1] = -1         # rb 0, p 0, n 1  -> high nibble of byte 0
    z[17, 3] = -7        # rb 0, p 1, m 17, c 1 -> n 35 -> piece 1, byte 1, high nibble
    z[40, 2] = 5         # rb 1, p 1, m 8, c 0 -> n 16 -> piece 0, byte 8, low nibble
    buf = L.pack_blocked(z, 4)
    assert len(buf) == 64 * 4 * 4 // 8
    expect = bytearray(len(buf))
    expect[0] = 0xF3
    expect[(0 * 4 + 1 * 2 + 1) * 16 + 1] = 0x90
    expect[(1 * 4 + 0 * 2 + 1) * 16 + 8] = 0x05
    assert buf == bytes(expect)
    np.testing.assert_array_equal(L.parse_blocked(buf, 4, 64, 4), z)
    h = np.zeros((32, 2))
    h[1, 0] = 1.5        # n 2 -> bits 32..47 of chunk (0,0) -> piece 0 bytes 4..5
    buf = L.pack_blocked(h, 16)
    assert buf[4:6] == np.float16(1.5).tobytes() and sum(buf) == sum(np.float16(1.5).tobytes())


@pytest.mark.parametrize("mode", ["uniform", "gdn", "kda", "window"])
def test_layout_round_trip(rng, mode):
    d = 32
    if mode == "uniform":
        desc = {"mode": "uniform", "heads": 2, "d_k": d, "d_v": d, "bits": 8}
        sts = [{"z": rng.integers(-127, 128, (d, d)).astype(float),
                "s": N.fp16(rng.uniform(0.1, 2, d))} for _ in range(2)]
    elif mode == "gdn":
        desc = {"mode": "step", "kind": "gdn", "heads": 3, "d_k": d, "d_v": d,
                "head_bits": [4, 16, 6]}
        sts = []
        for b in desc["head_bits"]:
            X = rng.standard_normal((d, d))
            e = Q.quantize_step(X, np.ones(d), np.full(d, b))
            sts.append({k: e[k] for k in ("z", "r", "c", "h")})
    elif mode == "kda":
        rb = rng.choice([2, 4, 6, 8, 16], size=(2, d))
        desc = {"mode": "step", "kind": "kda", "heads": 2, "d_k": d, "d_v": d, "row_bits": rb}
        sts = []
        for h in range(2):
            e = Q.quantize_step(rng.standard_normal((d, d)), np.ones(d), rb[h])
            sts.append({k: e[k] for k in ("z", "r", "c", "h")})
    else:
        desc = {"mode": "window", "heads": 2, "d_k": d, "d_v": d, "p": 4}
        sts = []
        for h in range(2):
            st = W.new_window_state(rng.standard_normal((d, d)), 4)
            st["ell"] = 3
            st["alpha"] = N.fp32(rng.uniform(0.9, 1, 4))
            st["kt"] = N.fp32(rng.standard_normal((4, d)))
            st["u"] = N.fp32(rng.standard_normal((4, d)))
            sts.append(st)
    buf = L.pack_slot(desc, sts)
    lay = L.slot_layout(desc)
    assert len(buf) == lay["slot_bytes"] and lay["slot_bytes"] % 256 == 0
    back = L.parse_slot(desc, buf)
    for h, (a, b) in enumerate(zip(sts, back)):
        keys = list(b)
        if mode == "gdn" and desc["head_bits"][h] == 16:
            keys = ["h"]                      # a pivot head stores its FP16 values only
        for key in keys:
            np.testing.assert_array_equal(np.asarray(a[key]), np.asarray(b[key]), err_msg=key)
