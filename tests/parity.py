"""Teacher-forced comparison of the GPU path against the oracle.

For a compared step the oracle starts from the GPU's own packed bytes before
the step (parsed by the oracle's independent layout parser), runs the step in
float64 and walks the quantizer one decision at a time:

* FP16 scales (r, c0, c, uniform s, pivot values): a GPU value that differs
  from the oracle's is accepted, and adopted for the later decisions, only if
  the oracle's unrounded value lies within 1e-5 relative of the midpoint of
  the two binary16 neighbours and the GPU chose the other neighbour.  The
  initial column scale c0 is not stored; where it is such a near-tie the
  oracle keeps whichever neighbour reproduces the GPU's codes of the column.
  An FP16 pivot value is formed from two terms, D S_hat and beta k e^T, and
  e_j = v_j - sum_i k_i (D S_hat)_ij is itself a float32 dot product; its tie
  window also covers 4 fp32 ulps of the magnitudes of all those terms (where
  they cancel, fp32 cannot decide the rounding that float64 decides).
* integer codes: identical, except |dz| = 1 where the oracle's pre-rounding
  value is within 1e-3 code units of a half-integer (an exact tie up to fp32
  arithmetic);
* float32 window scales C, B: within 1e-6 relative, then adopted;
* readouts: ||y_gpu - y||_2 / ||y||_2 <= 1e-5 per (slot, head); the window
  record u_i = v_i - S_{i-1}^T (alpha_i k_i) is a readout too and is judged
  the same way; the record key beta_i k_i is exact (one fp32 product).

Any other difference is a failure.  Counts of adoptions are returned.
"""
from __future__ import annotations

from collections import Counter

import numpy as np

from oracle import numerics as N
from oracle import quantizers as Q
from oracle import recurrence as R
from oracle import window as W
from oracle.layout import parse_head

SCALE_REL = 1e-5
CODE_TIE = 1e-3
Y_REL = 1e-5
F32_REL = 1e-6


def oracle_desc(d: dict) -> dict:
    """Oracle layout description from a plan query (binding dict)."""
    if d["mode"] == 0:
        return {"mode": "uniform", "heads": d["heads"], "d_k": d["d_k"], "d_v": d["d_v"],
                "bits": d["uniform_bits"]}
    if d["mode"] == 2:
        return {"mode": "window", "heads": d["heads"], "d_k": d["d_k"], "d_v": d["d_v"],
                "p": d["window"], "rank": d.get("window_rank", 0),
                "iters": d.get("window_iters", 0)}
    ub = d["unit_bits"]
    if d["kind"] == 0:
        return {"mode": "step", "kind": "gdn", "heads": d["heads"], "d_k": d["d_k"],
                "d_v": d["d_v"], "head_bits": list(ub)}
    return {"mode": "step", "kind": "kda", "heads": d["heads"], "d_k": d["d_k"],
            "d_v": d["d_v"], "row_bits": ub.reshape(d["heads"], d["d_k"])}


def row_bits_of(desc: dict, h: int) -> np.ndarray:
    d_k = desc["d_k"]
    if desc["mode"] == "step" and desc["kind"] == "gdn":
        return np.full(d_k, int(desc["head_bits"][h]))
    if desc["mode"] == "step":
        return np.asarray(desc["row_bits"][h])
    return np.full(d_k, int(desc.get("bits", 8)))


def _signed_neighbours(x):
    x = np.asarray(x, dtype=np.float64)
    r = N.fp16(x)
    up = np.nextafter(r.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(r.astype(np.float16), np.float16(-np.inf)).astype(np.float64)
    lo = np.where(r <= x, r, dn)
    hi = np.where(r >= x, r, up)
    return lo, hi


def adopt_fp16(pre, ora, gpu, clamp=True, abs_tol=0.0):
    """(values to continue with, number adopted, failure mask).  abs_tol widens
    the tie window to the fp32 evaluation error of the value's terms."""
    pre = np.asarray(pre, dtype=np.float64)
    if clamp:
        lo, hi = N.fp16_neighbours(pre)
        ref = np.clip(pre, N.FP16_MIN_NORMAL, N.FP16_MAX)
    else:
        lo, hi = _signed_neighbours(pre)
        ref = pre
    mid = 0.5 * (lo + hi)
    near = np.abs(ref - mid) <= np.maximum(SCALE_REL * np.abs(ref), abs_tol)
    diff = gpu != ora
    ok = ~diff | (near & ((gpu == lo) | (gpu == hi)))
    return np.where(diff & ok, gpu, ora), int((diff & ok).sum()), ~ok


def adopt_codes(pre, ora, gpu):
    d = gpu - ora
    frac = np.abs(np.abs(pre - np.floor(pre)) - 0.5)
    ok = (d == 0) | ((np.abs(d) == 1) & (frac <= CODE_TIE))
    return np.where(ok, gpu, ora), int(((d != 0) & ok).sum()), ~ok


def adopt_f32(ora, gpu):
    ok = np.abs(gpu - ora) <= F32_REL * np.maximum(np.abs(ora), 1e-30)
    return np.where(ok, gpu, ora), int(((gpu != ora) & ok).sum()), ~ok


class Report:
    def __init__(self):
        self.count = Counter()
        self.fail = []
        self.max_y_rel = 0.0

    def add(self, key, n):
        self.count[key] += n

    def bad(self, where, what, mask):
        n = int(np.sum(mask))
        if n:
            self.fail.append(f"{where}: {what} ({n} mismatches)")

    def y(self, where, y_gpu, y_ref):
        rel = float(np.linalg.norm(y_gpu - y_ref) / max(np.linalg.norm(y_ref), 1e-300))
        self.max_y_rel = max(self.max_y_rel, rel)
        if not rel <= Y_REL:
            self.fail.append(f"{where}: readout rel err {rel:.3e}")

    def assert_ok(self):
        assert not self.fail, "\n".join(self.fail[:20])


# ----------------------------------------------------------- quantizer checks
def check_uniform(where, X, bits, gpu, rep: Report):
    pre_s, s = Q.uniform_scale(X, bits)
    s, n, bad = adopt_fp16(pre_s, s, gpu["s"])
    rep.add("scale_adopted", n)
    rep.bad(where, "row scale s", bad)
    pre_z, z = Q.uniform_codes(X, s, bits)
    z, n, bad = adopt_codes(pre_z, z, gpu["z"])
    rep.add("tie_codes", n)
    rep.bad(where, "codes", bad)


def check_step(where, X, w, row_bits, gpu, rep: Report, mag=None):
    """mag: elementwise size of the terms X is formed from (|D S_hat|,
    |beta k e^T| and |beta k_i| times the terms of e_j); a pivot value within
    4 fp32 ulps of those terms of an FP16 rounding midpoint is an exact tie up
    to fp32 arithmetic."""
    row_bits = np.asarray(row_bits)
    piv = row_bits == N.PIVOT_BITS
    keep = ~piv
    if piv.any():
        tol = 0.0 if mag is None else 2.0 ** -22 * mag[piv]
        h, n, bad = adopt_fp16(X[piv], N.fp16(X[piv]), gpu["h"][piv], clamp=False, abs_tol=tol)
        rep.add("pivot_adopted", n)
        rep.bad(where, "FP16 pivot values", bad)
    if not keep.any():
        return
    pre_r, r = Q.step_row_scales(X, w, row_bits)
    r_k, n, bad = adopt_fp16(pre_r[keep], r[keep], gpu["r"][keep])
    rep.add("scale_adopted", n)
    rep.bad(where, "row scale r", bad)
    r = r.copy()
    r[keep] = r_k
    pre_c0, c0 = Q.step_col_init(X, r, row_bits)
    pre_z, z = Q.step_codes(X, r, c0, row_bits)
    # c0 near-ties: keep the neighbour that reproduces the GPU codes
    lo, hi = N.fp16_neighbours(pre_c0)
    ref = np.clip(pre_c0, N.FP16_MIN_NORMAL, N.FP16_MAX)
    near = np.abs(ref - 0.5 * (lo + hi)) <= SCALE_REL * ref
    for j in np.nonzero(near)[0]:
        alt = hi[j] if c0[j] == lo[j] else lo[j]
        c_alt = c0.copy()
        c_alt[j] = alt
        pz, zz = Q.step_codes(X, r, c_alt, row_bits)
        if (np.sum(zz[keep, j] != gpu["z"][keep, j]) < np.sum(z[keep, j] != gpu["z"][keep, j])):
            c0, pre_z, z = c_alt, pz, zz
            rep.add("c0_adopted", 1)
    z_k, n, bad = adopt_codes(pre_z[keep], z[keep], gpu["z"][keep])
    rep.add("tie_codes", n)
    rep.bad(where, "codes", bad)
    z = z.copy()
    z[keep] = z_k
    Nn, D, pre_c, c = Q.step_col_refit(X, w, r, z, c0, row_bits)
    pos = D > 0
    c_p, n, bad = adopt_fp16(pre_c[pos], c[pos], gpu["c"][pos])
    rep.add("scale_adopted", n)
    rep.bad(where, "column scale c", bad)
    rep.bad(where, "column scale c (D = 0)", gpu["c"][~pos] != c0[~pos])


def check_window_quant(where, S, gpu, rep: Report, c_floor=Q.WINDOW_C_FLOOR):
    C = Q.window_row_smoothing(S, c_floor)
    C, n, bad = adopt_f32(C, gpu["C"])
    rep.add("f32_adopted", n)
    rep.bad(where, "smoothing C", bad)
    T, B = Q.window_col_scales(S, C)
    B, n, bad = adopt_f32(B, gpu["B"])
    rep.add("f32_adopted", n)
    rep.bad(where, "column scale B", bad)
    pre_z, Z = Q.window_codes(T, B)
    Z, n, bad = adopt_codes(pre_z, Z, gpu["Z"])
    rep.add("tie_codes", n)
    rep.bad(where, "window codes", bad)


def comp_adopter(where, gpu: dict, iters: int, dim: int, rep: Report):
    """Teacher-forced check of the compensator pairs (LeapQuant notes Sec. 2.4):
    the GPU's stored FP16 pair h must be the oracle's binary16 rounding of its
    float64 fit, or a correct rounding of a value within the float32 error of
    the fit, taken as (2 iters + 1) dim 2^-24 of the pair vector's norm (each
    iteration is two dim-term sums, plus the final scaling).  The GPU's pair
    is adopted either way, so the residual and the next pairs follow the
    stored values."""
    tau = (2 * iters + 1) * dim * 2.0 ** -24

    def adopt(h, k, u):
        out = []
        for raw, g, name in ((k, gpu["Kc"][h], "Kc"), (u, gpu["Uc"][h], "Uc")):
            own = W.fp16_value(raw)
            half_ulp = 0.5 * np.spacing(np.abs(raw).astype(np.float16)).astype(np.float64)
            near = np.abs(g - raw) <= half_ulp + tau * np.linalg.norm(raw)
            ok = (g == own) | near
            rep.add("comp_adopted", int(np.sum((g != own) & ok)))
            rep.bad(where, f"compensator {name}[{h}]", ~ok)
            out.append(np.asarray(g, dtype=np.float64).copy())
        return out[0], out[1]
    return adopt


# --------------------------------------------------------------- step checks
def check_decode_head(where, desc, h, before: bytes, after: bytes, inp: dict, y_gpu, w,
                      rep: Report):
    """inp: q, k [d_k], v [d_v], beta scalar, gate scalar (GDN) or [d_k] (KDA), float64."""
    st0 = parse_head(desc, h, before)
    st1 = parse_head(desc, h, after)
    d_k = desc["d_k"]
    mode = desc["mode"]
    if mode == "window":
        rank, iters = int(desc.get("rank", 0)), int(desc.get("iters", 0))
        adopt = comp_adopter(where, st1, iters, max(d_k, desc["d_v"]), rep) if rank else None
        r = W.window_step(st0, inp["q"], inp["k"], inp["v"], float(inp["beta"]),
                          float(inp["gate"]), int(desc["p"]), iters, adopt=adopt)
        rep.y(where, y_gpu, r["o"])
        if r["flushed"] is not None:
            check_window_quant(where, r["flushed"]["R"], st1, rep)
            rep.bad(where, "l after flush", np.array([st1["ell"] != 0]))
        else:
            i = int(st0["ell"])
            rep.bad(where, "l", np.array([st1["ell"] != i + 1]))
            rep.bad(where, "record alpha", np.array([st1["alpha"][i] != N.fp32(inp["gate"])]))
            rep.bad(where, "record beta k", st1["kt"][i] != r["kt"])
            # u_i = v_i - S_{i-1}^T (alpha_i k_i) is a readout of the state: the
            # readout tolerance applies to it, norm-wise per (slot, head)
            rel = np.linalg.norm(st1["u"][i] - r["u"]) / max(np.linalg.norm(r["u"]), 1e-300)
            rep.bad(where, f"record u rel err {rel:.2e}", np.array([not rel <= Y_REL]))
            rep.bad(where, "boundary codes changed", st1["Z"] != st0["Z"])
            if rank:
                rep.bad(where, "compensators changed",
                        (st1["Kc"] != st0["Kc"]).ravel())
                rep.bad(where, "compensators changed", (st1["Uc"] != st0["Uc"]).ravel())
        return
    kind = desc.get("kind", "gdn")
    dvec = R.gate_vector(inp["gate"], "gdn" if mode == "uniform" else kind, d_k)
    if mode == "uniform":
        S_hat = Q.dequant_uniform(st0["z"], st0["s"])
    else:
        rb = row_bits_of(desc, h)
        S_hat = Q.dequant_step(st0["z"], st0["r"], st0["c"], rb, st0["h"])
    Sd = R.retained(S_hat, dvec)
    X = R.delta_update(Sd, inp["k"], inp["v"], inp["beta"])
    rep.y(where, y_gpu, R.readout(X, inp["q"]))
    if mode == "uniform":
        check_uniform(where, X, int(desc["bits"]), st1, rep)
    else:
        # terms of X: D S_hat, beta k e^T, and those of the dot product e_j
        e_terms = np.abs(inp["v"]) + np.abs(inp["k"]) @ np.abs(Sd)
        mag = np.abs(Sd) + np.abs(X - Sd) + np.outer(np.abs(inp["beta"] * inp["k"]), e_terms)
        check_step(where, X, w, row_bits_of(desc, h), st1, rep, mag=mag)


def check_window_encode(where, desc, S, gpu: dict, rep: Report, init=None):
    """A boundary re-encode of dense S: with compensators, the teacher-forced
    pair fit (started from `init`, the head's previous pairs, or the all-ones
    vector) comes first and the residual is what is quantized."""
    rank, iters = int(desc.get("rank", 0)), int(desc.get("iters", 0))
    if rank:
        adopt = comp_adopter(where, gpu, iters, max(desc["d_k"], desc["d_v"]), rep)
        S = W.encode_boundary(S, rank, iters, init, adopt=adopt)["R"]
    check_window_quant(where, S, gpu, rep)


def check_quantized_head(where, desc, h, X, packed: bytes, w, rep: Report):
    st = parse_head(desc, h, packed)
    if desc["mode"] == "uniform":
        check_uniform(where, X, int(desc["bits"]), st, rep)
    elif desc["mode"] == "window":
        check_window_encode(where, desc, X, st, rep)  # a pack starts from all-ones
        rep.bad(where, "l", np.array([st["ell"] != 0]))
    else:
        check_step(where, X, w, row_bits_of(desc, h), st, rep)


def dequant_head(desc, h, buf: bytes) -> np.ndarray:
    st = parse_head(desc, h, buf)
    if desc["mode"] == "uniform":
        return Q.dequant_uniform(st["z"], st["s"])
    if desc["mode"] == "window":
        return W.window_state_dense(st)
    return Q.dequant_step(st["z"], st["r"], st["c"], row_bits_of(desc, h), st["h"])
