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
  An FP16 pivot value X_ij = (D S_hat)_ij + beta k_i e_j is formed in fp32
  from e_j = v_j - sum_l k_l (D S_hat)_lj, a d_k-term fp32 sum; a GPU value
  is also accepted if it is the binary16 rounding of a value within the fp32
  error bound of that evaluation (below): where the terms cancel, fp32
  cannot decide the rounding that float64 decides, and the interval can
  span more than one binary16 step.
* float32 window scales C, B and codes after a rebuild: the rebuilt state
  S_p = Gamma S_hat_0 + sum_j Gamma k~_j u_j^T, minus the new compensator
  pairs, is a sum of at most 1 + p + 2r fp32 terms per element; where those
  terms cancel (a rank-r fit removes most of a column), its fp32 error is
  large against the residual that is quantized, so C, B and the codes also
  accept a GPU value within the error bound that follows from it (below).
* integer codes: identical, except |dz| = 1 where the oracle's pre-rounding
  value is within 1e-3 code units of a half-integer (an exact tie up to fp32
  arithmetic);
* float32 window scales C, B: within 1e-6 relative (or the rebuild's error
  bound), then adopted;

Error bounds (u = 2^-24; a sum of n fp32 terms in any order is within
(n - 1) u of the sum of the terms' magnitudes, Higham's gamma_{n-1}; each
product and the final rounding add u; everything is doubled for the second
order terms):

* pivot value: |X_gpu - X| <= 2u (|X| + |D S_hat| + |beta k_i| (3 |e_j| +
  (d_k + 2) A_j)), A_j = sum_l |k_l (D S_hat)_lj|;
* rebuilt residual: |R_gpu - R| <= 2u (2p + 2r + 6) M with M the same sum
  over the magnitudes of every term (1 + p + 2r terms; each carries a decay
  product Gamma of up to p fp32 factors and two more roundings); then C_a = sqrt(mean_j |R_aj|) moves by
  at most mean_j dR_aj / (2 C_a) + u C_a, T = R / C by dR / C + |T| dC / C,
  B_j = max_a |T_aj| by max_a dT_aj + u B_j, and the pre-rounding code
  127 T / B by 127 (dT + |T| dB / B) / B.
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
    """(values to continue with, number adopted, failure mask).

    Scales (clamp): a GPU value that differs must be the other binary16
    neighbour of an unrounded value within 1e-5 relative of their midpoint.
    Pivot values (no clamp) with an fp32 error bound abs_tol: a GPU value that
    differs must be the binary16 rounding of some value within abs_tol of the
    oracle's, i.e. lie between the roundings of pre - abs_tol and pre + abs_tol
    (where terms cancel that interval can span several binary16 steps)."""
    pre = np.asarray(pre, dtype=np.float64)
    diff = gpu != ora
    if clamp:
        lo, hi = N.fp16_neighbours(pre)
        ref = np.clip(pre, N.FP16_MIN_NORMAL, N.FP16_MAX)
        mid = 0.5 * (lo + hi)
        near = np.abs(ref - mid) <= SCALE_REL * np.abs(ref)
        ok = ~diff | (near & ((gpu == lo) | (gpu == hi)))
    else:
        lo, hi = _signed_neighbours(pre)
        mid = 0.5 * (lo + hi)
        near = np.abs(pre - mid) <= SCALE_REL * np.abs(pre)
        ok = ~diff | (near & ((gpu == lo) | (gpu == hi)))
        tol = np.broadcast_to(np.asarray(abs_tol, dtype=np.float64), pre.shape)
        if np.any(tol > 0):
            with np.errstate(over="ignore"):
                within = (gpu >= N.fp16(pre - tol)) & (gpu <= N.fp16(pre + tol))
            ok = ok | within
    return np.where(diff & ok, gpu, ora), int((diff & ok).sum()), ~ok


def adopt_codes(pre, ora, gpu, tie=None):
    """tie: per-element bound (code units, default 1e-3) on how far the GPU's
    unrounded code may lie from the oracle's `pre`.  A GPU code is accepted if
    it is a rounding of some value in that window, |gpu - pre| <= 1/2 + tie:
    the oracle's own code, or, when `pre` lies within the window of a
    half-integer, its neighbour across it (and, where the window exceeds half a
    code, e.g. on a residual at the level of its own float32 error, any code
    the window reaches)."""
    d = gpu - ora
    win = CODE_TIE if tie is None else np.maximum(CODE_TIE, tie)
    ok = (d == 0) | (np.abs(gpu - pre) <= 0.5 + win)
    return np.where(ok, gpu, ora), int(((d != 0) & ok).sum()), ~ok


def adopt_f32(ora, gpu, tol=None):
    """tol: per-element absolute error bound that widens the 1e-6 window."""
    win = F32_REL * np.maximum(np.abs(ora), 1e-30)
    if tol is not None:
        win = np.maximum(win, tol)
    ok = np.abs(gpu - ora) <= win
    return np.where(ok, gpu, ora), int(((gpu != ora) & ok).sum()), ~ok


class Report:
    def __init__(self):
        self.count = Counter()
        self.fail = []
        self.max_y_rel = 0.0

    def add(self, key, n):
        self.count[key] += n

    def bad(self, where, what, mask, detail=None):
        n = int(np.sum(mask))
        if n:
            extra = "" if detail is None else f"; {detail(mask)}"
            self.fail.append(f"{where}: {what} ({n} mismatches{extra})")

    def y(self, where, y_gpu, y_ref, bound=None):
        """Norm-wise Y_REL; `bound` (per element) is the float32 forward error
        bound of the readout, which exceeds Y_REL where the readout cancels."""
        rel = float(np.linalg.norm(y_gpu - y_ref) / max(np.linalg.norm(y_ref), 1e-300))
        if bound is not None and not rel <= Y_REL and np.all(np.abs(y_gpu - y_ref) <= bound):
            self.add("y_within_f32_bound", 1)
            return
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


def check_step(where, X, w, row_bits, gpu, rep: Report, err=None):
    """err: elementwise fp32 error bound of X (module docstring); a pivot value
    within it of an FP16 rounding midpoint is an exact tie up to fp32
    arithmetic."""
    row_bits = np.asarray(row_bits)
    piv = row_bits == N.PIVOT_BITS
    keep = ~piv
    if piv.any():
        tol = 0.0 if err is None else err[piv]
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


def check_window_quant(where, S, gpu, rep: Report, c_floor=Q.WINDOW_C_FLOOR, dR=None):
    """dR: elementwise fp32 error bound of the rebuilt residual S (module
    docstring), or None for an exactly known S (a pack)."""
    u = 2.0 ** -24
    C = Q.window_row_smoothing(S, c_floor)
    dC = None if dR is None else dR.mean(-1) / (2 * C) + 2 * u * C
    C, n, bad = adopt_f32(C, gpu["C"], dC)
    rep.add("f32_adopted", n)
    rep.bad(where, "smoothing C", bad,
            lambda m: f"max rel diff {np.max(np.abs(gpu['C'] - C)[m] / C[m]):.2e}")
    T, B = Q.window_col_scales(S, C)
    dT = dB = None
    if dR is not None:
        dT = dR / C[:, None] + np.abs(T) * (dC / C)[:, None]
        dB = dT.max(axis=0) + 2 * u * B
    B_ora = B
    B, n, bad = adopt_f32(B, gpu["B"], dB)
    rep.add("f32_adopted", n)
    rep.bad(where, "column scale B", bad,
            lambda m: f"max rel diff {np.max(np.abs(gpu['B'] - B_ora)[m] / B_ora[m]):.2e}"
            + ("" if dB is None else f", bound {np.max(dB[m] / B_ora[m]):.2e}"))
    pre_z, Z = Q.window_codes(T, B)
    tie = None
    if dT is not None:
        safe_B = np.where(B > 0, B, 1.0)
        tie = Q.WINDOW_CODE_MAX * (dT + np.abs(T) * (dB / safe_B)[None, :]) / safe_B[None, :]
    Z, n, bad = adopt_codes(pre_z, Z, gpu["Z"], tie)
    rep.add("tie_codes", n)
    rep.bad(where, "window codes", bad)


def comp_adopter(where, gpu: dict, iters: int, dim: int, rep: Report, noise: float = 0.0):
    """Teacher-forced check of the compensator pairs (LeapQuant notes Sec. 2.4):
    the GPU's stored FP16 pair h must be the oracle's binary16 rounding of its
    float64 fit, or a correct rounding of a value within the float32 error of
    the fit, taken as (2 iters + 1) dim 2^-24 of the pair vector's norm (each
    iteration is two dim-term sums, plus the final scaling).  The GPU's pair
    is adopted either way, so the residual and the next pairs follow the
    stored values.

    `noise` is the float32 error of the rebuilt state being fitted (Frobenius
    norm).  A pair whose weight |k| |u| lies below it in both fits fits only
    that error (a rank-deficient state, e.g. a zero gate at the window's last
    token), so its direction is not unique: it is accepted when the GPU's pair
    is as small, and adopted."""
    tau = (2 * iters + 1) * dim * 2.0 ** -24

    def adopt(h, k, u):
        gk = np.asarray(gpu["Kc"][h], dtype=np.float64)
        gu = np.asarray(gpu["Uc"][h], dtype=np.float64)
        if (noise > 0.0 and np.linalg.norm(k) * np.linalg.norm(u) <= noise
                and np.linalg.norm(gk) * np.linalg.norm(gu) <= noise):
            rep.add("comp_noise_level", 1)
            return gk.copy(), gu.copy()
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
        adopt = None
        if rank:
            # float32 error of the rebuild that the pairs are fitted to: the
            # flush check's elementwise bound 2 (2p + 2r + 6) 2^-24 per unit of
            # the terms' magnitudes, here on a norm bound of those terms
            p = int(desc["p"])
            a_, b_ = abs(float(inp["gate"])), abs(float(inp["beta"]))
            held = int(st0["ell"])
            mag = (np.linalg.norm(W.boundary_residual(st0))
                   + sum(np.linalg.norm(st0["kt"][j]) * np.linalg.norm(st0["u"][j])
                         for j in range(held))
                   + sum(np.linalg.norm(st0["Kc"][h_]) * np.linalg.norm(st0["Uc"][h_])
                         for h_ in range(rank)))
            nk = np.linalg.norm(inp["k"])
            scale = a_ * mag + b_ * nk * (np.linalg.norm(inp["v"]) + a_ * mag * nk)
            noise = 2 * (2 * p + 2 * rank + 6) * 2.0 ** -24 * scale
            adopt = comp_adopter(where, st1, iters, max(d_k, desc["d_v"]), rep, noise=noise)
        r = W.window_step(st0, inp["q"], inp["k"], inp["v"], float(inp["beta"]),
                          float(inp["gate"]), int(desc["p"]), iters, adopt=adopt)
        rep.y(where, y_gpu, r["o"])
        if r["flushed"] is not None:
            p = int(desc["p"])
            new = r["state"]
            M = W.window_dense(np.abs(r["S0"]), new["alpha"], np.abs(new["kt"]), np.abs(new["u"]),
                               p, None if not rank else np.abs(st0["Kc"]),
                               None if not rank else np.abs(st0["Uc"]))
            if rank:
                M = M + np.abs(r["flushed"]["Kc"]).T @ np.abs(r["flushed"]["Uc"])
            dR = 2 * 2.0 ** -24 * (2 * p + 2 * rank + 6) * M
            check_window_quant(where, r["flushed"]["R"], st1, rep, dR=dR)
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
    # fp32 error bound of X = D S_hat + beta k e^T with e_j a d_k-term sum, and
    # of the readout X^T q, a d_k-term sum of products of those elements
    u = 2.0 ** -24
    A = np.abs(inp["k"]) @ np.abs(Sd)
    e = inp["v"] - Sd.T @ inp["k"]
    err = 2 * u * (np.abs(X) + np.abs(Sd) + np.outer(np.abs(inp["beta"] * inp["k"]),
                                                    3 * np.abs(e) + (d_k + 2) * A))
    aq = np.abs(inp["q"])
    rep.y(where, y_gpu, R.readout(X, inp["q"]),
          bound=err.T @ aq + (d_k + 2) * u * (np.abs(X).T @ aq))
    if mode == "uniform":
        check_uniform(where, X, int(desc["bits"]), st1, rep)
    else:
        check_step(where, X, w, row_bits_of(desc, h), st1, rep, err=err)


def check_window_encode(where, desc, S, gpu: dict, rep: Report, init=None):
    """A boundary re-encode of dense S: with compensators, the teacher-forced
    pair fit (started from `init`, the head's previous pairs, or the all-ones
    vector) comes first and the residual is what is quantized."""
    rank, iters = int(desc.get("rank", 0)), int(desc.get("iters", 0))
    dR = None
    if rank:
        # the state the pairs are fitted to is exact here; the kernel forms the
        # residual S - sum_h kc_h uc_h^T with `rank` fp32 multiply-adds per
        # element, hence at most 2 rank 2^-24 of |S| + sum_h |kc_h| |uc_h|^T
        noise = 2 * (2 * rank + 2) * 2.0 ** -24 * np.linalg.norm(S)
        adopt = comp_adopter(where, gpu, iters, max(desc["d_k"], desc["d_v"]), rep, noise=noise)
        enc = W.encode_boundary(S, rank, iters, init, adopt=adopt)
        mag = np.abs(S) + np.abs(enc["Kc"]).T @ np.abs(enc["Uc"])
        dR = 2 * rank * 2.0 ** -24 * mag
        S = enc["R"]
    check_window_quant(where, S, gpu, rep, dR=dR)


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
