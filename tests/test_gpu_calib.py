"""GPU calibration statistics (STEPQuant Sec. 4, Eqs. 6-8; Sec. 4.1, App. B-C)
against the oracle: the per-step gate statistics (float64 on both sides), the
distortion of the library's own quantizer summed per unit, and the whole
statistics stream feeding sq_calibrate_bits."""
import numpy as np
import pytest

import quantized_recurrent_state_decode_amd as sq
from oracle import calibration as C
from oracle import quantizers as Q
from oracle import recurrence as R
from oracle.layout import parse_head
from synth import inputs as SI

from gpu_util import inputs_dev, to_dev
from parity import Report, check_quantized_head, oracle_desc

pytestmark = pytest.mark.gpu


def _zeros(shape):
    import torch
    return torch.zeros(shape, dtype=torch.float64, device="cuda")


@pytest.mark.parametrize("kind,d_k", [("gdn", 128), ("kda", 128), ("gdn", 64), ("kda", 64)])
def test_gate_stats_match_oracle(kind, d_k):
    """Sums over 6 steps of 3 sequences of log r (per unit) and g_i^2 with
    g = D (q - beta k (k . q)): float64 on both sides, so they agree to the
    order of the additions."""
    import torch
    w = SI.workload("gdn_mid_step6" if kind == "gdn" else "kda_step6", heads=4, d_k=d_k,
                    d_v=d_k, calib_seqs=3)
    params = SI.gate_params(w)
    U = w.heads if kind == "gdn" else w.heads * d_k
    ls, om = _zeros(U), _zeros((w.heads, d_k))
    ref_ls, ref_om = np.zeros(U), np.zeros((w.heads, d_k))
    kid = sq.SQ_KIND_GDN if kind == "gdn" else sq.SQ_KIND_KDA
    for t in range(6):
        inp = SI.calib_inputs(w, t, params)
        d = inputs_dev(inp)
        sq.sq_calib_gate_stats(kid, w.heads, d_k, 3, d["q"], d["k"], d["beta"], d["gate"], ls, om)
        x = {k: v.astype(np.float64) for k, v in inp.items()}
        ref_ls += np.log(x["gate"]).sum(0).reshape(-1)
        g = R.transported_query(x["q"], x["k"], x["beta"], R.gate_vector(x["gate"], kind, d_k))
        ref_om += (g * g).sum(0)
    torch.cuda.synchronize()
    np.testing.assert_allclose(ls.cpu().numpy(), ref_ls, rtol=1e-12, atol=0)
    np.testing.assert_allclose(om.cpu().numpy(), ref_om, rtol=1e-10, atol=0)


@pytest.mark.parametrize("bits", [2, 4, 6, 8])
def test_distortion_of_packed_heads(bits):
    """The library's quantizer packs n x H tiles at width b (checked
    teacher-forced against the oracle), and the distortion kernel's per-unit
    sums equal the float64 squared error of those packed heads against the
    tiles, per head and per key row."""
    import torch
    rng = np.random.default_rng(60 + bits)
    H, n, d = 3, 2, 128
    S = (rng.standard_normal((n, H, d, d)) * rng.lognormal(0, 1, (n, H, d, 1))
         * rng.lognormal(0, 0.5, (n, H, 1, d))).astype(np.float32)
    wts = C.impact_factors(rng.lognormal(0, 1.5, (H, d))).astype(np.float32)
    plan = sq.sq_plan_create_step(sq.SQ_KIND_GDN, H, d, d, np.full(H, bits), wts)
    dp = sq.device_plan(plan)
    mhb = sq.sq_max_head_bytes(plan)
    packed = torch.zeros(n * H * mhb, dtype=torch.uint8, device="cuda")
    Sd = to_dev(S)
    per_head, per_row = _zeros(H), _zeros(H * d)
    sq.sq_calib_distortion(plan, dp, n, Sd, packed, False, per_head)
    sq.sq_calib_distortion(plan, dp, n, Sd, packed, True, per_row)
    torch.cuda.synchronize()
    desc = oracle_desc(sq.sq_plan_query(plan))
    buf = packed.cpu().numpy().tobytes()
    rep = Report()
    ref_row = np.zeros((H, d))
    for t in range(n * H):
        h = t % H
        head = buf[t * mhb:(t + 1) * mhb]
        check_quantized_head(f"tile {t}", desc, h, S[t // H, h].astype(np.float64), head,
                             wts[h].astype(np.float64), rep)
        st = parse_head(desc, h, head)
        Xh = Q.dequant_step(st["z"], st["r"], st["c"], np.full(d, bits), st["h"])
        E = Xh - S[t // H, h].astype(np.float64)
        ref_row[h] += (E * E).sum(-1)
    rep.assert_ok()
    np.testing.assert_allclose(per_row.cpu().numpy().reshape(H, d), ref_row, rtol=1e-10)
    np.testing.assert_allclose(per_head.cpu().numpy(), ref_row.sum(-1), rtol=1e-10)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_statistics_stream_feeds_calibration(kind):
    """The oracle's two-pass statistics (pass 1: ell and omega over the stream,
    w from omega; pass 2: d_u(b) on snapshots of the unquantised recurrence at
    each candidate width) computed on the GPU: gate statistics per step, the
    fp32 dense step for the trajectory, the library's quantizer at each width
    for the distortion.  Compared with the oracle on the same inputs and the
    GPU's own snapshots: ell and omega to float64 summation order, d_u(b)
    within 1e-4 relative (the fp32 quantizer may take the other side of a
    rounding tie, which moves a unit's error by a hair), and the allocation
    sq_calibrate_bits makes from the GPU statistics equals the oracle
    allocator's from the oracle statistics."""
    import torch
    H, d, n, steps, start, every = 4, 128, 2, 40, 8, 16
    cand = (4, 6, 8)
    w = SI.workload("gdn_mid_step6" if kind == "gdn" else "kda_step6", heads=H, calib_seqs=n)
    params = SI.gate_params(w)
    kid = sq.SQ_KIND_GDN if kind == "gdn" else sq.SQ_KIND_KDA
    U = H if kind == "gdn" else H * d
    inputs = [SI.calib_inputs(w, t, params) for t in range(steps)]
    # pass 1
    ls, om = _zeros(U), _zeros((H, d))
    for inp in inputs:
        dv = inputs_dev(inp)
        sq.sq_calib_gate_stats(kid, H, d, n, dv["q"], dv["k"], dv["beta"], dv["gate"], ls, om)
    torch.cuda.synchronize()
    ell = ls.cpu().numpy() / (steps * n)
    omega = om.cpu().numpy() / (steps * n)
    wts = sq.sq_impact_factors(omega)
    ref_ls, ref_om = np.zeros(U), np.zeros((H, d))
    for inp in inputs:
        x = {k: v.astype(np.float64) for k, v in inp.items()}
        ref_ls += np.log(x["gate"]).sum(0).reshape(-1)
        g = R.transported_query(x["q"], x["k"], x["beta"], R.gate_vector(x["gate"], kind, d))
        ref_om += (g * g).sum(0)
    np.testing.assert_allclose(ell, ref_ls / (steps * n), rtol=1e-12)
    np.testing.assert_allclose(omega, ref_om / (steps * n), rtol=1e-10)
    np.testing.assert_allclose(wts, C.impact_factors(ref_om / (steps * n)), rtol=2e-7)
    # pass 2
    plans = [sq.sq_plan_create_step(sq.SQ_KIND_GDN, H, d, d, np.full(H, b), wts) for b in cand]
    dps = [sq.device_plan(p) for p in plans]
    mhb = max(sq.sq_max_head_bytes(p) for p in plans)
    packed = torch.zeros(n * H * mhb, dtype=torch.uint8, device="cuda")
    dist = [_zeros(U) for _ in cand]
    S = torch.zeros((n, H, d, d), dtype=torch.float32, device="cuda")
    ident = torch.arange(n, dtype=torch.int32, device="cuda")
    y = torch.empty((n, H, d), dtype=torch.float32, device="cuda")
    ref_dist = np.zeros((U, len(cand)))
    n_snap = 0
    for t, inp in enumerate(inputs):
        dv = inputs_dev(inp)
        sq.sq_dense_step(kid, H, d, d, S, n, ident, n, dv["q"], dv["k"], dv["v"], dv["beta"],
                         dv["gate"], y)
        done = t + 1
        if done > start and (done - start) % every == 0:
            n_snap += 1
            for ci, b in enumerate(cand):
                sq.sq_calib_distortion(plans[ci], dps[ci], n, S, packed, kind == "kda", dist[ci])
            Sh = S.cpu().numpy().astype(np.float64)
            for ci, b in enumerate(cand):
                enc = Q.quantize_step(Sh, wts.astype(np.float64)[None], np.full(Sh.shape[:-1], b))
                E = Q.dequant_step(enc["z"], enc["r"], enc["c"], np.full(Sh.shape[:-1], b),
                                   enc["h"]) - Sh
                e2 = (E * E).sum(-1)
                per = e2.sum(-1) if kind == "gdn" else e2
                ref_dist[:, ci] += per.mean(0).reshape(-1)
    torch.cuda.synchronize()
    gdist = np.stack([dd.cpu().numpy() for dd in dist], axis=1) / (n * n_snap)
    ref_dist /= n_snap
    assert n_snap == 2
    np.testing.assert_allclose(gdist, ref_dist, rtol=1e-4)
    stats = {"kind": kid, "heads": H, "d_k": d, "d_v": d, "cand_bits": list(cand),
             "ell": ell, "dist": gdist, "omega": omega}
    opts = {"nominal_bits": 6.0, "pivot_frac": 0.02}
    got = sq.sq_plan_query(sq.sq_calibrate_bits(stats, opts))["unit_bits"]
    ora = C.allocate(kind, H, d, d, ref_ls / (steps * n), ref_dist, ref_om / (steps * n), cand,
                     6.0, 0.02)
    np.testing.assert_array_equal(got, ora["bits"])
