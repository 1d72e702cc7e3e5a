"""Kernel branches that ordinary inputs never reach, checked teacher-forced
against the oracle.

* Saturated column scale.  STEPQuant App. B.5 clamps every FP16 scale to
  [2^-14, 65504].  When a column's largest |X_ij| / r_i exceeds 65504 the
  initial column scale saturates and codes beyond +-q_b are clamped; the GDN
  and KDA kernels then take their clamping code path.  A value column of
  magnitude 4e9 in v puts beta k_i e_j far beyond 65504 r_i in every row.
* Zero retention.  alpha = 0 (GDN) or d_i = 0 (KDA key rows) removes the
  reconstructed state, X = beta k v^T on those rows (STEPQuant Sec. 3,
  Eq. 1 with D_t = 0); the kernels keep the division by the retained row
  factor finite for it.
* FP16 pivot values beyond the binary16 range round to infinity on both
  sides (pivots store FP16(X) without a clamp, STEPQuant Sec. 4).
"""
import numpy as np
import pytest

import quantized_recurrent_state_decode_amd as sq
from oracle import calibration as C
from oracle import quantizers as Q
from oracle import recurrence as R
from oracle.layout import parse_head
from synth import inputs as SI

from gpu_util import Pool, head_inputs, inputs_dev, oracle_warmup, to_dev
from parity import Report, check_decode_head, oracle_desc, row_bits_of

pytestmark = pytest.mark.gpu

HUGE = 4.0e9


def _impact(rng, heads, d_k):
    return C.impact_factors(rng.lognormal(0.0, 1.5, (heads, d_k))).astype(np.float32)


def _decode_and_check(pool, w, slots, inp, tiles):
    """One decode step with the given inputs; every listed tile checked
    teacher-forced.  Returns the parsed heads after the step, the readouts
    and the oracle's unrounded initial column scales of each tile."""
    import torch
    desc = oracle_desc(pool.desc)
    sdev = to_dev(slots.astype(np.int32))
    y = torch.empty((w.batch, w.heads, w.d_v), dtype=torch.float32, device="cuda")
    need = sorted(set(b for b, _ in tiles))
    before = {b: pool.slot_bytes_of(int(slots[b])) for b in need}
    pool.decode(sdev, w.batch, inputs_dev(inp), y)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    after = {b: pool.slot_bytes_of(int(slots[b])) for b in need}
    rep = Report()
    parsed, pre_c0 = {}, {}
    wts = pool.desc["w"]
    for b, h in tiles:
        x = head_inputs(inp, b, h)
        check_decode_head(f"b {b} h {h}", desc, h, pool.head_bytes(before[b], h),
                          pool.head_bytes(after[b], h), x, yh[b, h].astype(np.float64),
                          wts[h].astype(np.float64), rep)
        parsed[(b, h)] = parse_head(desc, h, pool.head_bytes(after[b], h))
        st = parse_head(desc, h, pool.head_bytes(before[b], h))
        rb = row_bits_of(desc, h)
        X = R.delta_update(R.retained(Q.dequant_step(st["z"], st["r"], st["c"], rb, st["h"]),
                                      R.gate_vector(x["gate"], desc["kind"], w.d_k)),
                           x["k"], x["v"], x["beta"])
        _, r = Q.step_row_scales(X, wts[h].astype(np.float64), rb)
        pre_c0[(b, h)] = Q.step_col_init(X, r, rb)[0]
    print("adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()
    return parsed, yh, pre_c0


def _gdn_case(batch, heads_bits, seed):
    rng = np.random.default_rng(seed)
    H = len(heads_bits)
    w = SI.workload("gdn_mid_step6", batch=batch, n_slots=batch, heads=H, steps=1)
    plan = sq.sq_plan_create_step(sq.SQ_KIND_GDN, H, 128, 128, heads_bits, _impact(rng, H, 128))
    pool = Pool(plan, batch)
    slots = SI.slot_ids(w)
    S0 = oracle_warmup(SI.workload("gdn_mid_step6", batch=min(batch, 4), n_slots=min(batch, 4),
                                   heads=H), 16)
    S = to_dev(S0.astype(np.float32)).repeat(-(-batch // len(S0)), 1, 1, 1)[:batch].contiguous()
    pool.pack(to_dev(slots), S, batch)
    inp = SI.step_inputs(w, 0, SI.gate_params(w))
    return w, pool, slots, {k: v.copy() for k, v in inp.items()}, rng


@pytest.mark.parametrize("batch", [4, 512])
def test_saturated_column_gdn(batch):
    """A 4e9 value column on batch rows 0 and 1: every width (2, 4, 6, 8 bits)
    and the FP16 pivot head.  At batch 512 the 32 four-bit heads make a class
    of 16,384 tiles, so the decode runs the split launch and the 4-bit tiles
    the width-specialised body; at batch 4 every class shares one launch."""
    bits = [2, 4, 6, 8, 16] + ([4] * 31 if batch == 512 else [])
    w, pool, slots, inp, rng = _gdn_case(batch, bits, 70 + batch)
    inp["v"][0, :, 5] = HUGE
    inp["v"][1, :, 77] = -HUGE
    tiles = [(b, h) for b in (0, 1, 2) for h in range(5)] + [(batch - 1, len(bits) - 1)]
    parsed, _, pre_c0 = _decode_and_check(pool, w, slots, inp, tiles)
    for h in range(4):          # the column scale saturated and codes hit the clamp
        assert pre_c0[(0, h)][5] > 65504.0 and pre_c0[(1, h)][77] > 65504.0
        qb = 2 ** (bits[h] - 1) - 1
        assert np.abs(parsed[(0, h)]["z"][:, 5]).max() == qb
        assert np.abs(parsed[(1, h)]["z"][:, 77]).max() == qb
    # the pivot head holds infinities where |X| exceeds the binary16 range
    assert np.isinf(parsed[(0, 4)]["h"][:, 5]).any()


def test_saturated_column_kda():
    """KDA rows of every width and FP16 pivot rows sharing one saturated
    column scale."""
    rng = np.random.default_rng(75)
    H, d = 3, 128
    row_bits = rng.choice((2, 4, 6, 8, 16), size=H * d)
    row_bits[:5] = 16
    plan = sq.sq_plan_create_step(sq.SQ_KIND_KDA, H, d, d, row_bits, _impact(rng, H, d))
    w = SI.workload("kda_step6", batch=3, n_slots=3, heads=H, steps=1)
    pool = Pool(plan, 3)
    slots = SI.slot_ids(w)
    pool.pack(to_dev(slots), to_dev(oracle_warmup(w, 16).astype(np.float32)), 3)
    inp = {k: v.copy() for k, v in SI.step_inputs(w, 0, SI.gate_params(w)).items()}
    inp["v"][0, :, 9] = HUGE
    inp["v"][1, :, 100] = -HUGE
    _, _, pre_c0 = _decode_and_check(pool, w, slots, inp,
                                     [(b, h) for b in range(3) for h in range(H)])
    for h in range(H):
        assert pre_c0[(0, h)][9] > 65504.0 and pre_c0[(1, h)][100] > 65504.0


def test_zero_retention_gdn():
    """alpha = 0 on batch rows 0 and 2 (every width and the pivot head): the
    state is replaced by the write term beta k v^T."""
    w, pool, slots, inp, rng = _gdn_case(4, [2, 4, 6, 8, 16], 80)
    inp["gate"][0, :] = 0.0
    inp["gate"][2, :] = 0.0
    _, yh, _ = _decode_and_check(pool, w, slots, inp, [(b, h) for b in range(4) for h in range(5)])
    # with nothing retained the readout is (k . q) beta v exactly in the reals
    for h in range(5):
        ref = float(np.dot(inp["k"][0, h].astype(np.float64), inp["q"][0, h])) \
            * float(inp["beta"][0, h]) * inp["v"][0, h].astype(np.float64)
        assert np.linalg.norm(yh[0, h] - ref) <= 1e-5 * np.linalg.norm(ref)


def test_zero_retention_kda():
    """d_i = 0 on every third key row of one tile and on every row of
    another, beside ordinary rows; pivot rows included."""
    rng = np.random.default_rng(85)
    H, d = 3, 128
    row_bits = rng.choice((2, 4, 6, 8, 16), size=H * d)
    row_bits[:4] = 16
    plan = sq.sq_plan_create_step(sq.SQ_KIND_KDA, H, d, d, row_bits, _impact(rng, H, d))
    w = SI.workload("kda_step6", batch=3, n_slots=3, heads=H, steps=1)
    pool = Pool(plan, 3)
    slots = SI.slot_ids(w)
    pool.pack(to_dev(slots), to_dev(oracle_warmup(w, 16).astype(np.float32)), 3)
    inp = {k: v.copy() for k, v in SI.step_inputs(w, 0, SI.gate_params(w)).items()}
    inp["gate"][0, :, ::3] = 0.0
    inp["gate"][1, 2, :] = 0.0
    _decode_and_check(pool, w, slots, inp, [(b, h) for b in range(3) for h in range(H)])
