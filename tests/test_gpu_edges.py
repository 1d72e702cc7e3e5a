"""Edge cases of the GPU path: a slot id outside the pool on the KDA and window
kernels (its outputs are NaN, no slot but the valid ones changes, and the
valid tiles still match the oracle teacher-forced), empty batches on every
entry point, and all-zero tiles, where every FP16 scale sits at its clamp
(STEPQuant App. B.5: scales clamped to [2^-14, 65504]) and every code is 0."""
import numpy as np
import pytest

import quantized_recurrent_state_decode_amd as sq
from oracle import calibration as C
from synth import inputs as SI

from gpu_util import Pool, head_inputs, inputs_dev, oracle_warmup, to_dev
from parity import Report, check_decode_head, check_quantized_head, oracle_desc

pytestmark = pytest.mark.gpu


def _kda_plan(rng, heads, d):
    bits = rng.choice((2, 4, 6, 8, 16), size=heads * d)
    w = C.impact_factors(rng.lognormal(0.0, 1.5, (heads, d))).astype(np.float32)
    return sq.sq_plan_create_step(sq.SQ_KIND_KDA, heads, d, d, bits, w)


def _bad_slot_case(pool, w, rng):
    """Decode one step with slots [4, n_slots + 11, 1]; returns the inputs,
    outputs and pool bytes before and after."""
    import torch
    S0 = oracle_warmup(w, 12).astype(np.float32)
    pool.pack(to_dev(np.arange(w.batch, dtype=np.int32)), to_dev(S0), w.batch)
    before = pool.pool.cpu().numpy().copy()
    slots = np.array([4, pool.n_slots + 11, 1], dtype=np.int32)
    inp = SI.step_inputs(w, 0, SI.gate_params(w))
    inp = {k: np.ascontiguousarray(v[:3]) for k, v in inp.items()}
    y = torch.zeros((3, w.heads, w.d_v), dtype=torch.float32, device="cuda")
    pool.decode(to_dev(slots), 3, inputs_dev(inp), y)
    torch.cuda.synchronize()
    return slots, inp, y.cpu().numpy(), before, pool.pool.cpu().numpy()


@pytest.mark.parametrize("mode", ["kda", "window"])
def test_bad_slot_is_skipped(mode):
    rng = np.random.default_rng(91)
    if mode == "kda":
        w = SI.workload("kda_step6", batch=6, n_slots=6, heads=3)
        plan = _kda_plan(rng, 3, 128)
    else:
        w = SI.workload("gdn_window16", batch=6, n_slots=6, heads=3)
        plan = sq.sq_plan_create_window(3, 128, 128, 16)
    pool = Pool(plan, 6)
    slots, inp, yh, before, after = _bad_slot_case(pool, w, rng)
    assert np.isnan(yh[1]).all() and np.isfinite(yh[0]).all() and np.isfinite(yh[2]).all()
    sb = pool.slot_bytes
    for s in (0, 2, 3, 5):
        assert np.array_equal(after[s * sb:(s + 1) * sb], before[s * sb:(s + 1) * sb])
    desc = oracle_desc(pool.desc)
    rep = Report()
    for b in (0, 2):
        s = int(slots[b])
        for h in range(w.heads):
            check_decode_head(f"b {b} h {h}", desc, h,
                              pool.head_bytes(before[s * sb:(s + 1) * sb].tobytes(), h),
                              pool.head_bytes(after[s * sb:(s + 1) * sb].tobytes(), h),
                              head_inputs(inp, b, h), yh[b, h].astype(np.float64),
                              None if pool.desc["w"] is None else pool.desc["w"][h].astype(np.float64),
                              rep)
    rep.assert_ok()


@pytest.mark.parametrize("mode", ["uniform", "gdn", "kda", "window"])
def test_empty_batch_is_a_noop(mode):
    """B = 0 on decode, pack, unpack and (window) flush: no launch, no error,
    the pool unchanged."""
    import torch
    rng = np.random.default_rng(92)
    if mode == "uniform":
        plan = sq.sq_plan_create_uniform(2, 64, 64, 8)
    elif mode == "gdn":
        plan = sq.sq_plan_create_step(sq.SQ_KIND_GDN, 2, 64, 64, [4, 16],
                                      C.impact_factors(rng.lognormal(0, 1, (2, 64))).astype(np.float32))
    elif mode == "kda":
        plan = _kda_plan(rng, 2, 64)
    else:
        plan = sq.sq_plan_create_window(2, 64, 64, 4)
    pool = Pool(plan, 3)
    S = to_dev(rng.standard_normal((3, 2, 64, 64)).astype(np.float32))
    pool.pack(to_dev(np.arange(3, dtype=np.int32)), S, 3)
    snap = pool.pool.cpu().numpy().copy()
    none = torch.zeros(0, dtype=torch.int32, device="cuda")
    z = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda")
    gate = z(0, 2, 64) if mode == "kda" else z(0, 2)
    y = z(0, 2, 64)
    sq.sq_decode_step(pool.plan, pool.dev_plan, pool.pool, 3, none, 0, z(0, 2, 64), z(0, 2, 64),
                      z(0, 2, 64), z(0, 2), gate, y)
    pool.pack(none, z(0, 2, 64, 64), 0)
    sq.sq_pool_unpack(pool.plan, pool.dev_plan, pool.pool, 3, none, 0, z(0, 2, 64, 64))
    if mode == "window":
        sq.sq_window_flush(pool.plan, pool.dev_plan, pool.pool, 3, none, 0)
    torch.cuda.synchronize()
    assert np.array_equal(pool.pool.cpu().numpy(), snap)


@pytest.mark.parametrize("kind", ["gdn", "kda", "uniform", "window", "window_r2"])
def test_zero_tiles_quantize(kind):
    """All-zero tiles: m_i = 0, so r_i and c0_j clamp to 2^-14, every code is
    0, D_j = 0 keeps c_j = c0_j, and FP16 pivot units store zeros; checked
    against the oracle decision by decision."""
    import torch
    rng = np.random.default_rng(93)
    H, d, n = 3, 128, 6
    wts = C.impact_factors(rng.lognormal(0, 1.5, (H, d))).astype(np.float32)
    if kind == "gdn":
        plan = sq.sq_plan_create_step(sq.SQ_KIND_GDN, H, d, d, [4, 16, 8], wts)
    elif kind == "kda":
        plan = _kda_plan(rng, H, d)
        wts = sq.sq_plan_query(plan)["w"].astype(np.float32)
    elif kind == "uniform":       # every row scale clamps to 2^-14, every code 0
        plan = sq.sq_plan_create_uniform(H, d, d, 8)
    elif kind == "window":        # C at its floor, B_j = 0 and column codes 0
        plan = sq.sq_plan_create_window(H, d, d, 16)
    else:                         # and the pair fit of a zero state gives zero pairs
        plan = sq.sq_plan_create_window_lowrank(H, d, d, 16, 2, 3)
    pool = Pool(plan, 2)
    desc = oracle_desc(pool.desc)
    X = np.zeros((n, d, d), dtype=np.float32)
    X[n - 1, 5, 7] = 3.0          # one tile with a single non-zero element
    heads = (np.arange(n) % H).astype(np.int32)
    mhb = sq.sq_max_head_bytes(plan)
    out = torch.full((n * mhb,), 0xAB, dtype=torch.uint8, device="cuda")
    sq.sq_quantize_tiles(plan, pool.dev_plan, to_dev(X), n, to_dev(heads), out)
    torch.cuda.synchronize()
    ob = out.cpu().numpy().tobytes()
    rep = Report()
    for t in range(n):
        h = int(heads[t])
        check_quantized_head(f"tile {t}", desc, h, X[t].astype(np.float64),
                             ob[t * mhb:(t + 1) * mhb], wts[h].astype(np.float64), rep)
    rep.assert_ok()
