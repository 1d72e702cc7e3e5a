"""GPU parity of the STEP KDA path (per-key-row widths, channel-wise gates,
FP16 pivot rows, one shared column scale) against the oracle, teacher-forced."""
import json
import os

import numpy as np
import pytest

import quantized_recurrent_state_decode_amd as sq
from conftest import GOLDEN
from oracle import calibration as C
from synth import inputs as SI

from gpu_util import Pool, head_inputs, inputs_dev, oracle_warmup, to_dev
from parity import Report, check_decode_head, check_quantized_head, dequant_head, oracle_desc

pytestmark = pytest.mark.gpu


def _plan(rng, heads, dk, dv, choices=(2, 4, 6, 8, 16)):
    bits = rng.choice(choices, size=heads * dk)
    bits[:3] = 16                       # at least a few pivot rows
    w = C.impact_factors(rng.lognormal(0.0, 1.5, (heads, dk))).astype(np.float32)
    return sq.sq_plan_create_step(sq.SQ_KIND_KDA, heads, dk, dv, bits, w)


def _compare_steps(pool, w, slots, steps, tiles):
    import torch
    desc = oracle_desc(pool.desc)
    sdev = to_dev(slots.astype(np.int32))
    params = SI.gate_params(w)
    y = torch.empty((w.batch, w.heads, w.d_v), dtype=torch.float32, device="cuda")
    rep = Report()
    for t in range(steps):
        inp = SI.step_inputs(w, t, params)
        before = {b: pool.slot_bytes_of(int(slots[b])) for b, _ in tiles}
        pool.decode(sdev, w.batch, inputs_dev(inp), y)
        torch.cuda.synchronize()
        yh = y.cpu().numpy()
        for b, h in tiles:
            after = pool.slot_bytes_of(int(slots[b]))
            check_decode_head(f"step {t} b {b} h {h}", desc, h, pool.head_bytes(before[b], h),
                              pool.head_bytes(after, h), head_inputs(inp, b, h),
                              yh[b, h].astype(np.float64), pool.desc["w"][h].astype(np.float64),
                              rep)
    return rep


@pytest.mark.parametrize("shape", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_kda_decode_teacher_forced(shape):
    rng = np.random.default_rng(40 + shape[0])
    dk, dv = shape
    w = SI.workload("kda_step6", batch=5, n_slots=7, heads=3, d_k=dk, d_v=dv, steps=4)
    pool = Pool(_plan(rng, 3, dk, dv), 7)
    slots = SI.slot_ids(w)
    pool.pack(to_dev(slots), to_dev(oracle_warmup(w, 24).astype(np.float32)), w.batch)
    rep = _compare_steps(pool, w, slots, w.steps,
                         [(b, h) for b in range(w.batch) for h in range(w.heads)])
    print("adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()


def test_kda_quantize_only_and_unpack():
    import torch
    rng = np.random.default_rng(8)
    H = 4
    plan = _plan(rng, H, 128, 128)
    pool = Pool(plan, 3)
    desc = oracle_desc(pool.desc)
    n = 8
    X = (rng.standard_normal((n, 128, 128)) * rng.lognormal(0, 1.2, (n, 128, 1))
         * rng.lognormal(0, 1.2, (n, 1, 128))).astype(np.float32)
    heads = (np.arange(n) % H).astype(np.int32)
    mhb = sq.sq_max_head_bytes(plan)
    out = torch.zeros(n * mhb, dtype=torch.uint8, device="cuda")
    sq.sq_quantize_tiles(plan, pool.dev_plan, to_dev(X), n, to_dev(heads), out)
    torch.cuda.synchronize()
    ob = out.cpu().numpy().tobytes()
    rep = Report()
    for t in range(n):
        check_quantized_head(f"tile {t}", desc, int(heads[t]), X[t].astype(np.float64),
                             ob[t * mhb:(t + 1) * mhb],
                             pool.desc["w"][heads[t]].astype(np.float64), rep)
    rep.assert_ok()
    slots = to_dev(np.array([2, 0], dtype=np.int32))
    pool.pack(slots, to_dev(X.reshape(2, H, 128, 128)), 2)
    S = torch.empty((2, H, 128, 128), dtype=torch.float32, device="cuda")
    sq.sq_pool_unpack(plan, pool.dev_plan, pool.pool, 3, slots, 2, S)
    torch.cuda.synchronize()
    S = S.cpu().numpy()
    for b, slot in enumerate([2, 0]):
        buf = pool.slot_bytes_of(slot)
        for h in range(H):
            np.testing.assert_allclose(S[b, h], dequant_head(desc, h, pool.head_bytes(buf, h)),
                                       rtol=1e-6, atol=1e-30)


def test_full_size_kda_sampled():
    """The 256-request, 32-head KDA workload at full size with the calibrated
    allocation (rows in {4,6,8}, 1.4% FP16 rows), in the launch configuration
    the bench times: 3 steps, 24 sampled tiles compared on the last."""
    import torch
    with open(os.path.join(GOLDEN, "calib_kda_step6.json")) as f:
        st = json.load(f)
    stats = {"kind": 1, "heads": 32, "d_k": 128, "d_v": 128, "cand_bits": st["cand_bits"],
             "ell": np.array(st["ell"]), "dist": np.array(st["dist"]),
             "omega": np.array(st["omega"])}
    plan = sq.sq_calibrate_bits(stats, {"nominal_bits": 6.0, "pivot_frac": st["pivot_frac"]})
    w = SI.workload("kda_step6")
    pool = Pool(plan, w.n_slots)
    assert pool.desc["payload_bytes"] == 417024
    slots = SI.slot_ids(w)
    sdev = to_dev(slots)
    S = torch.zeros((w.batch, 32, 128, 128), dtype=torch.float32, device="cuda")
    y = torch.empty((w.batch, 32, 128), dtype=torch.float32, device="cuda")
    params = SI.gate_params(w)
    for t in range(16):
        d = inputs_dev(SI.warmup_inputs(w, t, params))
        sq.sq_dense_step(1, 32, 128, 128, S, w.batch, sdev, w.batch, d["q"], d["k"], d["v"],
                         d["beta"], d["gate"], y)
    pool.pack(sdev, S, w.batch)
    del S
    rng = np.random.default_rng(3)
    piv_heads = sorted(set(np.nonzero(pool.desc["unit_bits"] == 16)[0] // 128))
    sample = [(int(b), int(h)) for b, h in zip(rng.choice(w.batch, 20), rng.choice(32, 20))]
    sample += [(7, int(h)) for h in piv_heads[:4]]
    for t in range(2):
        pool.decode(sdev, w.batch, inputs_dev(SI.step_inputs(w, 100 + t, params)), y)
    w2 = SI.workload("kda_step6")
    rep = _compare_steps(pool, w2, slots, 1, sample)
    print("adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()


@pytest.mark.parametrize("shape", [(128, 128), (64, 128)])
def test_kda_single_width_blocks(shape):
    """Heads whose sorted rows fill whole 32-row blocks of one width (4 or 8
    bits, the blocks with their own read and code passes) beside mixed blocks,
    a 6-bit-only block and FP16 rows; all tiles teacher-forced on four steps,
    the last with a saturated value column (those blocks then take the
    clamping code pass after their own read)."""
    import torch
    dk, dv = shape
    rng = np.random.default_rng(90 + dk)
    runs = {128: [[(4, 64), (8, 64)], [(4, 40), (6, 56), (8, 32)], [(2, 8), (4, 24), (8, 93), (16, 3)]],
            64: [[(4, 32), (8, 32)], [(8, 32), (6, 32)], [(4, 30), (16, 2), (8, 32)]]}[dk]
    H = len(runs)
    bits = np.concatenate([rng.permutation(np.concatenate([np.full(n, b) for b, n in head]))
                           for head in runs]).astype(np.int32)
    assert bits.size == H * dk
    w8 = C.impact_factors(rng.lognormal(0.0, 1.5, (H, dk))).astype(np.float32)
    plan = sq.sq_plan_create_step(sq.SQ_KIND_KDA, H, dk, dv, bits, w8)
    w = SI.workload("kda_step6", batch=4, n_slots=5, heads=H, d_k=dk, d_v=dv, steps=4)
    pool = Pool(plan, 5)
    slots = SI.slot_ids(w)
    pool.pack(to_dev(slots), to_dev(oracle_warmup(w, 24).astype(np.float32)), w.batch)
    tiles = [(b, h) for b in range(w.batch) for h in range(H)]
    rep = _compare_steps(pool, w, slots, 3, tiles)
    print("adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()
    # a fourth step with a saturated value column on batch row 0
    desc = oracle_desc(pool.desc)
    inp = {k: v.copy() for k, v in SI.step_inputs(w, 3, SI.gate_params(w)).items()}
    inp["v"][0, :, 7] = 4.0e9
    sdev = to_dev(slots.astype(np.int32))
    y = torch.empty((w.batch, H, dv), dtype=torch.float32, device="cuda")
    before = {b: pool.slot_bytes_of(int(slots[b])) for b, _ in tiles}
    pool.decode(sdev, w.batch, inputs_dev(inp), y)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    rep = Report()
    for b, h in tiles:
        check_decode_head(f"saturated b {b} h {h}", desc, h, pool.head_bytes(before[b], h),
                          pool.head_bytes(pool.slot_bytes_of(int(slots[b])), h),
                          head_inputs(inp, b, h), yh[b, h].astype(np.float64),
                          pool.desc["w"][h].astype(np.float64), rep)
    print("saturated step: adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()


@pytest.mark.parametrize("shape", [(128, 128), (64, 128), (128, 64)])
def test_kda_extreme_heads(shape):
    """Heads at the extremes of the row widths: every row FP16 (the largest
    head, staged in more than one round at 128 x 128), every row 8 bits,
    every row 2 bits, and a head with a single integer row among FP16 rows;
    decode teacher-forced on three steps, then quantize-only and unpack."""
    import torch
    dk, dv = shape
    rng = np.random.default_rng(120 + dk + dv)
    one_int = np.full(dk, 16)
    one_int[dk // 2] = 4
    bits = np.concatenate([np.full(dk, 16), np.full(dk, 8), np.full(dk, 2), one_int]).astype(np.int32)
    H = 4
    w8 = C.impact_factors(rng.lognormal(0.0, 1.5, (H, dk))).astype(np.float32)
    plan = sq.sq_plan_create_step(sq.SQ_KIND_KDA, H, dk, dv, bits, w8)
    w = SI.workload("kda_step6", batch=3, n_slots=4, heads=H, d_k=dk, d_v=dv, steps=3)
    pool = Pool(plan, 4)
    slots = SI.slot_ids(w)
    pool.pack(to_dev(slots), to_dev(oracle_warmup(w, 16).astype(np.float32)), w.batch)
    rep = _compare_steps(pool, w, slots, w.steps, [(b, h) for b in range(w.batch) for h in range(H)])
    print("decode adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()
    # quantize-only of fresh tiles, and unpack of the pool against the oracle's dequantisation
    desc = oracle_desc(pool.desc)
    n = 8
    X = (rng.standard_normal((n, dk, dv)) * rng.lognormal(0, 1.0, (n, dk, 1))).astype(np.float32)
    heads = (np.arange(n) % H).astype(np.int32)
    mhb = sq.sq_max_head_bytes(plan)
    out = torch.zeros(n * mhb, dtype=torch.uint8, device="cuda")
    sq.sq_quantize_tiles(plan, pool.dev_plan, to_dev(X), n, to_dev(heads), out)
    torch.cuda.synchronize()
    ob = out.cpu().numpy().tobytes()
    rep = Report()
    wq = pool.desc["w"]
    for t in range(n):
        h = int(heads[t])
        check_quantized_head(f"tile {t}", desc, h, X[t].astype(np.float64),
                             ob[t * mhb:(t + 1) * mhb], wq[h].astype(np.float64), rep)
    print("quantize adoptions", dict(rep.count))
    rep.assert_ok()
    S_out = torch.empty((w.batch, H, dk, dv), dtype=torch.float32, device="cuda")
    sq.sq_pool_unpack(plan, pool.dev_plan, pool.pool, 4, to_dev(slots.astype(np.int32)), w.batch,
                      S_out)
    torch.cuda.synchronize()
    Sh = S_out.cpu().numpy()
    for b in range(w.batch):
        sb = pool.slot_bytes_of(int(slots[b]))
        for h in range(H):
            np.testing.assert_allclose(Sh[b, h], dequant_head(desc, h, pool.head_bytes(sb, h)),
                                       rtol=1e-6, atol=1e-30)
