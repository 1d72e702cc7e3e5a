"""GPU parity of the uniform and STEP GDN paths against the oracle.

Every compared step is teacher-forced (the oracle starts from the GPU's packed
bytes) and judged by the rules in tests/parity.py.  Sizes span several tiles,
a batch that is not a multiple of anything, pools larger than the batch, and
all code widths including FP16 pivot heads."""
import numpy as np
import pytest

import quantized_recurrent_state_decode_amd as sq
from oracle import calibration as C
from oracle import quantizers as Q
from oracle import recurrence as R
from synth import inputs as SI

from gpu_util import Pool, head_inputs, inputs_dev, oracle_warmup, to_dev
from parity import Report, check_decode_head, check_quantized_head, dequant_head, oracle_desc

pytestmark = pytest.mark.gpu


def _impact(rng, heads, d_k):
    return C.impact_factors(rng.lognormal(0.0, 1.5, (heads, d_k))).astype(np.float32)


def _run_teacher_forced(pool, w, slots, S0, steps, check_tiles=None, compare_steps=None):
    """Pack S0 into the slots, run `steps` decode steps and compare each
    compared step against the oracle, teacher-forced."""
    import torch
    desc = oracle_desc(pool.desc)
    wts = pool.desc["w"]
    slots_dev = to_dev(slots.astype(np.int32))
    pool.pack(slots_dev, to_dev(S0.astype(np.float32)), w.batch)
    params = SI.gate_params(w)
    rep = Report()
    y = torch.empty((w.batch, w.heads, w.d_v), dtype=torch.float32, device="cuda")
    tiles = check_tiles or [(b, h) for b in range(w.batch) for h in range(w.heads)]
    for t in range(steps):
        inp = SI.step_inputs(w, t, params)
        compare = compare_steps is None or t in compare_steps
        before = {b: pool.slot_bytes_of(int(slots[b])) for b, _ in tiles} if compare else None
        pool.decode(slots_dev, w.batch, inputs_dev(inp), y)
        if not compare:
            continue
        torch.cuda.synchronize()
        y_h = y.cpu().numpy()
        after = {b: pool.slot_bytes_of(int(slots[b])) for b, _ in tiles}
        for b, h in tiles:
            check_decode_head(f"step {t} b {b} h {h}", desc, h, pool.head_bytes(before[b], h),
                              pool.head_bytes(after[b], h), head_inputs(inp, b, h),
                              y_h[b, h].astype(np.float64),
                              None if wts is None else wts[h].astype(np.float64), rep)
    return rep


def test_tiny_uniform_int8_all_steps():
    """Batch 1, one 64 x 64 head, uniform INT8 rowwise, 256 steps, every step
    compared."""
    w = SI.workload("tiny_gdn_int8")
    pool = Pool(sq.sq_plan_create_uniform(1, 64, 64, 8), 1)
    S0 = oracle_warmup(w, w.warmup_steps)
    rep = _run_teacher_forced(pool, w, SI.slot_ids(w), S0, w.steps)
    print("adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()


@pytest.mark.parametrize("bits", [2, 4, 6, 8])
def test_uniform_widths_128(bits):
    w = SI.workload("tiny_gdn_int8", d_k=128, d_v=128, heads=3, batch=5, n_slots=8, steps=3)
    pool = Pool(sq.sq_plan_create_uniform(3, 128, 128, bits), 8)
    rep = _run_teacher_forced(pool, w, SI.slot_ids(w), oracle_warmup(w, 24), w.steps)
    rep.assert_ok()


def test_step_gdn_mixed_widths():
    """Heads at every width {2,4,6,8} plus FP16 pivot heads; half-lives
    log-uniform in [1, 4096]; 7 live slots in a pool of 11."""
    rng = np.random.default_rng(5)
    w = SI.workload("gdn_mid_step6", batch=7, n_slots=11, heads=6, steps=6)
    bits = [4, 16, 6, 8, 2, 4]
    plan = sq.sq_plan_create_step(sq.SQ_KIND_GDN, 6, 128, 128, bits, _impact(rng, 6, 128))
    pool = Pool(plan, 11)
    rep = _run_teacher_forced(pool, w, SI.slot_ids(w), oracle_warmup(w, 48), w.steps)
    print("adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()


@pytest.mark.parametrize("shape", [(64, 128), (128, 64)])
def test_step_gdn_rectangular(shape):
    rng = np.random.default_rng(9)
    dk, dv = shape
    w = SI.workload("gdn_mid_step6", batch=3, n_slots=3, heads=4, steps=3, d_k=dk, d_v=dv)
    plan = sq.sq_plan_create_step(sq.SQ_KIND_GDN, 4, dk, dv, [4, 6, 16, 8], _impact(rng, 4, dk))
    rep = _run_teacher_forced(Pool(plan, 3), w, SI.slot_ids(w), oracle_warmup(w, 16), w.steps)
    rep.assert_ok()


@pytest.mark.parametrize("mode", ["uniform", "step"])
def test_quantize_only_and_unpack(mode):
    """The quantizer alone on identical fp32 tiles (sq_quantize_tiles), and the
    dequantised state of sq_pool_unpack against the oracle's parse."""
    import torch
    rng = np.random.default_rng(21)
    H = 5
    if mode == "uniform":
        plan = sq.sq_plan_create_uniform(H, 128, 128, 6)
    else:
        plan = sq.sq_plan_create_step(sq.SQ_KIND_GDN, H, 128, 128, [2, 4, 6, 8, 16],
                                      _impact(rng, H, 128))
    pool = Pool(plan, 4)
    desc = oracle_desc(pool.desc)
    n = 2 * H
    X = (rng.standard_normal((n, 128, 128)) * rng.lognormal(0, 1, (n, 128, 1))
         * rng.lognormal(0, 1, (n, 1, 128))).astype(np.float32)
    X[3, 5, :] = 0.0                                    # an all-zero row
    heads = np.arange(n, dtype=np.int32) % H
    mhb = sq.sq_max_head_bytes(plan)
    out = torch.zeros(n * mhb, dtype=torch.uint8, device="cuda")
    sq.sq_quantize_tiles(plan, pool.dev_plan, to_dev(X), n, to_dev(heads), out)
    torch.cuda.synchronize()
    ob = out.cpu().numpy().tobytes()
    rep = Report()
    wts = pool.desc["w"]
    for t in range(n):
        check_quantized_head(f"tile {t}", desc, int(heads[t]), X[t].astype(np.float64),
                             ob[t * mhb:(t + 1) * mhb], None if wts is None else
                             wts[heads[t]].astype(np.float64), rep)
    rep.assert_ok()
    # pack two slots from X, unpack them, compare with the oracle's dequantisation
    slots = to_dev(np.array([3, 1], dtype=np.int32))
    pool.pack(slots, to_dev(X[:2 * H].reshape(2, H, 128, 128)), 2)
    S = torch.empty((2, H, 128, 128), dtype=torch.float32, device="cuda")
    sq.sq_pool_unpack(plan, pool.dev_plan, pool.pool, 4, slots, 2, S)
    torch.cuda.synchronize()
    S = S.cpu().numpy()
    for b, slot in enumerate([3, 1]):
        buf = pool.slot_bytes_of(slot)
        for h in range(H):
            ref = dequant_head(desc, h, pool.head_bytes(buf, h))
            np.testing.assert_allclose(S[b, h], ref, rtol=1e-6, atol=1e-30)


def test_beta_zero_is_pure_decay_and_recall():
    """beta = 0: X = alpha S_hat and y = (alpha S_hat)^T q.  beta = 1, |k| = 1,
    q = k: y = v for any stored state (associative recall)."""
    import torch
    rng = np.random.default_rng(2)
    H, B = 4, 3
    plan = sq.sq_plan_create_step(sq.SQ_KIND_GDN, H, 128, 128, [4, 6, 8, 16],
                                  _impact(rng, H, 128))
    pool = Pool(plan, B)
    desc = oracle_desc(pool.desc)
    slots = np.arange(B, dtype=np.int32)
    pool.pack(to_dev(slots), to_dev(rng.standard_normal((B, H, 128, 128)).astype(np.float32)), B)
    k = rng.standard_normal((B, H, 128))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((B, H, 128)).astype(np.float32)
    alpha = np.full((B, H), 0.9, np.float32)
    y = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    # beta = 0
    before = [pool.slot_bytes_of(s) for s in slots]
    inp = {"q": k, "k": k, "v": v, "beta": np.zeros((B, H), np.float32), "gate": alpha}
    pool.decode(to_dev(slots), B, inputs_dev(inp), y)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    for b in range(B):
        for h in range(H):
            S_hat = dequant_head(desc, h, pool.head_bytes(before[b], h))
            ref = R.readout(R.retained(S_hat, np.full(128, np.float64(np.float32(0.9)))),
                            k[b, h].astype(np.float64))
            assert np.linalg.norm(yh[b, h] - ref) <= 1e-5 * np.linalg.norm(ref)
    # associative recall
    inp = {"q": k, "k": k, "v": v, "beta": np.ones((B, H), np.float32), "gate": alpha}
    pool.decode(to_dev(slots), B, inputs_dev(inp), y)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    for b in range(B):
        for h in range(H):
            assert np.linalg.norm(yh[b, h] - v[b, h]) <= 1e-5 * np.linalg.norm(v[b, h])


def test_bad_slot_is_skipped_and_other_slots_untouched():
    import os
    import torch
    rng = np.random.default_rng(4)
    plan = sq.sq_plan_create_step(sq.SQ_KIND_GDN, 2, 128, 128, [4, 8], _impact(rng, 2, 128))
    pool = Pool(plan, 6)
    pool.pack(to_dev(np.arange(6, dtype=np.int32)),
              to_dev(rng.standard_normal((6, 2, 128, 128)).astype(np.float32)), 6)
    snap = pool.pool.cpu().numpy().copy()
    B = 3
    slots = np.array([4, 17, 1], dtype=np.int32)          # 17 is outside the pool
    inp = {"q": rng.standard_normal((B, 2, 128)).astype(np.float32),
           "k": rng.standard_normal((B, 2, 128)).astype(np.float32),
           "v": rng.standard_normal((B, 2, 128)).astype(np.float32),
           "beta": np.full((B, 2), 0.5, np.float32), "gate": np.full((B, 2), 0.9, np.float32)}
    y = torch.zeros((B, 2, 128), dtype=torch.float32, device="cuda")
    pool.decode(to_dev(slots), B, inputs_dev(inp), y)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.isnan(yh[1]).all() and np.isfinite(yh[0]).all() and np.isfinite(yh[2]).all()
    now = pool.pool.cpu().numpy()
    sb = pool.slot_bytes
    for s in (0, 2, 3, 5):
        assert np.array_equal(now[s * sb:(s + 1) * sb], snap[s * sb:(s + 1) * sb])
    assert not np.array_equal(now[4 * sb:5 * sb], snap[4 * sb:5 * sb])
    # with host validation the same call is refused before launching
    os.environ["SQ_VALIDATE"] = "1"
    try:
        with pytest.raises(sq.StepqError) as e:
            pool.decode(to_dev(slots), B, inputs_dev(inp), y)
        assert e.value.status == sq.SQ_ESLOT_RANGE
        with pytest.raises(sq.StepqError) as e:
            pool.decode(to_dev(np.array([1, 2, 1], np.int32)), B, inputs_dev(inp), y)
        assert e.value.status == sq.SQ_EDUP_SLOT
    finally:
        del os.environ["SQ_VALIDATE"]


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_dense_fp32_step(kind):
    """The FP32-state reference step against the float64 recurrence."""
    import torch
    w = (SI.workload("gdn_mid_step6", batch=5, n_slots=8, heads=3, steps=4) if kind == "gdn"
         else SI.workload("kda_step6", batch=5, n_slots=8, heads=3, steps=4))
    S0 = oracle_warmup(w, 8)
    slots = SI.slot_ids(w)
    S = np.zeros((w.n_slots, w.heads, 128, 128), np.float32)
    S[slots] = S0.astype(np.float32)
    S_dev = to_dev(S)
    ref = S[slots].astype(np.float64)
    y = torch.empty((w.batch, w.heads, 128), dtype=torch.float32, device="cuda")
    params = SI.gate_params(w)
    for t in range(w.steps):
        inp = SI.step_inputs(w, t, params)
        d = inputs_dev(inp)
        sq.sq_dense_step(0 if kind == "gdn" else 1, w.heads, 128, 128, S_dev, w.n_slots,
                         to_dev(slots), w.batch, d["q"], d["k"], d["v"], d["beta"], d["gate"], y)
        dvec = R.gate_vector(inp["gate"].astype(np.float64), kind, 128)
        ref, yr = R.dense_step(ref, inp["q"].astype(np.float64), inp["k"].astype(np.float64),
                               inp["v"].astype(np.float64), inp["beta"].astype(np.float64), dvec)
        torch.cuda.synchronize()
        yh = y.cpu().numpy()
        rel = np.linalg.norm(yh - yr, axis=-1) / np.linalg.norm(yr, axis=-1)
        assert rel.max() <= 1e-5
    Sh = S_dev.cpu().numpy()[slots]
    assert np.linalg.norm(Sh - ref) <= 1e-5 * np.linalg.norm(ref)


def _full_size_pool_sampled(plan, extra_tiles):
    """The 512-of-1024-slot, 48-head pool shape at full size, in the launch
    configuration the bench times: 8 fp32 dense warm-up steps on the GPU, pack,
    3 decode steps, 24 random tiles plus `extra_tiles` compared teacher-forced
    on the last."""
    import torch
    rng = np.random.default_rng(33)
    w = SI.workload("gdn_pool_step4")
    pool = Pool(plan, w.n_slots)
    slots = SI.slot_ids(w)
    # a state with the warm-up's scale: 8 fp32 dense steps on the GPU from S = 0
    S = torch.zeros((w.n_slots, 48, 128, 128), dtype=torch.float32, device="cuda")
    y = torch.empty((w.batch, 48, 128), dtype=torch.float32, device="cuda")
    sdev = to_dev(slots)
    params = SI.gate_params(w)
    for t in range(8):
        d = inputs_dev(SI.warmup_inputs(w, t, params))
        sq.sq_dense_step(0, 48, 128, 128, S, w.n_slots, sdev, w.batch, d["q"], d["k"], d["v"],
                         d["beta"], d["gate"], y)
    pool.pack(sdev, S[sdev.long()].contiguous(), w.batch)
    del S
    sample = [(int(b), int(h)) for b, h in zip(rng.choice(w.batch, 24), rng.choice(48, 24))]
    sample += extra_tiles
    desc = oracle_desc(pool.desc)
    wts = pool.desc["w"]
    for t in range(3):
        inp = SI.step_inputs(w, t, params)
        before = {b: pool.slot_bytes_of(int(slots[b])) for b, _ in sample} if t == 2 else None
        pool.decode(sdev, w.batch, inputs_dev(inp), y)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    rep = Report()
    for b, h in sample:
        after = pool.slot_bytes_of(int(slots[b]))
        check_decode_head(f"b {b} h {h}", desc, h, pool.head_bytes(before[b], h),
                          pool.head_bytes(after, h), head_inputs(inp, b, h),
                          yh[b, h].astype(np.float64),
                          None if wts is None else wts[h].astype(np.float64), rep)
    print("adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()


def test_full_size_gdn_pool_sampled():
    """Nominal 4-bit STEP at the pool shape, one split launch: the 45 4-bit
    heads in the width-specialised body, the two 2-bit heads and the FP16
    pivot head in the grid rows ahead of them."""
    rng = np.random.default_rng(34)
    bits = np.full(48, 4)
    bits[[5, 29]] = 2
    bits[17] = 16
    plan = sq.sq_plan_create_step(sq.SQ_KIND_GDN, 48, 128, 128, bits, _impact(rng, 48, 128))
    _full_size_pool_sampled(plan, [(3, 17), (100, 5), (511, 29)])


def test_full_size_uniform_int4_pool_sampled():
    """Uniform rowwise INT4 (the same-hardware baseline) at the pool shape."""
    _full_size_pool_sampled(sq.sq_plan_create_uniform(48, 128, 128, 4),
                            [(0, 0), (511, 47), (255, 20)])


def test_full_size_fp32_dense_pool_sampled():
    """The fp32 dense step (the other same-hardware baseline) at the pool
    shape, in place over the 1024-slot pool: 8 warm-up steps, then one step
    checked on sampled tiles against the float64 recurrence started from the
    GPU's state, and untouched slots checked unchanged."""
    import torch
    rng = np.random.default_rng(35)
    w = SI.workload("gdn_pool_fp32")
    slots = SI.slot_ids(w)
    S = torch.zeros((w.n_slots, 48, 128, 128), dtype=torch.float32, device="cuda")
    y = torch.empty((w.batch, 48, 128), dtype=torch.float32, device="cuda")
    sdev = to_dev(slots)
    params = SI.gate_params(w)
    for t in range(8):
        d = inputs_dev(SI.warmup_inputs(w, t, params))
        sq.sq_dense_step(0, 48, 128, 128, S, w.n_slots, sdev, w.batch, d["q"], d["k"], d["v"],
                         d["beta"], d["gate"], y)
    sample = [(int(b), int(h)) for b, h in zip(rng.choice(w.batch, 24), rng.choice(48, 24))]
    sample += [(0, 0), (511, 47)]
    torch.cuda.synchronize()
    before = {(b, h): S[int(slots[b]), h].cpu().numpy().astype(np.float64) for b, h in sample}
    idle = int(np.setdiff1d(np.arange(w.n_slots), slots)[0])
    idle_before = S[idle].cpu().numpy()
    inp = SI.step_inputs(w, 0, params)
    d = inputs_dev(inp)
    sq.sq_dense_step(0, 48, 128, 128, S, w.n_slots, sdev, w.batch, d["q"], d["k"], d["v"],
                     d["beta"], d["gate"], y)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    for b, h in sample:
        x = {k: inp[k][b, h].astype(np.float64) for k in ("q", "k", "v")}
        dvec = R.gate_vector(np.float64(inp["gate"][b, h]), "gdn", 128)
        ref, yr = R.dense_step(before[(b, h)][None], x["q"][None], x["k"][None], x["v"][None],
                               np.array([inp["beta"][b, h]], np.float64), dvec[None])
        got = S[int(slots[b]), h].cpu().numpy()
        assert np.linalg.norm(got - ref[0]) <= 1e-5 * np.linalg.norm(ref[0]), (b, h)
        assert np.linalg.norm(yh[b, h] - yr[0]) <= 1e-5 * np.linalg.norm(yr[0]), (b, h)
    assert np.array_equal(S[idle].cpu().numpy(), idle_before)


def _calibrated_plan(name):
    """The plan the bench builds for a workload: sq_calibrate_bits on the
    calibration statistics stored for it (written by the oracle)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", f"calib_{name}.json")) as f:
        st = json.load(f)
    stats = {"kind": 0 if st["kind"] == "gdn" else 1, "heads": st["heads"], "d_k": st["d_k"],
             "d_v": st["d_v"], "cand_bits": st["cand_bits"], "ell": np.array(st["ell"]),
             "dist": np.array(st["dist"]), "omega": np.array(st["omega"])}
    return sq.sq_calibrate_bits(stats, {"nominal_bits": st["nominal_bits"],
                                        "pivot_frac": st["pivot_frac"], "gamma": st["gamma"],
                                        "horizon": st["horizon"]})


def test_full_size_gdn_mid_all_tiles():
    """The mid workload at full size (64 slots x 16 heads, the calibrated
    nominal-6-bit plan: 4-, 6- and 8-bit heads and one FP16 head) in the launch
    configuration the bench times (every width class in one merged launch):
    8 fp32 dense warm-up steps on the GPU, pack, 6 decode steps, and every one
    of the 1,024 tiles compared teacher-forced on the first and the last."""
    import torch
    w = SI.workload("gdn_mid_step6", steps=6)
    plan = _calibrated_plan("gdn_mid_step6")
    pool = Pool(plan, w.n_slots)
    assert sorted(set(int(b) for b in pool.desc["unit_bits"])) == [4, 6, 8, 16]
    slots = SI.slot_ids(w)
    sdev = to_dev(slots)
    params = SI.gate_params(w)
    S = torch.zeros((w.n_slots, w.heads, 128, 128), dtype=torch.float32, device="cuda")
    y = torch.empty((w.batch, w.heads, 128), dtype=torch.float32, device="cuda")
    for t in range(8):
        d = inputs_dev(SI.warmup_inputs(w, t, params))
        sq.sq_dense_step(0, w.heads, 128, 128, S, w.n_slots, sdev, w.batch, d["q"], d["k"],
                         d["v"], d["beta"], d["gate"], y)
    S0 = S[sdev.long()].cpu().numpy().astype(np.float64)
    del S
    rep = _run_teacher_forced(pool, w, slots, S0, w.steps, compare_steps={0, w.steps - 1})
    print("adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()


def test_full_size_fp32_dense_kda_sampled():
    """The fp32 dense KDA step (the KDA workload's same-hardware baseline) at
    the KDA shape, 256 slots x 32 heads with per-row gates: 8 warm-up steps,
    then one step checked on sampled tiles against the float64 recurrence
    started from the GPU's state."""
    import torch
    rng = np.random.default_rng(36)
    w = SI.workload("kda_fp32")
    slots = SI.slot_ids(w)
    H = w.heads
    S = torch.zeros((w.n_slots, H, 128, 128), dtype=torch.float32, device="cuda")
    y = torch.empty((w.batch, H, 128), dtype=torch.float32, device="cuda")
    sdev = to_dev(slots)
    params = SI.gate_params(w)
    for t in range(8):
        d = inputs_dev(SI.warmup_inputs(w, t, params))
        sq.sq_dense_step(1, H, 128, 128, S, w.n_slots, sdev, w.batch, d["q"], d["k"], d["v"],
                         d["beta"], d["gate"], y)
    sample = [(int(b), int(h)) for b, h in zip(rng.choice(w.batch, 24), rng.choice(H, 24))]
    sample += [(0, 0), (w.batch - 1, H - 1)]
    torch.cuda.synchronize()
    before = {(b, h): S[int(slots[b]), h].cpu().numpy().astype(np.float64) for b, h in sample}
    inp = SI.step_inputs(w, 0, params)
    d = inputs_dev(inp)
    sq.sq_dense_step(1, H, 128, 128, S, w.n_slots, sdev, w.batch, d["q"], d["k"], d["v"],
                     d["beta"], d["gate"], y)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    for b, h in sample:
        x = {k: inp[k][b, h].astype(np.float64) for k in ("q", "k", "v")}
        dvec = R.gate_vector(inp["gate"][b, h].astype(np.float64), "kda", 128)
        ref, yr = R.dense_step(before[(b, h)][None], x["q"][None], x["k"][None], x["v"][None],
                               np.array([inp["beta"][b, h]], np.float64), dvec[None])
        got = S[int(slots[b]), h].cpu().numpy()
        assert np.linalg.norm(got - ref[0]) <= 1e-5 * np.linalg.norm(ref[0]), (b, h)
        assert np.linalg.norm(yh[b, h] - yr[0]) <= 1e-5 * np.linalg.norm(yr[0]), (b, h)


@pytest.mark.parametrize("case", ["one_width", "all_pivots", "split_fallback"])
def test_step_gdn_dispatch_paths(case):
    """The decode launch shapes a STEP GDN plan can take, teacher-forced:
    a plan of one width (its width-specialised kernel alone), a plan of FP16
    pivot heads only, and a plan whose largest class fills the chip many times
    over while the other classes' leading rows would exceed the grid's row
    limit (B + leading rows > 65535), which decodes the largest class alone
    and then the others in one merged launch."""
    import torch
    rng = np.random.default_rng(150)
    if case == "one_width":
        bits, B = [4] * 6, 7
    elif case == "all_pivots":
        bits, B = [16] * 3, 5
    else:
        bits, B = [4, 2, 6, 8, 16], 16384   # one head per class: 4 leading rows per batch row
    H = len(bits)
    w = SI.workload("gdn_mid_step6", batch=B, n_slots=B, heads=H, steps=1)
    plan = sq.sq_plan_create_step(sq.SQ_KIND_GDN, H, 128, 128, bits, _impact(rng, H, 128))
    pool = Pool(plan, B)
    slots = SI.slot_ids(w)
    S4 = oracle_warmup(SI.workload("gdn_mid_step6", batch=4, n_slots=4, heads=H), 16)
    S = to_dev(S4.astype(np.float32)).repeat(-(-B // 4), 1, 1, 1)[:B].contiguous()
    sdev = to_dev(slots.astype(np.int32))
    pool.pack(sdev, S, B)
    del S
    torch.cuda.empty_cache()
    tiles = [(b, h) for b in sorted({0, 1, B // 2, B - 1}) for h in range(H)]
    desc = oracle_desc(pool.desc)
    inp = SI.step_inputs(w, 0, SI.gate_params(w))
    y = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    before = {b: pool.slot_bytes_of(int(slots[b])) for b, _ in tiles}
    pool.decode(sdev, B, inputs_dev(inp), y)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    rep = Report()
    for b, h in tiles:
        check_decode_head(f"{case} b {b} h {h}", desc, h, pool.head_bytes(before[b], h),
                          pool.head_bytes(pool.slot_bytes_of(int(slots[b])), h),
                          head_inputs(inp, b, h), yh[b, h].astype(np.float64),
                          pool.desc["w"][h].astype(np.float64), rep)
    print(case, "adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()
    assert np.all(np.isfinite(yh))
