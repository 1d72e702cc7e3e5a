"""GPU parity at full size on exactly what bench.py times.

Each workload is built the way bench.py builds it: the plan from bench._plan
(sq_calibrate_bits on the stored calibration statistics for the STEP
workloads), the initial state from bench.build_state (128 fp32 dense warm-up
steps on the GPU from S = 0, then sq_pool_pack), and decode step t reading
input set t % 8 as the bench's timed loop does.  The decode then runs the
workload's whole step count in the launch configuration the bench times, and
on eight of those steps (the first, the last and steps between them; for the
window path the tokens around the first two rebuilds) at least 64 tiles are
compared teacher-forced against the oracle (every tile for the mid
workload), among them every FP16 pivot head, every 2-bit head and, for KDA,
every head that holds FP16 pivot rows.

A free-running comparison is reported beside it, not gated: the oracle runs
on its own from the same packed start, and the readouts drift apart as soon
as one rounding tie is taken differently (STEPQuant Proposition 1: an error
propagates through A_t).
"""
import numpy as np
import pytest

import bench
import quantized_recurrent_state_decode_amd as sq
from oracle import recurrence as R
from oracle import step as ST
from oracle import window as W
from oracle.layout import parse_head
from synth import inputs as SI

from gpu_util import Pool, head_inputs, inputs_dev, to_dev
from parity import Report, check_decode_head, oracle_desc, row_bits_of

pytestmark = pytest.mark.gpu

N_SETS = 8          # bench.py's --input-sets default: step t reads set t % 8


def _setup(name):
    w = SI.workload(name)
    plan = bench._plan(sq, w)
    pool = Pool(plan, w.n_slots)
    slots = SI.slot_ids(w)
    sdev = to_dev(slots)
    contrast = bench.build_state(sq, w, [{"plan": plan, "dev_plan": pool.dev_plan,
                                          "pool": pool.pool}], sdev, w.warmup_steps)
    params = SI.gate_params(w)
    sets = [SI.step_inputs(w, i, params) for i in range(N_SETS)]
    return w, pool, slots, sdev, sets, contrast


def _run(w, pool, slots, sdev, sets, tiles, compare_steps, track=()):
    """All w.steps decode steps; teacher-forced checks of `tiles` on the
    compare steps; the readouts of the `track` tiles at every step, and their
    packed bytes before the first step."""
    import torch
    desc = oracle_desc(pool.desc)
    wts = pool.desc["w"]
    devsets = [inputs_dev(s) for s in sets]
    y = torch.empty((w.batch, w.heads, w.d_v), dtype=torch.float32, device="cuda")
    rep = Report()
    need = sorted(set(b for b, _ in tiles))
    start = {(b, h): pool.head_bytes(pool.slot_bytes_of(int(slots[b])), h) for b, h in track}
    tb = torch.tensor([b for b, _ in track], dtype=torch.long, device="cuda")
    th = torch.tensor([h for _, h in track], dtype=torch.long, device="cuda")
    hist = []
    for t in range(w.steps):
        cmp = t in compare_steps
        before = {b: pool.slot_bytes_of(int(slots[b])) for b in need} if cmp else None
        pool.decode(sdev, w.batch, devsets[t % N_SETS], y)
        if track:
            hist.append(y[tb, th].clone())
        if not cmp:
            continue
        torch.cuda.synchronize()
        yh = y.cpu().numpy()
        after = {b: pool.slot_bytes_of(int(slots[b])) for b in need}
        inp = sets[t % N_SETS]
        for b, h in tiles:
            check_decode_head(f"step {t} b {b} h {h}", desc, h, pool.head_bytes(before[b], h),
                              pool.head_bytes(after[b], h), head_inputs(inp, b, h),
                              yh[b, h].astype(np.float64),
                              None if wts is None else wts[h].astype(np.float64), rep)
    hist = torch.stack(hist).cpu().numpy() if track else None
    return rep, start, hist


def _free_running(w, pool, sets, track, start, hist, upto):
    """The oracle on its own from the packed start of each tracked tile:
    relative readout difference to the GPU at each step (max over tiles)."""
    desc = oracle_desc(pool.desc)
    wts = pool.desc["w"]
    states = {bh: parse_head(desc, bh[1], start[bh]) for bh in track}
    rel = []
    for t in range(upto):
        inp = sets[t % N_SETS]
        worst = 0.0
        for n, (b, h) in enumerate(track):
            x = head_inputs(inp, b, h)
            st = states[(b, h)]
            if desc["mode"] == "window":
                r = W.window_step(st, x["q"], x["k"], x["v"], x["beta"], float(x["gate"]),
                                  int(desc["p"]), int(desc.get("iters", 0)))
                yo, states[(b, h)] = r["o"], r["state"]
            else:
                dvec = R.gate_vector(x["gate"], desc.get("kind", "gdn"), w.d_k)
                r = ST.step_step(st, x, wts[h].astype(np.float64), row_bits_of(desc, h), dvec)
                yo = r["y"]
                states[(b, h)] = {k: r["new"][k] for k in ("z", "r", "c", "h")}
            worst = max(worst, float(np.linalg.norm(hist[t, n] - yo) / np.linalg.norm(yo)))
        rel.append(worst)
    marks = [m for m in (1, 2, 4, 8, 16, 32, 64, 128, 256) if m <= upto]
    return {f"step {m}": f"{rel[m - 1]:.2e}" for m in marks}


def _sample(rng, w, n):
    return [(int(b), int(h)) for b, h in zip(rng.choice(w.batch, n), rng.choice(w.heads, n))]


def _report(name, rep, free=None, contrast=None):
    print(f"{name}: adoptions {dict(rep.count)}, max y rel {rep.max_y_rel:.2e}")
    if contrast is not None:
        print(f"{name}: warm-up state contrast {contrast}")
    if free is not None:
        print(f"{name}: free-running max readout rel diff {free}")


@pytest.mark.timeout(900)
def test_pool_step4_bench_plan():
    """High-concurrency GDN pool (512 of 1024 slots, 48 heads, nominal 4 bits,
    calibrated plan: FP16 pivot head, 2-bit and 4-bit heads) in the split
    launch the bench times: 256 steps, 80 tiles on 8 of them."""
    w, pool, slots, sdev, sets, contrast = _setup("gdn_pool_step4")
    ub = pool.desc["unit_bits"]
    assert (ub == 16).sum() == 1 and set(int(b) for b in ub) <= {2, 4, 6, 8, 16}
    rng = np.random.default_rng(40)
    special = [int(h) for h in np.nonzero((ub == 16) | (ub == 2))[0]]
    tiles = [(int(b), h) for h in special for b in rng.choice(w.batch, 8, replace=False)]
    tiles += _sample(rng, w, 80 - len(tiles)) + [(0, 0), (w.batch - 1, w.heads - 1)]
    steps = {0, 1, 2, 63, 128, 191, w.steps - 2, w.steps - 1}
    track = tiles[:4]
    rep, start, hist = _run(w, pool, slots, sdev, sets, tiles, steps, track)
    free = _free_running(w, pool, sets, track, start, hist, 64)
    _report("gdn_pool_step4", rep, free)
    rep.assert_ok()


@pytest.mark.timeout(900)
def test_mid_step6_bench_plan_all_tiles():
    """Mid GDN (64 slots x 16 heads, calibrated nominal-6-bit plan with an FP16
    head), one merged launch: 1,024 steps, every tile on 8 of them."""
    w, pool, slots, sdev, sets, contrast = _setup("gdn_mid_step6")
    assert 16 in set(int(b) for b in pool.desc["unit_bits"])
    tiles = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    steps = {0, 1, 2, 255, 511, 767, w.steps - 2, w.steps - 1}
    track = [(0, 0), (5, 7), (63, 15)]
    rep, start, hist = _run(w, pool, slots, sdev, sets, tiles, steps, track)
    free = _free_running(w, pool, sets, track, start, hist, 64)
    _report("gdn_mid_step6", rep, free)
    rep.assert_ok()


@pytest.mark.timeout(900)
def test_kda_step6_bench_plan():
    """KDA (256 slots x 32 heads, calibrated per-row {4,6,8} plan with 1.4%
    FP16 rows): 512 steps, 72+ tiles on 8 of them including a tile of every
    head that holds pivot rows; the warm-up state's magnitude contrast is
    printed."""
    w, pool, slots, sdev, sets, contrast = _setup("kda_step6")
    rows = pool.desc["unit_bits"].reshape(w.heads, w.d_k)
    piv_heads = [int(h) for h in np.nonzero((rows == 16).any(axis=1))[0]]
    assert piv_heads
    rng = np.random.default_rng(41)
    tiles = [(int(rng.integers(w.batch)), h) for h in piv_heads]
    tiles += _sample(rng, w, max(72 - len(tiles), 40)) + [(0, 0), (w.batch - 1, w.heads - 1)]
    steps = {0, 1, 2, 127, 255, 383, w.steps - 2, w.steps - 1}
    track = tiles[:3]
    rep, start, hist = _run(w, pool, slots, sdev, sets, tiles, steps, track)
    free = _free_running(w, pool, sets, track, start, hist, 32)
    _report("kda_step6", rep, free, contrast)
    rep.assert_ok()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["gdn_window16", "gdn_window16_r4"])
def test_window16_bench_plan(name):
    """Per-window path (256 slots x 32 heads, p = 16, INT8 boundary, fp32
    records; r = 4 FP16 compensator pairs in the second case): 1,024 tokens,
    72 tiles on the tokens around the first two rebuilds (tokens 15, 16, 17,
    31, 32, 33 counted from 1), the first and the last."""
    w, pool, slots, sdev, sets, contrast = _setup(name)
    rng = np.random.default_rng(42)
    tiles = _sample(rng, w, 70) + [(0, 0), (w.batch - 1, w.heads - 1)]
    steps = {0, 14, 15, 16, 30, 31, 32, w.steps - 1}
    track = tiles[:3]
    rep, start, hist = _run(w, pool, slots, sdev, sets, tiles, steps, track)
    free = _free_running(w, pool, sets, track, start, hist, 48)
    _report(name, rep, free)
    rep.assert_ok()
