"""GPU parity of the per-window variant (INT8 boundary with key-row smoothing,
float32 records, dense rebuild every p tokens, optional FP16 compensator
pairs refitted at every rebuild) against the oracle, teacher-forced, across
window flushes."""
import numpy as np
import pytest

import quantized_recurrent_state_decode_amd as sq
from oracle import window as W
from synth import inputs as SI

from gpu_util import Pool, head_inputs, inputs_dev, oracle_warmup, to_dev
from parity import (Report, check_decode_head, check_quantized_head, check_window_encode,
                    dequant_head, oracle_desc)

pytestmark = pytest.mark.gpu


def _run(pool, w, slots, steps, tiles=None, compare=None, edit=None):
    import torch
    desc = oracle_desc(pool.desc)
    sdev = to_dev(slots.astype(np.int32))
    params = SI.gate_params(w)
    y = torch.empty((w.batch, w.heads, w.d_v), dtype=torch.float32, device="cuda")
    tiles = tiles or [(b, h) for b in range(w.batch) for h in range(w.heads)]
    rep = Report()
    for t in range(steps):
        inp = SI.step_inputs(w, t, params)
        if edit is not None:
            inp = {k: v.copy() for k, v in inp.items()}
            edit(t, inp)
        cmp = compare is None or t in compare
        before = {b: pool.slot_bytes_of(int(slots[b])) for b, _ in tiles} if cmp else None
        pool.decode(sdev, w.batch, inputs_dev(inp), y)
        if not cmp:
            continue
        torch.cuda.synchronize()
        yh = y.cpu().numpy()
        for b, h in tiles:
            after = pool.slot_bytes_of(int(slots[b]))
            check_decode_head(f"step {t} b {b} h {h}", desc, h, pool.head_bytes(before[b], h),
                              pool.head_bytes(after, h), head_inputs(inp, b, h),
                              yh[b, h].astype(np.float64), None, rep)
    return rep


def _plan(heads, dk, dv, p, rank, iters=4):
    if rank == 0:
        return sq.sq_plan_create_window(heads, dk, dv, p)
    return sq.sq_plan_create_window_lowrank(heads, dk, dv, p, rank, iters)


@pytest.mark.parametrize("p,steps,rank,iters", [(4, 10, 0, 0), (16, 34, 0, 0), (1, 3, 0, 0),
                                                (4, 10, 4, 4), (16, 34, 4, 4), (8, 17, 8, 2),
                                                (32, 33, 1, 6)])
def test_window_decode_across_flushes(p, steps, rank, iters):
    w = SI.workload("gdn_window16", batch=3, n_slots=5, heads=2, window=p, steps=steps)
    pool = Pool(_plan(2, 128, 128, p, rank, iters), 5)
    slots = SI.slot_ids(w)
    pool.pack(to_dev(slots), to_dev(oracle_warmup(w, 32).astype(np.float32)), w.batch)
    rep = _run(pool, w, slots, w.steps)
    print("adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()


@pytest.mark.parametrize("rank", [0, 2])
def test_window_64_and_rectangular(rank):
    for dk, dv in ((64, 64), (128, 64), (64, 128)):
        w = SI.workload("gdn_window16", batch=2, n_slots=2, heads=2, d_k=dk, d_v=dv, window=3,
                        steps=7)
        pool = Pool(_plan(2, dk, dv, 3, rank, 3), 2)
        slots = SI.slot_ids(w)
        pool.pack(to_dev(slots), to_dev(oracle_warmup(w, 16).astype(np.float32)), w.batch)
        rep = _run(pool, w, slots, w.steps)
        rep.assert_ok()


@pytest.mark.parametrize("rank", [0, 4])
def test_window_flush_unpack_pack(rank):
    """sq_window_flush rebuilds partial windows (l = 0 heads untouched),
    sq_pool_unpack returns S_l, sq_pool_pack / quantize-only encode the
    boundary (with compensators: refitted from the head's previous pairs at
    a flush, from the all-ones vector at a pack)."""
    import torch
    rng = np.random.default_rng(12)
    w = SI.workload("gdn_window16", batch=4, n_slots=4, heads=2, window=8, steps=5)
    pool = Pool(_plan(2, 128, 128, 8, rank), 4)
    desc = oracle_desc(pool.desc)
    slots = SI.slot_ids(w)
    sdev = to_dev(slots)
    pool.pack(sdev, to_dev(oracle_warmup(w, 16).astype(np.float32)), w.batch)
    params = SI.gate_params(w)
    y = torch.empty((4, 2, 128), dtype=torch.float32, device="cuda")
    for t in range(5):                       # slots 0, 1 get 5 tokens; 2, 3 get 3
        bsz = 4 if t < 3 else 2
        inp = {k: v[:bsz] for k, v in SI.step_inputs(w, t, params).items()}
        pool.decode(to_dev(slots[:bsz]), bsz, inputs_dev(inp), y[:bsz])
    # unpack of open windows
    S = torch.empty((4, 2, 128, 128), dtype=torch.float32, device="cuda")
    sq.sq_pool_unpack(pool.plan, pool.dev_plan, pool.pool, 4, sdev, 4, S)
    torch.cuda.synchronize()
    Sh = S.cpu().numpy()
    bufs = [pool.slot_bytes_of(int(s)) for s in slots]
    for b in range(4):
        for h in range(2):
            ref = dequant_head(desc, h, pool.head_bytes(bufs[b], h))
            np.testing.assert_allclose(Sh[b, h], ref, rtol=2e-6, atol=2e-6 * np.abs(ref).max())
    # explicit flush of the partial windows
    from oracle.layout import parse_head
    sq.sq_window_flush(pool.plan, pool.dev_plan, pool.pool, 4, sdev, 4)
    rep = Report()
    for b in range(4):
        after = pool.slot_bytes_of(int(slots[b]))
        for h in range(2):
            st0 = parse_head(desc, h, pool.head_bytes(bufs[b], h))
            assert st0["ell"] == (5 if b < 2 else 3)
            st1 = parse_head(desc, h, pool.head_bytes(after, h))
            assert st1["ell"] == 0
            check_window_encode(f"flush b {b} h {h}", desc, W.window_state_dense(st0), st1, rep,
                                init=st0.get("Uc"))
    rep.assert_ok()
    # a second flush is a no-op (l = 0)
    snap = pool.pool.cpu().numpy().copy()
    sq.sq_window_flush(pool.plan, pool.dev_plan, pool.pool, 4, sdev, 4)
    assert np.array_equal(pool.pool.cpu().numpy(), snap)
    # quantize-only
    n = 4
    X = (rng.standard_normal((n, 128, 128)) * rng.lognormal(0, 1, (n, 128, 1))).astype(np.float32)
    X[1, :, 7] = 0.0                          # an all-zero column
    heads = (np.arange(n) % 2).astype(np.int32)
    mhb = sq.sq_max_head_bytes(pool.plan)
    out = torch.zeros(n * mhb, dtype=torch.uint8, device="cuda")
    sq.sq_quantize_tiles(pool.plan, pool.dev_plan, to_dev(X), n, to_dev(heads), out)
    torch.cuda.synchronize()
    ob = out.cpu().numpy().tobytes()
    rep = Report()
    for t in range(n):
        check_quantized_head(f"tile {t}", desc, int(heads[t]), X[t].astype(np.float64),
                             ob[t * mhb:(t + 1) * mhb], None, rep)
    rep.assert_ok()


@pytest.mark.parametrize("rank", [0, 4])
def test_full_size_window_sampled(rank):
    """Batch 256, 32 heads, p = 16 at full size: 20 tokens (one flush at token
    16), 16 sampled tiles compared at the flush and at the last token."""
    import torch
    w = SI.workload("gdn_window16")
    pool = Pool(_plan(32, 128, 128, 16, rank), w.n_slots)
    slots = SI.slot_ids(w)
    sdev = to_dev(slots)
    S = torch.zeros((w.batch, 32, 128, 128), dtype=torch.float32, device="cuda")
    y = torch.empty((w.batch, 32, 128), dtype=torch.float32, device="cuda")
    params = SI.gate_params(w)
    for t in range(16):
        d = inputs_dev(SI.warmup_inputs(w, t, params))
        sq.sq_dense_step(0, 32, 128, 128, S, w.batch, sdev, w.batch, d["q"], d["k"], d["v"],
                         d["beta"], d["gate"], y)
    pool.pack(sdev, S, w.batch)
    del S
    rng = np.random.default_rng(5)
    tiles = [(int(b), int(h)) for b, h in zip(rng.choice(w.batch, 16), rng.choice(32, 16))]
    rep = _run(pool, w, slots, 20, tiles=tiles, compare={15, 19})
    print("adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()


@pytest.mark.parametrize("rank", [0, 1])
def test_window_zero_gate_and_beta(rank):
    """Tokens with alpha = 0 (the boundary and every earlier record vanish from
    S, LeapQuant notes Sec. 2.3, Eq. 4 with a zero decay factor) and tokens
    with beta = 0 (no write), including the token that fills a window and so
    triggers the rebuild; all tiles teacher-forced.  A zero gate leaves the
    rebuilt state of rank one or two, so with one pair the residual is at the
    level of its own float32 error (its codes are then checked within that
    bound).  More pairs would be fitted to the near-degenerate rounding
    residual of the first, whose directions are not unique."""
    p = 4
    w = SI.workload("gdn_window16", batch=3, n_slots=4, heads=2, window=p, steps=10)
    pool = Pool(_plan(2, 128, 128, p, rank, 3), 4)
    slots = SI.slot_ids(w)
    pool.pack(to_dev(slots), to_dev(oracle_warmup(w, 16).astype(np.float32)), w.batch)

    def edit(t, inp):
        if t in (1, 3, 6):            # token 3 fills the first window
            inp["gate"][0, :] = 0.0
            inp["gate"][2, 1] = 0.0
        if t in (2, 3, 7):
            inp["beta"][1, :] = 0.0

    rep = _run(pool, w, slots, w.steps, edit=edit)
    print("adoptions", dict(rep.count), "max y rel", rep.max_y_rel)
    rep.assert_ok()
