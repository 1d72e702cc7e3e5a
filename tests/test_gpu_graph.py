"""Decode steps captured as a HIP graph, as bench.py times them.  Each case
packs one state into twin pools, captures three decode steps on the first,
then replays the graph three times; between replays the same three steps run
eagerly on the twin, with synchronisations.  After every replay the two pools
and the readouts must be bit-identical.  Cases: the split GDN launch (pool
shape), a uniform plan, KDA rows of mixed widths, and the window, whose
rebuild at p = 4 falls inside the captured steps.  The prefill forms are
captured and replayed the same way."""
import numpy as np
import pytest

import quantized_recurrent_state_decode_amd as sq
from oracle import calibration as C
from synth import inputs as SI

from gpu_util import Pool, inputs_dev, to_dev

pytestmark = pytest.mark.gpu


def _case(kind, rng):
    if kind == "gdn_split":
        # largest class 45 heads x 512 rows = 23,040 tiles: the split launch
        w = SI.workload("gdn_pool_step4", n_slots=512)
        bits = np.full(48, 4)
        bits[[5, 29]] = 2
        bits[17] = 16
        wts = C.impact_factors(rng.lognormal(0.0, 1.5, (48, 128))).astype(np.float32)
        return w, sq.sq_plan_create_step(sq.SQ_KIND_GDN, 48, 128, 128, bits, wts)
    if kind == "uniform":
        w = SI.workload("gdn_pool_int4", batch=16, n_slots=24, heads=6)
        return w, sq.sq_plan_create_uniform(6, 128, 128, 4)
    if kind == "kda":
        w = SI.workload("kda_step6", batch=8, n_slots=10, heads=4)
        bits = rng.choice((2, 4, 6, 8, 16), size=4 * 128)
        wts = C.impact_factors(rng.lognormal(0.0, 1.5, (4, 128))).astype(np.float32)
        return w, sq.sq_plan_create_step(sq.SQ_KIND_KDA, 4, 128, 128, bits, wts)
    w = SI.workload("gdn_window16", batch=8, n_slots=10, heads=4)
    return w, sq.sq_plan_create_window(4, 128, 128, 4)


@pytest.mark.parametrize("kind", ["gdn_split", "uniform", "kda", "window"])
def test_graph_replays_match_eager(kind):
    import torch
    rng = np.random.default_rng(95)
    w, plan = _case(kind, rng)
    slots = to_dev(SI.slot_ids(w))
    gen = torch.Generator(device="cuda").manual_seed(96)
    S = 0.3 * torch.randn((w.batch, w.heads, w.d_k, w.d_v), generator=gen, device="cuda")
    pa, pb = Pool(plan, w.n_slots), Pool(plan, w.n_slots)
    pa.pack(slots, S, w.batch)
    pb.pack(slots, S, w.batch)
    del S
    params = SI.gate_params(w)
    ins = [inputs_dev(SI.step_inputs(w, t, params)) for t in range(3)]
    ya = torch.zeros((3, w.batch, w.heads, w.d_v), dtype=torch.float32, device="cuda")
    yb = torch.zeros_like(ya)
    torch.cuda.synchronize()
    assert torch.equal(pa.pool, pb.pool)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(3):
            pa.decode(slots, w.batch, ins[t], ya[t])
    torch.cuda.synchronize()
    assert torch.equal(pa.pool, pb.pool), "capture must not execute the steps"
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        for t in range(3):
            pb.decode(slots, w.batch, ins[t], yb[t])
        torch.cuda.synchronize()
        assert torch.equal(pa.pool, pb.pool), f"pools differ after replay {r}"
        assert torch.equal(ya, yb), f"readouts differ after replay {r}"
        assert bool(torch.isfinite(ya).all())
    del g


@pytest.mark.parametrize("form,kind", [("sq_prefill_chunkwise", "gdn"), ("sq_prefill_chunkwise", "kda"),
                                       ("sq_prefill_chunk", "gdn")])
def test_prefill_graph_replays_match_eager(form, kind):
    """Two prefill chunks (37 tokens: two whole blocks and a ragged one of the
    matrix form) captured on one state and replayed three times; between
    replays the same chunks run eagerly on a twin state.  States and outputs
    must be bit-identical after every replay (neither form allocates, clears
    memory or sums with atomics)."""
    import torch
    B, H, d, T = 3, 4, 128, 37
    w = SI.workload("gdn_mid_step6" if kind == "gdn" else "kda_step6", batch=B, n_slots=B,
                    heads=H)
    params = SI.gate_params(w)
    chunks = []
    for c in range(2):
        steps = [SI.step_inputs(w, c * T + t, params) for t in range(T)]
        chunks.append({k: to_dev(np.ascontiguousarray(np.stack([s[k] for s in steps], axis=1)))
                       for k in steps[0]})
    gen = torch.Generator(device="cuda").manual_seed(97)
    Sa = 0.05 * torch.randn((B, H, d, d), generator=gen, device="cuda")
    Sb = Sa.clone()
    ya = torch.zeros((2, B, T, H, d), dtype=torch.float32, device="cuda")
    yb = torch.zeros_like(ya)
    knd = sq.SQ_KIND_GDN if kind == "gdn" else sq.SQ_KIND_KDA
    fn = getattr(sq, form)

    def run(S, y):
        for c, x in enumerate(chunks):
            fn(knd, H, d, d, B, T, S, x["q"], x["k"], x["v"], x["beta"], x["gate"], y[c])

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(Sa, ya)
    torch.cuda.synchronize()
    assert torch.equal(Sa, Sb), "capture must not execute the chunks"
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        run(Sb, yb)
        torch.cuda.synchronize()
        assert torch.equal(Sa, Sb), f"states differ after replay {r}"
        assert torch.equal(ya, yb), f"outputs differ after replay {r}"
        assert bool(torch.isfinite(ya).all())
    del g
