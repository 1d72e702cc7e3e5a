"""GPU prefill of a chunk (the middle step of "unpack active states, run the
chunk, pack boundary states", STEPQuant App. F.1) against the oracle's step
recurrence, alone and between sq_pool_unpack and sq_pool_pack."""
import numpy as np
import pytest

import quantized_recurrent_state_decode_amd as sq
from oracle import calibration as C
from oracle import recurrence as R
from synth import inputs as SI

from gpu_util import Pool, oracle_warmup, to_dev
from parity import Report, check_quantized_head, oracle_desc

pytestmark = pytest.mark.gpu

Y_REL = 1e-5   # readouts and states, norm-wise per (sequence, head): float32 over T steps


def _chunk(w, T, params):
    """Inputs of T tokens, sequence-major [B][T][H][...]."""
    steps = [SI.step_inputs(w, t, params) for t in range(T)]
    return {k: np.ascontiguousarray(np.stack([s[k] for s in steps], axis=1)) for k in steps[0]}


def _oracle(S0, x, kind, d_k):
    """Float64 recurrence over the chunk: outputs [B][T][H][d_v], final state."""
    S = S0.astype(np.float64)
    T = x["q"].shape[1]
    ys = []
    for t in range(T):
        xt = {k: v[:, t].astype(np.float64) for k, v in x.items()}
        dvec = R.gate_vector(xt["gate"], kind, d_k)
        S, y = R.dense_step(S, xt["q"], xt["k"], xt["v"], xt["beta"], dvec)
        ys.append(y)
    return np.stack(ys, axis=1), S


def _rel(a, b, axis):
    return np.linalg.norm(a - b, axis=axis) / np.maximum(np.linalg.norm(b, axis=axis), 1e-300)


@pytest.mark.parametrize("kind,shape,T", [("gdn", (128, 128), 1), ("gdn", (128, 128), 130),
                                          ("kda", (128, 128), 37), ("gdn", (64, 64), 5),
                                          ("kda", (128, 64), 64), ("gdn", (64, 128), 9)])
def test_prefill_chunk_matches_recurrence(kind, shape, T):
    import torch
    dk, dv = shape
    w = SI.workload("gdn_mid_step6" if kind == "gdn" else "kda_step6", batch=3, n_slots=3,
                    heads=2, d_k=dk, d_v=dv)
    params = SI.gate_params(w)
    S0 = oracle_warmup(w, 12)
    x = _chunk(w, T, params)
    S = to_dev(S0.astype(np.float32))
    y = torch.empty((3, T, 2, dv), dtype=torch.float32, device="cuda")
    d = {k: to_dev(v) for k, v in x.items()}
    sq.sq_prefill_chunk(sq.SQ_KIND_GDN if kind == "gdn" else sq.SQ_KIND_KDA, 2, dk, dv, 3, T, S,
                        d["q"], d["k"], d["v"], d["beta"], d["gate"], y)
    torch.cuda.synchronize()
    y_ref, S_ref = _oracle(S0.astype(np.float32), x, kind, dk)
    assert _rel(y.cpu().numpy(), y_ref, -1).max() <= Y_REL
    assert _rel(S.cpu().numpy().reshape(6, -1), S_ref.reshape(6, -1), -1).max() <= Y_REL


def test_prefill_between_unpack_and_pack():
    """A STEP pool (every width and an FP16 head): unpack the live slots, run a
    20-token chunk, pack the boundary states back.  The chunk's outputs and
    final states follow the recurrence from the unpacked states, and the pack
    is the plan's quantizer on those final states (teacher-forced)."""
    import torch
    rng = np.random.default_rng(71)
    H, d, T = 5, 128, 20
    w = SI.workload("gdn_mid_step6", batch=3, n_slots=6, heads=H)
    bits = np.array([2, 4, 6, 8, 16])
    wts = C.impact_factors(rng.lognormal(0.0, 1.5, (H, d))).astype(np.float32)
    pool = Pool(sq.sq_plan_create_step(sq.SQ_KIND_GDN, H, d, d, bits, wts), 6)
    slots = np.array([4, 0, 2], dtype=np.int32)
    sdev = to_dev(slots)
    pool.pack(sdev, to_dev(oracle_warmup(w, 16).astype(np.float32)), 3)
    S = torch.empty((3, H, d, d), dtype=torch.float32, device="cuda")
    sq.sq_pool_unpack(pool.plan, pool.dev_plan, pool.pool, 6, sdev, 3, S)
    torch.cuda.synchronize()
    S_start = S.cpu().numpy()
    x = _chunk(w, T, SI.gate_params(w))
    dx = {k: to_dev(v) for k, v in x.items()}
    y = torch.empty((3, T, H, d), dtype=torch.float32, device="cuda")
    sq.sq_prefill_chunk(sq.SQ_KIND_GDN, H, d, d, 3, T, S, dx["q"], dx["k"], dx["v"], dx["beta"],
                        dx["gate"], y)
    torch.cuda.synchronize()
    S_end = S.cpu().numpy()
    y_ref, S_ref = _oracle(S_start, x, "gdn", d)
    assert _rel(y.cpu().numpy(), y_ref, -1).max() <= Y_REL
    assert _rel(S_end.reshape(3 * H, -1), S_ref.reshape(3 * H, -1), -1).max() <= Y_REL
    pool.pack(sdev, S, 3)
    desc = oracle_desc(pool.desc)
    rep = Report()
    for b in range(3):
        buf = pool.slot_bytes_of(int(slots[b]))
        for h in range(H):
            check_quantized_head(f"b {b} h {h}", desc, h, S_end[b, h].astype(np.float64),
                                 pool.head_bytes(buf, h), wts[h].astype(np.float64), rep)
    rep.assert_ok()
