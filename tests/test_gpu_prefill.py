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


FORMS = {"serial": "sq_prefill_chunk", "chunkwise": "sq_prefill_chunkwise"}


def _run(form, kind, H, dk, dv, B, T, S0, x):
    """One call of the given prefill form on device copies; returns (y, S)."""
    import torch
    S = to_dev(np.ascontiguousarray(S0, dtype=np.float32))
    y = torch.full((B, T, H, dv), float("nan"), dtype=torch.float32, device="cuda")
    d = {k: to_dev(np.ascontiguousarray(v, dtype=np.float32)) for k, v in x.items()}
    getattr(sq, FORMS[form])(sq.SQ_KIND_GDN if kind == "gdn" else sq.SQ_KIND_KDA, H, dk, dv, B, T,
                             S, d["q"], d["k"], d["v"], d["beta"], d["gate"], y)
    torch.cuda.synchronize()
    return y.cpu().numpy(), S.cpu().numpy()


# T spans one token, ragged single blocks, whole blocks and ragged
# multi-block tails for the chunkwise form (blocks of 16 tokens)
@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("kind,shape,T", [("gdn", (128, 128), 1), ("gdn", (128, 128), 130),
                                          ("kda", (128, 128), 37), ("gdn", (64, 64), 5),
                                          ("kda", (128, 64), 64), ("gdn", (64, 128), 9),
                                          ("kda", (64, 64), 97), ("gdn", (128, 64), 32),
                                          ("kda", (64, 128), 33), ("kda", (128, 128), 160),
                                          ("kda", (128, 128), 1), ("kda", (64, 64), 16),
                                          ("gdn", (64, 64), 17)])
def test_prefill_chunk_matches_recurrence(form, kind, shape, T):
    dk, dv = shape
    w = SI.workload("gdn_mid_step6" if kind == "gdn" else "kda_step6", batch=3, n_slots=3,
                    heads=2, d_k=dk, d_v=dv)
    params = SI.gate_params(w)
    S0 = oracle_warmup(w, 12)
    x = _chunk(w, T, params)
    y, S = _run(form, kind, 2, dk, dv, 3, T, S0, x)
    y_ref, S_ref = _oracle(S0.astype(np.float32), x, kind, dk)
    assert _rel(y, y_ref, -1).max() <= Y_REL
    assert _rel(S.reshape(6, -1), S_ref.reshape(6, -1), -1).max() <= Y_REL


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_prefill_degenerate_gates(form, kind):
    """Gates of exactly 0 and 1 and write strengths of 0 and 1 inside one
    sequence: a zero gate erases the state (every decay product across it is
    0, with no division), beta = 0 leaves the token out, beta = 1 with a unit
    key overwrites the key's direction."""
    rng = np.random.default_rng(5)
    dk = dv = 128
    B, H, T = 2, 3, 75
    w = SI.workload("gdn_mid_step6" if kind == "gdn" else "kda_step6", batch=B, n_slots=B,
                    heads=H, d_k=dk, d_v=dv)
    S0 = oracle_warmup(w, 8)
    x = _chunk(w, T, SI.gate_params(w))
    for t, val in ((3, 0.0), (40, 1.0), (64, 0.0)):      # whole-token gates
        x["gate"][:, t] = val
    x["beta"][:, 10] = 0.0
    x["beta"][:, 50] = 1.0
    if kind == "kda":                                    # single channels at 0 and 1
        x["gate"][0, 20, 1, rng.integers(0, dk, 9)] = 0.0
        x["gate"][1, 70, 2, rng.integers(0, dk, 9)] = 1.0
    y, S = _run(form, kind, H, dk, dv, B, T, S0, x)
    y_ref, S_ref = _oracle(S0.astype(np.float32), x, kind, dk)
    assert np.isfinite(y).all() and np.isfinite(S).all()
    assert _rel(y, y_ref, -1).max() <= Y_REL
    assert _rel(S.reshape(B * H, -1), S_ref.reshape(B * H, -1), -1).max() <= Y_REL


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("kind,shape", [("gdn", (128, 128)), ("kda", (128, 64))])
def test_prefill_long_sequence(form, kind, shape):
    """One long prompt (2,048 tokens, 128 blocks of the chunkwise form) from
    the warm-up state: the error of the block products must not build up
    over the blocks."""
    dk, dv = shape
    B, H, T = 1, 2, 2048
    w = SI.workload("gdn_mid_step6" if kind == "gdn" else "kda_step6", batch=B, n_slots=B,
                    heads=H, d_k=dk, d_v=dv)
    S0 = oracle_warmup(w, 16)
    x = _chunk(w, T, SI.gate_params(w))
    y, S = _run(form, kind, H, dk, dv, B, T, S0, x)
    y_ref, S_ref = _oracle(S0.astype(np.float32), x, kind, dk)
    assert _rel(y, y_ref, -1).max() <= Y_REL
    assert _rel(S.reshape(B * H, -1), S_ref.reshape(B * H, -1), -1).max() <= Y_REL


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_chunkwise_prefill_at_bench_size(kind):
    """The launch bench.py times for --prefill 256 (64 sequences x 16 heads
    for GDN, 256 x 32 for KDA, d = 128): sampled (sequence, head) tiles
    against the float64 recurrence over all 256 tokens, every tile against
    the serial form."""
    import torch
    T = 256
    w = SI.workload("gdn_mid_step6" if kind == "gdn" else "kda_step6")
    B, H, dk, dv = w.batch, w.heads, w.d_k, w.d_v
    rng = np.random.default_rng(17)
    S0 = (rng.standard_normal((B, H, dk, dv)) * 0.05).astype(np.float32)
    x = _chunk(w, T, SI.gate_params(w))
    y_c, S_c = _run("chunkwise", kind, H, dk, dv, B, T, S0, x)
    y_s, S_s = _run("serial", kind, H, dk, dv, B, T, S0, x)
    torch.cuda.empty_cache()
    assert np.isfinite(y_c).all() and np.isfinite(S_c).all()
    # every tile: the two forms agree to the fp32 bar
    assert _rel(y_c, y_s, -1).max() <= 2 * Y_REL
    assert _rel(S_c.reshape(B * H, -1), S_s.reshape(B * H, -1), -1).max() <= 2 * Y_REL
    # sampled tiles: the float64 recurrence
    for b, h in ((0, 0), (B - 1, H - 1), (B // 2, H // 3)):
        xs = {k: v[b:b + 1, :, h:h + 1] for k, v in x.items()}
        y_ref, S_ref = _oracle(S0[b:b + 1, h:h + 1], xs, kind, dk)
        assert _rel(y_c[b:b + 1, :, h:h + 1], y_ref, -1).max() <= Y_REL
        assert _rel(S_c[b, h].ravel(), S_ref.ravel(), -1) <= Y_REL


@pytest.mark.parametrize("form", list(FORMS))
def test_prefill_between_unpack_and_pack(form):
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
    getattr(sq, FORMS[form])(sq.SQ_KIND_GDN, H, d, d, 3, T, S, dx["q"], dx["k"], dx["v"],
                             dx["beta"], dx["gate"], y)
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
