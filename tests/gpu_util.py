"""Helpers for the GPU tests: device buffers, seeded inputs, warm-up states."""
from __future__ import annotations

import numpy as np

import quantized_recurrent_state_decode_amd as sq
from oracle import recurrence as R
from synth import inputs as SI


def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(torch_dev())


def oracle_warmup(w: SI.Workload, steps: int) -> np.ndarray:
    """Float64 dense states [B, H, d_k, d_v] after `steps` unquantised steps
    from S = 0 (the initial state recipe of the workloads)."""
    params = SI.gate_params(w)
    S = np.zeros((w.batch, w.heads, w.d_k, w.d_v))
    for t in range(steps):
        inp = SI.warmup_inputs(w, t, params)
        dvec = R.gate_vector(inp["gate"].astype(np.float64), w.kind, w.d_k)
        S, _ = R.dense_step(S, inp["q"].astype(np.float64), inp["k"].astype(np.float64),
                            inp["v"].astype(np.float64), inp["beta"].astype(np.float64), dvec)
    return S


class Pool:
    """A plan, its device tables and a zeroed pool."""

    def __init__(self, plan, n_slots):
        import torch
        self.plan = plan
        self.desc = sq.sq_plan_query(plan)
        self.dev_plan = sq.device_plan(plan)
        self.n_slots = n_slots
        self.slot_bytes = self.desc["slot_bytes"]
        self.pool = torch.zeros(sq.sq_pool_bytes(plan, n_slots), dtype=torch.uint8,
                                device=torch_dev())
        sq.sq_pool_init(plan, self.dev_plan, self.pool, n_slots)

    def slot_bytes_of(self, slot: int) -> bytes:
        import torch
        torch.cuda.synchronize()
        s = self.slot_bytes
        return self.pool[slot * s:(slot + 1) * s].cpu().numpy().tobytes()

    def head_bytes(self, slot_buf: bytes, h: int) -> bytes:
        off = int(self.desc["head_off"][h])
        end = int(self.desc["head_off"][h + 1]) if h + 1 < self.desc["heads"] else self.slot_bytes
        return slot_buf[off:end]

    def pack(self, slots_dev, S_dev, batch):
        sq.sq_pool_pack(self.plan, self.dev_plan, self.pool, self.n_slots, slots_dev, batch, S_dev)

    def decode(self, slots_dev, batch, inp_dev, y_dev):
        sq.sq_decode_step(self.plan, self.dev_plan, self.pool, self.n_slots, slots_dev, batch,
                          inp_dev["q"], inp_dev["k"], inp_dev["v"], inp_dev["beta"],
                          inp_dev["gate"], y_dev)


def inputs_dev(inp: dict) -> dict:
    return {k: to_dev(v) for k, v in inp.items()}


def head_inputs(inp: dict, b: int, h: int) -> dict:
    """float64 inputs of one (batch row, head) from a batch of float32 inputs."""
    g = inp["gate"][b, h]
    return {"q": inp["q"][b, h].astype(np.float64), "k": inp["k"][b, h].astype(np.float64),
            "v": inp["v"][b, h].astype(np.float64), "beta": float(inp["beta"][b, h]),
            "gate": np.asarray(g, dtype=np.float64)}
