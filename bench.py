"""Throughput of the fused quantized recurrent-state decode step on one MI355X.

A step is one sq_decode_step call: every (slot, head) tile of the live batch
is reconstructed, updated, read out, refit, requantised and written back in
place.  The default workload is the high-concurrency GDN pool: 512 live
requests drawn from a 1024-slot pool by a seeded random permutation, 48 heads
of 128 x 128, nominal 4 bits with FP16 pivot heads, allocation from the
library's lifetime-aware calibration.

The timed loop cycles through `--layers` independent pools (one per layer, as
a model would) and `--input-sets` input batches, so that a pool is touched
again only after more bytes than the 256 MB Infinity Cache holds: the
achieved bandwidth is HBM bandwidth, not cache bandwidth.

Output: one JSON line (metric, value = steps/s, roofline of the decode kernel
with its launch duration from HIP events, the CPU oracle on a bounded sample).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "state-update steps/s and HBM GB/s (% of peak) at batch 512, 1 GPU"
# the kernel one decode step launches
KERNEL = {"step": "gdn_split_kernel<128,128,b> (largest code-width class in its width-specialised "
                  "body, the other classes in leading grid rows) when that class has >= 16,384 tiles, "
                  "else gdn_decode_kernel<128,128>",
          "uniform": "gdn_class_kernel<d,d,b,uniform>", "window": "window_tile_kernel<128,128,16>",
          "kda": "kda_tile_kernel<128,128>", "dense": "dense_kernel<128,128> (fp32 state)"}
# sources whose change invalidates a committed traffic measurement, per kernel family
TRAFFIC_SOURCES = {"gdn": ("tile_gdn.hip",), "kda": ("tile_kda.hip",), "window": ("tile_window.hip",),
                   "dense": ("dense.hip",)}
HBM_PEAK_GBS = 8000.0


def _plan(sq, w):
    if w.mode == "uniform":
        return sq.sq_plan_create_uniform(w.heads, w.d_k, w.d_v, w.bits)
    if w.mode == "window":
        if w.comp_rank:
            return sq.sq_plan_create_window_lowrank(w.heads, w.d_k, w.d_v, w.window, w.comp_rank,
                                                    w.power_iters)
        return sq.sq_plan_create_window(w.heads, w.d_k, w.d_v, w.window)
    with open(os.path.join(ROOT, "tests", "golden", f"calib_{w.calib or w.name}.json")) as f:
        st = json.load(f)
    stats = {"kind": 0 if st["kind"] == "gdn" else 1, "heads": st["heads"], "d_k": st["d_k"],
             "d_v": st["d_v"], "cand_bits": st["cand_bits"], "ell": np.array(st["ell"]),
             "dist": np.array(st["dist"]), "omega": np.array(st["omega"])}
    return sq.sq_calibrate_bits(stats, {"nominal_bits": st["nominal_bits"],
                                        "pivot_frac": st["pivot_frac"], "gamma": st["gamma"],
                                        "horizon": st["horizon"]})


def measured_traffic(workload: str, family: str):
    """HBM bytes per step from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary of this workload, if the decode kernel sources are still the ones
    the counters were taken on (else None)."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_step", "kernel_source_sha256_16"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash(family):
        return None
    return int(fields["traffic_bytes_per_step"])


def measured_valu(workload: str, family: str):
    """VALU instructions per decode step from the committed rocprofv3
    SQ_INSTS_VALU summary of this workload, if the decode kernel sources are
    still the ones the counter was taken on (else None)."""
    path = os.path.join(ROOT, "profiles", f"valu_issue_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("valu_instructions_per_step", "kernel_source_sha256_16"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash(family):
        return None
    return int(fields["valu_instructions_per_step"])


def kernel_source_hash(family: str) -> str:
    """First 16 hex digits of the sha256 of the decode sources of a kernel
    family (its kernel file, the shared tile header, the internal header and
    the host dispatcher)."""
    import hashlib
    csrc = os.path.join(ROOT, "quantized_recurrent_state_decode_amd", "csrc")
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[family] + ("tile_common.h", "sq_internal.h", "sq_host.cpp"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def algorithmic_bytes(desc, w) -> int:
    """Bytes one decode step must move: the packed state of every live slot
    read and written once (payload, no padding), q, k, v, beta, gate in, y out,
    slot ids.  Window mode: the boundary and C, B (and the compensator pairs)
    are read, the records held (mean (p-1)/2 per token) are read, one record
    is written, the boundary is rewritten once per p tokens."""
    B, H, dk, dv = w.batch, w.heads, w.d_k, w.d_v
    gate = B * H * (dk if w.kind == "kda" else 1) * 4
    io = B * H * (2 * dk + dv) * 4 + B * H * 4 + gate + B * H * dv * 4 + B * 4
    if w.mode == "dense":
        return 2 * B * H * dk * dv * 4 + io
    if w.mode != "window":
        return 2 * B * desc["payload_bytes"] + io
    p = w.window
    base = dk * dv + 4 * (dk + dv) + 2 * w.comp_rank * (dk + dv)
    rec = 4 * (dk + dv) + 4
    per_tile = base + rec * (p - 1) / 2.0 + rec + base / p + 16
    return int(B * H * per_tile) + io


def build_state(sq, w, pools, slots_dev, steps):
    """Warm-up state: `steps` fp32 dense steps from S = 0 with the library's
    dense kernel, then packed into every pool."""
    import torch
    from synth import inputs as SI
    params = SI.gate_params(w)
    S = torch.zeros((w.batch, w.heads, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    ident = torch.arange(w.batch, dtype=torch.int32, device="cuda")
    y = torch.empty((w.batch, w.heads, w.d_v), dtype=torch.float32, device="cuda")
    for t in range(steps):
        inp = {k: torch.from_numpy(v).cuda() for k, v in SI.warmup_inputs(w, t, params).items()}
        sq.sq_dense_step(0 if w.kind == "gdn" else 1, w.heads, w.d_k, w.d_v, S, w.batch, ident,
                         w.batch, inp["q"], inp["k"], inp["v"], inp["beta"], inp["gate"], y)
    for pl in pools:
        if w.mode == "dense":
            pl["pool"].index_copy_(0, slots_dev.long(), S)
        else:
            sq.sq_pool_pack(pl["plan"], pl["dev_plan"], pl["pool"], w.n_slots, slots_dev, w.batch, S)
    torch.cuda.synchronize()
    return S


def cpu_baseline(w, desc, pool_bytes: bytes, slots, budget_s: float) -> dict:
    """The float64 oracle, as it stands, on a bounded sample of the same
    workload: the first slots of the live batch (all heads), teacher-forced
    from the GPU's packed state, decode steps repeated until the time budget
    is spent.  Reported as equivalent full-batch steps/s."""
    from oracle import layout as OL
    from oracle import quantizers as Q
    from oracle import recurrence as R
    from oracle import window as OW
    from synth import inputs as SI
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import oracle_desc, row_bits_of
    od = oracle_desc(desc)
    nb = 1
    sb = desc["slot_bytes"]
    states = []
    for b in range(nb):
        s = int(slots[b])
        states.append(OL.parse_slot(od, pool_bytes[b * sb:(b + 1) * sb]))
    params = SI.gate_params(w)
    tiles = 0
    t0 = time.perf_counter()
    step = 0
    while time.perf_counter() - t0 < budget_s:
        inp = SI.step_inputs(w, step, params)
        for b in range(nb):
            for h in range(w.heads):
                st = states[b][h]
                q, k, v = (inp[x][b, h].astype(np.float64) for x in ("q", "k", "v"))
                beta = float(inp["beta"][b, h])
                if w.mode == "window":
                    r = OW.window_step(st, q, k, v, beta, float(inp["gate"][b, h]), w.window,
                                       w.power_iters)
                    states[b][h] = r["state"]
                    tiles += 1
                    continue
                dvec = R.gate_vector(inp["gate"][b, h].astype(np.float64),
                                     "gdn" if w.mode == "uniform" else w.kind, w.d_k)
                if w.mode == "uniform":
                    S_hat = Q.dequant_uniform(st["z"], st["s"])
                    X = R.delta_update(R.retained(S_hat, dvec), k, v, beta)
                    R.readout(X, q)
                    e = Q.quantize_uniform(X, w.bits)
                    states[b][h] = {"z": e["z"], "s": e["s"]}
                else:
                    rb = row_bits_of(od, h)
                    S_hat = Q.dequant_step(st["z"], st["r"], st["c"], rb, st["h"])
                    X = R.delta_update(R.retained(S_hat, dvec), k, v, beta)
                    R.readout(X, q)
                    e = Q.quantize_step(X, desc["w"][h].astype(np.float64), rb)
                    states[b][h] = {"z": e["z"], "r": e["r"], "c": e["c"], "h": e["h"]}
                tiles += 1
        step += 1
    dt = time.perf_counter() - t0
    tiles_per_s = tiles / dt
    return {"value": tiles_per_s / (w.batch * w.heads), "unit": "steps/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{nb} slot x {w.heads} heads, {step} steps ({tiles} tiles) in "
                      f"{dt:.1f} s, float64 numpy, one process; value = tiles/s / "
                      f"({w.batch} x {w.heads}) tiles per step"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="gdn_pool_step4")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed steps one by one instead of replaying them as a HIP graph")
    ap.add_argument("--input-sets", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the same-hardware runs: fp32-dense and uniform-INT4 at the pool "
                         "workload's shape, fp32-dense at the KDA and window shapes")
    ap.add_argument("--state-warmup", type=int, default=None,
                    help="fp32 steps that build the initial state (default: the workload's 128)")
    ap.add_argument("--prefill", type=int, default=0, metavar="T",
                    help="measure sq_prefill_chunk instead: one chunk of T tokens per sequence "
                         "over the workload's batch and heads (tokens/s)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before timing, copy MIB MiB device-to-device once (a plain copy of "
                         "known size for scaling HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode step has no cross-GPU exchange; see the sharding notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_recurrent_state_decode_amd as sq
    from synth import inputs as SI

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = SI.workload(args.workload)
    if args.prefill:
        print(json.dumps(measure_prefill(sq, w, args)))
        return
    m = measure(sq, w, args)
    abytes, ms_per_step, launch_ms, desc = m["abytes"], m["ms_per_step"], m["launch_ms"], m["desc"]
    family = "window" if w.mode == "window" else ("dense" if w.mode == "dense" else w.kind)
    gbs_step = abytes / (ms_per_step * 1e-3) / 1e9
    gbs_kernel = abytes / (launch_ms * 1e-3) / 1e9
    hist = None
    if desc is not None and desc["unit_bits"] is not None:
        hist = {str(b): int(c) for b, c in zip(*np.unique(desc["unit_bits"], return_counts=True))}
    out = {
        "metric": METRIC,
        "value": 1e3 / ms_per_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_slots": w.n_slots,
                   "heads": w.heads, "d_k": w.d_k, "d_v": w.d_v, "mode": w.mode,
                   "kind": w.kind, "nominal_bits": w.nominal_bits if w.mode == "step" else
                   (w.bits if w.mode == "uniform" else (32 if w.mode == "dense" else 8)),
                   "unit_bits_histogram": hist,
                   "slot_bytes": (w.heads * w.d_k * w.d_v * 4 if desc is None else desc["slot_bytes"]),
                   "layers_rotated": args.layers,
                   "input_sets": args.input_sets, "algorithmic_bytes_per_step": abytes,
                   "timed_loop": ("eager launches" if args.eager else
                                  "one HIP graph replay of the K steps (captured after warm-up)"),
                   "state_gbs": gbs_step, "pct_of_hbm_peak": 100.0 * gbs_step / HBM_PEAK_GBS},
        "roofline": {"bound": "hbm", "achieved": gbs_kernel, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs_kernel / HBM_PEAK_GBS,
                     "traffic": measured_traffic(w.name, family),
                     "kernel": KERNEL[w.mode if w.kind == "gdn" else "kda"],
                     "kernel_source_sha256_16": kernel_source_hash(family),
                     "launch_ms": launch_ms, "bytes_per_launch": abytes,
                     "launch": "one decode call (sq_decode_step with all its kernel launches, or "
                               "sq_dense_step in dense mode), HIP events on the launch stream"},
    }
    valu = measured_valu(w.name, family)
    if valu is not None:
        # the issue rate the decode launch sustains: 64 lanes per VALU
        # instruction over the launch, against the chip's non-packed lane rate
        lane_ops = 64.0 * valu / (launch_ms * 1e-3)
        out["roofline"]["alu_issue"] = {"achieved": lane_ops / 1e12, "peak": VALU_PEAK / 1e12,
                                        "unit": "T lane-ops/s", "frac": lane_ops / VALU_PEAK,
                                        "valu_instructions_per_launch": valu}
    if not args.no_cpu and desc is not None:
        torch.cuda.synchronize()
        sb = desc["slot_bytes"]
        pb = m["pools"][0]["pool"]
        s0 = int(m["slots"][0])
        host = pb[s0 * sb:(s0 + 1) * sb].cpu().numpy().tobytes()
        out["cpu_baseline"] = cpu_baseline(w, desc, host, m["slots"], args.cpu_seconds)
    del m
    if w.name == "gdn_pool_step4" and not args.no_compare:
        out["same_hardware"] = same_hardware(sq, args, out["value"])
    elif w.name in DENSE_TWIN and not args.no_compare:
        out["same_hardware"] = dense_twin(sq, args, out["value"], DENSE_TWIN[w.name])
    print(json.dumps(out))


def measure(sq, w, args) -> dict:
    """Time args.steps consecutive decode steps of workload w (after
    args.warmup untimed ones), rotating args.layers independent pools so that
    the live state exceeds the on-package cache, then time 64 single calls
    with HIP events on the launch stream."""
    import torch
    from synth import inputs as SI
    dense = w.mode == "dense"
    plan = None if dense else _plan(sq, w)
    desc = None if dense else sq.sq_plan_query(plan)
    slots = SI.slot_ids(w)
    slots_dev = torch.from_numpy(slots).cuda()
    pools = []
    for _ in range(args.layers):
        if dense:
            pools.append({"pool": torch.zeros((w.n_slots, w.heads, w.d_k, w.d_v),
                                              dtype=torch.float32, device="cuda")})
            continue
        dp = sq.device_plan(plan)
        pool = torch.empty(sq.sq_pool_bytes(plan, w.n_slots), dtype=torch.uint8, device="cuda")
        sq.sq_pool_init(plan, dp, pool, w.n_slots)
        pools.append({"plan": plan, "dev_plan": dp, "pool": pool})
    build_state(sq, w, pools, slots_dev,
                w.warmup_steps if args.state_warmup is None else args.state_warmup)
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    params = SI.gate_params(w)
    sets = []
    for i in range(args.input_sets):
        inp = SI.step_inputs(w, i, params)
        sets.append({k: torch.from_numpy(v).cuda() for k, v in inp.items()})
    y = torch.empty((args.input_sets, w.batch, w.heads, w.d_v), dtype=torch.float32,
                    device="cuda")
    stream = torch.cuda.current_stream()
    kind = 0 if w.kind == "gdn" else 1

    def step(i, st=None):
        st = stream if st is None else st
        pl = pools[i % len(pools)]
        s = sets[i % len(sets)]
        if dense:
            sq.sq_dense_step(kind, w.heads, w.d_k, w.d_v, pl["pool"], w.n_slots, slots_dev,
                             w.batch, s["q"], s["k"], s["v"], s["beta"], s["gate"],
                             y[i % len(sets)], st)
        else:
            sq.sq_decode_step(plan, pl["dev_plan"], pl["pool"], w.n_slots, slots_dev, w.batch,
                              s["q"], s["k"], s["v"], s["beta"], s["gate"], y[i % len(sets)],
                              st)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    graph = None
    if not args.eager:
        # the K timed steps captured once as a HIP graph (the same launches,
        # arguments and in-place pool updates); one untimed replay first
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for i in range(args.steps):
                step(args.warmup + i, cap)
        graph.replay()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    del graph

    # per-launch durations with events on the launch stream (second pass)
    n_ev = min(args.steps, 64)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_ev)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    return {"desc": desc, "pools": pools, "slots": slots, "ms_per_step": ms_per_step,
            "launch_ms": launch_ms, "abytes": algorithmic_bytes(desc, w)}


VALU_PEAK = 256 * 4 * 16 * 2.4e9   # non-packed fp32 lane-ops/s: CUs x SIMDs x lanes x clock


def measure_prefill(sq, w, args) -> dict:
    """One chunk of T tokens for every sequence of the workload's batch, on
    dense fp32 states (sq_prefill_chunk, the middle step between
    sq_pool_unpack and sq_pool_pack).  The chunk is arithmetic-bound: four
    fp32 lane-ops per state element and token (decayed update, write term,
    readout, next key retrieval)."""
    import torch
    from synth import inputs as SI
    T, B, H, dk, dv = args.prefill, w.batch, w.heads, w.d_k, w.d_v
    params = SI.gate_params(w)
    steps = [SI.step_inputs(w, t, params) for t in range(T)]
    x = {k: torch.from_numpy(np.ascontiguousarray(np.stack([st[k] for st in steps], axis=1))).cuda()
         for k in steps[0]}
    del steps
    S = torch.zeros((B, H, dk, dv), dtype=torch.float32, device="cuda")
    y = torch.empty((B, T, H, dv), dtype=torch.float32, device="cuda")
    kind = 0 if w.kind == "gdn" else 1

    def chunk():
        sq.sq_prefill_chunk(kind, H, dk, dv, B, T, S, x["q"], x["k"], x["v"], x["beta"],
                            x["gate"], y)

    for _ in range(max(args.warmup // 10, 1)):
        chunk()
    torch.cuda.synchronize()
    n = max(args.steps // 32, 2)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(n):
        chunk()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / n
    ops = 4.0 * dk * dv * B * H * T
    return {"metric": "prefill tokens/s (one chunk per sequence, state in registers)",
            "value": B * T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": n,
            "warmup": max(args.warmup // 10, 1), "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": w.name, "batch": B, "heads": H, "d_k": dk, "d_v": dv,
                       "kind": w.kind, "chunk_tokens": T},
            "roofline": {"bound": "alu", "achieved": ops / (ms * 1e-3) / 1e12,
                         "peak": VALU_PEAK / 1e12, "unit": "T lane-ops/s",
                         "frac": ops / (ms * 1e-3) / VALU_PEAK, "traffic": None,
                         "kernel": "prefill_kernel<d_k,d_v>", "launch_ms": ms,
                         "ops_per_launch": ops}}


def same_hardware(sq, args, value: float) -> dict:
    """The pool workload's shape (same batch, slots, heads, d, inputs and
    timing protocol) with the fp32 state kept dense, and with uniform rowwise
    INT4: the denominators of the packed path's speed-up on this GPU.  Then
    the 6-bit plan of the mid workload at batch 512 against the fp32 state of
    that shape (the setting of the pages' 6-bit, batch-512 comparison)."""
    import torch
    from synth import inputs as SI
    res = {}
    for key, name in (("fp32_dense", "gdn_pool_fp32"), ("uniform_int4", "gdn_pool_int4"),
                      ("step6_b512", "gdn_b512_step6"), ("fp32_dense_b512", "gdn_b512_fp32")):
        w = SI.workload(name)
        m = measure(sq, w, args)
        res[key] = {"workload": name, "steps_per_s": 1e3 / m["ms_per_step"],
                    "ms_per_step": m["ms_per_step"], "launch_ms": m["launch_ms"],
                    "algorithmic_bytes_per_step": m["abytes"],
                    "achieved_gbs": m["abytes"] / (m["launch_ms"] * 1e-3) / 1e9,
                    "kernel": KERNEL[w.mode]}
        del m
        torch.cuda.empty_cache()
    res["speedup_vs_fp32_dense"] = value / res["fp32_dense"]["steps_per_s"]
    res["speedup_vs_uniform_int4"] = value / res["uniform_int4"]["steps_per_s"]
    res["speedup_step6_b512_vs_fp32_dense"] = (res["step6_b512"]["steps_per_s"]
                                              / res["fp32_dense_b512"]["steps_per_s"])
    return res


# the fp32-dense workload of the same shape, inputs and gates as a packed one
DENSE_TWIN = {"kda_step6": "kda_fp32", "gdn_window16": "gdn_window_fp32",
              "gdn_window16_r4": "gdn_window_fp32"}


def dense_twin(sq, args, value: float, name: str) -> dict:
    """The workload's shape (batch, slots, heads, d, inputs, gates, timing
    protocol) with the fp32 state kept dense: the denominator of the packed
    step's speed-up on this GPU."""
    import torch
    from synth import inputs as SI
    w = SI.workload(name)
    m = measure(sq, w, args)
    dense = {"workload": name, "steps_per_s": 1e3 / m["ms_per_step"], "ms_per_step": m["ms_per_step"],
             "launch_ms": m["launch_ms"], "algorithmic_bytes_per_step": m["abytes"],
             "achieved_gbs": m["abytes"] / (m["launch_ms"] * 1e-3) / 1e9, "kernel": KERNEL["dense"]}
    del m
    torch.cuda.empty_cache()
    return {"fp32_dense": dense, "speedup_vs_fp32_dense": value / dense["steps_per_s"]}


if __name__ == "__main__":
    main()
