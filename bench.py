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
DEFAULT_WORKLOAD = "gdn_pool_step4"


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


def _state_key(w, steps):
    """Workloads whose warm-up states are identical (same seed, shape, gates,
    gains and batch) share one build."""
    return (w.kind, w.seed, w.batch, w.heads, w.d_k, w.d_v, w.half_life, w.half_life_range,
            w.key_gain_sigma, w.value_gain_sigma, steps)


def magnitude_contrast(S) -> dict:
    """Maximum-to-median RMS contrast of each state tile over key rows
    (sqrt(mean_j S_ij^2)) and over value columns, median linearly
    interpolated (STEPQuant Sec. 4.2 and appendix B); the median over tiles."""
    import torch
    r = S.pow(2).mean(-1).sqrt()
    c = S.pow(2).mean(-2).sqrt()
    rc = r.amax(-1) / torch.quantile(r, 0.5, dim=-1)
    cc = c.amax(-1) / torch.quantile(c, 0.5, dim=-1)
    return {"key_rows": float(torch.quantile(rc.flatten(), 0.5)),
            "value_columns": float(torch.quantile(cc.flatten(), 0.5)),
            "tiles": int(rc.numel())}


def build_state(sq, w, pools, slots_dev, steps, cache=None):
    """Warm-up state: `steps` fp32 dense steps from S = 0 with the library's
    dense kernel, then packed into every pool.  Returns the state's magnitude
    contrast."""
    import torch
    from synth import inputs as SI
    key = _state_key(w, steps)
    if cache is not None and key in cache:
        S, contrast = cache[key]
    else:
        params = SI.gate_params(w)
        S = torch.zeros((w.batch, w.heads, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
        ident = torch.arange(w.batch, dtype=torch.int32, device="cuda")
        y = torch.empty((w.batch, w.heads, w.d_v), dtype=torch.float32, device="cuda")
        for t in range(steps):
            inp = {k: torch.from_numpy(v).cuda() for k, v in SI.warmup_inputs(w, t, params).items()}
            sq.sq_dense_step(0 if w.kind == "gdn" else 1, w.heads, w.d_k, w.d_v, S, w.batch, ident,
                             w.batch, inp["q"], inp["k"], inp["v"], inp["beta"], inp["gate"], y)
        contrast = magnitude_contrast(S) if steps > 0 else None
        if cache is not None:
            cache[key] = (S, contrast)
    for pl in pools:
        if w.mode == "dense":
            pl["pool"].index_copy_(0, slots_dev.long(), S)
        else:
            sq.sq_pool_pack(pl["plan"], pl["dev_plan"], pl["pool"], w.n_slots, slots_dev, w.batch, S)
    torch.cuda.synchronize()
    return contrast


def _oracle_steps(w, od, states, sets, n_steps, deadline):
    """Decode steps of the float64 oracle on parsed slot states (a list of
    per-slot head lists), free-running from the packed state it was given;
    step t reads input set t % len(sets), whose batch rows are the states'
    slots in order (inputs are made before the clock starts, as the GPU's
    are resident).  Returns the number of (slot, head) tiles done before the
    deadline."""
    from oracle import quantizers as Q
    from oracle import recurrence as R
    from oracle import window as OW
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import row_bits_of
    tiles = 0
    for step in range(n_steps):
        inp = sets[step % len(sets)]
        for b, sl in enumerate(states):
            for h in range(w.heads):
                if time.perf_counter() > deadline:
                    return tiles
                st = sl[h]
                q, k, v = (inp[x][b, h] for x in ("q", "k", "v"))
                beta = float(inp["beta"][b, h])
                if w.mode == "window":
                    r = OW.window_step(st, q, k, v, beta, float(inp["gate"][b, h]), w.window,
                                       w.power_iters)
                    sl[h] = r["state"]
                    tiles += 1
                    continue
                dvec = R.gate_vector(inp["gate"][b, h], "gdn" if w.mode == "uniform" else w.kind,
                                     w.d_k)
                if w.mode == "uniform":
                    S_hat = Q.dequant_uniform(st["z"], st["s"])
                    X = R.delta_update(R.retained(S_hat, dvec), k, v, beta)
                    R.readout(X, q)
                    e = Q.quantize_uniform(X, w.bits)
                    sl[h] = {"z": e["z"], "s": e["s"]}
                else:
                    rb = row_bits_of(od, h)
                    S_hat = Q.dequant_step(st["z"], st["r"], st["c"], rb, st["h"])
                    X = R.delta_update(R.retained(S_hat, dvec), k, v, beta)
                    R.readout(X, q)
                    e = Q.quantize_step(X, od["w"][h], rb)
                    sl[h] = {"z": e["z"], "r": e["r"], "c": e["c"], "h": e["h"]}
                tiles += 1
    return tiles


def _rows(sets, idx):
    """The given batch rows of each input set, widened to float64."""
    return [{k: np.asarray(v[idx], dtype=np.float64) for k, v in st.items()} for st in sets]


def _cpu_worker(job):
    """One process of the multi-core oracle run: parse its slots from the
    shared host copy of the pool, then run the sampled decode steps."""
    from oracle import layout as OL
    from synth import inputs as SI
    w = SI.workload(job["workload"])
    od = job["od"]
    buf = np.load(job["path"], mmap_mode="r")
    sb = job["slot_bytes"]
    states = [OL.parse_slot(od, bytes(buf[i * sb:(i + 1) * sb])) for i in job["slots"]]
    t0 = time.perf_counter()
    tiles = _oracle_steps(w, od, states, job["sets"], job["steps"], t0 + job["budget_s"])
    return tiles, time.perf_counter() - t0


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, desc, host: np.ndarray, sample_slots: int, steps: int, budget_s: float,
                 single_s: float) -> dict:
    """The float64 oracle, as it stands, on a bounded sample of the same
    workload, free-running from the GPU's packed state: `steps` decode steps
    of the first `sample_slots` live slots (all heads) over every host core
    available to this process (a process pool, one BLAS thread per worker),
    then one slot on one core.  Step t reads the GPU loop's input set t % 8,
    made before the clock starts.  Reported as equivalent full-batch steps/s."""
    import multiprocessing as mp
    import tempfile
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import layout as OL
    from parity import oracle_desc
    od = oracle_desc(desc)
    if desc.get("w") is not None:
        od["w"] = desc["w"].astype(np.float64)
    sb = desc["slot_bytes"]
    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(16, affinity))
    full = w.batch * w.heads
    res = {"unit": "steps/s", "kind": "oracle", "cpu_model": _cpu_model(),
           "affinity_cpus": affinity}
    from synth import inputs as SI
    params = SI.gate_params(w)
    sets = [SI.step_inputs(w, i, params) for i in range(8)]   # the GPU loop's 8 input sets
    # single core: one slot, all heads, until the budget is spent
    states = [OL.parse_slot(od, host[:sb].tobytes())]
    t0 = time.perf_counter()
    tiles = _oracle_steps(w, od, states, _rows(sets, [0]), 1 << 30, t0 + single_s)
    dt = time.perf_counter() - t0
    single = {"value": tiles / dt / full, "cores": 1, "tiles": tiles, "seconds": dt,
              "sample": f"1 slot x {w.heads} heads, {tiles} tiles in {dt:.1f} s, one process"}
    # every core: sample_slots slots x all heads x `steps` steps, split by slot
    n = min(sample_slots, host.size // sb)
    with tempfile.TemporaryDirectory(dir="/tmp") as tmp:
        path = os.path.join(tmp, "slots.npy")
        np.save(path, host[:n * sb])
        jobs = [{"workload": w.name, "od": od, "path": path, "slot_bytes": sb,
                 "slots": list(range(k, n, workers)), "sets": _rows(sets[:max(1, steps)], list(range(k, n, workers))),
                 "steps": steps, "budget_s": budget_s} for k in range(workers)]
        env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                              "MKL_NUM_THREADS")}
        for k in env:
            os.environ[k] = "1"
        try:
            ctx = mp.get_context("forkserver")
            t0 = time.perf_counter()
            with ctx.Pool(workers) as pool:
                out = pool.map(_cpu_worker, jobs)
            dt = time.perf_counter() - t0
        finally:
            for k, v in env.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    tiles = sum(o[0] for o in out)
    busy = max(o[1] for o in out)
    res.update({"value": tiles / busy / full, "cores": workers, "tiles": tiles,
                "seconds": busy, "wall_seconds_with_startup": dt,
                "sample": f"{n} slots x {w.heads} heads x {steps} steps ({tiles} tiles done) "
                          f"over {workers} worker processes (one BLAS thread each) in "
                          f"{busy:.1f} s, float64 numpy; value = tiles/s / ({w.batch} x "
                          f"{w.heads}) tiles per step",
                "single_core": single})
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--runs", type=int, default=3,
                    help="timed runs of K steps each; the median is reported")
    ap.add_argument("--spin-ms", type=float, default=500.0,
                    help="after the W warm-up steps, keep launching untimed steps until this "
                         "much wall time has passed (clocks at steady state before timing)")
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed steps one by one instead of replaying them as a HIP graph")
    ap.add_argument("--input-sets", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=25.0,
                    help="time budget of the multi-core oracle run")
    ap.add_argument("--cpu-single-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads' block (mid, KDA, window, tiny)")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the same-hardware runs: fp32-dense and uniform-INT4 at the pool "
                         "workload's shape, fp32-dense at the KDA and window shapes")
    ap.add_argument("--state-warmup", type=int, default=None,
                    help="fp32 steps that build the initial state (default: the workload's 128)")
    ap.add_argument("--prefill", type=int, default=0, metavar="T",
                    help="measure the prefill instead: one chunk of T tokens per sequence over "
                         "the workload's batch and heads (tokens/s), the matrix form "
                         "(sq_prefill_chunkwise) with the token-serial form beside it")
    ap.add_argument("--prefill-form", choices=("both", "chunkwise", "serial"), default="both",
                    help="which prefill form(s) --prefill times")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill block of the default line (both prefill forms on the "
                         "64 x 16-head GDN and 64 x 32-head KDA shapes)")
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
    cache = {}
    m = measure(sq, w, args, cache=cache)
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
                   "timing": m["timing"],
                   "state_gbs": gbs_step, "pct_of_hbm_peak": 100.0 * gbs_step / HBM_PEAK_GBS},
        "roofline": {"bound": "hbm", "achieved": gbs_kernel, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs_kernel / HBM_PEAK_GBS,
                     "traffic": measured_traffic(w.name, family),
                     "kernel": KERNEL[w.mode if w.kind == "gdn" else "kda"],
                     "kernel_source_sha256_16": kernel_source_hash(family),
                     "launch_ms": launch_ms, "bytes_per_launch": abytes,
                     "launch": "one decode call = one kernel launch (sq_decode_step, or "
                               "sq_dense_step in dense mode); duration = HIP events on the launch "
                               "stream around the K-launch graph replay, divided by K (median of "
                               "the timed runs)"},
    }
    if m["contrast"] is not None and w.kind == "kda":
        out["config"]["state_contrast"] = m["contrast"]
    valu = measured_valu(w.name, family)
    if valu is not None:
        # the issue rate the decode launch sustains: 64 lanes per VALU
        # instruction over the launch, against the chip's non-packed lane rate
        lane_ops = 64.0 * valu / (launch_ms * 1e-3)
        out["roofline"]["alu_issue"] = {"achieved": lane_ops / 1e12, "peak": VALU_PEAK / 1e12,
                                        "unit": "T lane-ops/s", "frac": lane_ops / VALU_PEAK,
                                        "valu_instructions_per_launch": valu}
    host = None
    if not args.no_cpu and desc is not None:
        torch.cuda.synchronize()
        sb = desc["slot_bytes"]
        pb = m["pools"][0]["pool"]
        # the live slots in batch order, as host bytes
        idx = torch.from_numpy(m["slots"].astype(np.int64)).cuda()
        host = pb[:w.n_slots * sb].view(w.n_slots, sb).index_select(0, idx).cpu().numpy().reshape(-1)
    del m
    torch.cuda.empty_cache()
    if w.name == DEFAULT_WORKLOAD and not args.no_configs:
        out["configs"] = configs_block(sq, args, cache)
        out["cache_assisted"] = cache_assisted(sq, args, cache)
    if w.name == DEFAULT_WORKLOAD and not args.no_prefill:
        out["prefill"] = prefill_block(sq, args)
    if w.name == DEFAULT_WORKLOAD and not args.no_compare:
        out["same_hardware"] = same_hardware(sq, args, out["value"], cache)
    elif w.name in DENSE_TWIN and not args.no_compare:
        out["same_hardware"] = dense_twin(sq, args, out["value"], DENSE_TWIN[w.name], cache)
    cache.clear()
    torch.cuda.empty_cache()
    if host is not None:
        cb = cpu_baseline(w, desc, host, w.batch, 2, args.cpu_seconds, args.cpu_single_seconds)
        if cb.get("value"):
            # the same algorithmic bytes per step, and the GPU line over it
            cb["equivalent_gbs"] = cb["value"] * abytes / 1e9
            cb["gpu_over_cpu"] = out["value"] / cb["value"]
        if isinstance(cb.get("single_core"), dict) and cb["single_core"].get("value"):
            cb["single_core"]["equivalent_gbs"] = cb["single_core"]["value"] * abytes / 1e9
        out["cpu_baseline"] = cb
    print(json.dumps(out))


def measure(sq, w, args, steps=None, cache=None) -> dict:
    """Time K consecutive decode steps of workload w, K = `steps` (default
    args.steps), rotating args.layers independent pools so that the live state
    exceeds the on-package cache.  Protocol: args.warmup untimed steps, untimed
    steps until args.spin_ms of wall time has passed, then args.runs timed
    runs of exactly K steps, each between device synchronisations and timed
    with HIP events on the launch stream; the median run is reported.  A
    second pass times 64 single calls for the per-launch duration."""
    import torch
    from synth import inputs as SI
    K = args.steps if steps is None else steps
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
    contrast = build_state(sq, w, pools, slots_dev,
                           w.warmup_steps if args.state_warmup is None else args.state_warmup,
                           cache)
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
        # arguments and in-place pool updates)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for i in range(K):
                step(args.warmup + i, cap)

    def run():
        if graph is not None:
            graph.replay()
        else:
            for i in range(K):
                step(args.warmup + i)

    # untimed runs until the clocks have settled
    t0 = time.perf_counter()
    spins = 0
    while True:
        run()
        torch.cuda.synchronize()
        spins += 1
        if time.perf_counter() - t0 >= args.spin_ms * 1e-3:
            break
    runs = []
    for _ in range(max(1, args.runs)):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        run()
        end.record(stream)
        torch.cuda.synchronize()
        runs.append(start.elapsed_time(end) / K)
    ms_per_step = float(np.median(runs))
    graph_ok = graph is not None
    del graph

    # per-launch durations with events on the launch stream (second pass)
    n_ev = min(K, 64)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_ev)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    eager_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    # every decode step here is one kernel launch, so in the graph replay the
    # launch duration is the timed region over K (back-to-back launches, no
    # host gaps); eager launches each carry the host's launch gap
    launch_ms = eager_ms if graph_ok is False else ms_per_step
    timing = {"K": K, "runs_ms_per_step": runs, "median_ms_per_step": ms_per_step,
              "spin_runs": spins, "spin_s": time.perf_counter() - t0,
              "eager_launch_ms": eager_ms}
    return {"desc": desc, "pools": pools, "slots": slots, "ms_per_step": ms_per_step,
            "launch_ms": launch_ms, "abytes": algorithmic_bytes(desc, w), "timing": timing,
            "contrast": contrast}


VALU_PEAK = 256 * 4 * 16 * 2.4e9   # non-packed fp32 lane-ops/s: CUs x SIMDs x lanes x clock


MFMA_F32_PEAK = 157.3e12           # dense fp32 matrix-core FLOP/s (published)


def measure_prefill(sq, w, args) -> dict:
    """One chunk of T tokens for every sequence of the workload's batch, on
    dense fp32 states (the middle step between sq_pool_unpack and
    sq_pool_pack).  The matrix form (sq_prefill_chunkwise) is priced against
    the fp32 matrix-core peak by its three state products, W S, (Q o g) S and
    (K o G)^T U: 6 d_k d_v FLOP per token and tile (the intra-block L U, A
    and L and the triangular solves are not counted).  The token-serial form
    (sq_prefill_chunk) is priced against the vector issue peak by its four
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
    n = max(args.steps // 32, 2)
    warm = max(args.warmup // 10, 1)

    def timed(fn) -> float:
        def chunk():
            fn(kind, H, dk, dv, B, T, S, x["q"], x["k"], x["v"], x["beta"], x["gate"], y)
        for _ in range(warm):
            chunk()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(n):
            chunk()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n

    ops = 4.0 * dk * dv * B * H * T
    flops = 6.0 * dk * dv * B * H * T
    serial = None
    if args.prefill_form in ("both", "serial"):
        ms = timed(sq.sq_prefill_chunk)
        serial = {"kernel": "prefill_kernel<d_k,d_v>", "tokens_per_s": B * T / (ms * 1e-3),
                  "launch_ms": ms,
                  "roofline": {"bound": "alu", "achieved": ops / (ms * 1e-3) / 1e12,
                               "peak": VALU_PEAK / 1e12, "unit": "T lane-ops/s",
                               "frac": ops / (ms * 1e-3) / VALU_PEAK, "traffic": None,
                               "ops_per_launch": ops}}
    out = {"metric": "prefill tokens/s (one chunk per sequence, state in registers)",
           "n_gpus": 1, "steps": n, "warmup": warm, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "batch": B, "heads": H, "d_k": dk, "d_v": dv,
                      "kind": w.kind, "chunk_tokens": T}}
    if args.prefill_form == "serial":
        out.update({"value": serial["tokens_per_s"], "unit": "tokens/s",
                    "ms_per_step": serial["launch_ms"], "form": "serial",
                    "roofline": dict(serial["roofline"], kernel=serial["kernel"],
                                     launch_ms=serial["launch_ms"])})
        return out
    ms = timed(sq.sq_prefill_chunkwise)
    kname = "chunk_prefill_kernel<d_k,d_v,%s>" % ("true" if kind else "false")
    out.update({"value": B * T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
                "form": "chunkwise",
                "roofline": {"bound": "mfma", "achieved": flops / (ms * 1e-3) / 1e12,
                             "peak": MFMA_F32_PEAK / 1e12, "unit": "TFLOP/s",
                             "frac": flops / (ms * 1e-3) / MFMA_F32_PEAK, "traffic": None,
                             "kernel": kname, "launch_ms": ms, "flops_per_launch": flops}})
    if serial is not None:
        out["serial"] = serial
        out["chunkwise_over_serial"] = serial["launch_ms"] / ms
    return out


def _summary(w, m, kernel) -> dict:
    """steps/s (median run), GB/s per step and per launch, % of the HBM peak."""
    gbs = m["abytes"] / (m["ms_per_step"] * 1e-3) / 1e9
    out = {"workload": w.name, "batch": w.batch, "heads": w.heads, "d_k": w.d_k, "d_v": w.d_v,
           "mode": w.mode, "steps_per_s": 1e3 / m["ms_per_step"], "ms_per_step": m["ms_per_step"],
           "launch_ms": m["launch_ms"], "algorithmic_bytes_per_step": m["abytes"],
           "state_gbs": gbs, "pct_of_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
           "launch_gbs": m["abytes"] / (m["launch_ms"] * 1e-3) / 1e9,
           "timing": m["timing"], "kernel": kernel}
    if m["desc"] is not None and m["desc"]["unit_bits"] is not None:
        out["unit_bits_histogram"] = {str(b): int(c) for b, c in
                                      zip(*np.unique(m["desc"]["unit_bits"], return_counts=True))}
    if w.mode == "window":
        out["window"] = w.window
        out["comp_rank"] = w.comp_rank
    if m["contrast"] is not None and w.kind == "kda":
        out["state_contrast"] = m["contrast"]
    return out


# the other workloads reported beside the headline, with the K each one times
# (a multiple of layers x window for the window path, so that every timed run
# holds exactly one rebuild per layer pool)
CONFIGS = (("tiny_gdn_int8", 256, 1), ("gdn_mid_step6", 256, None), ("kda_step6", 64, None),
           ("gdn_window16", 64, None), ("gdn_window16_r4", 64, None))


def configs_block(sq, args, cache) -> dict:
    """The tiny uniform INT8 case, the mid GDN plan, KDA and the per-window
    path (without and with compensator tokens), each by the same protocol."""
    import argparse as _ap
    import torch
    from synth import inputs as SI
    res = {}
    for name, K, layers in CONFIGS:
        w = SI.workload(name)
        a = _ap.Namespace(**vars(args))
        if layers is not None:
            a.layers = layers
        K = max(K, args.steps) if w.mode != "window" else K * max(1, -(-args.steps // K))
        m = measure(sq, w, a, steps=K, cache=cache)
        kern = KERNEL["window"] if w.mode == "window" else KERNEL[
            w.mode if w.kind == "gdn" else "kda"]
        res[name] = _summary(w, m, kern)
        if name == "tiny_gdn_int8":
            res[name]["note"] = "one 64 x 64 tile per step: launch-latency bound, steps/s only"
        del m
        torch.cuda.empty_cache()
    return res


def prefill_block(sq, args) -> list:
    """The prefill chunk beside the decode line: both forms (matrix form on
    the fp32 matrix cores, token-serial on the vector units) on one chunk per
    sequence, 8 timed launches each."""
    import argparse as _ap
    import torch
    from synth import inputs as SI
    res = []
    for name, over, T in (("gdn_mid_step6", {}, 256),
                          ("kda_step6", {"batch": 64, "n_slots": 64}, 128)):
        a = _ap.Namespace(**vars(args))
        a.prefill, a.prefill_form, a.steps, a.warmup = T, "both", 256, 50
        r = measure_prefill(sq, SI.workload(name, **over), a)
        res.append({"config": r["config"], "tokens_per_s": r["value"], "launch_ms": r["ms_per_step"],
                    "roofline": r["roofline"], "serial": r["serial"],
                    "chunkwise_over_serial": r["chunkwise_over_serial"]})
        torch.cuda.empty_cache()
    return res


def cache_assisted(sq, args, cache) -> dict:
    """The headline workload on a single pool, without layer rotation: its
    222 MB of packed state can stay in the 256 MB on-package cache between
    steps.  Reported apart from the headline, which rotates args.layers pools
    so that every step reads its state from HBM."""
    import argparse as _ap
    import torch
    from synth import inputs as SI
    w = SI.workload(DEFAULT_WORKLOAD)
    a = _ap.Namespace(**vars(args))
    a.layers = 1
    m = measure(sq, w, a, cache=cache)
    res = _summary(w, m, KERNEL[w.mode if w.kind == "gdn" else "kda"])
    res["layers_rotated"] = 1
    res["label"] = "cache-assisted"
    del m
    torch.cuda.empty_cache()
    return res


def same_hardware(sq, args, value: float, cache=None) -> dict:
    """The pool workload's shape (same batch, slots, heads, d, inputs and
    timing protocol) with the fp32 state kept dense, and with uniform rowwise
    INT4: the denominators of the packed path's speed-up on this GPU.  Then
    the 6-bit plan of the mid workload at batch 512 against the fp32 state of
    that shape (the setting of the pages' 6-bit, batch-512 comparison), and the
    fp32 state at the KDA and window shapes."""
    import torch
    from synth import inputs as SI
    res = {}
    for key, name in (("fp32_dense", "gdn_pool_fp32"), ("uniform_int4", "gdn_pool_int4"),
                      ("step6_b512", "gdn_b512_step6"), ("fp32_dense_b512", "gdn_b512_fp32"),
                      ("fp32_dense_kda", "kda_fp32"), ("fp32_dense_window", "gdn_window_fp32")):
        w = SI.workload(name)
        m = measure(sq, w, args, cache=cache)
        res[key] = {"workload": name, "steps_per_s": 1e3 / m["ms_per_step"],
                    "ms_per_step": m["ms_per_step"], "launch_ms": m["launch_ms"],
                    "algorithmic_bytes_per_step": m["abytes"],
                    "achieved_gbs": m["abytes"] / (m["launch_ms"] * 1e-3) / 1e9,
                    "pct_of_hbm_peak": 100.0 * m["abytes"] / (m["launch_ms"] * 1e-3) / 1e9
                    / HBM_PEAK_GBS,
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


def dense_twin(sq, args, value: float, name: str, cache=None) -> dict:
    """The workload's shape (batch, slots, heads, d, inputs, gates, timing
    protocol) with the fp32 state kept dense: the denominator of the packed
    step's speed-up on this GPU."""
    import torch
    from synth import inputs as SI
    w = SI.workload(name)
    m = measure(sq, w, args, cache=cache)
    dense = {"workload": name, "steps_per_s": 1e3 / m["ms_per_step"], "ms_per_step": m["ms_per_step"],
             "launch_ms": m["launch_ms"], "algorithmic_bytes_per_step": m["abytes"],
             "achieved_gbs": m["abytes"] / (m["launch_ms"] * 1e-3) / 1e9, "kernel": KERNEL["dense"]}
    del m
    torch.cuda.empty_cache()
    return {"fp32_dense": dense, "speedup_vs_fp32_dense": value / dense["steps_per_s"]}


if __name__ == "__main__":
    main()
