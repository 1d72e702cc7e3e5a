"""Write the calibration statistics of the STEP workloads (calls only the oracle
and the seeded input generators).

STEPQuant calibrates offline on a separate stream (Sec. 5.1: segments of 2048
tokens): per unit the mean log retention l_u and the distortion d_u(b) at each
candidate width, per key row the row-impact score omega_i.  The library's
sq_calibrate_bits turns these into bit widths, pivots and impact factors.

usage: python tests/golden/make_calib_stats.py <workload> [...]
writes tests/golden/calib_<workload>.json
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import calibration as C  # noqa: E402
from synth import inputs as SI  # noqa: E402


def main(name: str) -> None:
    w = SI.workload(name)
    params = SI.gate_params(w)
    st = C.collect_stats(w.kind, w.heads, w.d_k, w.d_v, w.calib_steps,
                         lambda t: SI.calib_inputs(w, t, params), w.cand_bits,
                         snapshot_start=w.calib_snapshot_start,
                         snapshot_every=w.calib_snapshot_every, gamma=w.gamma)
    out = {
        "source": "oracle.calibration.collect_stats on the seeded calibration stream "
                  f"(seed {w.seed + 1000}, {w.calib_seqs} sequences x {w.calib_steps} steps)",
        "workload": name, "kind": w.kind, "heads": w.heads, "d_k": w.d_k, "d_v": w.d_v,
        "cand_bits": list(w.cand_bits), "nominal_bits": w.nominal_bits,
        "pivot_frac": w.pivot_frac, "gamma": w.gamma, "horizon": w.calib_horizon,
        "snapshots": int(st["snapshots"]),
        "ell": [float(x) for x in st["ell"]],
        "dist": [[float(x) for x in row] for row in st["dist"]],
        "omega": [[float(x) for x in row] for row in st["omega"]],
    }
    with open(os.path.join(HERE, f"calib_{name}.json"), "w") as f:
        json.dump(out, f)


if __name__ == "__main__":
    for n in sys.argv[1:]:
        main(n)
