"""CPU oracle of the quantized recurrent-state decode step.  TEST INFRASTRUCTURE.

A plain, slow, float64 numpy implementation of what the library computes,
written from the pages (STEPQuant: When and Where Errors Matter in Delta-Rule
Recurrent State Quantization; the LeapQuant reading notes; the Korean summary
of STEPQuant).  Only the tests, the smoke entry point and the bench's CPU
baseline leg may import it; the library and its binding never do, and it
shares no code, header, table or helper with them.

Modules:
  numerics     rounding helpers (fp16 with scale clamp, rne, q_b)
  recurrence   gated delta rule, transition A_t, transported query g_t
  quantizers   uniform rowwise INT-b, dual-axis STEP quantizer, smoothed INT8
  step         one quantized decode step (uniform / STEP)
  window       per-window variant: records, windowed readout, flush
  calibration  lifetime weights, impact factors, pivots, greedy allocation
  layout       independent packer/parser of the slot layout

Parity unpinned (only self-consistency and brute force pin these): the
distortion estimator d_u(b) used for allocation, the 2-bit candidate in the
4-bit candidate set, the resulting allocations, and the synthetic magnitude
structure of the KDA workload.
"""
from . import calibration, layout, numerics, quantizers, recurrence, step, window  # noqa: F401
