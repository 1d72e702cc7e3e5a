"""The allocation-free distortion entry point (sq_calib_distortion_noalloc)
against sq_calib_distortion with a caller-owned scratch buffer, through the C
ABI: two calls in a row on the same GPU, the second with fewer sequences
(the library's array keeps the first call's bytes), per head and per key
row, and the refusal of a call that needs more scratch than the array holds.
The distortion sums are float64 with atomic adds in no fixed order, so the
two entry points agree to float64 rounding, not bit for bit."""
import numpy as np
import pytest

import quantized_recurrent_state_decode_amd as sq
from oracle import calibration as C

from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("per_row", [False, True])
def test_noalloc_distortion_matches_caller_scratch(per_row):
    import torch
    rng = np.random.default_rng(123)
    H, d = 5, 128
    wts = C.impact_factors(rng.lognormal(0.0, 1.5, (H, d))).astype(np.float32)
    plan = sq.sq_plan_create_step(sq.SQ_KIND_GDN, H, d, d, [2, 4, 6, 8, 4], wts)
    dp = sq.device_plan(plan)
    mhb = sq.sq_max_head_bytes(plan)
    U = H * d if per_row else H
    for n in (7, 3):                       # the second call is smaller
        S = (rng.standard_normal((n, H, d, d)) * rng.lognormal(0, 1, (n, H, d, 1))
             * rng.lognormal(0, 1, (n, H, 1, d))).astype(np.float32)
        S_dev = to_dev(S)
        packed = torch.zeros(n * H * mhb, dtype=torch.uint8, device="cuda")
        ref = torch.zeros(U, dtype=torch.float64, device="cuda")
        got = torch.zeros(U, dtype=torch.float64, device="cuda")
        sq.sq_calib_distortion(plan, dp, n, S_dev, packed, per_row, ref)
        sq.sq_calib_distortion_noalloc(plan, dp, n, S_dev, per_row, got)
        torch.cuda.synchronize()
        r, g = ref.cpu().numpy(), got.cpu().numpy()
        assert np.all(r > 0)
        np.testing.assert_allclose(g, r, rtol=1e-12, atol=0)


def test_noalloc_refuses_beyond_its_scratch():
    import torch
    rng = np.random.default_rng(124)
    H, d = 4, 128
    wts = C.impact_factors(rng.lognormal(0.0, 1.0, (H, d))).astype(np.float32)
    plan = sq.sq_plan_create_step(sq.SQ_KIND_GDN, H, d, d, [8, 8, 8, 8], wts)
    dp = sq.device_plan(plan)
    mhb = sq.sq_max_head_bytes(plan)
    n_max = (16 << 20) // (H * mhb)
    S = torch.zeros((1, H, d, d), dtype=torch.float32, device="cuda")
    dist = torch.zeros(H, dtype=torch.float64, device="cuda")
    with pytest.raises(sq.StepqError) as e:
        # refused on the host from the sizes alone, before anything reads S
        sq.sq_calib_distortion_noalloc(plan, dp, n_max + 1, S, False, dist)
    assert e.value.status == sq.SQ_EINVAL
    assert "limit" in sq.sq_last_error() or "limit" in str(e.value)
    torch.cuda.synchronize()
    assert np.all(dist.cpu().numpy() == 0)
