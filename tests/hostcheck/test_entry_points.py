"""Every device entry point driven up to its kernel launch in the checked
host build (run by ``test_hostcheck.py`` in a child process with the
sanitizer runtime preloaded).  The launchers there are stubs that check the
launch arguments and report no device, so each call must come back with
SQ_EHIP after the host logic, its bounds asserts and the sanitizers have
run; nothing is dereferenced at the placeholder addresses passed for device
buffers.  Against any other build of the library this module skips: with
real kernels those addresses would be launched on."""
import os

import numpy as np
import pytest

import quantized_recurrent_state_decode_amd as sq

pytestmark = pytest.mark.skipif(os.environ.get("SQ_HOSTCHECK_CHILD") != "1",
                                reason="runs only in the checked host build's child process")

DEV = 0x10000  # placeholder device address (never dereferenced by the stubs)
STREAM = 0


@pytest.fixture(scope="module", autouse=True)
def _checked_library():
    assert hasattr(sq.lib(), "sq_hostcheck_build"), "not the checked host build"


def _ehip(fn, *args):
    with pytest.raises(sq.StepqError) as e:
        fn(*args)
    assert e.value.status == sq.SQ_EHIP, str(e.value)


def _step_bits(rng, kind, heads, d_k, weights=(0.1, 0.4, 0.3, 0.2), pivots=1):
    n_u = heads if kind == sq.SQ_KIND_GDN else heads * d_k
    bits = rng.choice([2, 4, 6, 8], size=n_u, p=list(weights)).astype(np.int32)
    bits[rng.choice(n_u, size=pivots, replace=False)] = 16
    return bits


def _plans(rng):
    out = []
    for d_k, d_v in ((64, 64), (128, 128), (128, 64), (64, 128)):
        for b in (2, 4, 6, 8):
            out.append(("uniform", sq.sq_plan_create_uniform(4, d_k, d_v, b)))
        w = rng.lognormal(0.0, 1.0, (6, d_k)).astype(np.float32)
        out.append(("gdn", sq.sq_plan_create_step(sq.SQ_KIND_GDN, 6, d_k, d_v,
                                                  _step_bits(rng, sq.SQ_KIND_GDN, 6, d_k), w)))
        out.append(("kda", sq.sq_plan_create_step(sq.SQ_KIND_KDA, 6, d_k, d_v,
                                                  _step_bits(rng, sq.SQ_KIND_KDA, 6, d_k, pivots=9),
                                                  w)))
        out.append(("window", sq.sq_plan_create_window(3, d_k, d_v, 16)))
        out.append(("window", sq.sq_plan_create_window_lowrank(3, d_k, d_v, 8, 4, 4)))
    # the pool's shape: one width class of 45 heads (split launch at 512 slots),
    # two 2-bit heads and one FP16 head
    bits = np.full(48, 4, np.int32)
    bits[[5, 29]] = 2
    bits[17] = 16
    w = rng.lognormal(0.0, 1.0, (48, 128)).astype(np.float32)
    out.append(("gdn", sq.sq_plan_create_step(sq.SQ_KIND_GDN, 48, 128, 128, bits, w)))
    # one width only (a solo launch) and every width (the merged launch)
    out.append(("gdn", sq.sq_plan_create_step(sq.SQ_KIND_GDN, 8, 128, 128,
                                              np.full(8, 6, np.int32), w[:8])))
    out.append(("gdn", sq.sq_plan_create_step(sq.SQ_KIND_GDN, 5, 128, 128,
                                              np.array([2, 4, 6, 8, 16], np.int32), w[:5])))
    return out


@pytest.mark.parametrize("batch", [1, 3, 64, 512, 1024])
def test_every_entry_point_reaches_its_launch(batch):
    rng = np.random.default_rng(batch)
    for mode, plan in _plans(rng):
        d = sq.sq_plan_query(plan)
        n_slots = 2 * batch
        _ehip(sq.sq_decode_step, plan, DEV, DEV, n_slots, DEV, batch, DEV, DEV, DEV, DEV, DEV,
              DEV, STREAM)
        _ehip(sq.sq_pool_pack, plan, DEV, DEV, n_slots, DEV, batch, DEV, STREAM)
        _ehip(sq.sq_pool_unpack, plan, DEV, DEV, n_slots, DEV, batch, DEV, STREAM)
        _ehip(sq.sq_quantize_tiles, plan, DEV, DEV, batch * d["heads"], DEV, DEV, STREAM)
        if mode == "window":
            _ehip(sq.sq_window_flush, plan, DEV, DEV, n_slots, DEV, batch, STREAM)
        else:
            with pytest.raises(sq.StepqError) as e:
                sq.sq_window_flush(plan, DEV, DEV, n_slots, DEV, batch, STREAM)
            assert e.value.status == sq.SQ_EPLAN_MISMATCH
        # an empty batch is a no-op that touches nothing
        sq.sq_decode_step(plan, DEV, DEV, n_slots, None, 0, None, None, None, None, None, None,
                          STREAM)


@pytest.mark.parametrize("kind", [sq.SQ_KIND_GDN, sq.SQ_KIND_KDA])
def test_dense_and_prefill_reach_their_launch(kind):
    for d_k, d_v in ((64, 64), (128, 128), (128, 64), (64, 128)):
        _ehip(sq.sq_dense_step, kind, 4, d_k, d_v, DEV, 8, DEV, 8, DEV, DEV, DEV, DEV, DEV, DEV,
              STREAM)
        _ehip(sq.sq_prefill_chunk, kind, 4, d_k, d_v, 3, 17, DEV, DEV, DEV, DEV, DEV, DEV, DEV,
              STREAM)
        _ehip(sq.sq_prefill_chunkwise, kind, 4, d_k, d_v, 3, 17, DEV, DEV, DEV, DEV, DEV, DEV,
              DEV, STREAM)
