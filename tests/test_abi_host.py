"""Host-only tests of the C ABI: the library loads, exports every symbol the
header declares, and its host logic (plans, byte accounting, calibration,
argument checks) agrees with the oracle and the pages.  No GPU is touched."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from conftest import ROOT, golden
from oracle import calibration as C
from oracle import layout as L

import quantized_recurrent_state_decode_amd as sq

HEADER = os.path.join(ROOT, "include", "stepq.h")


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(sq.LIB_PATH):
        from quantized_recurrent_state_decode_amd import _build
        _build.build()


def test_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(sq_[a-z_0-9]+)\s*\(", text))
    assert declared == set(sq.EXPORTED)
    lib = ctypes.CDLL(sq.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def _desc_for_oracle(d, unit_bits=None):
    if d["mode"] == sq.SQ_MODE_UNIFORM:
        return {"mode": "uniform", "heads": d["heads"], "d_k": d["d_k"], "d_v": d["d_v"],
                "bits": d["uniform_bits"]}
    if d["mode"] == sq.SQ_MODE_WINDOW:
        return {"mode": "window", "heads": d["heads"], "d_k": d["d_k"], "d_v": d["d_v"],
                "p": d["window"], "rank": d["window_rank"]}
    ub = d["unit_bits"]
    if d["kind"] == sq.SQ_KIND_GDN:
        return {"mode": "step", "kind": "gdn", "heads": d["heads"], "d_k": d["d_k"],
                "d_v": d["d_v"], "head_bits": list(ub)}
    return {"mode": "step", "kind": "kda", "heads": d["heads"], "d_k": d["d_k"],
            "d_v": d["d_v"], "row_bits": ub.reshape(d["heads"], d["d_k"])}


@pytest.mark.parametrize("case", ["uni64", "uni128_4", "gdn", "kda", "win", "win_r4", "win_r8_64"])
def test_layout_sizes_match_independent_parser(case):
    rng = np.random.default_rng(7)
    if case == "uni64":
        p = sq.sq_plan_create_uniform(1, 64, 64, 8)
    elif case == "uni128_4":
        p = sq.sq_plan_create_uniform(3, 128, 128, 4)
    elif case == "gdn":
        bits = [4, 6, 8, 16, 2, 4]
        p = sq.sq_plan_create_step(sq.SQ_KIND_GDN, 6, 128, 128, bits, np.ones((6, 128)))
    elif case == "kda":
        bits = rng.choice([4, 6, 8, 16], size=4 * 128)
        p = sq.sq_plan_create_step(sq.SQ_KIND_KDA, 4, 128, 128, bits, np.ones((4, 128)))
    elif case == "win":
        p = sq.sq_plan_create_window(5, 128, 128, 16)
    elif case == "win_r4":
        p = sq.sq_plan_create_window_lowrank(5, 128, 128, 16, 4, 4)
    else:
        p = sq.sq_plan_create_window_lowrank(3, 64, 64, 7, 8, 2)
    d = sq.sq_plan_query(p)
    lay = L.slot_layout(_desc_for_oracle(d))
    assert d["slot_bytes"] == lay["slot_bytes"]
    np.testing.assert_array_equal(d["head_off"], lay["head_off"])
    od = _desc_for_oracle(d)
    assert d["payload_bytes"] == sum(L.head_fields(od, h)["used"] for h in range(d["heads"]))
    assert sq.sq_pool_bytes(p, 10) == 10 * d["slot_bytes"]
    assert sq.sq_max_head_bytes(p) == max(f["bytes"] for f in lay["fields"])
    assert sq.sq_plan_device_bytes(p) % 256 == 0


def test_tiny_uniform_slot_is_4224_bytes():
    """64 x 64 INT8 codes + 64 FP16 row scales = 4,224 bytes, padded to 4,352."""
    d = sq.sq_plan_query(sq.sq_plan_create_uniform(1, 64, 64, 8))
    assert d["payload_bytes"] == 4224 and d["slot_bytes"] == 4352


def test_qwen_six_bit_bytes_from_library():
    """STEPQuant App. D / F.1: 2304 heads of 128 x 128 at nominal six bits with
    32 FP16 pivot heads -> 29,999,104 B per request, 30,015,488 B with the
    analytic scale slots of the pivot heads."""
    g = golden("state_bytes.json")
    U = g["qwen_heads"]
    # 2272 integer heads whose widths sum to 6*2304 - 8*32 head-bits
    bits = np.full(U, 6)
    bits[:32] = 16
    bits[32:64] = 4                     # 32 heads at 4 bits balance the 8-bit charge
    assert bits[bits != 16].sum() == 6 * U - 8 * 32
    p = sq.sq_plan_create_step(sq.SQ_KIND_GDN, U, 128, 128, bits, np.ones((U, 128)))
    d = sq.sq_plan_query(p)
    assert d["payload_bytes"] == g["qwen_serving_bytes_per_request"]
    assert d["analytic_bytes"] == g["qwen_analytic_bytes_per_request"]
    assert d["slot_bytes"] == d["payload_bytes"]          # every head is a 256-B multiple


@pytest.mark.parametrize("nominal,lo", [(6, 4), (4, 2)])
def test_kda_compact_bytes_from_library(nominal, lo):
    """STEPQuant App. D: 640 KDA heads, 512 FP16 pivot rows -> 6.30 / 4.30
    bits per value and 7.875 / 5.375 MiB per request."""
    g = golden("state_bytes.json")
    H, d, n_piv = g["kda_heads"], g["kda_d"], g["kda_pivot_rows"]
    U = H * d
    rows = U - n_piv
    n_lo = (nominal * rows - (nominal * U - 8 * n_piv)) // (nominal - lo)
    bits = np.full(U, nominal)
    bits[:n_lo] = lo
    bits[-n_piv:] = 16
    p = sq.sq_plan_create_step(sq.SQ_KIND_KDA, H, d, d, bits, np.ones((H, d)))
    tot = sq.sq_plan_query(p)["payload_bytes"]
    assert round(8 * tot / (U * d), 2) == g["kda_bits_per_value"][str(nominal)]
    assert tot / 2 ** 20 == g["kda_mib_per_request"][str(nominal)]


def _random_stats(rng, kind, heads, d, cand):
    U = heads if kind == sq.SQ_KIND_GDN else heads * d
    base = rng.uniform(0.2, 3.0, U)
    steps = np.array([4.0 ** (-(b - cand[0]) / 2) for b in cand])       # convex in b
    dist = base[:, None] * steps[None, :] * rng.uniform(0.9, 1.1, (U, len(cand)))
    dist = np.sort(dist, axis=1)[:, ::-1].copy()
    ell = -rng.uniform(1e-4, 0.7, U)
    omega = rng.lognormal(0.0, 1.5, (heads, d))
    return {"kind": kind, "heads": heads, "d_k": d, "d_v": d, "cand_bits": cand,
            "ell": ell, "dist": dist, "omega": omega}


@pytest.mark.parametrize("kind,heads,cand,nominal,frac", [
    (sq.SQ_KIND_GDN, 16, (4, 6, 8), 6.0, 0.02),
    (sq.SQ_KIND_GDN, 48, (2, 4, 6, 8), 4.0, 0.0139),
    (sq.SQ_KIND_KDA, 8, (4, 6, 8), 6.0, 0.014),
])
def test_calibrate_bits_matches_oracle_allocation(kind, heads, cand, nominal, frac):
    rng = np.random.default_rng(11 + heads)
    st = _random_stats(rng, kind, heads, 128, cand)
    p = sq.sq_calibrate_bits(st, {"nominal_bits": nominal, "pivot_frac": frac})
    d = sq.sq_plan_query(p)
    ora = C.allocate("gdn" if kind == sq.SQ_KIND_GDN else "kda", heads, 128, 128, st["ell"],
                     st["dist"], st["omega"], cand, nominal, frac)
    np.testing.assert_array_equal(d["unit_bits"], ora["bits"])
    np.testing.assert_allclose(d["w"], ora["w"], rtol=2e-7)
    U = len(ora["bits"])
    n_u = 128 * 128 if kind == sq.SQ_KIND_GDN else 128
    piv = ora["bits"] == 16
    assert piv.sum() == math.ceil(frac * U - 1e-12)
    assert (ora["bits"][~piv] * n_u).sum() <= nominal * n_u * U - 8 * n_u * piv.sum()


def test_calibrate_bits_uniform_heads_fill_budget():
    """Identical GDN heads at nominal 4 bits, candidates {2,4,6,8}, one pivot:
    47 integer heads share 184 head-bits -> 45 heads at 4 bits, 2 at 2 bits."""
    rng = np.random.default_rng(3)
    st = _random_stats(rng, sq.SQ_KIND_GDN, 48, 128, (2, 4, 6, 8))
    st["dist"] = np.tile(np.array([[16.0, 1.0, 0.0625, 0.004]]), (48, 1)) * (
        1 + 1e-6 * rng.standard_normal((48, 1)))
    st["ell"] = np.full(48, math.log(math.exp(-math.log(2) / 64)))
    p = sq.sq_calibrate_bits(st, {"nominal_bits": 4.0, "pivot_frac": 0.0139})
    b = sq.sq_plan_query(p)["unit_bits"]
    assert (b == 16).sum() == 1 and (b == 4).sum() == 45 and (b == 2).sum() == 2


def test_impact_factors_match_oracle():
    """sq_impact_factors (the function sq_calibrate_bits applies) equals the
    oracle's w = (omega' / geomean omega')^(gamma/2), relative floor included,
    to float32 rounding; an all-zero head gets w = 1."""
    rng = np.random.default_rng(21)
    om = rng.lognormal(0.0, 2.0, (5, 64))
    om[1, :7] = 0.0                               # below the relative floor
    om[2, 3] = 1e-30
    w = sq.sq_impact_factors(om, 0.25, 1e-12)
    np.testing.assert_allclose(w, C.impact_factors(om, 0.25, 1e-12), rtol=2e-7)
    om[4] = 0.0
    w = sq.sq_impact_factors(om)
    assert np.all(w[4] == 1.0)
    np.testing.assert_allclose(w[:4], C.impact_factors(om[:4]), rtol=2e-7)
    bad = om.copy()
    bad[0, 0] = np.nan
    with pytest.raises(sq.StepqError) as e:
        sq.sq_impact_factors(bad)
    assert e.value.status == sq.SQ_ENONFINITE


def test_error_codes():
    with pytest.raises(sq.StepqError) as e:
        sq.sq_plan_create_uniform(1, 96, 128, 8)
    assert e.value.status == sq.SQ_EUNSUPPORTED and "64 or 128" in sq.sq_last_error()
    with pytest.raises(sq.StepqError) as e:
        sq.sq_plan_create_uniform(1, 128, 128, 5)
    assert e.value.status == sq.SQ_EUNSUPPORTED
    with pytest.raises(sq.StepqError) as e:
        sq.sq_plan_create_uniform(0, 128, 128, 8)
    assert e.value.status == sq.SQ_EINVAL
    with pytest.raises(sq.StepqError) as e:
        sq.sq_plan_create_window(1, 128, 128, 0)
    assert e.value.status == sq.SQ_EUNSUPPORTED
    with pytest.raises(sq.StepqError) as e:
        sq.sq_plan_create_window_lowrank(1, 128, 128, 16, 9, 4)
    assert e.value.status == sq.SQ_EUNSUPPORTED and "rank" in sq.sq_last_error()
    with pytest.raises(sq.StepqError) as e:
        sq.sq_plan_create_window_lowrank(1, 128, 128, 16, 4, 0)
    assert e.value.status == sq.SQ_EUNSUPPORTED and "iterations" in sq.sq_last_error()
    d = sq.sq_plan_query(sq.sq_plan_create_window_lowrank(1, 128, 128, 16, 0, 0))
    assert d["window_rank"] == 0 and d["window_iters"] == 0
    assert d["slot_bytes"] == sq.sq_plan_query(sq.sq_plan_create_window(1, 128, 128, 16))["slot_bytes"]
    with pytest.raises(sq.StepqError) as e:
        sq.sq_plan_create_step(sq.SQ_KIND_GDN, 2, 128, 128, [4, 3], np.ones((2, 128)))
    assert e.value.status == sq.SQ_EUNSUPPORTED
    with pytest.raises(sq.StepqError) as e:
        sq.sq_plan_create_step(sq.SQ_KIND_GDN, 2, 128, 128, [4, 4], np.zeros((2, 128)))
    assert e.value.status == sq.SQ_EINVAL
    rng = np.random.default_rng(0)
    st = _random_stats(rng, sq.SQ_KIND_GDN, 4, 128, (4, 6, 8))
    with pytest.raises(sq.StepqError) as e:          # budget below the smallest width
        sq.sq_calibrate_bits(st, {"nominal_bits": 3.0, "pivot_frac": 0.0})
    assert e.value.status == sq.SQ_EBUDGET
    st["dist"][1, 2] = np.nan
    with pytest.raises(sq.StepqError) as e:
        sq.sq_calibrate_bits(st, {"nominal_bits": 6.0})
    assert e.value.status == sq.SQ_ENONFINITE
    # null device pointers are rejected before any HIP call
    p = sq.sq_plan_create_uniform(1, 64, 64, 8)
    lib = sq.lib()
    assert lib.sq_decode_step(p, None, None, 1, None, 1, None, None, None, None, None, None,
                              None) == sq.SQ_EINVAL
    assert lib.sq_pool_pack(p, None, None, 1, None, 1, None, None) == sq.SQ_EINVAL
    assert lib.sq_window_flush(p, 1, 1, 1, 1, 1, None) == sq.SQ_EPLAN_MISMATCH
    assert lib.sq_plan_query(None, None) == sq.SQ_EINVAL
    # batch 0 is a no-op, with or without batch arrays; batch 1 needs them
    assert lib.sq_decode_step(p, 1, 1, 1, 1, 0, 1, 1, 1, 1, 1, 1, None) == sq.SQ_OK
    assert lib.sq_decode_step(p, 1, 1, 1, None, 0, None, None, None, None, None, None,
                              None) == sq.SQ_OK
    assert lib.sq_decode_step(p, 1, 1, 1, None, 1, None, None, None, None, None, None,
                              None) == sq.SQ_EINVAL
    assert lib.sq_pool_pack(p, 1, 1, 1, None, 0, None, None) == sq.SQ_OK
    assert lib.sq_pool_unpack(p, 1, 1, 1, None, 0, None, None) == sq.SQ_OK
    assert lib.sq_quantize_tiles(p, 1, None, 0, None, None, None) == sq.SQ_OK
    assert lib.sq_quantize_tiles(p, 1, None, 2, None, None, None) == sq.SQ_EINVAL
    # both prefill forms: checked before any HIP call, T = 0 or batch 0 is a no-op
    for fn in (lib.sq_prefill_chunk, lib.sq_prefill_chunkwise):
        assert fn(2, 1, 64, 64, 1, 1, 1, 1, 1, 1, 1, 1, 1, None) == sq.SQ_EINVAL
        assert fn(0, 1, 96, 64, 1, 1, 1, 1, 1, 1, 1, 1, 1, None) == sq.SQ_EUNSUPPORTED
        assert fn(1, 1, 64, 64, 1, -1, 1, 1, 1, 1, 1, 1, 1, None) == sq.SQ_EINVAL
        assert fn(0, 1, 64, 64, 1, 0, None, None, None, None, None, None, None, None) == sq.SQ_OK
        assert fn(0, 1, 64, 64, 0, 5, None, None, None, None, None, None, None, None) == sq.SQ_OK
        assert fn(0, 1, 64, 64, 1, 5, 1, 1, 1, None, 1, 1, 1, None) == sq.SQ_EINVAL
        assert fn(0, 2, 64, 64, 2 ** 30, 5, 1, 1, 1, 1, 1, 1, 1, None) == sq.SQ_EINVAL
    # the plan, device tables and pool are still required
    assert lib.sq_decode_step(p, None, 1, 1, None, 0, None, None, None, None, None, None,
                              None) == sq.SQ_EINVAL


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(sq, "_lib", None)
    monkeypatch.setattr(sq, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        sq.lib()
