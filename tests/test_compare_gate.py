"""Pins of the parity gate itself (oracle/compare.py), on the CPU.

Every float verdict of the GPU tests goes through ``compare.metrics`` and
``compare.passes``; these checks fix their arithmetic from outside the module:

* ``ulp_of`` against numpy's own float32 spacing and against bf16 spacings
  derived from bit patterns (the next bf16 above a value, minus the value),
  including subnormal magnitudes;
* ``to_f64`` against hand-decoded bf16 patterns;
* ``metrics`` / ``passes`` on tensors built so that the answer is known by
  construction: an error of exactly 4 ulps passes and 4.01 fails; a near-zero
  element is judged at the ulp of the floor 2^-8 max|yref| (and 6 floor-ulps
  fail); the rel-L2 thresholds sit between two tensors whose relative error
  is a ratio of square roots worked by hand; a NaN fails.

``test_planted_gate_mistake_is_caught`` loads copies of compare.py with one
plausible slip each (bf16 precision 7, floor dropped, floor applied to the
error, dtype thresholds swapped, ...) and requires at least one pin to fail
for every copy.

The gate's reading (per-element ulp with the floor, rel-L2 over the compared
elements) follows the tolerance the scope sets for the per-row equation of
page "Multi-LoRA Serving: one base, many adapters", sections 2 and 3.1.
"""
import importlib.util
import os

import numpy as np
import pytest

from oracle import compare as COMPARE

SRC = os.path.join(os.path.dirname(os.path.abspath(COMPARE.__file__)), "compare.py")


def _bf16_bits(v: float) -> np.uint16:
    """bf16 pattern of a value that bf16 represents exactly (checked)."""
    f = np.array([v], np.float32)
    bits = f.view(np.uint32)[0]
    assert bits & 0xFFFF == 0, f"{v} is not a bf16 value"
    return np.uint16(bits >> 16)


def _bf16_value(bits) -> float:
    return float(np.array([np.uint32(bits) << 16], np.uint32).view(np.float32)[0])


def _bf16_tensor(values) -> np.ndarray:
    return np.array([_bf16_bits(v) for v in values], np.uint16)


# ------------------------------------------------------------------ the pins

def pin_to_f64(cmp):
    # hand-decoded patterns: sign | exponent (8 bits, bias 127) | 7 fraction bits
    cases = {0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x3F00: 0.5, 0x4040: 3.0,
             0x3FC0: 1.5, 0x0001: 2.0 ** -133, 0x0000: 0.0, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127}
    bits = np.array(list(cases), np.uint16)
    got = cmp.to_f64(bits, "bf16")
    np.testing.assert_array_equal(got, np.array(list(cases.values()), np.float64))
    f = np.array([1.25, -3.0e-7], np.float32)
    np.testing.assert_array_equal(cmp.to_f64(f, "f32"), f.astype(np.float64))


def pin_ulp_f32(cmp):
    rng = np.random.default_rng(5)
    mags = np.concatenate([
        np.float32(2.0) ** rng.integers(-125, 127, 200).astype(np.float32),
        (rng.random(200) * 1e4).astype(np.float32) + np.float32(1e-3),
        np.array([1.0, 1.5, 2.0, 3.999, 1e-38, 1e-42, 1e-45], np.float32),
    ]).astype(np.float32)
    got = cmp.ulp_of(mags.astype(np.float64), "f32")
    np.testing.assert_array_equal(got, np.spacing(mags).astype(np.float64))


def pin_ulp_bf16_hand(cmp):
    # spacing of bf16 in [2^e, 2^(e+1)) is 2^(e-7)
    cases = [(0.5, 2.0 ** -8), (1.0, 2.0 ** -7), (1.99, 2.0 ** -7), (2.0, 2.0 ** -6),
             (3.0, 2.0 ** -6), (100.0, 2.0 ** -1), (2.0 ** -126, 2.0 ** -133),
             (1e-40, 2.0 ** -133)]
    for mag, want in cases:
        got = float(cmp.ulp_of(np.array([mag]), "bf16")[0])
        assert got == want, (mag, got, want)


def pin_ulp_bf16_bits(cmp):
    # the next bf16 pattern above a positive normal value, minus the value
    rng = np.random.default_rng(6)
    bits = rng.integers(0x0080, 0x7F7F, 500).astype(np.uint32)
    vals = np.array([_bf16_value(b) for b in bits])
    nxt = np.array([_bf16_value(b + 1) for b in bits])
    np.testing.assert_array_equal(cmp.ulp_of(vals, "bf16"), nxt - vals)


def _ones_with_errors(n, m, off_ulps):
    """y = n bf16 ones; yref = 1 + off_ulps * 2^-7 on the first m elements, else 1."""
    y = _bf16_tensor([1.0] * n)
    ref = np.ones(n)
    ref[:m] = 1.0 + off_ulps * 2.0 ** -7
    return y, ref


def pin_max_ulp_edge(cmp):
    # one element 4 bf16 ulps away among 4096 exact ones: max_ulp is exactly 4
    y, ref = _ones_with_errors(4096, 1, 4.0)
    m = cmp.metrics(y, ref, "bf16")
    assert m["max_ulp"] == 4.0 and cmp.passes(m, "bf16"), m
    y, ref = _ones_with_errors(4096, 1, 4.01)
    m = cmp.metrics(y, ref, "bf16")
    assert abs(m["max_ulp"] - 4.01) < 1e-9 and not cmp.passes(m, "bf16"), m


def pin_floor(cmp):
    # max|yref| = 256, so the floor is 1.0 and its ulp 2^-7.  An element with
    # yref = 2^-4 and an error of 3 * 2^-7 is 3 floor-ulps (its own ulp would
    # make it 48); with 6 * 2^-7 it is 6 floor-ulps and fails.
    base = [256.0] + [1.0] * 4095
    for err_units, ok in ((3, True), (6, False)):
        yv = list(base) + [2.0 ** -4 + err_units * 2.0 ** -7]
        ref = np.array(base + [2.0 ** -4])
        y = _bf16_tensor(yv)
        m = cmp.metrics(y, ref, "bf16")
        assert m["max_ulp"] == float(err_units), m
        assert cmp.passes(m, "bf16") == ok, m
    # exact equality: zero error everywhere, whatever the floor
    ref = np.array(base + [0.0, 2.0 ** -20])
    y = _bf16_tensor(list(base) + [0.0, 2.0 ** -20])
    m = cmp.metrics(y, ref, "bf16")
    assert m["max_ulp"] == 0.0 and m["rel_l2"] == 0.0 and cmp.passes(m, "bf16"), m


def pin_rel_l2_bf16(cmp):
    # n = 4096 ones, m of them 1 ulp (2^-7) off: rel-L2 = sqrt(m) 2^-7 / |yref|
    # with |yref|^2 = (n - m) + m (1 + 2^-7)^2.  m = 256: 16 * 2^-7 / sqrt(4100.0)
    # = 1.952e-3 (passes); m = 289: 17 * 2^-7 / sqrt(4100.5) = 2.074e-3 (fails).
    for m_off, want, ok in ((256, 16 * 2.0 ** -7 / np.sqrt(3840 + 256 * (1 + 2.0 ** -7) ** 2), True),
                            (289, 17 * 2.0 ** -7 / np.sqrt(3807 + 289 * (1 + 2.0 ** -7) ** 2), False)):
        y, ref = _ones_with_errors(4096, m_off, 1.0)
        m = cmp.metrics(y, ref, "bf16")
        assert abs(m["rel_l2"] - want) < 1e-15, (m, want)
        assert m["max_ulp"] == 1.0
        assert cmp.passes(m, "bf16") == ok, m


def pin_rel_l2_f32(cmp):
    # 10000 ones; yref = 1 + e on the first element only: rel-L2 = e / |yref|
    n = 10000
    for e, ok in ((4e-4, True), (1.2e-3, False)):   # rel about 4e-6 / 1.2e-5 (|yref| ~ 100)
        y = np.ones(n, np.float32)
        ref = np.ones(n)
        ref[0] += e
        m = cmp.metrics(y, ref, "f32")
        want = e / np.sqrt(n - 1 + (1 + e) ** 2)
        assert abs(m["rel_l2"] - want) < 1e-15, m
        assert cmp.passes(m, "f32") == (want <= 1e-5), m
        assert ok == (want <= 1e-5)
    # 5e-6 passes, 2e-5 fails
    for rel, ok in ((5e-6, True), (2e-5, False)):
        y = np.ones(n, np.float32)
        ref = np.ones(n)
        e = rel * 100.0
        ref[0] += e
        assert cmp.passes(cmp.metrics(y, ref, "f32"), "f32") == ok


def pin_dtype_thresholds(cmp):
    # a bf16 tensor at rel-L2 1.95e-3 passes although it is far above the fp32 bar
    y, ref = _ones_with_errors(4096, 256, 1.0)
    assert cmp.passes(cmp.metrics(y, ref, "bf16"), "bf16")
    # an fp32 tensor at rel-L2 1e-3 fails although it is below the bf16 bar
    y = np.ones(4096, np.float32)
    ref = np.ones(4096)
    ref[:16] += 0.016
    m = cmp.metrics(y, ref, "f32")
    assert 5e-4 < m["rel_l2"] < 2e-3 and not cmp.passes(m, "f32"), m


def pin_nonfinite(cmp):
    y = _bf16_tensor([1.0] * 64)
    y[3] = 0x7FC0   # NaN
    m = cmp.metrics(y, np.ones(64), "bf16")
    assert not cmp.passes(m, "bf16")


def pin_check_raises(cmp):
    y, ref = _ones_with_errors(4096, 1, 5.0)
    try:
        cmp.check(y, ref, "bf16", "pin")
    except AssertionError:
        pass
    else:
        raise AssertionError("check() accepted an error of 5 bf16 ulps")
    y, ref = _ones_with_errors(4096, 1, 3.0)
    cmp.check(y, ref, "bf16", "pin")


PINS = [pin_to_f64, pin_ulp_f32, pin_ulp_bf16_hand, pin_ulp_bf16_bits, pin_max_ulp_edge,
        pin_floor, pin_rel_l2_bf16, pin_rel_l2_f32, pin_dtype_thresholds, pin_nonfinite,
        pin_check_raises]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_gate_pin(pin):
    pin(COMPARE)


# ------------------------------------------------------- planted mistakes

MUTATIONS = {
    "bf16_precision_7": ('p = 8 if dtype == "bf16" else 24', 'p = 7 if dtype == "bf16" else 24'),
    "f32_precision_23": ('p = 8 if dtype == "bf16" else 24', 'p = 8 if dtype == "bf16" else 23'),
    "ulp_exponent_off": ("return np.ldexp(1.0, e - p)", "return np.ldexp(1.0, e - p + 1)"),
    "floor_dropped": ("ulps = err / ulp_of(np.maximum(np.abs(r64), floor), dtype)",
                      "ulps = err / ulp_of(np.abs(r64), dtype)"),
    "floor_on_error": ("ulps = err / ulp_of(np.maximum(np.abs(r64), floor), dtype)",
                       "ulps = np.maximum(err, floor) / ulp_of(np.abs(r64), dtype)"),
    "floor_fraction_7": ("ULP_FLOOR_FRACTION = 2.0 ** -8", "ULP_FLOOR_FRACTION = 2.0 ** -7"),
    "thresholds_swapped": ('return m["rel_l2"] <= BF16_REL_L2 and m["max_ulp"] <= BF16_MAX_ULP',
                           'return m["rel_l2"] <= F32_REL_L2 and m["max_ulp"] <= BF16_MAX_ULP'),
    "f32_bar_bf16": ('return m["rel_l2"] <= F32_REL_L2\n', 'return m["rel_l2"] <= BF16_REL_L2\n'),
    "ulp_gate_dropped": ('return m["rel_l2"] <= BF16_REL_L2 and m["max_ulp"] <= BF16_MAX_ULP',
                         'return m["rel_l2"] <= BF16_REL_L2'),
    "ulp_gate_strict": ('m["max_ulp"] <= BF16_MAX_ULP', 'm["max_ulp"] < BF16_MAX_ULP'),
    "rel_l2_by_max": ("denom = np.linalg.norm(r64)", "denom = np.max(np.abs(r64))"),
    "rel_l2_abs": ("float(np.linalg.norm(y64 - r64) / denom) if denom > 0",
                   "float(np.linalg.norm(y64 - r64)) if denom > 0"),
    "bf16_shift_15": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "max_ulp_mean": ("max_ulp=float(np.max(ulps))", "max_ulp=float(np.mean(ulps))"),
}


def _load_mutated(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    path = tmp_path / f"compare_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"compare_{name}", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_gate_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    mod = _load_mutated(name, old, new, tmp_path)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted gate mistake {name}"
