"""The parity bar the GPU tests apply (tests/_parity.py), on the CPU: ulp
distances, the switch from bit identity to the stated tolerances when the
two sides' clip multipliers differ by one ulp, and that the tolerances are
neither too tight for that case nor loose enough to let a plausible mistake
through (both checked with the oracle's own update)."""
import numpy as np
import pytest

import oracle
from _parity import Bar, assert_close32, assert_within_ulp16, ordered16, ordered32, ulp32


def test_ordered_integers_follow_the_values():
    x = np.array([-np.inf, -3.0, -1e-40, -0.0, 0.0, 1e-45, 1.0, np.float32(3.4e38), np.inf], np.float32)
    o = ordered32(x)
    assert (np.diff(o) >= 0).all() and o[3] == o[4] == 0
    assert ulp32(np.float32(1.0), np.nextafter(np.float32(1.0), np.float32(2))) == 1
    tiny = np.float32(1e-45)
    assert ulp32(-tiny, tiny) == 2
    h = np.array([0xFC00, 0xBC00, 0x8001, 0x8000, 0x0000, 0x0001, 0x3C00, 0x7C00], np.uint16)   # fp16
    oh = ordered16(h)
    assert (np.diff(oh) >= 0).all() and oh[3] == oh[4] == 0


def test_bar_switches_to_tolerances_only_after_a_one_ulp_difference():
    bar = Bar()
    c = np.float32(0.625)
    bar.clip("same", c, c, applied=True)
    assert bar.exact and bar.steps_since == 0
    with pytest.raises(AssertionError, match="differ"):
        bar.state32(np.array([1.0], np.float32), np.array([np.nextafter(np.float32(1), np.float32(2))]), "m", "m")
    bar.clip("one ulp", c, np.nextafter(c, np.float32(1)), applied=True)
    assert not bar.exact and bar.steps_since == 1 and bar.rtol == 1e-6
    bar.clip("next", c, c, applied=False)    # a voided step does not count
    assert bar.steps_since == 1
    bar.clip("next", c, c, applied=True)
    assert bar.steps_since == 2 and bar.rtol == 5e-6
    with pytest.raises(AssertionError, match="2 ulps apart"):
        Bar().clip("two ulps", c, np.nextafter(np.nextafter(c, np.float32(1)), np.float32(1)), applied=True)


def test_tolerance_checks():
    w = np.array([0.02, -0.5, 1e-12, 0.0, np.nan], np.float32)
    g = w.copy()
    g[0] = np.float32(0.02 * (1 + 0.9e-6))
    g[2] = np.float32(1e-12 + 0.9e-6 * 1e-3)       # within the floor
    assert_close32(g, w, 1e-6, 1e-3, "ok")
    g[1] = np.float32(-0.5 * (1 + 3e-6))
    with pytest.raises(AssertionError, match="outside rtol"):
        assert_close32(g, w, 1e-6, 1e-3, "too far")
    g = w.copy()
    g[4] = 1.0
    with pytest.raises(AssertionError, match="NaN positions"):
        assert_close32(g, w, 1e-6, 1e-3, "nan")
    a = np.array([0x3C00, 0x8000, 0x0001], np.uint16)
    assert_within_ulp16(np.array([0x3C01, 0x0000, 0x0000], np.uint16), a, "one ulp, +-0")
    with pytest.raises(AssertionError, match="more than 1 ulp"):
        assert_within_ulp16(np.array([0x3C02, 0x8000, 0x0001], np.uint16), a, "two ulps")


def _run(n, steps, clip_of, t_of=lambda t: t, seed=0):
    """The oracle's update for `steps` steps with a per-step clip multiplier."""
    rng = np.random.Generator(np.random.PCG64(seed))
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    param = np.zeros(n, np.uint16)
    for t in range(1, steps + 1):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        oracle.adam_update(g, 1.0, master, m, v, t_of(t), 1e-3, 0.9, 0.999, 1e-8, 0.1, param=param,
                           param_dt=oracle.BF16, clip=clip_of(t))
    return master, m, v, param


def test_one_ulp_multiplier_stays_within_the_bar_for_ten_steps():
    c = np.float32(0.7)
    c1 = np.nextafter(c, np.float32(1))
    a = _run(50_000, 10, lambda t: float(c))
    b = _run(50_000, 10, lambda t: float(c1) if t == 1 else float(c))
    bar = Bar()
    bar.clip("call 1", c, c1, applied=True)
    for t in range(2, 11):
        bar.clip(f"call {t}", c, c, applied=True)
    bar.state32(b[0], a[0], "master", "master")
    bar.state32(b[1], a[1], "m", "m")
    bar.state32(b[2], a[2], "v", "v")
    bar.param16(b[3], a[3], "param")


def test_the_tolerances_still_catch_an_off_by_one_bias_correction():
    a = _run(20_000, 3, lambda t: 1.0)
    b = _run(20_000, 3, lambda t: 1.0, t_of=lambda t: t + 1)
    bar = Bar()
    bar.clip("c", np.float32(0.5), np.nextafter(np.float32(0.5), np.float32(1)), applied=True)
    with pytest.raises(AssertionError):
        bar.state32(b[0], a[0], "master", "master")
