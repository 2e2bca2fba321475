"""Oracle average, overflow flag and gradient norm, pinned by exact arithmetic.

* The rank's averaged shard is (1/N_d) * sum_r g_r^(k) (ZeRO reading notes,
  second part §4), and averaging the rank's N_d segments equals all-reducing the
  full copies and slicing (all-reduce = reduce-scatter then all-gather, same
  section).
* The overflow check scans the partition gradients for inf/NaN, and the norm is
  computed shard by shard as a sum of squares before the square root (DeepSpeed
  ZeRO stage 1/2 walkthrough, §6 steps 1-2).
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
from workloads import grads16_np, to16_bits_np

U32 = 2.0 ** -24  # unit roundoff of fp32


def _exact(bits, dt):
    return [Fraction(float(x)) for x in oracle.decode16(bits, dt)]


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
@pytest.mark.parametrize("n_d", [1, 2, 3, 4, 7, 8, 64])
def test_average_within_summation_bound(dt, n_d):
    rng = np.random.Generator(np.random.PCG64(n_d * 10 + dt))
    n = 257
    # wide dynamic range so that fp32 accumulation actually rounds
    reps = [to16_bits_np((rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 4, n)).astype(np.float32),
                         "f16" if dt == oracle.F16 else "bf16") for _ in range(n_d)]
    got = oracle.average(reps, dt)
    ex = [_exact(r, dt) for r in reps]
    for j in range(n):
        xs = [ex[r][j] for r in range(n_d)]
        mean = sum(xs) / n_d
        # Higham: |fl(sum) - sum| <= (n_d - 1) u sum|x|, then one division by N_d
        bound = (n_d - 1) * U32 * float(sum(abs(x) for x in xs)) / n_d + U32 * abs(float(mean))
        assert abs(float(Fraction(float(got[j])) - mean)) <= bound * 1.0000001 + 1e-45


@pytest.mark.parametrize("n_d", [1, 2, 4, 8, 64])
def test_average_of_small_gradients_is_exact(n_d):
    # N(0,1e-3) fp16 values: the fp32 running sum is exact, and dividing by a
    # power of two is exact, so the oracle returns the exact mean.
    reps = [grads16_np(1000, "f16", 1.0, seed=100 + r) for r in range(n_d)]
    got = oracle.average(reps, oracle.F16)
    ex = [_exact(r, oracle.F16) for r in reps]
    for j in range(0, 1000, 7):
        assert Fraction(float(got[j])) == sum(e[j] for e in ex) / n_d


def test_average_single_copy_is_identity():
    bits = grads16_np(5000, "bf16", 65536.0, seed=3)
    np.testing.assert_array_equal(oracle.average([bits], oracle.BF16), oracle.decode16(bits, oracle.BF16))


@pytest.mark.parametrize("n_d", [2, 3, 8])
def test_segment_average_equals_allreduce_then_slice(n_d):
    psi = 10_001
    full = [grads16_np(psi, "f16", 1.0, seed=50 + r) for r in range(n_d)]
    allreduced = oracle.average(full, oracle.F16)
    offs, sizes, _ = oracle.partition(psi, n_d)
    for r in range(n_d):
        o, s = int(offs[r]), int(sizes[r])
        seg = oracle.average([c[o:o + s] for c in full], oracle.F16)
        np.testing.assert_array_equal(seg.view(np.uint32), allreduced[o:o + s].view(np.uint32))


# ---------------------------------------------------------------- overflow flag

@pytest.mark.parametrize("case,flag", [
    ("finite", 0), ("pinf", 1), ("ninf", 1), ("nan", 1), ("inf_minus_inf", 1),
    ("bf16_sum_overflow", 1), ("f16_max_sum_ok", 0), ("first", 1), ("last", 1),
])
def test_overflow_truth_table(case, flag):
    n = 37
    dt = oracle.F16
    reps = [np.zeros(n, dtype=np.uint16) for _ in range(2)]
    if case == "pinf":
        reps[0][5] = 0x7C00
    elif case == "ninf":
        reps[1][9] = 0xFC00
    elif case == "nan":
        reps[0][3] = 0x7E00
    elif case == "inf_minus_inf":
        reps[0][4], reps[1][4] = 0x7C00, 0xFC00
    elif case == "bf16_sum_overflow":
        dt = oracle.BF16
        big = to16_bits_np(np.array([3.0e38], np.float32), "bf16")[0]
        reps[0][7] = reps[1][7] = big  # each finite, their fp32 sum is +inf
    elif case == "f16_max_sum_ok":
        reps[0][7] = reps[1][7] = 0x7BFF  # 65504 + 65504 is finite in fp32
    elif case == "first":
        reps[1][0] = 0x7C00
    elif case == "last":
        reps[0][n - 1] = 0xFC00
    avg = oracle.average(reps, dt)
    _, f = oracle.norm_overflow(avg, 1.0)
    assert f == flag


# ---------------------------------------------------------------- norm

def test_norm_closed_form_constant_vector():
    for c, n in ((0.125, 1000), (3.0, 7), (1e-3, 4096)):
        a = np.full(n, c, dtype=np.float32)
        n2, f = oracle.norm_overflow(a, 1.0)
        assert f == 0
        assert math.sqrt(n2) == pytest.approx(abs(float(np.float32(c))) * math.sqrt(n), rel=1e-15)


def test_norm_power_of_two_unscale_is_exact():
    a = np.array([65536.0 * 3, -65536.0 * 0.5, 0.0], dtype=np.float32)
    n2, _ = oracle.norm_overflow(a, oracle.inv_scale_of(65536.0))
    assert n2 == 9.0 + 0.25


def test_norm_exact_rational_tiny():
    rng = np.random.Generator(np.random.PCG64(7))
    a = (rng.standard_normal(3000) * 10.0 ** rng.uniform(-5, 3, 3000)).astype(np.float32)
    inv = oracle.inv_scale_of(1024.0)
    n2, _ = oracle.norm_overflow(a, inv)
    exact = sum(Fraction(float(np.float32(x * np.float32(inv)))) ** 2 for x in a)
    assert abs(Fraction(n2) - exact) / exact < Fraction(1, 10 ** 12)


def test_norm_chunked_equals_whole():
    a = np.random.Generator(np.random.PCG64(9)).standard_normal(10_000).astype(np.float32)
    whole = oracle.norm_overflow(a, 0.5)
    acc = (0.0, 0)
    for s in range(0, a.size, 999):
        acc = oracle.norm_overflow(a[s:s + 999], 0.5, *acc)
    assert acc == whole


def test_inv_scale():
    assert oracle.inv_scale_of(65536.0) == 2.0 ** -16
    assert oracle.inv_scale_of(3.0) == float(np.float32(1.0 / 3.0))
