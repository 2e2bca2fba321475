"""The oracle's whole step: ZeRO equivalence, skip-on-overflow and loss-scale
bookkeeping, multi-group norm.

* ZeRO equivalence: each rank stepping only its segment, concatenated, equals
  every rank stepping the whole vector as plain data parallelism does, because
  the update of one coordinate depends only on that coordinate (ZeRO reading
  notes, second part §3; DeepSpeed walkthrough §3 "each rank owns one segment").
* Overflow: inf/NaN anywhere in the group's partition gradients lowers the loss
  scale and voids the step (DeepSpeed walkthrough §6 step 1).
"""
import numpy as np
import pytest

import oracle
from workloads import grads16_np, normal_f32_np, to16_bits_np


def _group(n, n_d, dt, seed, scale=1.0, wd=0.0, param=None):
    reps = [grads16_np(n, dt, scale, seed=(seed, r)) for r in range(n_d)]
    master = normal_f32_np(n, 0.02, (seed, "master"))
    odt = oracle.F16 if dt == "f16" else oracle.BF16
    return oracle.Group(replicas=reps, grad_dt=odt, master=master,
                        m=np.zeros(n, np.float32), v=np.zeros(n, np.float32),
                        param=param, param_dt=odt, weight_decay=wd)


@pytest.mark.parametrize("n_d,psi", [(2, 1001), (3, 10_000), (4, 787_971 // 16), (8, 4099)])
def test_zero_equivalence(n_d, psi):
    dt = "f16"
    steps = 3
    full_reps = [[grads16_np(psi, dt, 1.0, seed=(k, r)) for r in range(n_d)] for k in range(steps)]
    master0 = normal_f32_np(psi, 0.02, "m0")
    # plain data parallelism: the whole vector, averaged over all copies
    full = oracle.Group(replicas=None, grad_dt=oracle.F16, master=master0.copy(),
                        m=np.zeros(psi, np.float32), v=np.zeros(psi, np.float32),
                        param=np.zeros(psi, np.uint16))
    st_full = oracle.State()
    full_norms = []
    for k in range(steps):
        full.replicas = full_reps[k]
        oracle.step([full], oracle.Policy(), st_full)
        full_norms.append(st_full.norm2)
    # ZeRO: each rank steps its own segment
    offs, sizes, _ = oracle.partition(psi, n_d)
    flat_param = np.zeros(psi, np.uint16)
    master, m, v = np.empty(psi, np.float32), np.empty(psi, np.float32), np.empty(psi, np.float32)
    rank_norms = np.zeros(steps)
    for r in range(n_d):
        o, s = int(offs[r]), int(sizes[r])
        g = oracle.Group(replicas=None, grad_dt=oracle.F16, master=master0[o:o + s].copy(),
                         m=np.zeros(s, np.float32), v=np.zeros(s, np.float32),
                         param=flat_param[o:o + s])
        st = oracle.State()
        for k in range(steps):
            g.replicas = [c[o:o + s] for c in full_reps[k]]
            oracle.step([g], oracle.Policy(), st)
            rank_norms[k] += st.norm2
        master[o:o + s], m[o:o + s], v[o:o + s] = g.master, g.m, g.v
        assert st.step == steps
    for a, b in ((master, full.master), (m, full.m), (v, full.v)):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    np.testing.assert_array_equal(flat_param, full.param)
    # the global norm is the sum of the shard-local sums of squares
    np.testing.assert_allclose(rank_norms, full_norms, rtol=1e-12)


def _inject(group, replica, idx, bits):
    group.replicas[replica] = group.replicas[replica].copy()
    group.replicas[replica][idx] = bits


def test_skip_on_overflow_leaves_everything():
    n = 3000
    g = _group(n, 4, "f16", 1, scale=65536.0, param=np.zeros(n, np.uint16))
    pol = oracle.Policy(skip_on_overflow=True, growth_interval=1000)
    st = oracle.State(loss_scale=65536.0)
    oracle.step([g], pol, st)
    assert st.step == 1 and st.skipped == 0 and st.loss_scale == 65536.0 and st.good_steps == 1
    snap = [x.copy() for x in (g.master, g.m, g.v, g.param)]
    g.replicas = [grads16_np(n, "f16", 65536.0, seed=(2, r)) for r in range(4)]
    _inject(g, 2, n // 2, 0x7C00)
    oracle.step([g], pol, st)
    assert st.overflow == 1 and st.skipped == 1
    assert st.step == 1 and st.loss_scale == 32768.0 and st.good_steps == 0
    assert not np.isfinite(st.norm2)
    for a, b in zip((g.master, g.m, g.v, g.param), snap):
        np.testing.assert_array_equal(a, b)


def test_fp16_sum_overflow_and_nan_are_caught():
    n = 100
    for bits, dt in ((0x7E00, "f16"), (0xFC00, "f16")):
        g = _group(n, 2, dt, 3)
        _inject(g, 0, 99, bits)
        st = oracle.State()
        oracle.step([g], oracle.Policy(skip_on_overflow=True), st)
        assert st.skipped == 1
    g = _group(n, 2, "bf16", 4)
    big = to16_bits_np(np.array([3.0e38], np.float32), "bf16")[0]
    _inject(g, 0, 0, big)
    _inject(g, 1, 0, big)
    st = oracle.State()
    oracle.step([g], oracle.Policy(skip_on_overflow=True), st)
    assert st.skipped == 1 and st.overflow == 1


def test_scale_growth_and_floor():
    n = 64
    g = _group(n, 1, "f16", 5, scale=4.0)
    pol = oracle.Policy(skip_on_overflow=True, growth_interval=2, min_scale=1.0)
    st = oracle.State(loss_scale=4.0)
    oracle.step([g], pol, st)
    assert (st.loss_scale, st.good_steps) == (4.0, 1)
    oracle.step([g], pol, st)
    assert (st.loss_scale, st.good_steps, st.step) == (8.0, 0, 2)
    for expect in (4.0, 2.0, 1.0, 1.0):
        bad = _group(n, 1, "f16", 6)
        _inject(bad, 0, 1, 0x7C00)
        oracle.step([bad], pol, st)
        assert st.loss_scale == expect and st.step == 2


def test_static_scale_applies_even_on_overflow():
    n = 16
    g = _group(n, 1, "f16", 7)
    _inject(g, 0, 3, 0x7C00)
    st = oracle.State(loss_scale=2.0)
    oracle.step([g], oracle.Policy(skip_on_overflow=False), st)
    assert st.step == 1 and st.skipped == 0 and st.loss_scale == 2.0
    assert not np.isfinite(g.master[3]) and np.isfinite(np.delete(g.master, 3)).all()


def test_multi_group_norm_and_shared_skip():
    a = _group(1000, 1, "bf16", 8, wd=0.1)
    b = _group(37, 1, "bf16", 9)
    st = oracle.State()
    oracle.step([a, b], oracle.Policy(), st)
    na, _ = oracle.norm_overflow(oracle.average(a.replicas, oracle.BF16), 1.0)
    nb, _ = oracle.norm_overflow(oracle.average(b.replicas, oracle.BF16), 1.0, na)
    assert st.norm2 == nb
    # a non-finite gradient in the small group voids the step for both groups
    snap = a.master.copy()
    _inject(b, 0, 36, 0xFF80)
    oracle.step([a, b], oracle.Policy(skip_on_overflow=True), st)
    assert st.skipped == 1
    np.testing.assert_array_equal(a.master, snap)


def test_group_hyperparameters_apply_per_group():
    a = _group(200, 1, "f16", 10, wd=0.1)
    b = _group(200, 1, "f16", 10, wd=0.0)  # same inputs, no decay
    oracle.step([a, b], oracle.Policy(), oracle.State())
    assert not np.array_equal(a.master, b.master)
    a2 = _group(200, 1, "f16", 10, wd=0.1)
    oracle.step([a2], oracle.Policy(), oracle.State())
    np.testing.assert_array_equal(a.master, a2.master)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_loss_scale_is_unscaled_before_the_update(dt):
    """The loss scale only protects the 16-bit gradients; the step unscales
    first (DeepSpeed walkthrough §6 step 3), so with a power-of-two scale the
    update equals the update of the unscaled gradients, bit for bit. Scaling a
    16-bit value by 2^16 is exact while it stays in range, as here."""
    n, scale = 4000, 65536.0
    odt = oracle.F16 if dt == "f16" else oracle.BF16
    master0 = normal_f32_np(n, 0.02, "ls-master")
    plain = [grads16_np(n, dt, 1.0, seed=("ls", r)) for r in range(3)]
    scaled = [to16_bits_np(oracle.decode16(b, odt) * np.float32(scale), dt) for b in plain]
    for b, s in zip(plain, scaled):  # the scaled copies hold exactly scale x the plain values
        np.testing.assert_array_equal(oracle.decode16(s, odt), oracle.decode16(b, odt) * np.float32(scale))
    runs = []
    for reps, ls in ((plain, 1.0), (scaled, scale)):
        g = oracle.Group(replicas=reps, grad_dt=odt, master=master0.copy(), m=np.zeros(n, np.float32),
                         v=np.zeros(n, np.float32), param=np.zeros(n, np.uint16), param_dt=odt,
                         weight_decay=0.1)
        st = oracle.State(loss_scale=ls)
        for _ in range(3):
            oracle.step([g], oracle.Policy(), st)
        runs.append((g, st))
    (a, sa), (b, sb) = runs
    for x, y in ((a.master, b.master), (a.m, b.m), (a.v, b.v)):
        np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32))
    np.testing.assert_array_equal(a.param, b.param)
    assert sa.norm2 == sb.norm2


def _decode64(bits, dt):
    """16-bit patterns -> float64, independently of the oracle (numpy's binary16, bfloat16 by shifting)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("dt,wd", [("bf16", 0.1), ("f16", 0.0)])
def test_whole_step_against_float64_brute_force(dt, wd):
    # the whole step -- average of the N_d copies, unscale, AdamW with bias correction, skip on an
    # overflowing call with the scale halved, writeback -- recomputed in float64 from the definitions
    # (the reading notes' per-coordinate Adam, the walkthrough's step() actions), against the oracle
    # within the error fp32 arithmetic can add
    n, n_d, steps, lr, b1, b2, eps = 3000, 4, 6, 1e-3, 0.9, 0.999, 1e-8
    u = 2.0 ** -24
    odt = oracle.F16 if dt == "f16" else oracle.BF16
    scale = 1024.0
    g = _group(n, n_d, dt, 61, scale=scale, wd=wd, param=np.zeros(n, np.uint16))
    st = oracle.State(loss_scale=scale)
    pol = oracle.Policy(skip_on_overflow=True, growth_interval=1000)
    theta = g.master.astype(np.float64)
    m = np.zeros(n)
    v = np.zeros(n)
    m_mag = np.zeros(n)      # the moment's recursion on absolute values: its rounding error scales with this
    t, s = 0, scale
    for k in range(steps):
        g.replicas = [grads16_np(n, dt, s, seed=(62, k, r)) for r in range(n_d)]
        if k == 2:
            g.replicas[1] = g.replicas[1].copy()
            g.replicas[1][123] = 0x7C00 if dt == "f16" else 0x7F80     # +inf in one copy
        avg = sum(_decode64(r, dt) for r in g.replicas) / n_d
        oracle.step([g], pol, st)
        if not np.isfinite(avg).all():
            s = max(s / 2, 1.0)                 # the step is void, the scale halves
        else:
            grad = avg / s
            t += 1
            theta = theta * (1 - lr * wd)
            m = b1 * m + (1 - b1) * grad
            m_mag = b1 * m_mag + (1 - b1) * np.abs(grad)
            v = b2 * v + (1 - b2) * grad * grad
            theta = theta - lr * (m / (1 - b1 ** t)) / (np.sqrt(v / (1 - b2 ** t)) + eps)
        assert (st.step, st.loss_scale, st.skipped) == (t, s, int(k == 2)), k
        # fp32 rounding: each step adds a few ulps of |theta| and of the update (lr times a ratio of
        # order one, whose own error grows with the moments' by a few ulps per step); the moments
        # carry a few ulps per step of the magnitude of their terms (m may cancel, v cannot)
        tol_theta = (k + 1) * (3 * u * np.abs(theta) + 32 * (k + 2) * u * lr)
        assert (np.abs(g.master - theta) <= tol_theta).all(), (k, np.abs(g.master - theta).max())
        assert (np.abs(g.m - m) <= 4 * (k + 1) * u * m_mag + 1e-30).all(), k
        assert (np.abs(g.v - v) <= 8 * (k + 1) * u * np.abs(v) + 1e-30).all(), k
        np.testing.assert_array_equal(g.param, oracle.encode16(g.master, odt))
    assert t == steps - 1
