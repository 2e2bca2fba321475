"""Oracle Adam/AdamW update, pinned by closed forms and by a library routine.

The update is the per-coordinate rule of the ZeRO reading notes (second part,
§3): m <- b1 m + (1-b1) g, v <- b2 v + (1-b2) g^2, theta <- theta - lr *
mhat / (sqrt(vhat) + eps); the fp32 master/m/v come from the paper's
mixed-precision ledger (paper translation §3.1). Pins:

* step-1 closed form: m1 = (1-b1) g, v1 = (1-b2) g^2, theta1 = theta0 -
  lr g / (|g| + eps), i.e. about lr * sign(g) when |g| >> eps;
* constant gradient for t steps: mhat = g and vhat = g^2 exactly in real
  arithmetic, so theta_t = theta0 - t lr g / (|g| + eps);
* the moving averages' sum form m_t = (1-b1) sum_i b1^(t-i) g_i (same for v);
* torch.optim.Adam / AdamW in float64 on the same inputs (an independent
  implementation), within a bound derived from fp32 rounding;
* g = 0 leaves every coordinate unchanged.
"""
import numpy as np
import pytest
import torch

import oracle

U = 2.0 ** -24
LR, B1, B2, EPS = 1e-3, 0.9, 0.999, 1e-8


def _state(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    return master, np.zeros(n, np.float32), np.zeros(n, np.float32), g


def _run(g_seq, master, m, v, wd=0.0, t0=0, param=None, param_dt=oracle.F16):
    for k, g in enumerate(g_seq):
        oracle.adam_update(g, 1.0, master, m, v, t0 + k + 1, LR, B1, B2, EPS, wd,
                           param=param, param_dt=param_dt)


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_step_one_closed_form(wd):
    master, m, v, g = _state(4096, 1)
    th0 = master.astype(np.float64).copy()
    _run([g], master, m, v, wd=wd)
    g64 = g.astype(np.float64)
    np.testing.assert_allclose(m, (1 - B1) * g64, rtol=3 * U, atol=0)
    np.testing.assert_allclose(v, (1 - B2) * g64 * g64, rtol=6 * U, atol=0)
    want = th0 * (1 - LR * wd) - LR * g64 / (np.abs(g64) + EPS)
    err = np.abs(master - want)
    assert (err <= 2 * U * np.abs(want) + LR * 16 * U).all()


def test_step_one_is_about_lr_sign_g():
    master, m, v, g = _state(4096, 2)
    th0 = master.copy()
    _run([g], master, m, v)
    step = (th0.astype(np.float64) - master) / LR
    big = np.abs(g) > 1e-5  # |g| >> eps
    # |g|/(|g|+eps) = 1 - eps/|g| + ...; rounding theta1 to fp32 adds up to
    # u*|theta1|/lr, the fp32 lr and quotient a few u more
    mag = np.maximum(np.abs(th0[big]), np.abs(master[big])).astype(np.float64)
    tol = EPS / np.abs(g[big]) + 2 * U * mag / LR + 16 * U
    assert (np.abs(step[big] - np.sign(g[big])) <= tol).all()


@pytest.mark.parametrize("t", [2, 5, 10])
def test_constant_gradient_closed_form(t):
    master, m, v, g = _state(2048, 3)
    th0 = master.astype(np.float64).copy()
    _run([g] * t, master, m, v)
    g64 = g.astype(np.float64)
    want = th0 - t * LR * g64 / (np.abs(g64) + EPS)
    assert (np.abs(master - want) <= t * (2 * U * np.abs(want) + LR * 16 * U)).all()
    np.testing.assert_allclose(m, (1 - B1 ** t) * g64, rtol=4 * t * U)
    np.testing.assert_allclose(v, (1 - B2 ** t) * g64 * g64, rtol=8 * t * U)


def test_moving_average_sum_form():
    n, t = 1024, 7
    rng = np.random.Generator(np.random.PCG64(4))
    gs = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(t)]
    master, m, v, _ = _state(n, 5)
    _run(gs, master, m, v)
    G = np.stack([x.astype(np.float64) for x in gs])
    w1 = np.array([B1 ** (t - i) for i in range(1, t + 1)])
    w2 = np.array([B2 ** (t - i) for i in range(1, t + 1)])
    m_want = (1 - B1) * (w1[:, None] * G).sum(0)
    v_want = (1 - B2) * (w2[:, None] * G * G).sum(0)
    # error bound ~ few u per step on the sum of magnitudes
    m_mag = (1 - B1) * (w1[:, None] * np.abs(G)).sum(0)
    v_mag = (1 - B2) * (w2[:, None] * G * G).sum(0)
    assert (np.abs(m - m_want) <= 4 * t * U * m_mag).all()
    assert (np.abs(v - v_want) <= 6 * t * U * v_mag).all()


@pytest.mark.parametrize("wd", [0.0, 0.1])
@pytest.mark.parametrize("t", [1, 3, 10])
def test_matches_torch_optim_float64(wd, t):
    n = 3000
    rng = np.random.Generator(np.random.PCG64(11 + t))
    master, m, v, _ = _state(n, 6)
    gs = [(rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 0, n)).astype(np.float32) for _ in range(t)]
    p = torch.nn.Parameter(torch.from_numpy(master.astype(np.float64)))
    cls = torch.optim.AdamW if wd else torch.optim.Adam
    opt = cls([p], lr=LR, betas=(B1, B2), eps=EPS, weight_decay=wd, foreach=False)
    for g in gs:
        p.grad = torch.from_numpy(g.astype(np.float64))
        opt.step()
    _run(gs, master, m, v, wd=wd)
    st = opt.state[p]
    want = p.detach().numpy()
    assert (np.abs(master - want) <= t * (2 * U * np.abs(want) + LR * 32 * U)).all()
    m_ref = st["exp_avg"].numpy()
    v_ref = st["exp_avg_sq"].numpy()
    G = np.abs(np.stack(gs)).astype(np.float64)
    assert (np.abs(m - m_ref) <= 4 * t * U * G.max(0)).all()
    assert (np.abs(v - v_ref) <= 6 * t * U * (G * G).max(0)).all()


def test_zero_gradient_changes_nothing():
    master, m, v, _ = _state(500, 7)
    before = master.copy()
    _run([np.zeros(500, np.float32)] * 3, master, m, v)
    np.testing.assert_array_equal(master, before)
    assert not m.any() and not v.any()


def test_writeback_is_rounded_master():
    master, m, v, g = _state(5000, 8)
    for dt, name in ((oracle.F16, np.float16), (oracle.BF16, None)):
        ms, mm, vv = master.copy(), m.copy(), v.copy()
        param = np.zeros(5000, np.uint16)
        _run([g], ms, mm, vv, param=param, param_dt=dt)
        if name is not None:
            np.testing.assert_array_equal(param, ms.astype(np.float16).view(np.uint16))
        else:
            want = torch.from_numpy(ms).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            np.testing.assert_array_equal(param, want)
