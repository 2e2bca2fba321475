"""Gradient clipping by the global norm in the oracle.

The DeepSpeed walkthrough (§6 step 3) unscales and clips the rank's gradient
shard before the update, with the norm of step 2, but gives no formula. The
reading: multiplier c = min(1, max_norm / (norm + 1e-6)), formed in fp64 and
rounded once, applied to the unscaled gradient. Pins: torch's
clip_grad_norm_ followed by torch.optim.Adam/AdamW, both in float64 (an
independent implementation of the same rule); bit-identity with the unclipped
step when the norm is below the threshold; the clipped gradient's norm equals
the threshold."""
import numpy as np
import pytest
import torch

import oracle
from workloads import grads16_np, normal_f32_np

U = 2.0 ** -24
LR, B1, B2, EPS = 1e-3, 0.9, 0.999, 1e-8


def _group(n, n_d, seed, wd=0.0, scale=1.0):
    reps = [grads16_np(n, "bf16", scale, seed=(seed, r)) for r in range(n_d)]
    return oracle.Group(replicas=reps, grad_dt=oracle.BF16, master=normal_f32_np(n, 0.02, (seed, "m")),
                        m=np.zeros(n, np.float32), v=np.zeros(n, np.float32), weight_decay=wd)


@pytest.mark.parametrize("wd", [0.0, 0.1])
@pytest.mark.parametrize("max_norm", [0.01, 0.03])
def test_clip_matches_torch_float64(wd, max_norm):
    n, steps, scale = 5000, 4, 1024.0
    g = _group(n, 2, 1, wd=wd, scale=scale)
    p = torch.nn.Parameter(torch.from_numpy(g.master.astype(np.float64)))
    cls = torch.optim.AdamW if wd else torch.optim.Adam
    opt = cls([p], lr=LR, betas=(B1, B2), eps=EPS, weight_decay=wd, foreach=False)
    st = oracle.State(loss_scale=scale)
    pol = oracle.Policy(max_grad_norm=max_norm)
    clipped = 0
    for k in range(steps):
        g.replicas = [grads16_np(n, "bf16", scale, seed=(1, k, r)) for r in range(2)]
        a = oracle.average(g.replicas, oracle.BF16)
        grad = (a.astype(np.float64) / scale)   # exact: power-of-two scale
        p.grad = torch.from_numpy(grad.copy())
        total = torch.nn.utils.clip_grad_norm_([p], max_norm)
        opt.step()
        oracle.step([g], pol, st)
        assert np.sqrt(st.norm2) == pytest.approx(float(total), rel=1e-12)
        clipped += st.clip < 1.0
    assert clipped == steps  # the gradient norm (~0.05) is above both thresholds
    want = p.detach().numpy()
    assert (np.abs(g.master - want) <= steps * (2 * U * np.abs(want) + LR * 32 * U)).all()
    m_ref = opt.state[p]["exp_avg"].numpy()
    assert (np.abs(g.m - m_ref) <= 8 * steps * U * np.abs(m_ref).max()).all()


def test_clip_is_a_no_op_below_the_threshold():
    a, b = _group(3000, 4, 2), _group(3000, 4, 2)
    sa, sb = oracle.State(), oracle.State()
    oracle.step([a], oracle.Policy(), sa)
    oracle.step([b], oracle.Policy(max_grad_norm=1e6), sb)
    assert sb.clip == 1.0
    for x, y in ((a.master, b.master), (a.m, b.m), (a.v, b.v)):
        np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32))


def test_clipped_gradient_has_the_threshold_norm():
    g = _group(20_000, 2, 3)
    st = oracle.State()
    oracle.step([g], oracle.Policy(max_grad_norm=0.02), st)
    norm = np.sqrt(st.norm2)
    assert norm > 0.02 and st.clip < 1
    # m after one step is (1 - beta1) * clip * g exactly up to rounding
    a = oracle.average(g.replicas, oracle.BF16).astype(np.float64)
    clipped = a * np.float64(st.clip)
    assert np.sqrt((clipped ** 2).sum()) == pytest.approx(0.02 * norm / (norm + 1e-6), rel=1e-6)
    np.testing.assert_allclose(g.m, (1 - B1) * clipped, rtol=4 * U, atol=1e-30)


def test_clip_ignored_on_overflow_and_in_skip():
    g = _group(100, 1, 4)
    g.replicas[0] = g.replicas[0].copy()
    g.replicas[0][7] = 0x7F80
    st = oracle.State()
    oracle.step([g], oracle.Policy(skip_on_overflow=True, max_grad_norm=0.01), st)
    assert st.skipped == 1 and st.clip == 1.0


@pytest.mark.parametrize("max_norm", [0.0, 0.01, 1e6])
def test_sampled_step_with_the_shard_norm_equals_the_full_step(max_norm):
    # stepping a sample of coordinates with the whole shard's norm² and flag
    # (oracle_step_given_norm) gives exactly the full step's values there, over
    # calls with clipping, an overflow (skip) and scale growth, two groups
    pol = oracle.Policy(skip_on_overflow=True, growth_interval=2, max_grad_norm=max_norm)
    full = [_group(6000, 3, 31, wd=0.1, scale=64.0), _group(1500, 3, 32, scale=64.0)]
    idx = [np.array([0, 1, 2999, 5998, 5999]), np.array([0, 750, 1499])]
    smp = [oracle.Group(replicas=None, grad_dt=g.grad_dt, master=g.master[i].copy(), m=g.m[i].copy(),
                        v=g.v[i].copy(), param=None, weight_decay=g.weight_decay) for g, i in zip(full, idx)]
    sf, ss = oracle.State(loss_scale=64.0), oracle.State(loss_scale=64.0)
    for k in range(5):
        for gi, (g, s, i) in enumerate(zip(full, smp, idx)):
            g.replicas = [grads16_np(g.master.size, "bf16", sf.loss_scale, (33, k, gi, r)) for r in range(3)]
            if k == 2 and gi == 1:
                g.replicas[0] = g.replicas[0].copy()
                g.replicas[0][100] = 0x7F80         # outside the sample: only the shard flag sees it
            s.replicas = [r[i].copy() for r in g.replicas]
        oracle.step(full, pol, sf)
        oracle.step(smp, pol, ss, norm2=sf.norm2, flag=sf.overflow)
        assert (ss.step, ss.skipped, ss.loss_scale, ss.good_steps, ss.clip) == \
               (sf.step, sf.skipped, sf.loss_scale, sf.good_steps, sf.clip)
        for g, s, i in zip(full, smp, idx):
            for a, b in ((g.master[i], s.master), (g.m[i], s.m), (g.v[i], s.v)):
                np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    assert sf.skipped == 0 and sf.step == 4
    if max_norm == 0.01:
        assert sf.clip < 1.0


@pytest.mark.parametrize("max_norm", [0.0, 0.01])
def test_chunked_step_from_averages_equals_the_full_step(max_norm):
    # the full-size GPU tests' use of the oracle: average every chunk of a
    # shard once (oracle_average), add the chunks' fp64 norm sums in chunk
    # order, then step each chunk from its average with the whole shard's
    # norm² and flag (oracle_step_from_average, every chunk from the same
    # state before the call). The chunks' values equal the full step's bit
    # for bit, and their states the full step's state; the chunked norm equals
    # the full one within fp64 reassociation. Over calls with clipping, an
    # overflow (skip), scale growth and two groups.
    pol = oracle.Policy(skip_on_overflow=True, growth_interval=2, max_grad_norm=max_norm)
    full = [_group(6001, 3, 41, wd=0.1, scale=64.0), _group(1499, 3, 42, scale=64.0)]
    part = [oracle.Group(replicas=None, grad_dt=g.grad_dt, master=g.master.copy(), m=g.m.copy(), v=g.v.copy(),
                         param=np.zeros(g.master.size, np.uint16), param_dt=oracle.BF16,
                         weight_decay=g.weight_decay) for g in full]
    for g in full:
        g.param, g.param_dt = np.zeros(g.master.size, np.uint16), oracle.BF16
    chunk = 1000
    sf, sc = oracle.State(loss_scale=64.0), oracle.State(loss_scale=64.0)
    for k in range(6):
        for gi, g in enumerate(full):
            g.replicas = [grads16_np(g.master.size, "bf16", sf.loss_scale, (43, k, gi, r)) for r in range(3)]
            if k == 2 and gi == 1:
                g.replicas[2] = g.replicas[2].copy()
                g.replicas[2][1400] = 0xFFC0       # a NaN in the last chunk of the second group
        oracle.step(full, pol, sf)
        inv = oracle.inv_scale_of(sc.loss_scale)
        chunks, n2, flag = [], 0.0, 0
        for gi, g in enumerate(full):
            for s in range(0, g.master.size, chunk):
                e = min(g.master.size, s + chunk)
                a = oracle.average([r[s:e] for r in g.replicas], g.grad_dt)
                c2, cf = oracle.norm_overflow(a, inv)
                n2, flag = n2 + c2, flag | cf
                chunks.append((gi, s, e, a))
        after = []
        for gi, s, e, a in chunks:
            p = part[gi]
            cg = oracle.Group(replicas=None, grad_dt=p.grad_dt, master=p.master[s:e], m=p.m[s:e], v=p.v[s:e],
                              param=p.param[s:e], param_dt=p.param_dt, weight_decay=p.weight_decay)
            st = oracle.State(**vars(sc))
            oracle.step_from_average([cg], [a], pol, st, n2, flag)
            after.append(st)
        def same(x, y):   # NaN norms compare equal
            return all(a == b or (a != a and b != b) for a, b in zip(vars(x).values(), vars(y).values()))
        assert all(same(st, after[0]) for st in after)
        sc = after[0]
        assert abs(sc.norm2 - sf.norm2) <= 1e-12 * sf.norm2 or not np.isfinite(sf.norm2)
        assert (sc.step, sc.skipped, sc.loss_scale, sc.good_steps, sc.overflow) == \
               (sf.step, sf.skipped, sf.loss_scale, sf.good_steps, sf.overflow)
        assert sc.clip == sf.clip
        for g, p in zip(full, part):
            for a, b in ((g.master, p.master), (g.m, p.m), (g.v, p.v)):
                np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
            np.testing.assert_array_equal(g.param, p.param)
    assert sf.step == 5
    if max_norm == 0.01:
        assert sf.clip < 1.0
