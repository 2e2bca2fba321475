"""The step as a production training loop uses it: captured in a HIP graph and
replayed, and checkpointed / resumed mid-run.

* The library allocates nothing and never synchronises inside a call, so a
  fused step can be captured once and replayed; every replay (with eager work
  and synchronisations between replays) must give the eager step's bits.
* The rank's whole optimizer state is the fp32 master / m / v shard plus the
  176-byte step state; copying them out and back into fresh buffers must
  continue bit-identically, loss scale, step count and beta powers included."""
import numpy as np
import pytest
import torch

import zero_dp_partitioned_amd as zdp
from workloads import grads16_np, normal_f32_np, to16_bits_np

from _gpu_helpers import DEV, assert_bits_equal, assert_u16_equal, down16, down32, up16, up32

pytestmark = pytest.mark.gpu


def _setup(n, n_d, seed, dt="bf16"):
    master0 = normal_f32_np(n, 0.02, (seed, "master"))
    grp = zdp.Group(up32(master0), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV),
                    replicas=[torch.empty(n, dtype=torch.bfloat16, device=DEV) for _ in range(n_d)],
                    flat_param=up16(to16_bits_np(master0, dt), dt), weight_decay=0.1)
    return grp


def _load_grads(grp, k, seed, scale=1.0):
    for r, t in enumerate(grp.replicas):
        t.copy_(up16(grads16_np(t.numel(), "bf16", scale, (seed, "g", k, r)), "bf16"))


def test_graph_capture_and_replay_matches_eager():
    n, n_d, steps = 300_001, 4, 4
    eager, graphed = _setup(n, n_d, 21), _setup(n, n_d, 21)
    ws_e, st_e = zdp.new_workspace(1), zdp.new_state(1.0)
    ws_g, st_g = zdp.new_workspace(1), zdp.new_state(1.0)
    # capture one step of the graphed copy (its gradient buffers are refilled between replays)
    _load_grads(graphed, 0, 21)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        zdp.adam_step([graphed], ws_g, st_g)
    torch.cuda.synchronize()
    # capturing does not run the step: state untouched
    assert zdp.read_state(st_g)["step"] == 0
    for k in range(steps):
        _load_grads(eager, k, 21)
        zdp.adam_step([eager], ws_e, st_e)
        _load_grads(graphed, k, 21)
        graph.replay()
        junk = torch.randn(1000, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        tag = f"replay {k + 1}"
        assert_bits_equal(down32(graphed.master), down32(eager.master), tag + " master")
        assert_bits_equal(down32(graphed.exp_avg), down32(eager.exp_avg), tag + " exp_avg")
        assert_bits_equal(down32(graphed.exp_avg_sq), down32(eager.exp_avg_sq), tag + " exp_avg_sq")
        assert_u16_equal(down16(graphed.flat_param), down16(eager.flat_param), tag + " param")
        np.testing.assert_array_equal(st_g.cpu().numpy(), st_e.cpu().numpy())
    assert zdp.read_state(st_g)["step"] == steps


@pytest.mark.parametrize("optimistic", [False, True])
def test_static_step_captured_in_a_graph(optimistic):
    """zero_adam_step_static, the entry point for callers that cannot
    allocate, captured once and replayed: every replay gives the bits of the
    eager zero_adam_step with a workspace (an overflowing call voids a step
    of the optimistic pipeline, whose restore launch is in the graph). The
    first call on the device, which looks the static array up, is made before
    the capture."""
    n, n_d, steps = 300_001, 4, 4
    eager, graphed = _setup(n, n_d, 22), _setup(n, n_d, 22)
    pol = zdp.policy(True, optimistic=True, growth_interval=2) if optimistic else None
    if optimistic:
        for g in (eager, graphed):
            g.master_alt, g.exp_avg_alt, g.exp_avg_sq_alt = (torch.zeros(n, device=DEV) for _ in range(3))
    ws_e, st_e = zdp.new_workspace(1), zdp.new_state(1024.0 if optimistic else 1.0)
    st_g = zdp.new_state(1024.0 if optimistic else 1.0)
    # the first call on the device, outside the capture
    tiny = _setup(4099, 1, 23)
    zdp.adam_step_static([tiny], zdp.new_state(1.0))
    _load_grads(graphed, 0, 22)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        zdp.adam_step_static([graphed], st_g, pol)
    torch.cuda.synchronize()
    assert zdp.read_state(st_g)["step"] == 0
    for k in range(steps):
        scale = zdp.read_state(st_e)["loss_scale"]
        for g in (eager, graphed):
            _load_grads(g, k, 22, scale)
            if optimistic and k == 1:
                g.replicas[2][n // 3] = float("inf")
        zdp.adam_step([eager], ws_e, st_e, pol)
        graph.replay()
        junk = torch.randn(1000, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        tag = f"replay {k + 1}"
        se, sg = zdp.read_state(st_e), zdp.read_state(st_g)
        for x, y, name in zip(zdp.current_state(graphed, sg), zdp.current_state(eager, se),
                              ("master", "exp_avg", "exp_avg_sq")):
            assert_bits_equal(down32(x), down32(y), f"{tag} {name}")
        assert_u16_equal(down16(graphed.flat_param), down16(eager.flat_param), tag + " param")
        np.testing.assert_array_equal(st_g.cpu().numpy(), st_e.cpu().numpy())
    se = zdp.read_state(st_e)
    assert se["step"] == (steps - 1 if optimistic else steps)


@pytest.mark.parametrize("optimistic", [False, True])
def test_checkpoint_resume_is_bit_identical(optimistic):
    n, n_d, steps, cut = 200_003, 2, 6, 3
    pol = zdp.policy(True, growth_interval=2, optimistic=optimistic)

    def make():
        g = _setup(n, n_d, 22)
        if optimistic:
            g.master_alt, g.exp_avg_alt, g.exp_avg_sq_alt = (torch.zeros(n, device=DEV) for _ in range(3))
        return g

    def step(g, ws, st, k):
        _load_grads(g, k, 22, scale=zdp.read_state(st)["loss_scale"])
        if k == 1:
            g.replicas[1][77] = float("inf")   # one voided step inside the first half
        if optimistic:
            zdp.adam_step([g], ws, st, pol)
            return
        avg = torch.empty(n, device=DEV)
        zdp.reduce_grad_segment(g.replicas, avg, ws, 0, st)
        zdp.grad_norm_overflow(None, ws, 1, st, pol)
        reps, g.replicas, g.avg = g.replicas, None, avg
        zdp.adam_step([g], ws, st, pol)
        g.replicas, g.avg = reps, None

    # uninterrupted run
    a, ws_a, st_a = make(), zdp.new_workspace(1), zdp.new_state(1024.0)
    for k in range(steps):
        step(a, ws_a, st_a, k)
    # run, checkpoint to the host, resume into fresh buffers
    b, ws_b, st_b = make(), zdp.new_workspace(1), zdp.new_state(1024.0)
    for k in range(cut):
        step(b, ws_b, st_b, k)
    torch.cuda.synchronize()
    s = zdp.read_state(st_b)
    cm, cmm, cv = zdp.current_state(b, s)
    ckpt = {"master": cm.cpu(), "exp_avg": cmm.cpu(), "exp_avg_sq": cv.cpu(), "state": st_b.cpu(),
            "flat": b.flat_param.cpu()}
    del b, ws_b, st_b
    c = make()
    c.master.copy_(ckpt["master"].to(DEV))
    c.exp_avg.copy_(ckpt["exp_avg"].to(DEV))
    c.exp_avg_sq.copy_(ckpt["exp_avg_sq"].to(DEV))
    c.flat_param.copy_(ckpt["flat"].to(DEV))
    # the restored buffers are the primary set: point the state at it
    raw = ckpt["state"].numpy().copy()
    state = zdp.StepState.from_buffer_copy(raw.tobytes())
    state.cur = 0
    st_c = torch.from_numpy(np.frombuffer(bytes(state), dtype=np.uint8).copy()).to(DEV)
    ws_c = zdp.new_workspace(1)
    for k in range(cut, steps):
        step(c, ws_c, st_c, k)
    torch.cuda.synchronize()
    sa, sc = zdp.read_state(st_a), zdp.read_state(st_c)
    for key in ("step", "loss_scale", "good_steps", "beta1_pow", "beta2_pow", "grad_norm_sq", "skipped"):
        assert sa[key] == sc[key], key
    assert sa["step"] == steps - 1
    for x, y, what in zip(zdp.current_state(a, sa), zdp.current_state(c, sc), ("master", "exp_avg", "exp_avg_sq")):
        assert_bits_equal(down32(y), down32(x), "resumed " + what)
    assert_u16_equal(down16(c.flat_param), down16(a.flat_param), "resumed param")
