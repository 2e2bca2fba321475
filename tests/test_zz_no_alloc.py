"""The allocation-free step (zero_adam_step_static, norm partials in the
library's static device scratch) against the workspace step (zero_adam_step)
through the C ABI: the same inputs on two sides, two calls in a row, the
second with a smaller shard (the scratch still holds the first call's
partials), every element of master, m, v and the parameters and the whole
step state bit for bit. Fused pipeline over two groups, and the optimistic
pipeline with clipping and an overflowing first call (restore and second
pass)."""
import numpy as np
import pytest
import torch

import zero_dp_partitioned_amd as zdp
from workloads import grads16_np, normal_f32_np, to16_bits_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _groups(sizes, n_d, dt, seed, call, optimistic, inf_at=None):
    """Two identical device copies of a step's inputs: (groups_a, groups_b)."""
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    sides = ([], [])
    for gi, n in enumerate(sizes):
        master = normal_f32_np(n, 0.02, (seed, call, gi, "master"))
        flat = to16_bits_np(normal_f32_np(n + 9, 0.02, (seed, call, gi, "flat")), dt)
        flat[5:5 + n] = to16_bits_np(master, dt)
        reps = [grads16_np(n, dt, 1024.0, (seed, call, gi, r)) for r in range(n_d)]
        if inf_at is not None and gi == 0:
            reps[0] = reps[0].copy()
            reps[0][inf_at % n] = 0x7C00 if dt == "f16" else 0x7F80
        for side in sides:
            up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)  # noqa: E731
            f32 = lambda: torch.zeros(n, device=DEV)  # noqa: E731
            alt = dict(master_alt=f32(), exp_avg_alt=f32(), exp_avg_sq_alt=f32()) if optimistic else {}
            side.append(zdp.Group(up(master), f32(), f32(),
                                  replicas=[up(r.view(np.int16)).view(tdt) for r in reps],
                                  flat_param=up(flat.view(np.int16)).view(tdt), param_offset=5,
                                  weight_decay=0.1 * gi, **alt))
    return sides


def _same(tag, a, b):
    ia = a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16)
    ib = b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)
    if not torch.equal(ia, ib):
        i = int(torch.nonzero(ia != ib)[0])
        raise AssertionError(f"{tag}: differ at element {i}")


@pytest.mark.parametrize("pipeline", ["fused", "optimistic"])
def test_static_scratch_step_equals_the_workspace_step(pipeline):
    optimistic = pipeline == "optimistic"
    pol = zdp.policy(True, optimistic=True, max_grad_norm=0.05, growth_interval=3) if optimistic else None
    ws = zdp.new_workspace(2)
    st_a, st_b = zdp.new_state(1024.0), zdp.new_state(1024.0)
    # the second call's shard is smaller than the first's
    calls = [((3_000_017, 40_961), 8, "f16", 123), ((100_003, 777), 4, "bf16", None)]
    for call, (sizes, n_d, dt, inf_at) in enumerate(calls):
        tag = f"{pipeline} call {call + 1} sizes {sizes}"
        print(f"[case] no-alloc {tag}", flush=True)
        ga, gb = _groups(sizes, n_d, dt, 51, call, optimistic, inf_at if optimistic else None)
        zdp.adam_step(ga, ws, st_a, pol)
        zdp.adam_step_static(gb, st_b, pol)
        torch.cuda.synchronize()
        sa, sb = zdp.read_state(st_a), zdp.read_state(st_b)
        assert bytes(st_a.cpu().numpy()) == bytes(st_b.cpu().numpy()), (tag, sa, sb)
        for gi, (a, b) in enumerate(zip(ga, gb)):
            for name, x, y in zip(("master", "exp_avg", "exp_avg_sq"), zdp.current_state(a, sa),
                                  zdp.current_state(b, sb)):
                _same(f"{tag} group {gi} {name}", x, y)
            _same(f"{tag} group {gi} param", a.flat_param, b.flat_param)
        if optimistic and call == 0:
            assert sa["skipped"] == 1          # the overflowing call was voided on both sides
        if optimistic and call == 1:
            assert sa["skipped"] == 0 and sa["clip_coef"] < 1.0   # a clipped step: the second pass ran
        print(f"  {tag}: ok (step {sa['step']}, norm {sa['grad_norm']:.6g}, skipped {sa['skipped']}, "
              f"clip {sa['clip_coef']:.6g})", flush=True)


def test_static_scratch_refuses_too_many_groups():
    g = zdp.Group(torch.zeros(4, device=DEV), torch.zeros(4, device=DEV), torch.zeros(4, device=DEV),
                  replicas=[torch.zeros(4, dtype=torch.float16, device=DEV)])
    with pytest.raises(zdp.ZeroError) as e:
        zdp.adam_step_static([g] * (zdp.MAX_GROUPS + 1), zdp.new_state())
    assert e.value.code == zdp.ERR_INVALID_ARG and "static scratch" in str(e.value)
