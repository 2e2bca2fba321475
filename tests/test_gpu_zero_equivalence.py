"""ZeRO equivalence on the device: N_d ranks each stepping only their own
segment, with the segment of every gradient copy, give, concatenated, the
bits of one rank stepping the whole flat vector on the averaged gradient (the
plain data-parallel step). The update of a coordinate depends on that
coordinate alone (the reading notes, second part, §3), so partitioning the
optimizer state must not change a single bit of master, exp_avg, exp_avg_sq
or the written parameters; the rank-local squared norms add up to the whole
vector's (the two sums differ only in order).

The library is compared with itself through the C ABI, so these run at sizes
beyond the oracle's reach (50M elements, 64 copies), with odd segment offsets
(element path next to the quad path), the 8192-element tile of 32 or more
copies, and the pages' alignment padding; with a dynamic loss scale and no
overflow, through the checked and the optimistic pipelines as well."""
import pytest
import torch

import zero_dp_partitioned_amd as zdp
from workloads import fill_normal_

from _gpu_helpers import DEV, TORCH16

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _assert_same(got, want, what):
    diff = torch.nonzero(_bits(got) != _bits(want))
    if diff.numel():
        i = int(diff[0, 0])
        raise AssertionError(f"{what}: {diff.shape[0]} of {got.numel()} differ; first at {i}: "
                             f"{got[i].item()!r} vs {want[i].item()!r}")


@pytest.mark.parametrize("psi,n_d,dt,align,wd,steps,pipeline", [
    (1_000_003, 4, "bf16", 1, 0.1, 3, "fused"),      # remainder 3: odd offsets, element path next to quads
    (1_000_003, 8, "f16", 16, 0.0, 3, "fused"),      # padded to a multiple of 2 N_d, as the pages pad
    (2_097_189, 32, "f16", 1, 0.0, 2, "fused"),      # 32 copies: wide tiles in both steps
    (50_000_017, 64, "f16", 1, 0.0, 2, "fused"),     # 64 copies at 50M elements
    (1_000_003, 4, "bf16", 1, 0.1, 3, "checked"),    # average pass, verdict, update from the average
    (2_097_189, 32, "f16", 1, 0.0, 3, "optimistic"),  # second state set, committed every step
])
def test_segments_concatenate_to_the_whole_vector_step(psi, n_d, dt, align, wd, steps, pipeline):
    tag = f"equivalence psi={psi} n_d={n_d} {dt} align={align} {pipeline}"
    print(f"[case] {tag}", flush=True)
    segs, padded = zdp.partition(psi, n_d, align)
    assert sum(s for _, s in segs) == padded and segs[-1][0] + segs[-1][1] == padded
    f16 = TORCH16[dt]

    def fp32(seed=None):
        t = torch.zeros(padded, dtype=torch.float32, device=DEV)
        if seed is not None:
            fill_normal_(t[:psi], 0.02, seed)          # the padding stays 0
        return t

    scale = 1.0 if pipeline == "fused" else 1024.0
    pol = None if pipeline == "fused" else zdp.policy(True, optimistic=pipeline == "optimistic")
    master0 = fp32((50, psi, n_d, "master"))

    def buffers():
        b = dict(master=master0.clone(), m=fp32(), v=fp32(), flat=master0.to(f16))
        if pipeline == "optimistic":
            b.update(master_alt=fp32(), m_alt=fp32(), v_alt=fp32())
        return b

    whole, parts = buffers(), buffers()
    ws_w, st_w = zdp.new_workspace(1), zdp.new_state(scale)
    ranks = [(zdp.new_workspace(1), zdp.new_state(scale)) for _ in range(n_d)]

    def step(b, lo, hi, reps, ws, st):
        sl = slice(lo, hi)
        alt = {}
        if pipeline == "optimistic":
            alt = dict(master_alt=b["master_alt"][sl], exp_avg_alt=b["m_alt"][sl], exp_avg_sq_alt=b["v_alt"][sl])
        g = zdp.Group(b["master"][sl], b["m"][sl], b["v"][sl], replicas=[r[sl] for r in reps],
                      flat_param=b["flat"], param_offset=lo, weight_decay=wd, **alt)
        if pipeline == "checked":
            avg = torch.empty(hi - lo, dtype=torch.float32, device=DEV)
            zdp.reduce_grad_segment(g.replicas, avg, ws, 0, st)
            zdp.grad_norm_overflow(None, ws, 1, st, pol)
            g.replicas, g.avg = None, avg
        zdp.adam_step([g], ws, st, pol)

    def current(b, s):
        if s["cur"]:
            return dict(master=b["master_alt"], m=b["m_alt"], v=b["v_alt"], flat=b["flat"])
        return b

    for k in range(steps):
        reps = []
        for r in range(n_d):
            g = torch.zeros(padded, dtype=f16, device=DEV)
            fill_normal_(g[:psi], 1e-3, (50, psi, n_d, "grad", k, r), scale=scale)
            reps.append(g)
        step(whole, 0, padded, reps, ws_w, st_w)
        for r, (o, s) in enumerate(segs):
            step(parts, o, o + s, reps, *ranks[r])
        torch.cuda.synchronize()
        sw = zdp.read_state(st_w)
        sr = [zdp.read_state(st) for _, st in ranks]
        assert all(x["step"] == sw["step"] == k + 1 for x in sr)
        assert sw["overflow"] == 0 and not any(x["overflow"] for x in sr)
        assert all(x["cur"] == sw["cur"] for x in sr)
        total = sum(x["grad_norm_sq"] for x in sr)
        assert abs(total - sw["grad_norm_sq"]) <= 1e-12 * sw["grad_norm_sq"], (total, sw["grad_norm_sq"])
        cw, cp = current(whole, sw), current(parts, sw)
        for name in ("master", "m", "v", "flat"):
            _assert_same(cp[name], cw[name], f"{tag} step {k + 1} {name}")
    cp = current(parts, sw)
    if padded > psi:
        # zero gradients leave zero state: the padding never moves
        for name in ("master", "m", "v"):
            assert torch.count_nonzero(cp[name][psi:]) == 0, f"{tag}: padding of {name} moved"
    assert not torch.equal(cp["master"], master0), "the step changed nothing"
