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
copies, and the pages' alignment padding."""
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


@pytest.mark.parametrize("psi,n_d,dt,align,wd,steps", [
    (1_000_003, 4, "bf16", 1, 0.1, 3),      # remainder 3: odd offsets, element path next to quads
    (1_000_003, 8, "f16", 16, 0.0, 3),      # padded to a multiple of 2 N_d, as the pages pad
    (2_097_189, 32, "f16", 1, 0.0, 2),      # 32 copies: wide tiles in the whole-vector and the segment steps
    (50_000_017, 64, "f16", 1, 0.0, 2),     # 64 copies at 50M elements
])
def test_segments_concatenate_to_the_whole_vector_step(psi, n_d, dt, align, wd, steps):
    tag = f"equivalence psi={psi} n_d={n_d} {dt} align={align}"
    print(f"[case] {tag}", flush=True)
    segs, padded = zdp.partition(psi, n_d, align)
    assert sum(s for _, s in segs) == padded and segs[-1][0] + segs[-1][1] == padded
    f16 = TORCH16[dt]

    def fp32(seed=None):
        t = torch.zeros(padded, dtype=torch.float32, device=DEV)
        if seed is not None:
            fill_normal_(t[:psi], 0.02, seed)          # the padding stays 0
        return t

    master0 = fp32((50, psi, n_d, "master"))
    whole = dict(master=master0.clone(), m=fp32(), v=fp32(), flat=master0.to(f16))
    parts = dict(master=master0.clone(), m=fp32(), v=fp32(), flat=master0.to(f16))
    ws_w, st_w = zdp.new_workspace(1), zdp.new_state(1.0)
    ranks = [(zdp.new_workspace(1), zdp.new_state(1.0)) for _ in range(n_d)]
    for k in range(steps):
        reps = []
        for r in range(n_d):
            g = torch.zeros(padded, dtype=f16, device=DEV)
            fill_normal_(g[:psi], 1e-3, (50, psi, n_d, "grad", k, r))
            reps.append(g)
        zdp.adam_step([zdp.Group(whole["master"], whole["m"], whole["v"], replicas=reps,
                                 flat_param=whole["flat"], weight_decay=wd)], ws_w, st_w)
        for r, (o, s) in enumerate(segs):
            ws, st = ranks[r]
            zdp.adam_step([zdp.Group(parts["master"][o:o + s], parts["m"][o:o + s], parts["v"][o:o + s],
                                     replicas=[g[o:o + s] for g in reps], flat_param=parts["flat"],
                                     param_offset=o, weight_decay=wd)], ws, st)
        torch.cuda.synchronize()
        sw = zdp.read_state(st_w)
        sr = [zdp.read_state(st) for _, st in ranks]
        assert all(x["step"] == sw["step"] == k + 1 for x in sr)
        assert sw["overflow"] == 0 and not any(x["overflow"] for x in sr)
        total = sum(x["grad_norm_sq"] for x in sr)
        assert abs(total - sw["grad_norm_sq"]) <= 1e-12 * sw["grad_norm_sq"], (total, sw["grad_norm_sq"])
        for name in ("master", "m", "v", "flat"):
            _assert_same(parts[name], whole[name], f"{tag} step {k + 1} {name}")
    if padded > psi:
        # zero gradients leave zero state: the padding never moves
        for name in ("master", "m", "v"):
            assert torch.count_nonzero(parts[name][psi:]) == 0, f"{tag}: padding of {name} moved"
    assert not torch.equal(parts["master"], master0), "the step changed nothing"
