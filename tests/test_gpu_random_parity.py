"""Random parity sweep: 1,000 seeded random configurations (and 24 large ones) of the whole step against
the oracle, bit for bit, three calls each. Each case draws 1-3 groups (shard
length 1..40,000, or 1.5M..6M in the large cases, N_d per group from 1-9, 32, 48, 64 or 65, parameter offset and
alignment, unaligned fp32 state), a gradient dtype, a copy layout (pointer
table, equally spaced buffer, packed unaligned, or each copy as far past
alignment as the fp32 state, which the kernels peel as a short head), a pipeline (fused, checked,
optimistic) with or without clipping, a loss scale, an inf or NaN written
into a copy now and then, and the parameter vector's dtype (the gradients'
most of the time, the other 16-bit type, or no fused writeback at all). About
half of the cases also cap every launch's grid (zdp.set_grid_limit) at a few
blocks or just either side of 256 (on the small shards only the caps of a few
blocks bind), so that blocks loop over tiles and launches write their level-2
norm partials themselves or leave them to a fold. The bar
is test_gpu_parity's: bit for bit, unless the two sides' clip multipliers are
one ulp apart (then the stated tolerances from that call on)."""
import numpy as np
import pytest
import torch

import oracle
import zero_dp_partitioned_amd as zdp
from workloads import grads16_np, normal_f32_np, to16_bits_np

from _gpu_helpers import DEV, ORACLE_DT, assert_u16_equal, carve, down16, up16, up32
from _parity import Bar
from test_gpu_parity import NEG_NAN, POS_INF, _compare_group, _compare_state, _replicas_on_device

pytestmark = pytest.mark.gpu

N_CASES = 1000


N_LARGE = 24


def _case(seed, large=False):
    rng = np.random.Generator(np.random.PCG64(seed + (1 << 20 if large else 0)))
    dt = ["f16", "bf16"][rng.integers(2)]
    pipeline = ["fused", "checked", "optimistic"][rng.integers(3)]
    clip = bool(rng.integers(2)) and pipeline != "fused"
    groups = []
    for _ in range(int(rng.integers(1, 3 if large else 4))):
        if large:   # beyond the restore kernel's 1,024-block grid: its blocks loop over tiles
            n, n_d = int(rng.integers(1_500_000, 6_000_000)), int(rng.choice([1, 2, 4, 8]))
        else:
            n = int(rng.choice([1, 7, 8, 9, 255, 4096, 4097, int(rng.integers(1, 40_000))]))
            n_d = int(rng.choice([1, 1, 2, 3, 4, 5, 8, 9, 32, 48, 64, 65]))
        layout = "strided" if n_d > 64 else ["table", "strided", "packed", "shift"][rng.integers(4)]
        groups.append(dict(n=n, n_d=n_d, layout=layout, off=int(rng.integers(0, 9)),
                           mis=int(rng.choice([0, 0, 0, 1, 2])), wd=float(rng.choice([0.0, 0.1]))))
    scale = float(rng.choice([1.0, 1024.0] + ([65536.0] if dt == "f16" else [2.0 ** 20])))
    total = sum(g["n"] / g["n_d"] for g in groups)
    max_norm = 1e-3 * np.sqrt(total) * float(rng.uniform(0.5, 2.0)) if clip else 0.0
    inject = [bool(rng.random() < 0.25) for _ in range(3)]
    pdt = [dt, dt, dt, {"f16": "bf16", "bf16": "f16"}[dt], None][rng.integers(5)]
    return dt, pipeline, clip, groups, scale, max_norm, inject, pdt


def _grid_limit(seed, large=False):
    """The case's block cap (0: none), drawn from a stream of its own so that
    the case's other draws are unchanged."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7, int(large)])))
    return int(rng.choice([0, 0, 0, 0, 0, 0, 0, 1, 2, 3, 7, 255, 256, 257]))


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration(seed):
    run_case(seed, _case(seed), _grid_limit(seed))


@pytest.mark.parametrize("seed", range(N_LARGE))
def test_random_large_configuration(seed):
    run_case(seed, _case(seed, large=True), _grid_limit(seed, large=True))


def run_case(seed, case, grid_limit=0):
    zdp.set_grid_limit(grid_limit)
    try:
        _run_case(seed, case, grid_limit)
    finally:
        zdp.set_grid_limit(0)


def _run_case(seed, case, grid_limit):
    dt, pipeline, clip, specs, scale, max_norm, inject, pdt = case
    dynamic = pipeline != "fused" and (pipeline == "optimistic" or seed % 2 == 0)
    tag = (f"seed {seed}: {dt} params {pdt} {pipeline} dynamic={dynamic} clip={max_norm:.3g} scale={scale} "
           f"grid limit {grid_limit} groups={specs}")
    print(f"[case] {tag}", flush=True)
    odt = ORACLE_DT[dt]
    opdt = ORACLE_DT[pdt] if pdt else odt
    pol = oracle.Policy(skip_on_overflow=dynamic, growth_interval=2, max_grad_norm=max_norm)
    sc = (zdp.policy(dynamic, growth_interval=2, max_grad_norm=max_norm, optimistic=pipeline == "optimistic")
          if pipeline != "fused" else None)
    if pipeline == "checked" and not dynamic and max_norm == 0.0:
        sc = None   # nothing asks for the norm first: the fused pipeline
        pol = oracle.Policy()
    grps, ogs, flats0 = [], [], []
    for gi, g in enumerate(specs):
        n, off, mis = g["n"], g["off"], g["mis"]
        master0 = normal_f32_np(n, 0.02, (40, seed, gi, "master"))
        flat0 = to16_bits_np(normal_f32_np(off + n + 3, 0.02, (40, seed, gi, "flat")), pdt or dt)
        flat0[off:off + n] = to16_bits_np(master0, pdt or dt)

        def fp32(x=None):
            t = carve(n + 8, mis, n, torch.float32)
            return t.copy_(up32(x)) if x is not None else t.zero_()

        alt = {}
        if pipeline == "optimistic":
            alt = dict(master_alt=fp32(), exp_avg_alt=fp32(), exp_avg_sq_alt=fp32())
        grps.append(zdp.Group(fp32(master0), fp32(), fp32(), flat_param=up16(flat0, pdt) if pdt else None,
                              param_offset=off if pdt else 0, weight_decay=g["wd"], **alt))
        ogs.append(oracle.Group(replicas=None, grad_dt=odt, master=master0.copy(), m=np.zeros(n, np.float32),
                                v=np.zeros(n, np.float32), param=flat0[off:off + n].copy() if pdt else None,
                                param_dt=opdt, weight_decay=g["wd"]))
        flats0.append(flat0)
    ws, st = zdp.new_workspace(len(specs)), zdp.new_state(scale)
    ost = oracle.State(loss_scale=scale)
    bar = Bar()   # bit for bit, or the tolerances once the clip multipliers differ by an ulp
    checked = zdp.is_checked(sc) if sc is not None else False
    avgs = [torch.empty(g["n"], dtype=torch.float32, device=DEV) for g in specs] if checked else None
    for k in range(3):
        host, dev = [], []
        for gi, (g, spec) in enumerate(zip(grps, specs)):
            reps = [grads16_np(spec["n"], dt, ost.loss_scale, (40, seed, gi, k, r)) for r in range(spec["n_d"])]
            if inject[k] and gi == 0:
                r = (seed + k) % spec["n_d"]
                reps[r] = reps[r].copy()
                reps[r][(seed * 7919 + k) % spec["n"]] = (POS_INF if (seed + k) % 2 else NEG_NAN)[dt]
            host.append(reps)
            lay = f"shift{spec['mis']}" if spec["layout"] == "shift" else spec["layout"]
            dev.append(_replicas_on_device(reps, dt, lay))
        if checked:
            scans = []
            for gi, (g, spec) in enumerate(zip(grps, specs)):
                if spec["n_d"] == 1 and gi % 2 == 0:
                    scans.append(dev[gi][0])          # single copy: the norm pass scans it
                    g.replicas, g.avg = dev[gi], None
                else:
                    zdp.reduce_grad_segment(dev[gi], avgs[gi], ws, gi, st)
                    scans.append(None)
                    g.replicas, g.avg = None, avgs[gi]
            zdp.grad_norm_overflow(scans if any(x is not None for x in scans) else None, ws, len(grps), st, sc,
                                   grad_dtype=zdp.DT_F16 if dt == "f16" else zdp.DT_BF16)
        else:
            for g, d in zip(grps, dev):
                g.replicas, g.avg = d, None
        zdp.adam_step(grps, ws, st, sc)
        for og, reps in zip(ogs, host):
            og.replicas = reps
        oracle.step(ogs, pol, ost)
        torch.cuda.synchronize()
        s = _compare_state(f"{tag} call {k + 1}", st, ost, bar)
        for gi, (g, og, spec) in enumerate(zip(grps, ogs, specs)):
            cm, cmm, cv = zdp.current_state(g, s)
            _compare_group(f"{tag} call {k + 1} group {gi}", cm, cmm, cv, og, bar)
            if pdt is None:
                continue
            got = down16(g.flat_param)
            off, n = spec["off"], spec["n"]
            bar.param16(got[off:off + n], og.param, f"{tag} call {k + 1} group {gi} param")
            outside = np.r_[0:off, off + n:flats0[gi].size]
            assert_u16_equal(got[outside], flats0[gi][outside], f"{tag} group {gi} outside the slice")


@pytest.mark.parametrize("pipeline", ["fused", "checked", "optimistic"])
def test_the_maximum_number_of_groups(pipeline):
    """ZERO_MAX_GROUPS (8) groups in one step, of assorted lengths, copy
    counts, layouts and decays: one shared norm and verdict, eight sets of β
    powers, every level-2 slot of the workspace. The second call carries an
    inf in group 0 (voided under the dynamic scale of the checked and
    optimistic pipelines, which also clip)."""
    assert zdp.MAX_GROUPS == 8
    shapes = [(1, 1, "table", 0, 0.0), (4097, 2, "strided", 3, 0.1), (30_011, 3, "packed", 1, 0.1),
              (7, 4, "table", 5, 0.0), (300_001, 8, "shift", 2, 0.1), (255, 1, "table", 8, 0.0),
              (65_536, 32, "table", 0, 0.1), (2, 5, "strided", 7, 0.0)]
    specs = [dict(n=n, n_d=nd, layout=lay, off=off, mis=1 if lay == "shift" else 0, wd=wd)
             for n, nd, lay, off, wd in shapes]
    total = sum(g["n"] / g["n_d"] for g in specs)
    max_norm = 1e-3 * np.sqrt(total) * 0.8 if pipeline != "fused" else 0.0
    case = ("bf16", pipeline, pipeline != "fused", specs, 1024.0, max_norm, [False, True, False], "bf16")
    run_case(2 * 4321, case)   # an even seed: the checked pipeline takes the dynamic scale
