"""The HBM placement helper zero_plan_arena on the host: the layout it returns
is valid (aligned, disjoint, inside its region and below max_bytes), spreads a
step's traffic over the regions, and rejects bad arguments."""
import ctypes

import pytest
from hypothesis import given, settings, strategies as st

import zero_dp_partitioned_amd as zdp

A = zdp.ARENA_ALIGN
R = zdp.HBM_REGION_BYTES
GiB = 1 << 30


def _up(x):
    return (x + A - 1) // A * A


def _check_layout(sizes, traffic, offs, regs, total, region, max_bytes):
    spans = sorted((o, o + _up(b)) for o, b in zip(offs, sizes))
    for (a0, a1), (b0, _) in zip(spans, spans[1:]):
        assert a1 <= b0, "buffers overlap"
    for o, b, r in zip(offs, sizes, regs):
        assert o % A == 0
        assert r * region <= o and o + _up(b) <= (r + 1) * region, "buffer leaves its region"
        assert o + _up(b) <= max_bytes
    assert total == max(o + _up(b) for o, b in zip(offs, sizes))


def test_struct_layout():
    assert ctypes.sizeof(zdp.ArenaBuffer) == 32


def test_gpt2_shard_in_two_regions():
    n = 1_557_611_200
    sizes = [4 * n, 4 * n, 4 * n, 2 * n, 2 * n]   # master, exp_avg, exp_avg_sq, gradient, parameters
    traffic = [8 * n, 8 * n, 8 * n, 2 * n, 2 * n]
    offs, regs, total = zdp.plan_arena(sizes, traffic, 280 * GiB)
    assert regs == [0, 1, 0, 1, 1]
    assert offs == [0, R, _up(4 * n), R + _up(4 * n), R + _up(4 * n) + _up(2 * n)]
    _check_layout(sizes, traffic, offs, regs, total, R, 280 * GiB)
    # each region carries part of the traffic; neither carries all of it
    load = [sum(t for t, r in zip(traffic, regs) if r == k) for k in (0, 1)]
    assert load == [16 * n, 12 * n]


def test_auto_region_count_and_limits():
    # buffers that need three regions
    big = [40 * GiB] * 6
    offs, regs, total = zdp.plan_arena(big, [1] * 6, 280 * GiB)
    assert sorted(set(regs)) == [0, 1, 2]
    _check_layout(big, [1] * 6, offs, regs, total, R, 280 * GiB)
    # max_bytes below one region: everything in region 0
    offs, regs, total = zdp.plan_arena([GiB, GiB], [5, 5], 50 * GiB)
    assert regs == [0, 0] and total == 2 * GiB
    # the last region is cut at max_bytes
    with pytest.raises(zdp.ZeroError) as e:
        zdp.plan_arena([90 * GiB, 90 * GiB, 20 * GiB], [3, 2, 1], 2 * R + 10 * GiB, n_regions=3)
    assert e.value.code == zdp.ERR_UNSUPPORTED
    offs, regs, total = zdp.plan_arena([90 * GiB, 90 * GiB, 8 * GiB], [3, 2, 1], 2 * R + 10 * GiB, n_regions=3)
    assert regs == [0, 1, 2] and total == 2 * R + 8 * GiB


def test_small_regions_and_explicit_count():
    region = 64 << 20
    offs, regs, total = zdp.plan_arena([3 << 20] * 4, [4, 3, 2, 1], 1 << 30, region_bytes=region, n_regions=4)
    assert regs == [0, 1, 2, 3]
    assert offs == [0, region, 2 * region, 3 * region]
    assert total == 3 * region + (4 << 20)


def test_rejects_bad_arguments():
    cases = [
        dict(sizes=[], traffic=[], max_bytes=GiB),
        dict(sizes=[0], traffic=[1], max_bytes=GiB),
        dict(sizes=[1], traffic=[-1], max_bytes=GiB),
        dict(sizes=[1], traffic=[1], max_bytes=GiB, region_bytes=A + 1),
        dict(sizes=[1], traffic=[1], max_bytes=GiB, n_regions=17),
        dict(sizes=[1], traffic=[1], max_bytes=A - 1),
    ]
    for c in cases:
        with pytest.raises(zdp.ZeroError) as e:
            zdp.plan_arena(**c)
        assert e.value.code == zdp.ERR_INVALID_ARG, c
    with pytest.raises(zdp.ZeroError) as e:   # a region count that does not start below max_bytes
        zdp.plan_arena([1], [1], R, n_regions=2)
    assert e.value.code == zdp.ERR_UNSUPPORTED
    with pytest.raises(zdp.ZeroError) as e:   # a buffer larger than any region
        zdp.plan_arena([R + 1], [1], 3 * R)
    assert e.value.code == zdp.ERR_UNSUPPORTED


@settings(max_examples=300, deadline=None)
@given(items=st.lists(st.tuples(st.integers(1, 40 << 20), st.integers(0, 1000)), min_size=1, max_size=24),
       n_regions=st.integers(1, 5))
def test_layout_is_valid_and_balanced(items, n_regions):
    # regions large enough for everything: the balance bound of greedy
    # heaviest-first assignment holds: max load - min load <= largest traffic
    region = 1 << 30
    sizes = [s for s, _ in items]
    traffic = [t for _, t in items]
    max_bytes = n_regions * region
    offs, regs, total = zdp.plan_arena(sizes, traffic, max_bytes, region_bytes=region, n_regions=n_regions)
    _check_layout(sizes, traffic, offs, regs, total, region, max_bytes)
    load = [sum(t for t, r in zip(traffic, regs) if r == k) for k in range(n_regions)]
    assert max(load) - min(load) <= max(traffic)
    assert zdp.plan_arena(sizes, traffic, max_bytes, region_bytes=region, n_regions=n_regions) == (offs, regs, total)


@pytest.mark.parametrize("pipeline,extra", [("fused", 0), ("optimistic", 0), ("checked", 8)])
@pytest.mark.parametrize("n_d,table", [(1, True), (8, True), (64, True), (100, False)])
def test_step_specs_traffic_is_the_bytes_model(pipeline, extra, n_d, table):
    # the traffic weights of a step's buffers add up to what the step moves:
    # 2*N_d + 26 bytes per parameter, plus the fp32 average written and read
    # back in the checked pipeline
    import torch
    from zero_dp_partitioned_amd import layout
    shards = [(1000, 10, 333), (70, 0, 70)]
    specs = layout.step_specs(shards, n_d, torch.float16, torch.bfloat16, pipeline, table)
    for gi, (psi, _, n) in enumerate(shards):
        mine = [s for s in specs if s.key[0] == gi]
        assert sum(s.traffic for s in mine) == (2 * n_d + 26 + extra) * n
        keys = {s.key for s in mine}
        assert (gi, "flat") in keys and next(s for s in mine if s.key == (gi, "flat")).numel == psi
        assert ((gi, "gradbuf") in keys) == (not table)
        assert ((gi, "master_alt") in keys) == (pipeline == "optimistic")
        assert ((gi, "avg") in keys) == (pipeline == "checked")


def test_free_ranges_are_the_gaps():
    from zero_dp_partitioned_amd import layout
    MiB = 1 << 20
    assert A == 2 * MiB
    # buffers at 0 (3 MiB), 20 MiB (1 byte), 40 MiB (4 MiB) in a 60 MiB arena: each gap starts at the
    # next 2 MiB boundary after a buffer's end
    offs, sizes, total = [0, 20 * MiB, 40 * MiB], [3 * MiB, 1, 4 * MiB], 60 * MiB
    assert layout.free_ranges(offs, sizes, total) == [(4 * MiB, 16 * MiB), (22 * MiB, 18 * MiB),
                                                      (44 * MiB, 16 * MiB)]
    # unsorted input, touching buffers, a tail shorter than the alignment
    assert layout.free_ranges([4 * MiB, 0], [4 * MiB, 4 * MiB], 8 * MiB + 1) == []
    assert layout.free_ranges([0], [1], 1) == []


@settings(max_examples=200, deadline=None)
@given(items=st.lists(st.tuples(st.integers(1, 40 << 20), st.integers(0, 100)), min_size=1, max_size=16),
       n_regions=st.integers(1, 4))
def test_free_ranges_cover_the_rest_of_a_plan(items, n_regions):
    from zero_dp_partitioned_amd import layout
    region = 1 << 30
    sizes = [s for s, _ in items]
    offs, regs, total = zdp.plan_arena(sizes, [t for _, t in items], n_regions * region,
                                      region_bytes=region, n_regions=n_regions)
    free = layout.free_ranges(offs, sizes, total)
    used = [(o, o + _up(b)) for o, b in zip(offs, sizes)]
    for fo, fb in free:
        assert fo % A == 0 and fb % A == 0 and fb >= A
        assert all(fo + fb <= lo or hi <= fo for lo, hi in used), "free range overlaps a buffer"
    # buffers plus free ranges account for the whole arena (plans are aligned)
    assert sum(_up(b) for b in sizes) + sum(fb for _, fb in free) == total
