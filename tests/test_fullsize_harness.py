"""The full-size verification harness (tests/_fullsize.py) on the CPU: host
tensors stand in for the device, holding the result of an independent,
unchunked oracle run over the whole shard. The chunked harness must agree
with it exactly over several calls (static scale in one pass; dynamic scale
with an overflowing call, and clipping, in two passes; two groups; a chunk
sample), and must catch a single planted one-ulp difference anywhere,
naming the chunk. Also the fallback plan for a host short of memory: which
chunks it samples and when it is taken."""
import numpy as np
import pytest
import torch

import oracle
import _fullsize as _fs
from _fullsize import FullCheck, GroupCheck, HostStager
from _parity import Bar
from workloads import grads16_np, normal_f32_np, to16_bits_np


class Side:
    """A whole-shard oracle run kept in torch CPU tensors (the stand-in for
    the device's buffers)."""

    def __init__(self, sizes, n_d, seed, wds):
        self.n_d, self.seed = n_d, seed
        self.groups = []
        for gi, (n, wd) in enumerate(zip(sizes, wds)):
            master = normal_f32_np(n, 0.02, (seed, gi, "master"))
            param = to16_bits_np(master, "bf16")
            self.groups.append(oracle.Group(replicas=None, grad_dt=oracle.BF16, master=master,
                                            m=np.zeros(n, np.float32), v=np.zeros(n, np.float32), param=param,
                                            param_dt=oracle.BF16, weight_decay=wd))
        self.state = None

    def tensors(self, gi):
        g = self.groups[gi]
        return (torch.from_numpy(g.master), torch.from_numpy(g.m), torch.from_numpy(g.v),
                torch.from_numpy(g.param.view(np.int16)).view(torch.bfloat16))

    def draw(self, call, scale, inf_at=None):
        reps = []
        for gi, g in enumerate(self.groups):
            r = [grads16_np(g.master.size, "bf16", scale, (self.seed, call, gi, k)) for k in range(self.n_d)]
            if inf_at is not None and inf_at[0] == gi:
                r[1] = r[1].copy()
                r[1][inf_at[1]] = 0x7F80
            g.replicas = r
            reps.append([torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) for x in r])
        return reps


def _make(side, reps, policy, scale, ranges=None, chunk=700):
    checks = []
    for gi, g in enumerate(side.groups):
        n = g.master.size
        master, m, v, param = side.tensors(gi)
        gc = GroupCheck(n, reps[gi], param, 0, (ranges or {}).get(gi, [(0, n)]), chunk, oracle.BF16, oracle.BF16,
                        1e-3, 0.9, 0.999, 1e-8, g.weight_decay)
        gc.state = (lambda master=master, m=m, v=v: (master, m, v))
        checks.append(gc)
    fc = FullCheck(checks, policy, scale, workers=3, stager=HostStager())
    return fc


def _run(policy, calls, sizes=(5000, 1234), scale=1024.0, inf_call=None, ranges=None, plant=None):
    side = Side(sizes, 3, 7, (0.1, 0.0))
    reps = [[torch.zeros(n, dtype=torch.bfloat16) for _ in range(3)] for n in sizes]
    fc = _make(side, reps, policy, scale, ranges)
    fc.load_initial()
    bar = Bar()
    st = oracle.State(loss_scale=scale)
    try:
        for call in range(1, calls + 1):
            drawn = side.draw(call, st.loss_scale, inf_at=(1, 1000) if call == inf_call else None)
            for gi in range(len(sizes)):
                for r, d in zip(reps[gi], drawn[gi]):
                    r.copy_(d)
            oracle.step(side.groups, policy, st)      # the stand-in device: the whole shard at once
            if plant is not None and plant[0] == call:
                g = side.groups[plant[1]]
                g.master[plant[2]] = np.nextafter(g.master[plant[2]], np.float32(1))
            gpu = {"clip_coef": st.clip}
            post = fc.step_and_compare(f"call {call}", bar, gpu)
            assert (post.step, post.skipped, post.overflow, post.loss_scale, post.good_steps, post.clip) == \
                   (st.step, st.skipped, st.overflow, st.loss_scale, st.good_steps, st.clip)
            if np.isfinite(st.norm2):
                assert abs(post.norm2 - st.norm2) <= 1e-12 * st.norm2
            else:
                assert not np.isfinite(post.norm2)
    finally:
        fc.close()
    return st


def test_static_scale_one_pass():
    st = _run(oracle.Policy(), calls=3)
    assert st.step == 3


def test_dynamic_scale_with_an_overflow_and_clipping_two_passes():
    st = _run(oracle.Policy(skip_on_overflow=True, growth_interval=2, max_grad_norm=0.01), calls=5, inf_call=3)
    assert st.step == 4 and st.clip < 1.0


def test_a_chunk_sample_still_takes_the_norm_over_every_element():
    st = _run(oracle.Policy(skip_on_overflow=True), calls=3, inf_call=2,
              ranges={0: [(0, 700), (2100, 2800), (4900, 5000)]})
    assert st.step == 2 and st.skipped == 0


@pytest.mark.parametrize("policy", [oracle.Policy(), oracle.Policy(skip_on_overflow=True, max_grad_norm=0.01)])
@pytest.mark.parametrize("where", [(0, 0), (0, 4321), (1, 1233)])
def test_a_single_planted_ulp_is_caught(policy, where):
    with pytest.raises(AssertionError, match=r"elements \[\d+, \d+\) master"):
        _run(policy, calls=2, plant=(2, *where))


# --------------------------------------------------------------------------
# the fallback when the host cannot hold the oracle's copy of every element
# --------------------------------------------------------------------------

def test_sample_ranges_cover_the_sampled_chunks_in_order():
    c = _fs.SAMPLE_CHUNK
    n = 300 * c + 5
    r = _fs.sample_ranges(n, [3 * c + 7, 130 * c, n - 1, n, -1])
    assert r == [(0, c), (3 * c, 4 * c), (64 * c, 65 * c), (128 * c, 129 * c), (130 * c, 131 * c),
                 (192 * c, 193 * c), (256 * c, 257 * c), (300 * c, n)]
    assert _fs.sample_ranges(0, [0]) == []
    assert _fs.sample_ranges(10, []) == [(0, 10)]
    assert _fs.sample_ranges(3 * c, [c]) == [(0, 3 * c)]     # adjacent sampled chunks merge


def test_plan_ranges_falls_back_only_when_the_state_does_not_fit():
    shards = [(1_000_000, [10]), (300, [])]
    need = _fs.oracle_bytes(1_000_300, False) + 20 * _fs.STAGE_BYTES
    full, msg = _fs.plan_ranges(shards, False, 16, int(need / 0.8) + 1)
    assert msg is None and full == [[(0, 1_000_000)], [(0, 300)]]
    full, msg = _fs.plan_ranges(shards, False, 16, None)
    assert msg is None and full == [[(0, 1_000_000)], [(0, 300)]]
    part, msg = _fs.plan_ranges(shards, True, 16, int(need / 0.8) + 1)   # the kept averages tip it over
    assert msg and "chunk sample" in msg and part == [_fs.sample_ranges(1_000_000, [10]), [(0, 300)]]


@pytest.mark.parametrize("where,caught", [(500, True), (2000, False)])
def test_a_sampled_run_compares_only_its_chunks(where, caught):
    """A planted difference inside the sample is caught; one outside it is
    not looked at (its element still enters the norm, unchanged)."""
    ranges = {0: [(0, 1024), (3072, 4096)]}
    if caught:
        with pytest.raises(AssertionError, match=r"elements \[\d+, \d+\) master"):
            _run(oracle.Policy(), calls=2, ranges=ranges, plant=(2, 0, where))
    else:
        assert _run(oracle.Policy(), calls=2, ranges=ranges, plant=(2, 0, where)).step == 2
