"""The C-ABI library on the host (no GPU): it loads, exports every symbol
include/zero_dp.h declares, its host-only partition calls agree exactly with the
oracle, and argument errors come back before anything touches a device."""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import zero_dp_partitioned_amd as zdp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero_dp.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(zero_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_five_step_calls():
    names = _declared()
    for must in ("zero_partition", "zero_reduce_grad_segment", "zero_grad_norm_overflow",
                 "zero_adam_step", "zero_cast_writeback"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = zdp.load()
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(_declared()) == set(zdp.EXPORTS)


def test_struct_sizes_match_header_layout():
    assert ctypes.sizeof(zdp.Segment) == 16
    assert ctypes.sizeof(zdp.TensorSlice) == 32
    assert ctypes.sizeof(zdp.StepState) == 176
    assert ctypes.sizeof(zdp.Policy) == 48
    assert ctypes.sizeof(zdp._Group) == 144


@settings(max_examples=400, deadline=None)
@given(numel=st.integers(0, 2 ** 40), n_d=st.integers(1, 1100), align=st.sampled_from([1, 2, 8, 64]))
def test_partition_matches_oracle(numel, n_d, align):
    segs, padded = zdp.partition(numel, n_d, align)
    offs, sizes, opad = oracle.partition(numel, n_d, align)
    assert padded == opad
    assert [s[0] for s in segs] == offs.tolist()
    assert [s[1] for s in segs] == sizes.tolist()


def test_partition_workload_segments():
    assert zdp.partition(787_971, 4)[0][1] == (196_993, 196_993)
    assert zdp.partition(7_500_000_000, 64)[0][63] == (7_382_812_500, 117_187_500)
    assert zdp.partition(13_000_000_000, 8)[0][7] == (11_375_000_000, 1_625_000_000)


@settings(max_examples=200, deadline=None)
@given(numels=st.lists(st.integers(0, 5000), min_size=0, max_size=12), n_d=st.integers(1, 9),
       data=st.data())
def test_partition_tensors_matches_oracle(numels, n_d, data):
    rank = data.draw(st.integers(0, n_d - 1))
    assert zdp.partition_tensors(numels, n_d, rank) == oracle.tensor_slices(numels, n_d, rank)


def test_partition_errors():
    L = zdp.load()
    segs = (zdp.Segment * 4)()
    assert L.zero_partition(-1, 4, 1, segs, None) == zdp.ERR_INVALID_ARG
    assert L.zero_partition(10, 0, 1, segs, None) == zdp.ERR_INVALID_ARG
    assert L.zero_partition(10, 4, 0, segs, None) == zdp.ERR_INVALID_ARG
    assert L.zero_partition(10, 4, 1, None, None) == zdp.ERR_INVALID_ARG
    assert L.zero_partition(2 ** 63 - 1, 4, 8, segs, None) == zdp.ERR_INVALID_ARG
    assert "overflow" in zdp.last_error()
    with pytest.raises(zdp.ZeroError):
        zdp.partition_tensors([3, 4], 2, 2)
    out = (zdp.TensorSlice * 1)()
    n = ctypes.c_int32()
    arr = (ctypes.c_int64 * 3)(5, 5, 5)
    assert L.zero_partition_tensors(arr, 3, 1, 0, 1, out, 1, ctypes.byref(n)) == zdp.ERR_INVALID_ARG


def test_workspace_bytes():
    assert zdp.workspace_bytes(0) == 0
    assert zdp.workspace_bytes(zdp.MAX_GROUPS + 1) == 0
    w1, w8 = zdp.workspace_bytes(1), zdp.workspace_bytes(8)
    assert w1 == w8 > 0 and w1 % 256 == 0
    assert w1 < 32 << 20  # constant, independent of the shard size


def test_device_calls_reject_bad_arguments_before_launch():
    """Every one of these returns from the host checks; no HIP call is made."""
    L = zdp.load()
    vp = ctypes.c_void_p
    fake = vp(0x100000)  # never dereferenced: the checks fail first
    W = zdp.workspace_bytes(8)
    assert L.zero_state_init(None, 1.0, None) == zdp.ERR_INVALID_ARG
    assert L.zero_state_init(vp(0x100004), 1.0, None) == zdp.ERR_ALIGNMENT
    assert L.zero_state_init(fake, -1.0, None) == zdp.ERR_INVALID_ARG
    reps = (vp * 2)(0x100000, 0x100000)
    assert L.zero_reduce_grad_segment(reps, 2, 7, 10, fake, fake, W, 0, fake, None) == zdp.ERR_INVALID_ARG
    assert L.zero_reduce_grad_segment(reps, 0, 1, 10, fake, fake, W, 0, fake, None) == zdp.ERR_INVALID_ARG
    assert L.zero_reduce_grad_segment(reps, 2, 1, 10, fake, None, W, 0, fake, None) == zdp.ERR_WORKSPACE
    assert L.zero_reduce_grad_segment(reps, 2, 1, 10, fake, vp(0x100010), W, 0, fake, None) == zdp.ERR_WORKSPACE
    assert L.zero_reduce_grad_segment(reps, 2, 1, 10, fake, fake, W, 9, fake, None) == zdp.ERR_WORKSPACE
    assert L.zero_reduce_grad_segment(reps, 2, 1, 10, vp(0x100002), fake, W, 0, fake, None) == zdp.ERR_ALIGNMENT
    odd = (vp * 1)(0x100001)
    assert L.zero_reduce_grad_segment(odd, 1, 1, 10, fake, fake, W, 0, fake, None) == zdp.ERR_ALIGNMENT
    assert L.zero_reduce_grad_segment(reps, 5000, 1, 10, fake, fake, W, 0, fake, None) == zdp.ERR_UNSUPPORTED
    assert L.zero_grad_norm_overflow(None, None, 1, 0, fake, W, None, fake, None) == zdp.ERR_INVALID_ARG
    assert L.zero_grad_norm_overflow(None, None, 1, 1, None, W, None, fake, None) == zdp.ERR_WORKSPACE
    assert L.zero_adam_step(None, 1, None, fake, W, fake, None) == zdp.ERR_INVALID_ARG
    g = zdp._Group()
    g.n = 10
    g.master = g.exp_avg = g.exp_avg_sq = 0x100000
    garr = (zdp._Group * 1)(g)
    # neither replicas nor avg
    assert L.zero_adam_step(garr, 1, None, fake, W, fake, None) == zdp.ERR_INVALID_ARG
    g.avg = 0x100000
    g.lr, g.beta1, g.beta2, g.eps = 1e-3, 0.9, 0.999, 1e-8
    g.master = 0x100002
    garr = (zdp._Group * 1)(g)
    assert L.zero_adam_step(garr, 1, None, fake, W, fake, None) == zdp.ERR_ALIGNMENT
    g.master = 0x100000
    g.beta1 = 1.0
    garr = (zdp._Group * 1)(g)
    assert L.zero_adam_step(garr, 1, None, fake, W, fake, None) == zdp.ERR_INVALID_ARG
    assert L.zero_adam_step(garr, 9, None, fake, W, fake, None) == zdp.ERR_INVALID_ARG
    bad = zdp.policy(True, backoff=0.0)
    g.beta1 = 0.9
    garr = (zdp._Group * 1)(g)
    assert L.zero_adam_step(garr, 1, ctypes.byref(bad), fake, W, fake, None) == zdp.ERR_INVALID_ARG
    for clip in (-1.0, float("inf"), float("nan")):
        badclip = zdp.policy(max_grad_norm=clip)
        assert L.zero_adam_step(garr, 1, ctypes.byref(badclip), fake, W, fake, None) == zdp.ERR_INVALID_ARG
        assert L.zero_grad_norm_overflow(None, None, 1, 1, fake, W, ctypes.byref(badclip), fake,
                                         None) == zdp.ERR_INVALID_ARG
    # optimistic needs skip and the second state set (with or without clipping)
    pol = zdp.policy(False, optimistic=True)
    assert L.zero_adam_step(garr, 1, ctypes.byref(pol), fake, W, fake, None) == zdp.ERR_INVALID_ARG
    assert "skip_on_overflow" in zdp.last_error()
    g.beta1 = 0.9
    garr = (zdp._Group * 1)(g)
    for opt in (zdp.policy(True, optimistic=True), zdp.policy(True, optimistic=True, max_grad_norm=1.0)):
        assert L.zero_adam_step(garr, 1, ctypes.byref(opt), fake, W, fake, None) == zdp.ERR_INVALID_ARG
        assert "_alt" in zdp.last_error()
    # a workspace smaller than zero_workspace_bytes()
    g.beta1 = 0.9
    garr2 = (zdp._Group * 2)(g, g)
    small = zdp.workspace_bytes(1) - 256
    assert L.zero_adam_step(garr2, 2, None, fake, small, fake, None) == zdp.ERR_WORKSPACE
    assert L.zero_reduce_grad_segment(reps, 2, 1, 10, fake, fake, small, 1, fake, None) == zdp.ERR_WORKSPACE
    assert L.zero_grad_norm_overflow(None, None, 1, 2, fake, small, None, fake, None) == zdp.ERR_WORKSPACE
    assert L.zero_cast_writeback(fake, 10, fake, 0, 3, None) == zdp.ERR_INVALID_ARG
    assert L.zero_cast_writeback(fake, -1, fake, 0, 1, None) == zdp.ERR_INVALID_ARG
    assert L.zero_cast_writeback(vp(0x100001), 10, fake, 0, 1, None) == zdp.ERR_ALIGNMENT
    assert L.zero_cast_writeback(fake, 10, vp(0x100001), 0, 1, None) == zdp.ERR_ALIGNMENT


def test_binding_has_no_cpu_path():
    src = open(os.path.join(ROOT, "zero_dp_partitioned_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("no fallback", "")
    for f in os.listdir(os.path.join(ROOT, "zero_dp_partitioned_amd", "csrc")):
        text = open(os.path.join(ROOT, "zero_dp_partitioned_amd", "csrc", f)).read()
        assert "oracle" not in text.lower()
