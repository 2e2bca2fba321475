"""The Python binding's marshalling, without a GPU: the zero_group structs it
builds from torch tensors carry the right counts, dtypes and pointers, and its
own checks fire before any pointer reaches the library: length (the library
cannot bound device writes), dtype (an fp32 array given as bf16 would be read
and written at twice its size), device (a host pointer given to a kernel
faults) and contiguity (a strided view would be read as if it were dense).
The structs are built here against the CPU device so that they can be
inspected; the device calls demand the state's GPU."""
import ctypes

import pytest
import torch

import zero_dp_partitioned_amd as zdp


CPU = torch.device("cpu")


def _structs(groups, device=CPU):
    keep = []
    arr = zdp._array_type(zdp._Group, len(groups))()
    for g, s in zip(groups, arr):
        zdp._group_struct(g, keep, s, device)
    return arr, keep


def _group(n=1000, n_d=3, dt=torch.bfloat16, flat_dt=torch.float16, off=7, alt=False, **kw):
    f = lambda: torch.zeros(n)  # noqa: E731
    extra = dict(master_alt=f(), exp_avg_alt=f(), exp_avg_sq_alt=f()) if alt else {}
    return zdp.Group(f(), f(), f(), replicas=[torch.zeros(n + r, dtype=dt) for r in range(n_d)],
                     flat_param=torch.zeros(n + off + 5, dtype=flat_dt), param_offset=off, lr=2e-3,
                     beta1=0.8, beta2=0.99, eps=1e-7, weight_decay=0.05, **extra, **kw)


def test_fields_of_two_groups():
    a, b = _group(), _group(n=17, n_d=1, dt=torch.float16, flat_dt=torch.bfloat16, off=0, alt=True)
    b.flat_param = None
    arr, keep = _structs([a, b])
    s = arr[0]
    assert (s.n, s.n_d, s.grad_dt, s.param_dt, s.param_offset) == (1000, 3, zdp.DT_BF16, zdp.DT_F16, 7)
    assert [s.replicas[r] for r in range(3)] == [t.data_ptr() for t in a.replicas]
    assert (s.master, s.exp_avg, s.exp_avg_sq) == (a.master.data_ptr(), a.exp_avg.data_ptr(),
                                                   a.exp_avg_sq.data_ptr())
    assert s.flat_param == a.flat_param.data_ptr() and not s.avg and not s.master_alt
    assert (s.lr, s.beta1, s.beta2, s.eps, s.weight_decay) == (2e-3, 0.8, 0.99, 1e-7, 0.05)
    s = arr[1]
    assert (s.n, s.n_d, s.grad_dt, s.param_dt, s.param_offset) == (17, 1, zdp.DT_F16, 0, 0)
    assert not s.flat_param
    assert (s.master_alt, s.exp_avg_alt, s.exp_avg_sq_alt) == (b.master_alt.data_ptr(), b.exp_avg_alt.data_ptr(),
                                                               b.exp_avg_sq_alt.data_ptr())
    assert ctypes.sizeof(arr) == 2 * ctypes.sizeof(zdp._Group)


def test_average_source_and_struct_reuse_across_calls():
    g = _group()
    g.replicas, g.avg = None, torch.zeros(1000)
    arr, _ = _structs([g])
    assert not arr[0].replicas and arr[0].n_d == 0 and arr[0].avg == g.avg.data_ptr()
    # a fresh struct each call: nothing of the previous call's group leaks into the next
    g2 = _group(n=10, n_d=2)
    arr2, _ = _structs([g2])
    assert arr2[0].avg is None or arr2[0].avg == 0
    assert arr2[0].n == 10 and arr2[0].n_d == 2


@pytest.mark.parametrize("break_it,msg", [
    (lambda g: g.replicas.__setitem__(1, torch.zeros(999, dtype=torch.bfloat16)), "shorter than the shard"),
    (lambda g: setattr(g, "exp_avg", torch.zeros(999)), "length 999 differs"),
    (lambda g: setattr(g, "param_offset", 13), "exceeds the flat parameter vector"),  # 1013 > 1012
    (lambda g: setattr(g, "param_offset", -1), "exceeds the flat parameter vector"),
    (lambda g: setattr(g, "master_alt", torch.zeros(1000)), "exp_avg_alt missing"),
    (lambda g: setattr(g, "avg", torch.zeros(999)), "shorter than the shard"),
    (lambda g: setattr(g, "exp_avg_alt", torch.zeros(1001)) or setattr(g, "master_alt", torch.zeros(1000))
     or setattr(g, "exp_avg_sq_alt", torch.zeros(1000)), "length 1001 differs"),
])
def test_length_checks(break_it, msg):
    g = _group()
    break_it(g)
    with pytest.raises(ValueError, match=msg):
        _structs([g])


@pytest.mark.parametrize("break_it,msg", [
    (lambda g: setattr(g, "master", torch.zeros(1000, dtype=torch.bfloat16)), "master: dtype"),
    (lambda g: setattr(g, "exp_avg", torch.zeros(1000, dtype=torch.float64)), "exp_avg: dtype"),
    (lambda g: setattr(g, "exp_avg_sq", torch.zeros(1000, dtype=torch.float16)), "exp_avg_sq: dtype"),
    (lambda g: setattr(g, "avg", torch.zeros(1000, dtype=torch.bfloat16)), "avg: dtype"),
    (lambda g: (setattr(g, "master_alt", torch.zeros(1000, dtype=torch.bfloat16)),
                setattr(g, "exp_avg_alt", torch.zeros(1000)), setattr(g, "exp_avg_sq_alt", torch.zeros(1000))),
     "master_alt: dtype"),
    (lambda g: g.replicas.__setitem__(0, torch.zeros(1000, dtype=torch.float32)), r"replicas\[0\]: dtype"),
    (lambda g: g.replicas.__setitem__(2, torch.zeros(1002, dtype=torch.float16)), r"replicas\[2\]: dtype"),
    (lambda g: setattr(g, "flat_param", torch.zeros(2000, dtype=torch.float32)), "flat_param: dtype"),
])
def test_dtype_checks(break_it, msg):
    g = _group()
    break_it(g)
    with pytest.raises(TypeError, match=msg):
        _structs([g])


@pytest.mark.parametrize("break_it,msg", [
    (lambda g: setattr(g, "master", torch.zeros(2000)[::2]), "master: not contiguous"),
    (lambda g: setattr(g, "exp_avg_sq", torch.zeros(2000)[::2]), "exp_avg_sq: not contiguous"),
    (lambda g: g.replicas.__setitem__(1, torch.zeros(2002, dtype=torch.bfloat16)[::2]), r"replicas\[1\]: not contiguous"),
    (lambda g: setattr(g, "flat_param", torch.zeros(4000, dtype=torch.float16)[::2]), "flat_param: not contiguous"),
])
def test_contiguity_checks(break_it, msg):
    g = _group()
    break_it(g)
    with pytest.raises(ValueError, match=msg):
        _structs([g])


def test_host_tensors_are_refused_for_a_device_step():
    g = _group()
    with pytest.raises(ValueError, match="master: tensor on cpu, expected cuda:0"):
        _structs([g], device=torch.device("cuda", 0))
    # the device calls take the device from the state, which must be a device tensor
    st, ws = torch.zeros(ctypes.sizeof(zdp.StepState), dtype=torch.uint8), torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="state must be a device tensor"):
        zdp.adam_step([g], ws, st)
    with pytest.raises(ValueError, match="state must be a device tensor"):
        zdp.reduce_grad_segment(g.replicas, torch.zeros(1000), ws, 0, st)
    with pytest.raises(ValueError, match="state must be a device tensor"):
        zdp.grad_norm_overflow(None, ws, 1, st)
    with pytest.raises(ValueError, match="state must be a device tensor"):
        zdp.state_init(st)
    with pytest.raises(ValueError, match="master must be a device tensor"):
        zdp.cast_writeback(torch.zeros(10), torch.zeros(10, dtype=torch.float16), 0)
