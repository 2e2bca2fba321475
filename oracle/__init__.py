"""CPU oracle for the ZeRO-DP partitioned optimizer step.

TEST INFRASTRUCTURE: the slow, plain reference the GPU library is checked
against. Only the tests, the smoke check and the benchmark's CPU-baseline leg
use it; the library never imports it and shares no code with it.

The arithmetic lives in ``zero_oracle.c`` (scalar C); this module marshals
numpy arrays into it. 16-bit floats travel as raw ``uint16`` bit patterns.
"""
import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

from . import build as _build

F16 = 1
BF16 = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)


class _Group(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int64),
        ("n_d", ctypes.c_int32),
        ("grad_dt", ctypes.c_int32),
        ("replicas", ctypes.POINTER(_u16p)),
        ("master", _f32p),
        ("m", _f32p),
        ("v", _f32p),
        ("param", _u16p),
        ("param_dt", ctypes.c_int32),
        ("pad_", ctypes.c_int32),
        ("lr", ctypes.c_double),
        ("beta1", ctypes.c_double),
        ("beta2", ctypes.c_double),
        ("eps", ctypes.c_double),
        ("weight_decay", ctypes.c_double),
    ]


class _Policy(ctypes.Structure):
    _fields_ = [
        ("skip_on_overflow", ctypes.c_int32),
        ("growth_interval", ctypes.c_int32),
        ("backoff", ctypes.c_double),
        ("growth", ctypes.c_double),
        ("min_scale", ctypes.c_double),
        ("max_grad_norm", ctypes.c_double),
    ]


class _State(ctypes.Structure):
    _fields_ = [
        ("step", ctypes.c_int64),
        ("norm2", ctypes.c_double),
        ("loss_scale", ctypes.c_float),
        ("overflow", ctypes.c_int32),
        ("skipped", ctypes.c_int32),
        ("good_steps", ctypes.c_int32),
        ("clip", ctypes.c_float),
        ("pad_", ctypes.c_int32),
    ]


def lib():
    """Load liboracle.so, compiling it first if it is missing or stale.
    ZDP_ORACLE_LIB names another build of the oracle source to load instead
    (the mutation tests use it to run the pins against planted mistakes)."""
    global _LIB
    if _LIB is None:
        path = os.environ.get("ZDP_ORACLE_LIB")
        if not path:
            path = _build.LIB
            if (not os.path.exists(path)
                    or os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
                _build.build()
        L = ctypes.CDLL(path)
        L.oracle_f16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_f16_decode.restype = ctypes.c_float
        L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_decode.restype = ctypes.c_float
        L.oracle_f16_encode.argtypes = [ctypes.c_float]
        L.oracle_f16_encode.restype = ctypes.c_uint16
        L.oracle_bf16_encode.argtypes = [ctypes.c_float]
        L.oracle_bf16_encode.restype = ctypes.c_uint16
        L.oracle_partition.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                       _i64p, _i64p, _i64p]
        L.oracle_partition.restype = ctypes.c_int
        L.oracle_tensor_slices.argtypes = [_i64p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                           _i32p, _i64p, _i64p, _i64p]
        L.oracle_tensor_slices.restype = ctypes.c_int
        L.oracle_average.argtypes = [ctypes.POINTER(_u16p), ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int64, _f32p]
        L.oracle_average.restype = None
        L.oracle_norm_overflow.argtypes = [_f32p, ctypes.c_int64, ctypes.c_float,
                                           _f64p, _i32p]
        L.oracle_norm_overflow.restype = None
        L.oracle_adam_update.argtypes = [ctypes.c_int64, _f32p, ctypes.c_float, ctypes.c_float,
                                         _f32p, _f32p, _f32p, _u16p, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                                         ctypes.c_double, ctypes.c_double, ctypes.c_double]
        L.oracle_adam_update.restype = None
        L.oracle_decode16.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int32, _f32p]
        L.oracle_decode16.restype = None
        L.oracle_cast.argtypes = [_f32p, ctypes.c_int64, _u16p, ctypes.c_int32]
        L.oracle_cast.restype = None
        L.oracle_step.argtypes = [ctypes.POINTER(_Group), ctypes.c_int32,
                                  ctypes.POINTER(_Policy), ctypes.POINTER(_State)]
        L.oracle_step.restype = ctypes.c_int
        L.oracle_step_given_norm.argtypes = [ctypes.POINTER(_Group), ctypes.c_int32, ctypes.POINTER(_Policy),
                                             ctypes.POINTER(_State), ctypes.c_double, ctypes.c_int32]
        L.oracle_step_given_norm.restype = ctypes.c_int
        L.oracle_step_from_average.argtypes = [ctypes.POINTER(_Group), ctypes.c_int32, ctypes.POINTER(_f32p),
                                               ctypes.POINTER(_Policy), ctypes.POINTER(_State), ctypes.c_double,
                                               ctypes.c_int32]
        L.oracle_step_from_average.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


# --------------------------------------------------------------------------
# 16-bit encodings
# --------------------------------------------------------------------------

def decode16(bits, dt):
    """uint16 bit patterns -> float32 values (exact)."""
    bits = _c(bits, np.uint16).ravel()
    out = np.empty(bits.size, dtype=np.float32)
    lib().oracle_decode16(_ptr(bits, ctypes.c_uint16), bits.size, dt, _ptr(out, ctypes.c_float))
    return out


def encode16(x, dt):
    """float32 values -> uint16 bit patterns, round to nearest even."""
    x = _c(x, np.float32).ravel()
    out = np.empty(x.size, dtype=np.uint16)
    lib().oracle_cast(_ptr(x, ctypes.c_float), x.size, _ptr(out, ctypes.c_uint16), dt)
    return out


# --------------------------------------------------------------------------
# Partition
# --------------------------------------------------------------------------

def partition(numel, n_d, align_elems=1):
    """Return (offsets[n_d], sizes[n_d], padded_numel)."""
    offs = np.empty(n_d, dtype=np.int64)
    sizes = np.empty(n_d, dtype=np.int64)
    padded = ctypes.c_int64(0)
    rc = lib().oracle_partition(int(numel), int(n_d), int(align_elems),
                                _ptr(offs, ctypes.c_int64), _ptr(sizes, ctypes.c_int64),
                                ctypes.byref(padded))
    if rc != 0:
        raise ValueError(f"oracle_partition rc={rc}")
    return offs, sizes, padded.value


def tensor_slices(numels, n_d, rank, align_elems=1):
    """List of (tensor, shard_begin, tensor_begin, length) inside rank's segment."""
    numels = np.asarray(numels, dtype=np.int64)
    cap = max(1, len(numels))
    t = np.empty(cap, dtype=np.int32)
    sb = np.empty(cap, dtype=np.int64)
    tb = np.empty(cap, dtype=np.int64)
    ln = np.empty(cap, dtype=np.int64)
    rc = lib().oracle_tensor_slices(_ptr(numels, ctypes.c_int64), len(numels), n_d, rank,
                                    align_elems, cap, _ptr(t, ctypes.c_int32),
                                    _ptr(sb, ctypes.c_int64), _ptr(tb, ctypes.c_int64),
                                    _ptr(ln, ctypes.c_int64))
    if rc < 0:
        raise ValueError(f"oracle_tensor_slices rc={rc}")
    return [(int(t[i]), int(sb[i]), int(tb[i]), int(ln[i])) for i in range(rc)]


# --------------------------------------------------------------------------
# Step pieces
# --------------------------------------------------------------------------

def _replica_array(replicas):
    reps = [_c(r, np.uint16) for r in replicas]
    arr = (_u16p * len(reps))(*[_ptr(r, ctypes.c_uint16) for r in reps])
    return reps, arr


def average(replicas, grad_dt):
    """fp32 average of N_d uint16 replica arrays of equal length."""
    reps, arr = _replica_array(replicas)
    n = reps[0].size if reps else 0
    for r in reps:
        if r.size != n:
            raise ValueError("replica lengths differ")
    out = np.empty(n, dtype=np.float32)
    lib().oracle_average(arr, len(reps), grad_dt, n, _ptr(out, ctypes.c_float))
    return out


def norm_overflow(avg, inv_scale, norm2=0.0, flag=0):
    """Continue the in-order fp64 sum of squares and the overflow flag."""
    avg = _c(avg, np.float32)
    n2 = ctypes.c_double(norm2)
    fl = ctypes.c_int32(flag)
    lib().oracle_norm_overflow(_ptr(avg, ctypes.c_float), avg.size,
                               ctypes.c_float(inv_scale), ctypes.byref(n2), ctypes.byref(fl))
    return n2.value, fl.value


def inv_scale_of(loss_scale):
    """The unscale multiplier: 1/S rounded once to fp32."""
    return float(np.float32(1.0 / float(loss_scale)))


def adam_update(avg, inv_scale, master, m, v, t, lr, beta1, beta2, eps, weight_decay,
                param=None, param_dt=F16, clip=1.0):
    """In-place update of master/m/v (and param, a uint16 array) for applied step t."""
    avg = _c(avg, np.float32)
    for a in (master, m, v):
        if a.dtype != np.float32 or not a.flags.c_contiguous or a.size != avg.size:
            raise ValueError("state arrays must be contiguous float32 of the shard length")
    pp = None
    if param is not None:
        if param.dtype != np.uint16 or not param.flags.c_contiguous or param.size != avg.size:
            raise ValueError("param must be contiguous uint16 of the shard length")
        pp = _ptr(param, ctypes.c_uint16)
    lib().oracle_adam_update(avg.size, _ptr(avg, ctypes.c_float), ctypes.c_float(inv_scale),
                             ctypes.c_float(clip), _ptr(master, ctypes.c_float), _ptr(m, ctypes.c_float),
                             _ptr(v, ctypes.c_float), pp, param_dt, int(t), lr, beta1,
                             beta2, eps, weight_decay)


# --------------------------------------------------------------------------
# Whole step
# --------------------------------------------------------------------------

@dataclass
class Policy:
    skip_on_overflow: bool = False
    growth_interval: int = 1000
    backoff: float = 0.5
    growth: float = 2.0
    min_scale: float = 1.0
    max_grad_norm: float = 0.0


@dataclass
class State:
    step: int = 0
    norm2: float = 0.0
    loss_scale: float = 1.0
    overflow: int = 0
    skipped: int = 0
    good_steps: int = 0
    clip: float = 1.0

    @property
    def grad_norm(self):
        return float(np.sqrt(self.norm2))


@dataclass
class Group:
    """One parameter group's shard. Arrays are numpy, updated in place."""
    replicas: list            # N_d uint16 arrays of length n
    grad_dt: int
    master: np.ndarray        # float32 [n]
    m: np.ndarray
    v: np.ndarray
    param: object = None      # uint16 [n] view of the rank's slice, or None
    param_dt: int = F16
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    _keep: list = field(default_factory=list, repr=False)


def _groups_struct(groups, keep, with_replicas=True):
    G = (_Group * len(groups))()
    for i, g in enumerate(groups):
        n = g.master.size
        for a in (g.master, g.m, g.v):
            if a.dtype != np.float32 or not a.flags.c_contiguous or a.size != n:
                raise ValueError("state arrays must be contiguous float32 of equal length")
        G[i].n = n
        G[i].grad_dt = g.grad_dt
        if with_replicas:
            reps, arr = _replica_array(g.replicas)
            keep.append((reps, arr))
            for r in reps:
                if r.size != n:
                    raise ValueError("replica length differs from shard length")
            G[i].n_d = len(reps)
            G[i].replicas = ctypes.cast(arr, ctypes.POINTER(_u16p))
        else:
            G[i].n_d = 0
            G[i].replicas = None
        G[i].master = _ptr(g.master, ctypes.c_float)
        G[i].m = _ptr(g.m, ctypes.c_float)
        G[i].v = _ptr(g.v, ctypes.c_float)
        if g.param is not None:
            p = g.param
            if p.dtype != np.uint16 or not p.flags.c_contiguous or p.size != n:
                raise ValueError("param slice must be contiguous uint16 of the shard length")
            G[i].param = _ptr(p, ctypes.c_uint16)
        else:
            G[i].param = None
        G[i].param_dt = g.param_dt
        G[i].lr, G[i].beta1, G[i].beta2 = g.lr, g.beta1, g.beta2
        G[i].eps, G[i].weight_decay = g.eps, g.weight_decay
    return G


def _policy_state(policy, state):
    P = _Policy(int(policy.skip_on_overflow), int(policy.growth_interval),
                policy.backoff, policy.growth, policy.min_scale, policy.max_grad_norm)
    S = _State(state.step, state.norm2, state.loss_scale, state.overflow,
               state.skipped, state.good_steps, state.clip, 0)
    return P, S


def _state_back(S, state):
    state.step, state.norm2, state.loss_scale = S.step, S.norm2, S.loss_scale
    state.overflow, state.skipped, state.good_steps = S.overflow, S.skipped, S.good_steps
    state.clip = S.clip
    return state


def step(groups, policy, state, norm2=None, flag=None):
    """Run one full step over ``groups`` in place; updates ``state``. With
    ``norm2`` and ``flag`` given, the groups hold a sample of a shard's
    coordinates and these are the whole shard's norm² and overflow flag, which
    the skip verdict and the clip multiplier then use."""
    keep = []
    G = _groups_struct(groups, keep)
    P, S = _policy_state(policy, state)
    if (norm2 is None) != (flag is None):
        raise ValueError("give both norm2 and flag, or neither")
    if norm2 is None:
        rc = lib().oracle_step(G, len(groups), ctypes.byref(P), ctypes.byref(S))
    else:
        rc = lib().oracle_step_given_norm(G, len(groups), ctypes.byref(P), ctypes.byref(S),
                                          ctypes.c_double(norm2), ctypes.c_int32(int(bool(flag))))
    if rc != 0:
        raise RuntimeError(f"oracle_step rc={rc}")
    return _state_back(S, state)


def step_from_average(groups, avgs, policy, state, norm2, flag):
    """One step over ``groups`` in place from their averaged gradients
    ``avgs`` (float32 arrays, as ``average`` returns them; the groups'
    ``replicas`` are not used) and the whole shard's norm² and overflow flag
    (``norm_overflow`` over every group in order, or over a shard the groups
    are a part of). Updates ``state``."""
    if len(avgs) != len(groups):
        raise ValueError("one average per group")
    keep = []
    G = _groups_struct(groups, keep, with_replicas=False)
    avs = [_c(a, np.float32) for a in avgs]
    for a, g in zip(avs, groups):
        if a.size != g.master.size:
            raise ValueError("average length differs from shard length")
    arr = (_f32p * len(avs))(*[_ptr(a, ctypes.c_float) for a in avs])
    P, S = _policy_state(policy, state)
    rc = lib().oracle_step_from_average(G, len(groups), arr, ctypes.byref(P), ctypes.byref(S),
                                        ctypes.c_double(norm2), ctypes.c_int32(int(bool(flag))))
    if rc != 0:
        raise RuntimeError(f"oracle_step_from_average rc={rc}")
    return _state_back(S, state)
