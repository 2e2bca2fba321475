"""Python binding of libzero_dp.so, the ZeRO-DP partitioned optimizer step for
AMD MI355X (gfx950).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch supplies device memory (``tensor.data_ptr()``) and the stream
(``torch.cuda.current_stream()``). Importing this module needs the built
library; there is no fallback.
"""
import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzero_dp.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_ALIGNMENT = -2
ERR_WORKSPACE = -3
ERR_HIP = -4
ERR_UNSUPPORTED = -5
MAX_GROUPS = 8
MAX_REPLICAS = 4096
DT_F16 = 1
DT_BF16 = 2
HBM_REGION_BYTES = 96 << 30
ARENA_ALIGN = 2 << 20

EXPORTS = ("zero_partition", "zero_partition_tensors", "zero_workspace_bytes",
           "zero_last_error", "zero_state_init", "zero_reduce_grad_segment",
           "zero_grad_norm_overflow", "zero_adam_step", "zero_cast_writeback", "zero_plan_arena",
           "zero_set_grid_limit", "zero_adam_step_static", "zero_copy_probe")


class ZeroError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"zero_dp error {code}: {msg}")
        self.code = code


class Segment(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("size", ctypes.c_int64)]


class TensorSlice(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("shard_begin", ctypes.c_int64), ("tensor_begin", ctypes.c_int64),
                ("length", ctypes.c_int64)]


class ArenaBuffer(ctypes.Structure):
    _fields_ = [("bytes", ctypes.c_int64), ("traffic", ctypes.c_int64), ("offset", ctypes.c_int64),
                ("region", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class StepState(ctypes.Structure):
    _fields_ = [("beta1_pow", ctypes.c_double * MAX_GROUPS),
                ("beta2_pow", ctypes.c_double * MAX_GROUPS),
                ("grad_norm_sq", ctypes.c_double),
                ("grad_norm", ctypes.c_float),
                ("loss_scale", ctypes.c_float),
                ("step", ctypes.c_int64),
                ("overflow", ctypes.c_int32),
                ("skipped", ctypes.c_int32),
                ("good_steps", ctypes.c_int32),
                ("clip_coef", ctypes.c_float),
                ("cur", ctypes.c_int32),
                ("redo", ctypes.c_int32)]


class Policy(ctypes.Structure):
    _fields_ = [("skip_on_overflow", ctypes.c_int32), ("growth_interval", ctypes.c_int32),
                ("optimistic", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("backoff", ctypes.c_double), ("growth", ctypes.c_double),
                ("min_scale", ctypes.c_double), ("max_grad_norm", ctypes.c_double)]


class _Group(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64),
                ("replicas", ctypes.POINTER(ctypes.c_void_p)),
                ("n_d", ctypes.c_int32),
                ("grad_dt", ctypes.c_int32),
                ("avg", ctypes.c_void_p),
                ("master", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p),
                ("master_alt", ctypes.c_void_p),
                ("exp_avg_alt", ctypes.c_void_p),
                ("exp_avg_sq_alt", ctypes.c_void_p),
                ("flat_param", ctypes.c_void_p),
                ("param_offset", ctypes.c_int64),
                ("param_dt", ctypes.c_int32),
                ("reserved", ctypes.c_int32),
                ("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


_LIB = None


def load():
    """Load the built library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              f"`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.zero_partition.argtypes = [i64, i32, i64, ctypes.POINTER(Segment), ctypes.POINTER(i64)]
        L.zero_partition_tensors.argtypes = [ctypes.POINTER(i64), i32, i32, i32, i64,
                                             ctypes.POINTER(TensorSlice), i32, ctypes.POINTER(i32)]
        L.zero_workspace_bytes.argtypes = [i32]
        L.zero_workspace_bytes.restype = ctypes.c_size_t
        L.zero_last_error.argtypes = []
        L.zero_last_error.restype = ctypes.c_char_p
        L.zero_state_init.argtypes = [vp, ctypes.c_float, vp]
        sz = ctypes.c_size_t
        L.zero_reduce_grad_segment.argtypes = [ctypes.POINTER(vp), i32, i32, i64, vp, vp, sz, i32, vp, vp]
        L.zero_grad_norm_overflow.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(i64), i32, i32, vp, sz,
                                              ctypes.POINTER(Policy), vp, vp]
        L.zero_adam_step.argtypes = [ctypes.POINTER(_Group), i32, ctypes.POINTER(Policy), vp, sz, vp, vp]
        L.zero_cast_writeback.argtypes = [vp, i64, vp, i64, i32, vp]
        L.zero_plan_arena.argtypes = [ctypes.POINTER(ArenaBuffer), i32, i64, i32, i64, ctypes.POINTER(i64)]
        L.zero_set_grid_limit.argtypes = [i32]
        L.zero_adam_step_static.argtypes = [ctypes.POINTER(_Group), i32, ctypes.POINTER(Policy), vp, vp]
        L.zero_copy_probe.argtypes = [vp, vp, vp, vp, i64, vp]
        for name in EXPORTS:
            fn = getattr(L, name)
            if name not in ("zero_workspace_bytes", "zero_last_error"):
                fn.restype = ctypes.c_int
        _LIB = L
    return _LIB


def last_error():
    return load().zero_last_error().decode()


def _check(rc):
    if rc != OK:
        raise ZeroError(rc, last_error())


# --------------------------------------------------------------------------
# host calls
# --------------------------------------------------------------------------

def partition(numel, n_d, align_elems=1):
    """[(offset, size)] for each rank, and the padded length."""
    segs = (Segment * n_d)()
    padded = ctypes.c_int64(0)
    _check(load().zero_partition(numel, n_d, align_elems, segs, ctypes.byref(padded)))
    return [(s.offset, s.size) for s in segs], padded.value


def partition_tensors(numels, n_d, rank, align_elems=1):
    """[(tensor, shard_begin, tensor_begin, length)] inside rank's segment."""
    arr = (ctypes.c_int64 * max(1, len(numels)))(*numels)
    cap = max(1, len(numels))
    out = (TensorSlice * cap)()
    n_out = ctypes.c_int32(0)
    _check(load().zero_partition_tensors(arr, len(numels), n_d, rank, align_elems, out, cap,
                                         ctypes.byref(n_out)))
    return [(out[i].tensor, out[i].shard_begin, out[i].tensor_begin, out[i].length)
            for i in range(n_out.value)]


def set_grid_limit(max_blocks):
    """Cap the blocks of every streaming launch (0: no cap); for tests."""
    _check(load().zero_set_grid_limit(int(max_blocks)))


def copy_probe(src0, src1, dst0, dst1, stream=None):
    """Copy src0 -> dst0 and src1 -> dst1 (uint8 device tensors of one size,
    a multiple of 16 bytes) with the update kernel's access shape: the
    bandwidth reference for a step of half reads, half writes."""
    torch = _torch()
    dev = src0.device if isinstance(src0, torch.Tensor) else None
    nb = _nbytes(src0) if isinstance(src0, torch.Tensor) else 0
    if dev is None or dev.type != "cuda":
        raise ValueError("copy_probe: src0 must be a device tensor")
    for name, t in (("src0", src0), ("src1", src1), ("dst0", dst0), ("dst1", dst1)):
        _need(t, name, (torch.uint8,), dev, nb, exact=True)
    _check(load().zero_copy_probe(_ptr(src0), _ptr(src1), _ptr(dst0), _ptr(dst1), ctypes.c_int64(nb),
                                  _stream(stream)))


def workspace_bytes(n_groups):
    return int(load().zero_workspace_bytes(n_groups))


def plan_arena(sizes, traffic, max_bytes, region_bytes=0, n_regions=0):
    """Offsets of buffers of `sizes` bytes, moving `traffic` bytes per step, in
    one arena of at most `max_bytes`: ([offset], [region], arena_bytes)."""
    if len(sizes) != len(traffic):
        raise ValueError("sizes and traffic differ in length")
    arr = (ArenaBuffer * max(1, len(sizes)))()
    for i, (b, t) in enumerate(zip(sizes, traffic)):
        arr[i].bytes, arr[i].traffic = int(b), int(t)
    total = ctypes.c_int64(0)
    _check(load().zero_plan_arena(arr, len(sizes), int(region_bytes), int(n_regions), int(max_bytes),
                                  ctypes.byref(total)))
    return [arr[i].offset for i in range(len(sizes))], [arr[i].region for i in range(len(sizes))], total.value


def arena_view(arena, offset, numel, dtype):
    """A `numel`-element view of dtype at byte `offset` of a uint8 arena tensor."""
    torch = _torch()
    nbytes = numel * torch.empty((), dtype=dtype).element_size()
    if offset < 0 or offset + nbytes > arena.numel():
        raise ValueError("view outside the arena")
    return arena[offset:offset + nbytes].view(dtype)


# --------------------------------------------------------------------------
# device calls (torch tensors for memory, torch's current stream)
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


_DTYPES = {}


def _dt_code(dtype):
    torch = _torch()
    if dtype == torch.float16:
        return DT_F16
    if dtype == torch.bfloat16:
        return DT_BF16
    raise TypeError(f"16-bit dtype expected, got {dtype}")


def _dt(t):
    code = _DTYPES.get(t.dtype)
    if code is not None:
        return code
    torch = _torch()
    _DTYPES.update({torch.float16: DT_F16, torch.bfloat16: DT_BF16})
    if t.dtype == torch.float16:
        return DT_F16
    if t.dtype == torch.bfloat16:
        return DT_BF16
    raise TypeError(f"16-bit tensor expected, got {t.dtype}")


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _nbytes(t):
    return t.numel() * t.element_size()


_ARRAY_TYPES = {}


def _array_type(ctype, n):
    """ctype * n, built once per length (building the type costs more than filling it)."""
    key = (ctype, n)
    t = _ARRAY_TYPES.get(key)
    if t is None:
        t = _ARRAY_TYPES[key] = ctype * n
    return t


def _ptr_array(tensors):
    return _array_type(ctypes.c_void_p, len(tensors))(*[t.data_ptr() for t in tensors])


def _f32():
    return (_torch().float32,)


def _half():
    torch = _torch()
    return (torch.float16, torch.bfloat16)


def _need(t, name, dtypes, device, n=None, exact=False):
    """Refuse a tensor the kernels would misread before its pointer reaches
    the library: a dtype other than `dtypes`, another device than `device`
    (a host pointer handed to a kernel faults), a non-contiguous view (read as
    if it were contiguous), or fewer than `n` elements (exactly `n` with
    `exact`): the library knows pointers and counts, not allocation sizes."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: a torch tensor is expected, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if t.device != device:
        raise ValueError(f"{name}: tensor on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous")
    if n is not None:
        if exact and t.numel() != n:
            raise ValueError(f"{name}: length {t.numel()} differs from the shard's {n}")
        if t.numel() < n:
            raise ValueError(f"{name}: {t.numel()} elements, shorter than the shard's {n}")
    return t


def _state_device(state, workspace=None):
    """The device of a step state (a device tensor of at least
    sizeof(zero_step_state) bytes); the workspace must be on it too."""
    torch = _torch()
    if not isinstance(state, torch.Tensor) or not state.is_cuda:
        raise ValueError("state must be a device tensor (from new_state)")
    dev = state.device
    _need(state, "state", (torch.uint8,), dev, ctypes.sizeof(StepState))
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8,), dev)
    return dev


def _same_half(tensors, name, device, n):
    """16-bit tensors of one dtype, on `device`, each at least n elements."""
    if not tensors:
        raise ValueError(f"{name}: empty list")
    first = _need(tensors[0], f"{name}[0]", _half(), device, n)
    for r, t in enumerate(tensors[1:], 1):
        _need(t, f"{name}[{r}]", (first.dtype,), device, n)
    return first.dtype


def new_state(loss_scale=1.0, device="cuda", stream=None):
    """Allocate and initialise a device zero_step_state (a uint8 tensor)."""
    torch = _torch()
    st = torch.empty(ctypes.sizeof(StepState), dtype=torch.uint8, device=device)
    _check(load().zero_state_init(_ptr(st), float(loss_scale), _stream(stream)))
    return st


def state_init(state, loss_scale=1.0, stream=None):
    _state_device(state)
    _check(load().zero_state_init(_ptr(state), float(loss_scale), _stream(stream)))


def read_state(state):
    """Copy the device state to the host (synchronises) and decode it."""
    raw = bytes(state.cpu().numpy().tobytes())
    s = StepState.from_buffer_copy(raw)
    return {"beta1_pow": list(s.beta1_pow), "beta2_pow": list(s.beta2_pow),
            "grad_norm_sq": s.grad_norm_sq, "grad_norm": s.grad_norm, "loss_scale": s.loss_scale,
            "step": s.step, "overflow": s.overflow, "skipped": s.skipped, "good_steps": s.good_steps,
            "clip_coef": s.clip_coef, "cur": s.cur, "redo": s.redo}


def new_workspace(n_groups, device="cuda"):
    torch = _torch()
    nbytes = workspace_bytes(n_groups)
    if nbytes == 0:
        raise ValueError(f"n_groups={n_groups} out of range")
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def policy(skip_on_overflow=False, growth_interval=1000, backoff=0.5, growth=2.0, min_scale=1.0,
           max_grad_norm=0.0, optimistic=False):
    """Loss-scale and clipping policy. Skipping or clipping selects the checked
    pipeline (reduce_grad_segment / grad_norm_overflow before adam_step), or,
    with optimistic=True (needs skip), the optimistic pipeline, which needs
    each group's *_alt state set and, when clipping triggers, runs a second
    pass."""
    return Policy(int(bool(skip_on_overflow)), int(growth_interval), int(bool(optimistic)), 0,
                  float(backoff), float(growth), float(min_scale), float(max_grad_norm))


def is_checked(policy_):
    return (policy_ is not None and not policy_.optimistic
            and (policy_.skip_on_overflow or policy_.max_grad_norm > 0))


def reduce_grad_segment(replicas, avg_out, workspace, group, state, stream=None):
    """Average N_d gradient copies (list of 16-bit tensors of equal length)."""
    dev = _state_device(state, workspace)
    _need(avg_out, "avg_out", _f32(), dev)
    n = avg_out.numel()
    _same_half(list(replicas), "replicas", dev, n)
    arr = _ptr_array(replicas)
    _check(load().zero_reduce_grad_segment(arr, len(replicas), _dt(replicas[0]), n, _ptr(avg_out),
                                           _ptr(workspace), _nbytes(workspace), group, _ptr(state),
                                           _stream(stream)))


def grad_norm_overflow(grads, workspace, n_groups, state, policy_=None, stream=None, grad_dtype=None):
    """Finalise the norm / overflow flag. ``grads``: None, or a list of n_groups
    entries (a 16-bit tensor to scan, or None for a slot already filled)."""
    dev = _state_device(state, workspace)
    if grads is None:
        gp, cp, dt = None, None, DT_F16 if grad_dtype is None else grad_dtype
    else:
        if len(grads) != n_groups:
            raise ValueError("grads must have one entry per group")
        _same_half([g for g in grads if g is not None], "grads", dev, 0)
        # an empty gradient still marks its slot for scanning: give it a
        # non-NULL address (never read, there are no elements)
        gp = (ctypes.c_void_p * n_groups)(*[
            (g.data_ptr() or workspace.data_ptr()) if g is not None else 0 for g in grads])
        cp = (ctypes.c_int64 * n_groups)(*[g.numel() if g is not None else 0 for g in grads])
        dt = _dt(next(g for g in grads if g is not None))
    sc = ctypes.byref(policy_) if policy_ is not None else None
    _check(load().zero_grad_norm_overflow(gp, cp, dt, n_groups, _ptr(workspace), _nbytes(workspace), sc,
                                          _ptr(state), _stream(stream)))


@dataclass
class Group:
    """One parameter group's shard. Tensors are device tensors."""
    master: object
    exp_avg: object
    exp_avg_sq: object
    replicas: list = None      # N_d 16-bit tensors (fused average)
    avg: object = None         # or an fp32 average from reduce_grad_segment
    master_alt: object = None  # optimistic pipeline: second state set
    exp_avg_alt: object = None
    exp_avg_sq_alt: object = None
    flat_param: object = None  # 16-bit flat vector (whole group) or None
    param_offset: int = 0
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0


def _group_struct(g, keep, s, device):
    """Fill the zero-initialised zero_group `s` from Group `g` after checking
    every tensor's dtype, device (`device`), contiguity and length; arrays the
    struct points into are appended to `keep` (alive until the call returns)."""
    f32 = _f32()
    _need(g.master, "master", f32, device)
    n = g.master.numel()
    s.n = n
    _need(g.exp_avg, "exp_avg", f32, device, n, exact=True)
    _need(g.exp_avg_sq, "exp_avg_sq", f32, device, n, exact=True)
    if g.replicas is not None:
        s.grad_dt = _dt_code(_same_half(list(g.replicas), "replicas", device, n))
        arr = _ptr_array(g.replicas)
        keep.append(arr)
        s.replicas = arr
        s.n_d = len(g.replicas)
    if g.avg is not None:
        _need(g.avg, "avg", f32, device, n)
        s.avg = g.avg.data_ptr()
    s.master, s.exp_avg, s.exp_avg_sq = g.master.data_ptr(), g.exp_avg.data_ptr(), g.exp_avg_sq.data_ptr()
    if g.master_alt is not None:
        for name in ("master_alt", "exp_avg_alt", "exp_avg_sq_alt"):
            if getattr(g, name) is None:
                raise ValueError(f"{name} missing")
            _need(getattr(g, name), name, f32, device, n, exact=True)
        s.master_alt = g.master_alt.data_ptr()
        s.exp_avg_alt = g.exp_avg_alt.data_ptr()
        s.exp_avg_sq_alt = g.exp_avg_sq_alt.data_ptr()
    if g.flat_param is not None:
        _need(g.flat_param, "flat_param", _half(), device)
        if g.param_offset < 0 or g.param_offset + n > g.flat_param.numel():
            raise ValueError("param_offset + n exceeds the flat parameter vector")
        s.flat_param = g.flat_param.data_ptr()
        s.param_offset = g.param_offset
        s.param_dt = _dt(g.flat_param)
    s.lr, s.beta1, s.beta2, s.eps, s.weight_decay = g.lr, g.beta1, g.beta2, g.eps, g.weight_decay


def adam_step(groups, workspace, state, policy_=None, stream=None):
    dev = _state_device(state, workspace)
    keep = []
    arr = _array_type(_Group, len(groups))()
    for g, s in zip(groups, arr):
        _group_struct(g, keep, s, dev)
    sc = ctypes.byref(policy_) if policy_ is not None else None
    _check(load().zero_adam_step(arr, len(groups), sc, _ptr(workspace), _nbytes(workspace), _ptr(state),
                                 _stream(stream)))


def adam_step_static(groups, state, policy_=None, stream=None):
    """adam_step without a workspace: the library's static scratch holds the
    norm partials (for callers that cannot allocate; calls that overlap on
    one GPU race)."""
    dev = _state_device(state)
    keep = []
    arr = _array_type(_Group, len(groups))()
    for g, s in zip(groups, arr):
        _group_struct(g, keep, s, dev)
    sc = ctypes.byref(policy_) if policy_ is not None else None
    _check(load().zero_adam_step_static(arr, len(groups), sc, _ptr(state), _stream(stream)))


def current_state(group, state_dict):
    """(master, exp_avg, exp_avg_sq) tensors holding the current state of a
    group, given read_state()'s result (the optimistic pipeline alternates)."""
    if state_dict.get("cur", 0) and group.master_alt is not None:
        return group.master_alt, group.exp_avg_alt, group.exp_avg_sq_alt
    return group.master, group.exp_avg, group.exp_avg_sq


def cast_writeback(master, flat_param, offset, stream=None):
    torch = _torch()
    if not isinstance(master, torch.Tensor) or not master.is_cuda:
        raise ValueError("master must be a device tensor")
    _need(master, "master", _f32(), master.device)
    _need(flat_param, "flat_param", _half(), master.device)
    n = master.numel()
    if offset < 0 or offset + n > flat_param.numel():
        raise ValueError("offset + n exceeds the flat parameter vector")
    _check(load().zero_cast_writeback(_ptr(master), n, _ptr(flat_param), offset, _dt(flat_param),
                                      _stream(stream)))
