"""Device buffers of one rank's step, laid out in HBM.

A step streams every buffer once: the N_d 16-bit gradient copies are read,
fp32 master / exp_avg / exp_avg_sq are read and written (or, in the
optimistic pipeline, one state set is read and the other written), an fp32
average is written and read back (checked pipeline), and the rank's slice of
the 16-bit flat parameter vector is written.

placement "regions": one arena spanning all free HBM, allocated before
anything else large, with every buffer at the offset zero_plan_arena gives, so
that the step's traffic spreads over MI355X's 96 GiB HBM regions (the region
helper in the C ABI says why). placement "packed": one allocation per buffer
in order, which typically puts a small shard's buffers side by side in one
region.

Only marshalling happens here: the plan comes from the C library and the
arena is an ordinary torch allocation.
"""
from dataclasses import dataclass

from . import ARENA_ALIGN, arena_view, plan_arena

PLACEMENTS = ("regions", "packed")
INLINE_COPIES = 64  # gradient copies the kernels take as a pointer table
SMALL_STEP_BYTES = 1 << 30


@dataclass
class BufferSpec:
    key: tuple      # (group, name) or (group, "grad", r)
    numel: int
    dtype: object   # torch dtype
    traffic: int    # bytes a step moves through the buffer


def step_specs(shards, n_d, grad_dtype, param_dtype, pipeline, copies_as_table):
    """Buffers of a step over groups `shards` = [(psi, offset, n)]:
    pipeline "fused", "checked" (adds an fp32 average) or "optimistic" (adds a
    second state set). The gradient copies of a group are separate buffers
    when copies_as_table (N_d <= 64), else one buffer of N_d copies spaced by n
    rounded up to 64 elements (key (g, "gradbuf"))."""
    import torch
    f32 = torch.float32
    out = []
    for gi, (psi, _, n) in enumerate(shards):
        state = 4 * n if pipeline == "optimistic" else 8 * n
        for name in ("master", "exp_avg", "exp_avg_sq"):
            out.append(BufferSpec((gi, name), n, f32, state))
        if pipeline == "optimistic":
            for name in ("master_alt", "exp_avg_alt", "exp_avg_sq_alt"):
                out.append(BufferSpec((gi, name), n, f32, 4 * n))
        if pipeline == "checked":
            out.append(BufferSpec((gi, "avg"), n, f32, 8 * n))
        if copies_as_table:
            for r in range(n_d):
                out.append(BufferSpec((gi, "grad", r), n, grad_dtype, 2 * n))
        else:
            out.append(BufferSpec((gi, "gradbuf"), n_d * copy_stride(n), grad_dtype, 2 * n * n_d))
        out.append(BufferSpec((gi, "flat"), psi, param_dtype, 2 * n))
    return out


def copy_stride(n):
    """Elements between gradient copies in one shared buffer."""
    return (n + 63) // 64 * 64


def allocate(specs, device, placement="regions", reserve_bytes=4 << 30, whole=True, n_regions=0):
    """({key: tensor}, info) for `specs`. With "regions" the dict also holds
    "arena" (the uint8 arena) and "free" (its unused (offset, bytes) ranges,
    see free_ranges) for carving the caller's other tensors with arena_view.

    "regions": with `whole` (the default) the arena is all free memory but
    `reserve_bytes`: an allocation that size is backed across the whole of
    HBM in address order, so the planned offsets fall into the physical
    regions. A smaller arena (whole=False: up to the end of the last buffer)
    is backed wherever the driver finds room, which can put every planned
    region into one physical one; it is also what `whole` falls back to if
    the whole-memory allocation fails. info["arena"] names the arena that was
    obtained ("whole: ...", "sized: ...", "sized: FALLBACK ...", or "none:
    ..." for packed placement). The space
    after the planned buffers stays free for the caller's other data. A step
    under SMALL_STEP_BYTES gets a small arena in one region. `n_regions` > 0
    asks the planner for exactly that many regions (0: the fewest, at least
    two, that hold the buffers)."""
    import torch
    if placement not in PLACEMENTS:
        raise ValueError(f"unknown placement {placement!r}")
    sizes = [max(1, s.numel) * torch.empty((), dtype=s.dtype).element_size() for s in specs]
    bufs = {}
    info = {"placement": placement}
    if placement == "regions":
        # blocks torch has cached but not handed out count as used for the
        # driver: return them first, so the arena spans all memory not in use
        torch.cuda.empty_cache()
        free, _ = torch.cuda.mem_get_info(device)
        # a step under SMALL_STEP_BYTES is bound by launch latency, not HBM: one region
        small = not n_regions and sum(sizes) < SMALL_STEP_BYTES
        offs, regs, total = plan_arena(sizes, [s.traffic for s in specs], free - reserve_bytes,
                                       n_regions=1 if small else n_regions)
        arena = None
        if small:
            info["arena"] = "sized: a step under 1 GiB, one region"
        elif not whole:
            info["arena"] = "sized: ends at the last planned buffer (asked for)"
        else:
            try:
                arena = torch.empty((free - reserve_bytes) // ARENA_ALIGN * ARENA_ALIGN, dtype=torch.uint8,
                                    device=device)
                total = arena.numel()
                info["arena"] = "whole: all free device memory but the reserve"
            except torch.cuda.OutOfMemoryError:
                info["arena"] = ("sized: FALLBACK, the whole-memory arena could not be allocated, so the "
                                 "planned regions need not be physical ones")
        if arena is None:
            arena = torch.empty(total, dtype=torch.uint8, device=device)
        for s, o in zip(specs, offs):
            bufs[s.key] = arena_view(arena, o, max(1, s.numel), s.dtype)
        info.update(arena_bytes=total, regions=len(set(regs)))
        # the arena itself and its unused byte ranges, for the caller's other data
        bufs["arena"] = arena
        bufs["free"] = free_ranges(offs, sizes, total)
    else:
        info["arena"] = "none: one allocation per buffer, wherever the driver finds room"
        for s in specs:
            bufs[s.key] = torch.empty(max(1, s.numel), dtype=s.dtype, device=device)
    return bufs, info


def free_ranges(offsets, sizes, total):
    """[(offset, bytes)] of the ARENA_ALIGN-aligned gaps of at least
    ARENA_ALIGN bytes that buffers at `offsets` of `sizes` leave in an arena
    of `total` bytes, in address order."""
    spans = sorted((o, o + s) for o, s in zip(offsets, sizes))
    out, at = [], 0
    for lo, hi in spans + [(total, total)]:
        start = (at + ARENA_ALIGN - 1) // ARENA_ALIGN * ARENA_ALIGN
        if lo - start >= ARENA_ALIGN:
            out.append((start, (lo - start) // ARENA_ALIGN * ARENA_ALIGN))
        at = max(at, hi)
    return out


def copies_of(bufs, gi, n_d, n):
    """The N_d gradient copy views of group gi."""
    if (gi, "gradbuf") in bufs:
        b, stride = bufs[(gi, "gradbuf")], copy_stride(n)
        return [b[r * stride:r * stride + n] for r in range(n_d)]
    return [bufs[(gi, "grad", r)][:n] for r in range(n_d)]
