"""Shared pieces of the GPU parity tests: moving uint16 bit patterns between
numpy and torch, running the library and the oracle side by side."""
import numpy as np
import torch

import oracle
import zero_dp_partitioned_amd as zdp

DEV = torch.device("cuda:0")
TORCH16 = {"f16": torch.float16, "bf16": torch.bfloat16}
ORACLE_DT = {"f16": oracle.F16, "bf16": oracle.BF16}


def up16(bits, dt, dev=DEV):
    """uint16 numpy bits -> 16-bit torch tensor on the device."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).to(dev).view(TORCH16[dt])


def down16(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16).copy()


def up32(x, dev=DEV):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32).copy()).to(dev)


def down32(t):
    return t.detach().cpu().numpy().copy()


def bits32(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def assert_bits_equal(got, want, what):
    got, want = bits32(got), bits32(want)
    bad = np.nonzero(got != want)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {got.size} differ; first at {i}: "
                             f"got {got.view(np.float32)[i]!r} want {want.view(np.float32)[i]!r}")


def assert_u16_equal(got, want, what):
    bad = np.nonzero(got != want)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {got.size} differ; first at {i}: "
                             f"got {got[i]:#06x} want {want[i]:#06x}")


def carve(buf_elems, offset, n, dtype, dev=DEV):
    """A length-n view starting `offset` elements into a fresh buffer, so the
    pointer alignment can be chosen."""
    base = torch.empty(buf_elems, dtype=dtype, device=dev)
    return base[offset:offset + n]
