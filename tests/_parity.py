"""The parity bar between the GPU library and the CPU oracle (host code only,
numpy; usable without a GPU).

The kernels and the oracle perform the same fp32 operations in the same
order, so master, m, v and the 16-bit parameters are compared bit for bit.
One input of the update is not fixed by the operations alone: the gradient
clipping multiplier min(1, max_norm / (norm + 1e-6)) is rounded to fp32 from
an fp64 norm that the two sides sum in different orders (the same squares,
grouped differently; they agree to about 1e-10 relative). Either fp32
rounding of the multiplier is then a correct result. When the two
multipliers differ they must be at most one fp32 ulp apart, and from that
call on the run is held to the stated tolerances instead of bit identity:

* master, m, v: |x - o| <= rtol * max(|o|, floor), rtol 1e-6 for the first
  step after the divergence and 5e-6 from the second on (the bar allows 5e-6
  after ten steps; a one-ulp multiplier difference moves the update by far
  less), with floors lr for master, (1 - beta1) * 1e-3 for m (the gradient
  draws' scale) and the smallest normal fp32 for v;
* the 16-bit parameters: at most one ulp apart as ordered integers, +0 and
  -0 equal;
* NaN positions identical.
"""
import numpy as np

GRAD_SIGMA = 1e-3
FLT_MIN = float(np.finfo(np.float32).tiny)


def ordered32(x):
    """float32 values as integers ordered like the floats (-0 and +0 both 0)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.where(b < 0, -(b & 0x7FFFFFFF), b)


def ordered16(bits):
    """uint16 bit patterns of fp16 or bf16 as integers ordered like the values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp32(a, b):
    """Distance in fp32 ulps between two finite float32 scalars or arrays
    (a Python int for scalars)."""
    d = np.abs(ordered32(np.atleast_1d(a)) - ordered32(np.atleast_1d(b)))
    return int(d[0]) if np.ndim(a) == 0 and np.ndim(b) == 0 else d


def assert_close32(got, want, rtol, floor, what):
    got = np.ascontiguousarray(got, dtype=np.float32)
    want = np.ascontiguousarray(want, dtype=np.float32)
    nan = np.isnan(want)
    if not (np.isnan(got) == nan).all():
        raise AssertionError(f"{what}: NaN positions differ")
    g, w = got[~nan].astype(np.float64), want[~nan].astype(np.float64)
    inf = np.isinf(w)
    if not (g[inf] == w[inf]).all():
        raise AssertionError(f"{what}: infinities differ")
    g, w = g[~inf], w[~inf]
    bound = rtol * np.maximum(np.abs(w), floor)
    bad = np.nonzero(np.abs(g - w) > bound)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {g.size} outside rtol {rtol:g} (floor {floor:g}); "
                             f"first: got {g[i]!r} want {w[i]!r}")


def assert_within_ulp16(got, want, what, ulps=1):
    d = np.abs(ordered16(got) - ordered16(want))
    bad = np.nonzero(d > ulps)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {d.size} more than {ulps} ulp apart; first at {i}: "
                             f"got {int(got[i]):#06x} want {int(want[i]):#06x}")


def assert_bits32(got, want, what):
    g = np.ascontiguousarray(got, dtype=np.float32).view(np.uint32)
    w = np.ascontiguousarray(want, dtype=np.float32).view(np.uint32)
    bad = np.nonzero(g != w)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {g.size} differ; first at {i}: "
                             f"got {g.view(np.float32)[i]!r} want {w.view(np.float32)[i]!r}")


def assert_bits16(got, want, what):
    bad = np.nonzero(np.asarray(got) != np.asarray(want))[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {len(got)} differ; first at {i}: "
                             f"got {int(got[i]):#06x} want {int(want[i]):#06x}")


class Bar:
    """The bar of one run (one GPU state next to one oracle state): exact
    until the clip multipliers first differ, the tolerances afterwards."""

    def __init__(self, lr=1e-3, beta1=0.9):
        self.exact = True
        self.steps_since = 0      # applied steps since the multipliers first differed
        self.lr = lr
        self.beta1 = beta1

    def clip(self, tag, gpu_clip, oracle_clip, applied):
        """Compare the multipliers of one call; `applied`: the step was applied."""
        g, o = np.float32(gpu_clip), np.float32(oracle_clip)
        if g != o:
            d = ulp32(g, o)
            if d > 1:
                raise AssertionError(f"{tag}: clip multipliers {g!r} and {o!r} are {d} ulps apart")
            self.exact = False
        if not self.exact and applied:
            self.steps_since += 1

    @property
    def rtol(self):
        return 1e-6 if self.steps_since <= 1 else 5e-6

    def state32(self, got, want, what, kind):
        """kind: "master", "m" or "v"."""
        if self.exact:
            nan = np.isnan(np.asarray(want, dtype=np.float32))
            if not (np.isnan(np.asarray(got, dtype=np.float32)) == nan).all():
                raise AssertionError(f"{what}: NaN positions differ")
            assert_bits32(np.where(nan, 0, got), np.where(nan, 0, want), what)
            return
        floor = {"master": self.lr, "m": (1.0 - self.beta1) * GRAD_SIGMA, "v": FLT_MIN}[kind]
        assert_close32(got, want, self.rtol, floor, what)

    def param16(self, got, want, what):
        if self.exact:
            assert_bits16(got, want, what)
        else:
            assert_within_ulp16(got, want, what)
