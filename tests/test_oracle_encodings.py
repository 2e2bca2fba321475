"""The oracle's fp16/bf16 encoders and decoders against library routines
(numpy's IEEE binary16 cast, torch's CPU bfloat16 cast), both round to nearest
even."""
import numpy as np
import pytest
import torch

import oracle


def _edge_floats():
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e9, -1e9,
            2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -26, 3e-8, 6e-8,
            2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11,
            np.finfo(np.float32).max, np.finfo(np.float32).tiny, 1e-45,
            3.3895314e38, 3.4e38, np.inf, -np.inf]
    return np.array(vals, dtype=np.float32)


def _random_floats(n=200_000, seed=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # plus values near fp16 range and at ties
    y = (rng.standard_normal(n) * 10.0 ** rng.uniform(-9, 5, n)).astype(np.float32)
    return np.concatenate([x, y])


@pytest.mark.parametrize("xs", [_edge_floats(), _random_floats()], ids=["edges", "random"])
def test_f16_encode_matches_numpy(xs):
    with np.errstate(over="ignore"):
        want = xs.astype(np.float16).view(np.uint16)
    got = oracle.encode16(xs, oracle.F16)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("xs", [_edge_floats(), _random_floats()], ids=["edges", "random"])
def test_bf16_encode_matches_torch(xs):
    want = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.encode16(xs, oracle.BF16)
    np.testing.assert_array_equal(got, want)


def test_nan_canonical():
    x = np.array([np.nan, -np.nan], dtype=np.float32)
    assert set(oracle.encode16(x, oracle.F16).tolist()) <= {0x7E00, 0xFE00}
    assert set(oracle.encode16(x, oracle.BF16).tolist()) <= {0x7FC0, 0xFFC0}
    assert (oracle.encode16(x, oracle.F16) & 0x7FFF == 0x7E00).all()


def test_decode_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got16 = oracle.decode16(bits, oracle.F16)
    want16 = bits.view(np.float16).astype(np.float32)
    fin = np.isfinite(want16)
    np.testing.assert_array_equal(got16[fin].view(np.uint32), want16[fin].view(np.uint32))
    assert np.isnan(got16[np.isnan(want16)]).all()
    assert (got16[np.isinf(want16)] == want16[np.isinf(want16)]).all()
    gotb = oracle.decode16(bits, oracle.BF16)
    wantb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    fin = np.isfinite(wantb)
    np.testing.assert_array_equal(gotb[fin].view(np.uint32), wantb[fin].view(np.uint32))
    assert np.isnan(gotb[np.isnan(wantb)]).all()


def test_round_trip_every_finite_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for dt in (oracle.F16, oracle.BF16):
        vals = oracle.decode16(bits, dt)
        fin = np.isfinite(vals)
        np.testing.assert_array_equal(oracle.encode16(vals[fin], dt), bits[fin])
