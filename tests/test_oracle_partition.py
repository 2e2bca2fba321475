"""Partition and tensor-slice map of the oracle, pinned by brute force and by the
pages' rules: the flat vector split into N_d contiguous segments, base =
numel // N_d with the remainder going to the first ranks (DeepSpeed ZeRO stage
1/2 walkthrough, §4 ②), concatenation giving back the flat vector (same page,
§3), optional padding of the flat length to a multiple of an alignment (§4 ①,
§7)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def _brute_partition(numel, n_d):
    """Deal elements out one at a time: rank r gets elements while its quota lasts."""
    quota = [numel // n_d + (1 if r < numel % n_d else 0) for r in range(n_d)]
    owner = []
    for r in range(n_d):
        owner += [r] * quota[r]
    return owner


@pytest.mark.parametrize("numel", [0, 1, 2, 3, 7, 8, 9, 63, 64, 65, 1000, 4097])
@pytest.mark.parametrize("n_d", [1, 2, 3, 4, 7, 8, 64])
def test_partition_brute_force(numel, n_d):
    offs, sizes, padded = oracle.partition(numel, n_d)
    assert padded == numel
    owner = _brute_partition(numel, n_d)
    for r in range(n_d):
        idx = [j for j, o in enumerate(owner) if o == r]
        assert sizes[r] == len(idx)
        if idx:
            assert offs[r] == idx[0] and idx == list(range(idx[0], idx[0] + len(idx)))
    # contiguity and coverage
    assert offs[0] == 0
    assert (offs[1:] == offs[:-1] + sizes[:-1]).all()
    assert sizes.sum() == numel
    assert sizes.max() - sizes.min() <= 1
    # the larger segments are the first ones
    assert (np.diff(sizes) <= 0).all()


@settings(max_examples=300, deadline=None)
@given(numel=st.integers(0, 10 ** 13), n_d=st.integers(1, 1100))
def test_partition_properties(numel, n_d):
    offs, sizes, _ = oracle.partition(numel, n_d)
    base, rem = divmod(numel, n_d)
    assert sizes.tolist() == [base + (1 if r < rem else 0) for r in range(n_d)]
    assert int(offs[-1] + sizes[-1]) == numel
    for r in (0, n_d // 2, n_d - 1):
        assert offs[r] == r * base + min(r, rem)


def test_concatenation_reproduces_flat_vector():
    rng = np.random.Generator(np.random.PCG64(1))
    flat = rng.integers(0, 1 << 16, size=10_007).astype(np.uint16)
    for n_d in (1, 3, 4, 8, 13):
        offs, sizes, _ = oracle.partition(flat.size, n_d)
        segs = [flat[o:o + s] for o, s in zip(offs, sizes)]
        np.testing.assert_array_equal(np.concatenate(segs), flat)


def test_alignment_padding():
    offs, sizes, padded = oracle.partition(787_971, 4, align_elems=8)
    assert padded == 787_976 and padded % 8 == 0
    assert sizes.tolist() == [196_994] * 4
    offs, sizes, padded = oracle.partition(10, 4, align_elems=2 * 4)
    assert padded == 16 and sizes.tolist() == [4, 4, 4, 4]


def test_workload_segments():
    # tiny: Psi = 787,971 = 4 * 196,992 + 3 -> ranks 0..2 get one extra element
    offs, sizes, _ = oracle.partition(787_971, 4)
    assert (int(offs[1]), int(sizes[1])) == (196_993, 196_993)
    offs, sizes, _ = oracle.partition(786_435, 4)
    assert (int(offs[1]), int(sizes[1])) == (196_609, 196_609)
    offs, sizes, _ = oracle.partition(7_500_000_000, 64)
    assert (int(offs[63]), int(sizes[63])) == (7_382_812_500, 117_187_500)
    offs, sizes, _ = oracle.partition(13_000_000_000, 8)
    assert (int(offs[7]), int(sizes[7])) == (11_375_000_000, 1_625_000_000)


def test_invalid_arguments():
    with pytest.raises(ValueError):
        oracle.partition(-1, 4)
    with pytest.raises(ValueError):
        oracle.partition(10, 0)


def _brute_slices(numels, n_d, rank):
    offs, sizes, _ = oracle.partition(sum(numels), n_d)
    lo, hi = int(offs[rank]), int(offs[rank] + sizes[rank])
    out = []
    start = 0
    for t, n in enumerate(numels):
        members = [j for j in range(start, start + n) if lo <= j < hi]
        if members:
            out.append((t, members[0] - lo, members[0] - start, len(members)))
        start += n
    return out


@pytest.mark.parametrize("numels", [[5], [3, 4, 5], [0, 7, 0, 2], [10, 1, 1, 1, 30], [1] * 9])
@pytest.mark.parametrize("n_d", [1, 2, 3, 5, 8])
def test_tensor_slices_brute_force(numels, n_d):
    for rank in range(n_d):
        assert oracle.tensor_slices(numels, n_d, rank) == _brute_slices(numels, n_d, rank)


def test_tiny_slices_straddle():
    # tensors occupy [0,393216) [393216,393984) [393984,787968) [787968,787971)
    numels = [512 * 768, 768, 768 * 513, 3]
    sl = oracle.tensor_slices(numels, 4, 1)  # rank 1 owns [196993, 393986)
    assert sl == [(0, 0, 196_993, 196_223), (1, 196_223, 0, 768), (2, 196_991, 0, 2)]
    assert oracle.tensor_slices(numels, 4, 2) == [(2, 0, 2, 196_993)]
    assert oracle.tensor_slices(numels, 4, 3) == [(2, 0, 196_995, 196_989), (3, 196_989, 0, 3)]
