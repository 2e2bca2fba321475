"""The bandwidth reference bench.py reports beside the step (zero_copy_probe):
it must copy both streams exactly, tails and grid-stride rounds included, and
refuse what its kernel cannot take."""
import ctypes

import pytest
import torch

import zero_dp_partitioned_amd as zdp

from _gpu_helpers import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_bytes,limit", [(16, 0), (16 * 1024 * 16, 0), (16 * 1_000_003, 0),
                                           (16 * 1_000_003, 3), (64 << 20, 0),
                                           ((2 << 30) + 16 * 4097, 0)])   # past 2^31 bytes: a 64-bit size
def test_copy_probe_copies_both_streams(n_bytes, limit):
    print(f"[case] copy probe {n_bytes} bytes, grid limit {limit}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(n_bytes + limit)
    src = [torch.randint(0, 256, (n_bytes,), dtype=torch.uint8, device=DEV, generator=g) for _ in range(2)]
    dst = [torch.zeros(n_bytes + 64, dtype=torch.uint8, device=DEV) for _ in range(2)]
    zdp.set_grid_limit(limit)
    try:
        zdp.copy_probe(src[0], src[1], dst[0][:n_bytes], dst[1][:n_bytes])
        torch.cuda.synchronize()
    finally:
        zdp.set_grid_limit(0)
    for s, d in zip(src, dst):
        assert torch.equal(d[:n_bytes], s)
        assert not torch.any(d[n_bytes:])      # nothing past the end


def test_copy_probe_refuses_what_it_cannot_take():
    a = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    b = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    L = zdp.load()

    def vp(t, k=0):
        return ctypes.c_void_p(t.data_ptr() + k)
    n = ctypes.c_int64
    assert L.zero_copy_probe(vp(a), vp(b), vp(a, 2048), vp(b, 2048), n(17), None) == zdp.ERR_INVALID_ARG
    assert L.zero_copy_probe(vp(a, 8), vp(b), vp(a, 2048), vp(b, 2048), n(32), None) == zdp.ERR_ALIGNMENT
    with pytest.raises(TypeError):
        zdp.copy_probe(a.view(torch.float32), b, a, b)
    with pytest.raises(ValueError):
        zdp.copy_probe(a, b[:16], a, b)
