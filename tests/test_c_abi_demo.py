"""The library driven from plain C: ``tests/c_abi/step_demo`` calls only the
C ABI with hipMalloc'd buffers, no torch -- zero_partition, zero_plan_arena,
zero_workspace_bytes, zero_state_init and, per step, zero_adam_step on the
copies (fused pipeline) or zero_reduce_grad_segment, zero_grad_norm_overflow
and zero_adam_step on the average (checked pipeline, dynamic loss scale, an
inf in a copy on the second step), then zero_cast_writeback into a bf16
vector. Its results are checked bit for bit against the CPU oracle run on
inputs this test regenerates on its own from the program's integer recipe
(MurmurHash3's 64-bit finalizer)."""
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "step_demo")

_C1 = np.uint64(0xFF51AFD7ED558CCD)
_C2 = np.uint64(0xC4CEB9FE1A85EC53)
_S33 = np.uint64(33)


def _fmix64(x):
    """MurmurHash3 fmix64 (uint64 arrays; products wrap mod 2^64), low 32 bits."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        x = x ^ (x >> _S33)
        x = x * _C1
        x = x ^ (x >> _S33)
        x = x * _C2
        x = x ^ (x >> _S33)
    return (x & np.uint64(0xFFFFFFFF)).astype(np.uint32)


def _grad_bits(keys):
    h = _fmix64(keys)
    sign = (h >> 31) << 15
    expo = 5 + (h >> 10) % 10
    frac = h & 0x3FF
    return (sign | (expo << 10) | frac).astype(np.uint16)


def _inputs(psi, n_d, off, n, steps, checked=False):
    flat0 = _grad_bits(np.uint64(0x5EED0000) + np.arange(psi, dtype=np.uint64))
    master0 = ((_fmix64(np.uint64(0xABC) + np.arange(n, dtype=np.uint64)) % 20001).astype(np.float32)
               - np.float32(10000.0)) * np.float32(2e-6)
    j = np.uint64(off) + np.arange(n, dtype=np.uint64)
    reps = np.empty((steps, n_d, n), np.uint16)
    for k in range(steps):
        for r in range(n_d):
            reps[k, r] = _grad_bits((np.uint64(k) << np.uint64(48)) ^ (np.uint64(r) << np.uint64(40)) ^ j)
    if checked and steps >= 2:
        reps[1, n_d - 1, n // 2] = 0x7C00   # +inf: the program's second step overflows
    return flat0, master0.astype(np.float32), reps


def _read(path):
    with open(path, "rb") as f:
        raw = f.read()
    hdr = np.frombuffer(raw, np.int64, 7)
    psi, n_d, rank, off, n, steps, checked = (int(x) for x in hdr)
    pos = 56

    def take(dtype, count):
        nonlocal pos
        a = np.frombuffer(raw, dtype, count, pos).copy()
        pos += a.nbytes
        return a

    out = dict(psi=psi, n_d=n_d, rank=rank, off=off, n=n, steps=steps, checked=checked)
    out["reps"] = take(np.uint16, steps * n_d * n).reshape(steps, n_d, n)
    out["master0"] = take(np.float32, n)
    out["master"] = take(np.float32, n)
    out["m"] = take(np.float32, n)
    out["v"] = take(np.float32, n)
    out["flat"] = take(np.uint16, psi)
    out["flat0"] = take(np.uint16, psi)
    out["cast"] = take(np.uint16, psi)
    out["norm2"] = float(take(np.float64, 1)[0])
    out["step"] = int(take(np.int64, 1)[0])
    out["loss_scale"] = float(take(np.float32, 1)[0])
    out["overflow"] = int(take(np.int32, 1)[0])
    out["skipped"] = int(take(np.int32, 1)[0])
    assert pos == len(raw)
    return out


def test_demo_is_built_and_rejects_bad_arguments():
    assert os.path.exists(EXE), "tests/c_abi/step_demo is not built (run __graft_entry__.build())"
    r = subprocess.run([EXE, "/dev/null", "10", "0", "0", "1"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "bad arguments" in r.stderr


def test_generator_matches_a_direct_evaluation():
    # the vectorised fmix64 against Python integers
    def ref(x):
        m = (1 << 64) - 1
        x ^= x >> 33
        x = (x * 0xFF51AFD7ED558CCD) & m
        x ^= x >> 33
        x = (x * 0xC4CEB9FE1A85EC53) & m
        x ^= x >> 33
        return x & 0xFFFFFFFF
    keys = [0, 1, 0x5EED0000, (3 << 48) ^ (7 << 40) ^ 12345, (1 << 64) - 1]
    assert [int(v) for v in _fmix64(np.array(keys, dtype=np.uint64))] == [ref(k) for k in keys]


@pytest.mark.gpu
@pytest.mark.parametrize("psi,n_d,rank,steps,pipeline", [(70_001, 3, 2, 3, "fused"), (4_099, 8, 0, 2, "fused"),
                                                         (70_001, 3, 2, 4, "checked"), (40_003, 8, 7, 3, "checked")])
def test_c_program_matches_oracle(tmp_path, psi, n_d, rank, steps, pipeline):
    out = tmp_path / "demo.bin"
    checked = pipeline == "checked"
    print(f"step_demo psi={psi} n_d={n_d} rank={rank} steps={steps} {pipeline}", flush=True)
    r = subprocess.run([EXE, str(out), str(psi), str(n_d), str(rank), str(steps)] + (["checked"] if checked else []),
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    d = _read(out)
    assert d["checked"] == int(checked)
    off, n = d["off"], d["n"]
    o_off, o_size, _ = oracle.partition(psi, n_d)
    assert (off, n) == (int(o_off[rank]), int(o_size[rank]))

    flat0, master0, reps = _inputs(psi, n_d, off, n, steps, checked)
    np.testing.assert_array_equal(d["flat0"], flat0)
    np.testing.assert_array_equal(d["master0"].view(np.uint32), master0.view(np.uint32))
    np.testing.assert_array_equal(d["reps"], reps)

    g = oracle.Group(replicas=None, grad_dt=oracle.F16, master=master0.copy(), m=np.zeros(n, np.float32),
                     v=np.zeros(n, np.float32), param=flat0[off:off + n].copy(), param_dt=oracle.F16,
                     lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    policy = oracle.Policy(skip_on_overflow=True, growth_interval=1000) if checked else oracle.Policy()
    st = oracle.State(loss_scale=1024.0 if checked else 1.0)
    skipped = 0
    for k in range(steps):
        g.replicas = [reps[k, q].copy() for q in range(n_d)]
        oracle.step([g], policy, st)
        skipped += st.skipped

    np.testing.assert_array_equal(d["master"].view(np.uint32), g.master.view(np.uint32))
    np.testing.assert_array_equal(d["m"].view(np.uint32), g.m.view(np.uint32))
    np.testing.assert_array_equal(d["v"].view(np.uint32), g.v.view(np.uint32))
    np.testing.assert_array_equal(d["flat"][off:off + n], g.param)
    np.testing.assert_array_equal(np.delete(d["flat"], np.s_[off:off + n]), np.delete(flat0, np.s_[off:off + n]))
    # the cast of the final master into the bf16 vector, and nothing outside the slice
    np.testing.assert_array_equal(d["cast"][off:off + n], oracle.encode16(g.master, oracle.BF16))
    np.testing.assert_array_equal(np.delete(d["cast"], np.s_[off:off + n]), np.delete(flat0, np.s_[off:off + n]))
    assert d["step"] == st.step == steps - skipped
    assert d["loss_scale"] == np.float32(st.loss_scale) and d["skipped"] == st.skipped
    assert d["overflow"] == st.overflow
    if checked:
        assert skipped == 1 and st.loss_scale == 512.0
    assert abs(d["norm2"] - st.norm2) <= 1e-12 * st.norm2
