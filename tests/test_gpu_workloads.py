"""The five workloads at full size, in the launch configuration bench.py times.

* tiny (and its literal shape list): every element against the oracle.
* GPT-2 1.5B, 7.5B at N_d=64, 13B at N_d=8 (dynamic loss scale with one
  overflowing call), LLaMA-3 8B (AdamW, two groups): the elementwise outputs
  on a fixed sample of coordinates (first and last 64, tensor and group
  boundaries, the injected inf, 4096 random ones) stepped by the oracle from
  the same inputs -- each coordinate's update depends only on that coordinate,
  so a sample is checked exactly; the gradient norm and the overflow flag over
  all elements by the oracle on the first call and on the overflowing call
  (chunked, chunk sums added in order); the flag, skip verdict, step count and
  loss scale on every call.
"""
import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import zero_dp_partitioned_amd as zdp
from zero_dp_partitioned_amd import layout
from workloads import WORKLOADS, derive_seed, fill_normal_, torch_dtype

from _gpu_helpers import DEV, ORACLE_DT, assert_bits_equal, assert_u16_equal, down16, down32

pytestmark = pytest.mark.gpu

WORKERS = min(16, os.cpu_count() or 1)


def _u16(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16).copy()


def full_norm_flag(rep_lists, dt, inv_scale):
    """The oracle's norm^2 and flag over every element of every group."""
    odt = ORACLE_DT[dt]

    def job(host):
        a = oracle.average(host, odt)
        return oracle.norm_overflow(a, inv_scale)

    results = []
    with ThreadPoolExecutor(WORKERS) as ex:
        pending = []
        for reps in rep_lists:
            n = reps[0].numel()
            chunk = max(1 << 20, (1 << 27) // len(reps))
            for s in range(0, n, chunk):
                e = min(n, s + chunk)
                host = [_u16(r[s:e]) for r in reps]
                pending.append(ex.submit(job, host))
                if len(pending) >= 2 * WORKERS:
                    results.append(pending.pop(0).result())
            print(f"  oracle scan: group of {n} elements queued", flush=True)
        results += [p.result() for p in pending]
    n2, flag = 0.0, 0
    for r2, rf in results:
        n2 += r2
        flag |= rf
    return n2, flag


def _sample(n, boundaries, seed, k=4096):
    idx = set(range(min(n, 64))) | set(range(max(0, n - 64), n))
    for b in boundaries:
        for d in (-1, 0, 1):
            if 0 <= b + d < n:
                idx.add(b + d)
    rng = np.random.Generator(np.random.PCG64(seed))
    if n > 0:
        idx |= set(rng.integers(0, n, size=min(k, n)).tolist())
    return np.array(sorted(idx), dtype=np.int64)


class Run:
    """Device buffers of a workload (laid out as bench.py lays them out: one
    arena over HBM's regions, gradient copies as a pointer table) and the
    oracle's copy of the sampled coordinates."""

    def __init__(self, key, full=False, optimistic=False, max_grad_norm=0.0, rank=None):
        self.wl = wl = WORKLOADS[key] if rank is None else dataclasses.replace(WORKLOADS[key], rank=rank)
        self.full = full
        self.optimistic = optimistic
        self.max_grad_norm = max_grad_norm
        gdt, pdt = torch_dtype(wl.grad_dt), torch_dtype(wl.param_dt)
        self.odt = ORACLE_DT[wl.grad_dt]
        self.groups, self.ogroups, self.samples, self.outside = [], [], [], []
        shards = []
        for spec in wl.groups:
            psi = sum(spec.numels)
            segs, _ = zdp.partition(psi, wl.n_d)
            o_off, o_size, _ = oracle.partition(psi, wl.n_d)
            assert segs[wl.rank] == (int(o_off[wl.rank]), int(o_size[wl.rank]))
            shards.append((psi, *segs[wl.rank]))
        pipeline = ("optimistic" if optimistic else "checked") if wl.dynamic_loss_scale or max_grad_norm > 0 \
            else "fused"
        spec_pipeline = "fused" if pipeline == "checked" and wl.n_d == 1 else pipeline
        specs = layout.step_specs(shards, wl.n_d, gdt, pdt, spec_pipeline, wl.n_d <= layout.INLINE_COPIES)
        buf, self.placement = layout.allocate(specs, DEV, "regions")
        print(f"  layout: {self.placement}", flush=True)
        for gi, (spec, (psi, off, n)) in enumerate(zip(wl.groups, shards)):
            master = buf[(gi, "master")][:n]
            fill_normal_(master, 0.02, derive_seed(wl.key, gi, "master"))
            flat = buf[(gi, "flat")][:psi]
            fill_normal_(flat, 0.02, derive_seed(wl.key, gi, "flat"))
            flat[off:off + n].copy_(master)
            reps = layout.copies_of(buf, gi, wl.n_d, n)
            alt = {}
            if optimistic:
                alt = {name: buf[(gi, name)][:n] for name in ("master_alt", "exp_avg_alt", "exp_avg_sq_alt")}
            self.groups.append(zdp.Group(master=master, exp_avg=buf[(gi, "exp_avg")][:n].zero_(),
                                         exp_avg_sq=buf[(gi, "exp_avg_sq")][:n].zero_(), replicas=reps,
                                         flat_param=flat, param_offset=off, lr=wl.lr, beta1=wl.beta1,
                                         beta2=wl.beta2, eps=wl.eps, weight_decay=spec.weight_decay, **alt))
            # sample: tensor boundaries inside the shard, the middle (inf site)
            bounds = [sl[1] for sl in zdp.partition_tensors(list(spec.numels), wl.n_d, wl.rank)]
            idx = np.arange(n, dtype=np.int64) if full else _sample(n, bounds + [n // 2], gi + 17)
            self.samples.append(idx)
            tidx = torch.from_numpy(idx).to(DEV)
            og = oracle.Group(replicas=None, grad_dt=self.odt, master=down32(master[tidx]),
                              m=np.zeros(idx.size, np.float32), v=np.zeros(idx.size, np.float32),
                              param=np.zeros(idx.size, np.uint16), param_dt=ORACLE_DT[wl.param_dt],
                              lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                              weight_decay=spec.weight_decay)
            self.ogroups.append(og)
            outs = np.unique(np.array([0, off - 1, off + n, psi - 1], dtype=np.int64))
            outs = outs[(outs >= 0) & (outs < psi) & ((outs < off) | (outs >= off + n))]
            self.outside.append((outs, _u16(flat[torch.from_numpy(outs).to(DEV)]) if outs.size else None))
        self.ws = zdp.new_workspace(len(self.groups))
        self.state = zdp.new_state(wl.loss_scale)
        self.ostate = oracle.State(loss_scale=wl.loss_scale)
        self.policy = oracle.Policy(skip_on_overflow=wl.dynamic_loss_scale, max_grad_norm=max_grad_norm)
        self.policy_ = (zdp.policy(wl.dynamic_loss_scale, optimistic=optimistic, max_grad_norm=max_grad_norm)
                        if wl.dynamic_loss_scale or max_grad_norm > 0 else None)
        self.avg = ([buf[(gi, "avg")][:g.master.numel()] for gi, g in enumerate(self.groups)]
                    if spec_pipeline == "checked" else None)

    def draw_grads(self, call):
        wl = self.wl
        scale = self.ostate.loss_scale  # the scale in force (asserted equal on both sides)
        for gi, g in enumerate(self.groups):
            for r, t in enumerate(g.replicas):
                fill_normal_(t, 1e-3, derive_seed(wl.key, gi, "grad", call, r), scale=scale)
        if wl.inf_at is not None and wl.inf_at[0] == call:
            _, rep, where = wl.inf_at
            g = self.groups[0]
            pos = g.master.numel() // 2 if where == "mid" else int(where)
            g.replicas[rep][pos] = float("inf")
            print(f"  call {call}: +inf in copy {rep} at {pos}", flush=True)
            return True
        return False

    def gpu_step(self):
        if self.policy_ is None or self.optimistic:
            zdp.adam_step(self.groups, self.ws, self.state, self.policy_)
            return
        if self.wl.n_d == 1:
            # checked pipeline with a single copy: scan it, then the update reads it again (as bench.py)
            zdp.grad_norm_overflow([g.replicas[0] for g in self.groups], self.ws, len(self.groups), self.state,
                                   self.policy_)
            zdp.adam_step(self.groups, self.ws, self.state, self.policy_)
            return
        for gi, g in enumerate(self.groups):
            zdp.reduce_grad_segment(g.replicas, self.avg[gi], self.ws, gi, self.state)
        zdp.grad_norm_overflow(None, self.ws, len(self.groups), self.state, self.policy_)
        saved = [g.replicas for g in self.groups]
        for gi, g in enumerate(self.groups):
            g.replicas, g.avg = None, self.avg[gi]
        try:
            zdp.adam_step(self.groups, self.ws, self.state, self.policy_)
        finally:
            for gi, g in enumerate(self.groups):
                g.replicas, g.avg = saved[gi], None

    def run(self, steps=None, full_scan_calls=(1,)):
        wl = self.wl
        steps = wl.steps if steps is None else steps
        for call in range(1, steps + 1):
            injected = self.draw_grads(call)
            # clipping depends on the whole shard's norm: scan it on every call
            want_full = call in full_scan_calls or injected or self.max_grad_norm > 0
            if want_full:
                inv = oracle.inv_scale_of(self.ostate.loss_scale)
                full_n2, full_flag = full_norm_flag([g.replicas for g in self.groups], wl.grad_dt, inv)
            # oracle inputs at the sampled coordinates
            for g, og, idx in zip(self.groups, self.ogroups, self.samples):
                tidx = torch.from_numpy(idx).to(DEV)
                og.replicas = [_u16(r[tidx]) for r in g.replicas]
            self.gpu_step()
            if self.max_grad_norm > 0:
                # the sampled coordinates stepped with the whole shard's norm and flag
                oracle.step(self.ogroups, self.policy, self.ostate, norm2=full_n2, flag=full_flag)
            else:
                oracle.step(self.ogroups, self.policy, self.ostate)
            torch.cuda.synchronize()
            s = zdp.read_state(self.state)
            tag = f"{wl.key} call {call}"
            assert s["step"] == self.ostate.step, tag
            assert s["skipped"] == self.ostate.skipped, tag
            assert s["overflow"] == self.ostate.overflow, tag
            assert s["loss_scale"] == np.float32(self.ostate.loss_scale), tag
            assert s["clip_coef"] == np.float32(self.ostate.clip), (tag, s["clip_coef"], self.ostate.clip)
            assert s["redo"] == 0, tag
            if want_full:
                assert s["overflow"] == full_flag, tag
                if np.isfinite(full_n2):
                    assert abs(s["grad_norm_sq"] - full_n2) <= 1e-10 * full_n2, (tag, s["grad_norm_sq"], full_n2)
                    assert s["grad_norm"] == pytest.approx(np.sqrt(full_n2), rel=1e-6)
                else:
                    assert not np.isfinite(s["grad_norm_sq"])
            if self.full:
                assert abs(s["grad_norm_sq"] - self.ostate.norm2) <= 1e-10 * self.ostate.norm2, tag
            for g, og, idx in zip(self.groups, self.ogroups, self.samples):
                tidx = torch.from_numpy(idx).to(DEV)
                cm, cmm, cv = zdp.current_state(g, s)
                assert_bits_equal(down32(cm[tidx]), og.master, tag + " master")
                assert_bits_equal(down32(cmm[tidx]), og.m, tag + " exp_avg")
                assert_bits_equal(down32(cv[tidx]), og.v, tag + " exp_avg_sq")
                # the slice always holds the rounded master (initially too)
                got = _u16(g.flat_param[tidx + g.param_offset])
                want = oracle.encode16(og.master, ORACLE_DT[wl.param_dt])
                assert_u16_equal(got, want, tag + " param")
            print(f"  {tag}: ok (step {s['step']}, norm {s['grad_norm']:.6g}, scale {s['loss_scale']}, "
                  f"skipped {s['skipped']})", flush=True)
        for g, (outs, before) in zip(self.groups, self.outside):
            if before is not None:
                assert_u16_equal(_u16(g.flat_param[torch.from_numpy(outs).to(DEV)]), before,
                                 wl.key + " flat vector outside the shard")
        return self.ostate


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("key", ["tiny", "tiny_literal"])
def test_tiny_every_element(key):
    print(f"[workload] {key}", flush=True)
    st = Run(key, full=True).run()
    assert st.step == 3
    _free()


@pytest.mark.timeout(600)
def test_gpt2_1_5b():
    print("[workload] gpt2_1.5b", flush=True)
    st = Run("gpt2_1.5b").run(full_scan_calls=(1,))
    assert st.step == 10 and st.loss_scale == 65536.0
    _free()


@pytest.mark.timeout(600)
def test_7_5b_nd64():
    print("[workload] 7.5b_nd64", flush=True)
    st = Run("7.5b_nd64").run(full_scan_calls=(1,))
    assert st.step == 10
    _free()


@pytest.mark.timeout(900)
def test_7_5b_nd64_rank0():
    # rank 0: offset 0, every buffer 16-byte aligned (rank 63's parameter slice is only 8-byte aligned)
    print("[workload] 7.5b_nd64 rank 0", flush=True)
    st = Run("7.5b_nd64", rank=0).run(steps=3, full_scan_calls=(1,))
    assert st.step == 3
    _free()


@pytest.mark.timeout(900)
def test_13b_nd8_rank0():
    print("[workload] 13b_nd8 rank 0 (checked)", flush=True)
    st = Run("13b_nd8", rank=0).run(steps=5, full_scan_calls=(1,))
    assert st.step == 4 and st.loss_scale == 32768.0
    _free()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("pipeline", ["checked", "optimistic"])
def test_13b_nd8_overflow_skip(pipeline):
    print(f"[workload] 13b_nd8 ({pipeline})", flush=True)
    st = Run("13b_nd8", optimistic=pipeline == "optimistic").run(full_scan_calls=(1,))
    # ten calls, the fourth overflows: nine applied steps, scale halved once
    assert st.step == 9 and st.loss_scale == 32768.0
    _free()


@pytest.mark.timeout(900)
def test_gpt2_1_5b_clipping():
    # clipping on the single-copy shard (the norm is about 39, the threshold 1): the checked pipeline
    # scans the copy first (the wide-load scan loops its capped grid over 380,277 tiles), then updates
    print("[workload] gpt2_1.5b clipping", flush=True)
    run = Run("gpt2_1.5b", max_grad_norm=1.0)
    st = run.run(steps=3)
    assert st.step == 3 and st.clip < 1.0
    del run
    _free()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("pipeline", ["checked", "optimistic"])
def test_13b_nd8_clipping(pipeline):
    # clipping at full size (the norm is about 14, the threshold 10: every applied call clips),
    # five calls with the overflow on the fourth; the optimistic pipeline's second pass loops over
    # the shard's 396,729 tiles with its capped grid
    print(f"[workload] 13b_nd8 clipping ({pipeline})", flush=True)
    run = Run("13b_nd8", optimistic=pipeline == "optimistic", max_grad_norm=10.0)
    st = run.run(steps=5)
    assert st.step == 4 and st.loss_scale == 32768.0 and st.clip < 1.0
    del run
    _free()


@pytest.mark.timeout(900)
def test_llama3_8b_adamw_two_groups():
    print("[workload] llama3_8b", flush=True)
    st = Run("llama3_8b").run(full_scan_calls=(1,))
    assert st.step == 5
    _free()
