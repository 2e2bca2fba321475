"""The five workloads at full size, in the launch configuration bench.py times.

* GPT-2 1.5B, 7.5B at N_d=64 (rank 63), 13B at N_d=8 (rank 7; dynamic loss
  scale with one overflowing call; the checked and the optimistic pipeline on
  the same gradient copies; with and without clipping): every element of
  master, m, v and the parameter slice on every call, against the oracle
  stepped chunk by chunk on the host (tests/_fullsize.py). The two 13B
  pipelines are also compared with each other on the device.
* LLaMA-3 8B (AdamW, two groups): every element of both groups on every
  call, with one block per 4096-element tile, and on the last two calls with
  the grid capped at 2^20 blocks, so that blocks loop over a second tile past
  element 2^32.
* tiny (and its literal shape list): every element.
* Rank 0 of the 7.5B and 13B shards (offset 0): a fixed sample of coordinates
  (first and last 64, tensor boundaries, 4096 random ones) stepped by the
  oracle from the same inputs, norm and flag over all elements on the first
  call.
On every call: the overflow flag, skip verdict, step count, loss scale and
clip multiplier; the norm within 1e-10 relative.
"""
import dataclasses
import gc
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import zero_dp_partitioned_amd as zdp
from zero_dp_partitioned_amd import layout
from workloads import WORKLOADS, derive_seed, fill_normal_, torch_dtype

from _fullsize import FullCheck, GroupCheck, chunk_for, cpu_workers, host_bytes_available, plan_ranges
from _gpu_helpers import DEV, ORACLE_DT, assert_bits_equal, assert_u16_equal, down16, down32
from _parity import Bar

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


class FullRun:
    """A workload at full size for one or two pipelines on the same gradient
    copies (laid out as bench.py lays them out: one arena over HBM's regions,
    copies as a pointer table), with the oracle stepping every checked
    element on the host (tests/_fullsize.py). The last pipeline named is the
    one compared with the oracle; the others are compared with it on the
    device, bit for bit."""

    def __init__(self, key, pipelines=("fused",), max_grad_norm=0.0):
        gc.collect()          # a previous run's arena must be gone before this one takes all free memory
        torch.cuda.empty_cache()
        self.wl = wl = WORKLOADS[key]
        self.pipelines = pipelines
        self.max_grad_norm = max_grad_norm
        gdt, pdt = torch_dtype(wl.grad_dt), torch_dtype(wl.param_dt)
        self.odt = ORACLE_DT[wl.grad_dt]
        shards = []
        for spec in wl.groups:
            psi = sum(spec.numels)
            segs, _ = zdp.partition(psi, wl.n_d)
            o_off, o_size, _ = oracle.partition(psi, wl.n_d)
            assert segs[wl.rank] == (int(o_off[wl.rank]), int(o_size[wl.rank]))
            shards.append((psi, *segs[wl.rank]))
        specs = []
        for p in pipelines:
            sp = "fused" if p == "checked" and wl.n_d == 1 else p
            for b in layout.step_specs(shards, wl.n_d, gdt, pdt, sp, wl.n_d <= layout.INLINE_COPIES):
                if b.key[1] == "grad":
                    if p == pipelines[0]:
                        specs.append(b)            # one set of copies for every pipeline
                else:
                    specs.append(dataclasses.replace(b, key=(p,) + b.key))
        buf, self.placement = layout.allocate(specs, DEV, "regions")
        print(f"  layout: {self.placement}", flush=True)
        self.reps = []
        self.side = {p: dict(groups=[], avg=None) for p in pipelines}
        self.outside = []
        for gi, (spec, (psi, off, n)) in enumerate(zip(wl.groups, shards)):
            self.reps.append(layout.copies_of(buf, gi, wl.n_d, n))
            for p in pipelines:
                master = buf[(p, gi, "master")][:n]
                fill_normal_(master, 0.02, derive_seed(wl.key, gi, "master"))
                flat = buf[(p, gi, "flat")][:psi]
                fill_normal_(flat, 0.02, derive_seed(wl.key, gi, "flat"))
                flat[off:off + n].copy_(master)
                alt = {}
                if p == "optimistic":
                    alt = {name: buf[(p, gi, name)][:n] for name in ("master_alt", "exp_avg_alt", "exp_avg_sq_alt")}
                self.side[p]["groups"].append(zdp.Group(
                    master=master, exp_avg=buf[(p, gi, "exp_avg")][:n].zero_(),
                    exp_avg_sq=buf[(p, gi, "exp_avg_sq")][:n].zero_(), replicas=self.reps[gi], flat_param=flat,
                    param_offset=off, lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                    weight_decay=spec.weight_decay, **alt))
            outs = np.unique(np.array([0, off - 1, off + n, psi - 1], dtype=np.int64))
            outs = outs[(outs >= 0) & (outs < psi) & ((outs < off) | (outs >= off + n))]
            flat = self.side[pipelines[-1]]["groups"][gi].flat_param
            self.outside.append((outs, _u16(flat[torch.from_numpy(outs).to(DEV)]) if outs.size else None))
        for p in pipelines:
            d = self.side[p]
            d["ws"] = zdp.new_workspace(len(wl.groups))
            d["state"] = zdp.new_state(wl.loss_scale)
            needs_norm = wl.dynamic_loss_scale or max_grad_norm > 0
            d["policy"] = (zdp.policy(wl.dynamic_loss_scale, optimistic=p == "optimistic", max_grad_norm=max_grad_norm)
                           if needs_norm else None)
            if p == "checked" and wl.n_d > 1:
                d["avg"] = [buf[(p, gi, "avg")][:g.master.numel()] for gi, g in enumerate(d["groups"])]
        # the oracle's side: the last pipeline, element by element (or a chunk sample if the host
        # cannot hold the oracle's copy of every element's state)
        main = self.side[pipelines[-1]]
        self.last_state = {"cur": 0}
        checks = []
        bounds = []
        for spec, (psi, off, n) in zip(wl.groups, shards):
            ends = np.cumsum(np.array(spec.numels, dtype=np.int64)) - off
            bounds.append((n, [int(x) for x in ends if 0 < x < n] + [1 << 32]))
        plan, msg = plan_ranges(bounds, wl.dynamic_loss_scale or max_grad_norm > 0, min(16, cpu_workers()),
                                host_bytes_available())
        if msg:
            print(f"  {msg}", flush=True)
        for gi, (spec, (psi, off, n)) in enumerate(zip(wl.groups, shards)):
            g = main["groups"][gi]
            ranges = plan[gi]

            def state(g=g):
                return zdp.current_state(g, self.last_state)
            chk = GroupCheck(n, self.reps[gi], g.flat_param, off, ranges, chunk_for(wl.n_d), self.odt,
                             ORACLE_DT[wl.param_dt], wl.lr, wl.beta1, wl.beta2, wl.eps, spec.weight_decay)
            chk.state = state
            checks.append(chk)
            print(f"  group {gi}: {chk.elements()} of {n} elements checked element by element", flush=True)
        self.check = FullCheck(checks, oracle.Policy(skip_on_overflow=wl.dynamic_loss_scale,
                                                     max_grad_norm=max_grad_norm), wl.loss_scale)
        self.check.load_initial()
        self.bar = Bar(lr=wl.lr, beta1=wl.beta1)

    def draw_grads(self, call):
        wl = self.wl
        scale = self.check.ostate.loss_scale  # the scale in force (asserted equal on every side)
        for gi, reps in enumerate(self.reps):
            for r, t in enumerate(reps):
                fill_normal_(t, 1e-3, derive_seed(wl.key, gi, "grad", call, r), scale=scale)
        if wl.inf_at is not None and wl.inf_at[0] == call:
            _, rep, where = wl.inf_at
            pos = self.reps[0][0].numel() // 2 if where == "mid" else int(where)
            self.reps[0][rep][pos] = float("inf")
            print(f"  call {call}: +inf in copy {rep} at {pos}", flush=True)

    def gpu_step(self, p):
        d = self.side[p]
        groups, ws, st, pol = d["groups"], d["ws"], d["state"], d["policy"]
        if pol is None or p == "optimistic":
            zdp.adam_step(groups, ws, st, pol)
            return
        if self.wl.n_d == 1:
            zdp.grad_norm_overflow([g.replicas[0] for g in groups], ws, len(groups), st, pol)
            zdp.adam_step(groups, ws, st, pol)
            return
        for gi, g in enumerate(groups):
            zdp.reduce_grad_segment(g.replicas, d["avg"][gi], ws, gi, st)
        zdp.grad_norm_overflow(None, ws, len(groups), st, pol)
        saved = [g.replicas for g in groups]
        for gi, g in enumerate(groups):
            g.replicas, g.avg = None, d["avg"][gi]
        try:
            zdp.adam_step(groups, ws, st, pol)
        finally:
            for gi, g in enumerate(groups):
                g.replicas, g.avg = saved[gi], None

    def _device_equal(self, tag, a, b, step=1 << 28):
        """Bitwise equality of two device tensors, compared in pieces."""
        iv = torch.int32 if a.dtype == torch.float32 else torch.int16
        av, bv = a.view(iv), b.view(iv)
        for s in range(0, av.numel(), step):
            x, y = av[s:s + step], bv[s:s + step]
            if not torch.equal(x, y):
                i = int(torch.nonzero(x != y)[0])
                raise AssertionError(f"{tag}: pipelines differ at element {s + i}: {int(x[i])} vs {int(y[i])}")

    def run(self, steps=None, grid_limits=None):
        """Step ``steps`` times; ``grid_limits`` maps a call to a block cap
        (zdp.set_grid_limit) that holds for that call's launches only."""
        wl = self.wl
        steps = wl.steps if steps is None else steps
        main = self.pipelines[-1]
        for call in range(1, steps + 1):
            t0 = time.perf_counter()
            self.draw_grads(call)
            limit = (grid_limits or {}).get(call, 0)
            if limit:
                print(f"  call {call}: at most {limit} blocks per launch", flush=True)
            zdp.set_grid_limit(limit)
            try:
                for p in self.pipelines:
                    self.gpu_step(p)
                torch.cuda.synchronize()
            finally:
                zdp.set_grid_limit(0)
            states = {p: zdp.read_state(self.side[p]["state"]) for p in self.pipelines}
            s = states[main]
            tag = f"{wl.key} call {call}"
            for p in self.pipelines[:-1]:
                o = states[p]
                for k in ("step", "skipped", "overflow", "loss_scale", "good_steps", "clip_coef"):
                    assert o[k] == s[k], (tag, p, k, o[k], s[k])
                for gi, (ga, gb) in enumerate(zip(self.side[p]["groups"], self.side[main]["groups"])):
                    for name, x, y in zip(("master", "exp_avg", "exp_avg_sq"), zdp.current_state(ga, o),
                                          zdp.current_state(gb, s)):
                        self._device_equal(f"{tag} group {gi} {name} ({p} vs {main})", x, y)
                    n, off = ga.master.numel(), ga.param_offset
                    self._device_equal(f"{tag} group {gi} param ({p} vs {main})", ga.flat_param[off:off + n],
                                       gb.flat_param[off:off + n])
            t1 = time.perf_counter()
            self.last_state = s
            ost = self.check.step_and_compare(tag, self.bar, s)
            assert s["step"] == ost.step, tag
            assert s["skipped"] == ost.skipped, tag
            assert s["overflow"] == ost.overflow, tag
            assert s["loss_scale"] == np.float32(ost.loss_scale), tag
            assert s["good_steps"] == ost.good_steps, tag
            assert s["redo"] == 0, tag
            if np.isfinite(ost.norm2):
                assert abs(s["grad_norm_sq"] - ost.norm2) <= 1e-10 * ost.norm2, (tag, s["grad_norm_sq"], ost.norm2)
                assert s["grad_norm"] == pytest.approx(np.sqrt(ost.norm2), rel=1e-6)
            else:
                assert not np.isfinite(s["grad_norm_sq"]), tag
            print(f"  {tag}: ok (step {s['step']}, norm {s['grad_norm']:.6g}, scale {s['loss_scale']}, "
                  f"skipped {s['skipped']}, clip {s['clip_coef']:.6g}, exact {self.bar.exact}; device "
                  f"{t1 - t0:.1f} s, oracle {time.perf_counter() - t1:.1f} s)", flush=True)
        for gi, (outs, before) in enumerate(self.outside):
            if before is not None:
                flat = self.side[main]["groups"][gi].flat_param
                assert_u16_equal(_u16(flat[torch.from_numpy(outs).to(DEV)]), before,
                                 wl.key + " flat vector outside the shard")
        return self.check.ostate

    def close(self):
        """Shut the oracle's pool and drop every reference to device memory
        (the state functions refer back to the run)."""
        self.check.close()
        for g in self.check.groups:
            g.state = g.reps = g.flat = None
            g.host.clear()
        self.check.groups = []
        self.side = self.reps = self.outside = None


def _done(run):
    run.close()
    del run
    gc.collect()
    _free()


@pytest.mark.parametrize("key", ["tiny", "tiny_literal"])
def test_tiny_every_element(key):
    print(f"[workload] {key}", flush=True)
    st = Run(key, full=True).run()
    assert st.step == 3
    _free()


@pytest.mark.timeout(900)
def test_gpt2_1_5b_every_element():
    print("[workload] gpt2_1.5b", flush=True)
    run = FullRun("gpt2_1.5b")
    st = run.run()
    assert st.step == 10 and st.loss_scale == 65536.0
    _done(run)


@pytest.mark.timeout(900)
def test_7_5b_nd64_every_element():
    print("[workload] 7.5b_nd64", flush=True)
    run = FullRun("7.5b_nd64")
    st = run.run()
    assert st.step == 10
    _done(run)


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


@pytest.mark.timeout(1200)
def test_13b_nd8_overflow_skip_every_element():
    # both dynamic-scale pipelines on the same copies: ten calls, the fourth overflows:
    # nine applied steps, the scale halved once
    print("[workload] 13b_nd8 (checked and optimistic)", flush=True)
    run = FullRun("13b_nd8", pipelines=("checked", "optimistic"))
    st = run.run()
    assert st.step == 9 and st.loss_scale == 32768.0
    _done(run)


@pytest.mark.timeout(900)
def test_gpt2_1_5b_clipping_every_element():
    # clipping on the single-copy shard (the norm is about 39, the threshold 1): the checked pipeline
    # scans the copy first (the wide-load scan loops its capped grid over 380,277 tiles), then updates
    print("[workload] gpt2_1.5b clipping", flush=True)
    run = FullRun("gpt2_1.5b", pipelines=("checked",), max_grad_norm=1.0)
    st = run.run(steps=3)
    assert st.step == 3 and st.clip < 1.0
    _done(run)


@pytest.mark.timeout(1200)
def test_13b_nd8_clipping_every_element():
    # clipping at full size (the norm is about 14, the threshold 10: every applied call clips), five
    # calls with the overflow on the fourth, both dynamic-scale pipelines on the same copies; the
    # optimistic pipeline's second pass loops over the shard's 396,729 tiles with its capped grid
    print("[workload] 13b_nd8 clipping (checked and optimistic)", flush=True)
    run = FullRun("13b_nd8", pipelines=("checked", "optimistic"), max_grad_norm=10.0)
    st = run.run(steps=5)
    assert st.step == 4 and st.loss_scale == 32768.0 and st.clip < 1.0
    _done(run)


@pytest.mark.timeout(1200)
def test_llama3_8b_adamw_two_groups_every_element():
    # 8,030,261,248 elements, one block per 4096-element tile (1,960,448 blocks for the matrix group);
    # on the last two calls a cap of 2^20 blocks makes 911,872 blocks loop over a second tile, past
    # element 2^32. The oracle's copy of the state takes 112 GB of host memory.
    print("[workload] llama3_8b", flush=True)
    run = FullRun("llama3_8b")
    st = run.run(grid_limits={4: 1 << 20, 5: 1 << 20})
    assert st.step == 5
    _done(run)
