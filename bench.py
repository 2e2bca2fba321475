#!/usr/bin/env python3
"""Throughput of the ZeRO-DP partitioned optimizer step on one MI355X.

One step is the whole path for one rank's shard: average the N_d gradient
copies, overflow flag and gradient norm, fp32 Adam/AdamW on master / m / v,
16-bit writeback into the flat parameter vector, step bookkeeping. Inputs are
seeded synthetic tensors already resident in HBM when timing starts.

Prints one JSON line: params updated per second (value), with the achieved
HBM bandwidth of the step against the bytes model (2*N_d + 26 bytes per
parameter: the 16-bit copies read once, fp32 master/m/v read and written, the
16-bit parameter written) and against MI355X's 8 TB/s, and the CPU oracle
timed on a bounded sample of the same workload on this host.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama3_8b]

The default workload is the largest shard one GPU holds: LLaMA-3 8B at
N_d = 1 (AdamW over two groups, 8,030,261,248 parameters, 224.85 GB per step).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
DEFAULT_WORKLOAD = "llama3_8b"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "zero_dp_partitioned_amd", "csrc")
KERNEL_SRCS = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "zero_dp_internal.h")]


def bytes_per_param(n_d):
    """Algorithmic HBM bytes of one step per parameter of the shard."""
    return 2 * n_d + 12 + 12 + 2


def kernel_source_hash():
    """Hash of the kernels' code and of the header that fixes their launch
    shapes (tile sizes, grid caps): comments and whitespace are removed first,
    so that only a change to the code invalidates recorded counters."""
    import re
    src = "\n".join(open(f).read() for f in KERNEL_SRCS)
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=25)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--cpu-sample", type=int, default=1 << 29,
                   help="elements of the shard the CPU oracle steps once on every thread of the CPU "
                        "share (0: skip)")
    p.add_argument("--cpu-single", type=int, default=1 << 28,
                   help="elements of the shard the CPU oracle steps once on one thread")
    p.add_argument("--pipeline", choices=["checked", "optimistic"], default="optimistic",
                   help="dynamic-loss-scale workloads: an update into a second state set committed "
                        "afterwards (optimistic, one pass) or the verdict before the update (checked, "
                        "an extra pass over an fp32 average: 2*N_d + 34 bytes per parameter)")
    p.add_argument("--max-grad-norm", type=float, default=0.0,
                   help="clip the gradient to this global norm (0: off); selects the checked pipeline, or "
                        "with --pipeline optimistic on a dynamic-scale workload the optimistic one")
    p.add_argument("--arena", choices=["whole", "sized"], default="whole",
                   help="regions placement: the arena is all free memory but 4 GiB (whole) or ends "
                        "at the last planned buffer (sized)")
    p.add_argument("--placement", choices=["regions", "packed"], default="regions",
                   help="buffers carved from one arena spread over HBM's 96 GiB regions (regions), or "
                        "one allocation each in order (packed)")
    p.add_argument("--regions", type=int, default=0,
                   help="regions placement: spread the buffers over exactly this many 96 GiB regions "
                        "(0: the fewest, at least two, that hold them)")
    p.add_argument("--quiet", action="store_true")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES bytes --steps times (to calibrate "
                        "HBM byte counters against a kernel of known traffic)")
    return p.parse_args()


def copy_calibration(args):
    """A plain copy of known size: BYTES read and BYTES written per launch."""
    import torch
    src = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": args.copy_calibration, "launches": args.steps}), flush=True)


COPY_BYTES = 2 << 30


def copy_ceiling(setup, reps=10):
    """The bandwidth (bytes read + bytes written per second) of the library's
    two-stream copy probe in the step's own arena: src0 -> dst0 and src1 ->
    dst1 from unused ranges, each stream from one HBM region into the other
    where the arena has two, so that each region serves one read and one
    write stream as in a step of half reads, half writes. None if the arena
    has no room."""
    import torch

    import zero_dp_partitioned_amd as zdp
    if setup.arena is None:
        return None
    A = zdp.ARENA_ALIGN
    spans = []   # (offset, region) of COPY_BYTES-sized pieces of the free ranges
    for off, nb in setup.free:
        o = (off + A - 1) // A * A
        while o + COPY_BYTES <= off + nb:
            spans.append((o, o // zdp.HBM_REGION_BYTES))
            o += COPY_BYTES
    if len(spans) < 4:
        return None
    by = {}
    for sp in spans:
        by.setdefault(sp[1], []).append(sp)
    regs = sorted(by, key=lambda r: -len(by[r]))
    if len(regs) >= 2 and len(by[regs[0]]) >= 2 and len(by[regs[1]]) >= 2:
        (s0, d1), (d0, s1) = by[regs[0]][:2], by[regs[1]][:2]
    else:
        s0, s1, d0, d1 = spans[:4]
    view = [zdp.arena_view(setup.arena, sp[0], COPY_BYTES, torch.uint8) for sp in (s0, s1, d0, d1)]
    zdp.copy_probe(*view)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        zdp.copy_probe(*view)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    moved = 4 * COPY_BYTES
    return {"gbps": moved / (ms / 1e3) / 1e9, "bytes": moved,
            "what": f"zero_copy_probe: two {COPY_BYTES >> 30} GiB streams in unused ranges of the step's arena "
                    f"(region {s0[1]} -> {d0[1]} and {s1[1]} -> {d1[1]}), bytes read + written per second, mean "
                    f"of {reps} launches"}


def log(args, *a):
    if not args.quiet:
        print("[bench]", *a, file=sys.stderr, flush=True)


class Setup:
    """Device buffers of one workload. Per group: fp32 master (seeded), m and v
    (zero), the N_d 16-bit gradient copies of the shard, and the group's whole
    16-bit flat parameter vector (plus a second state set for the optimistic
    pipeline, or an fp32 average for the checked one), placed by
    zero_dp_partitioned_amd.layout: "regions" (one arena over all free HBM,
    buffers spread over its 96 GiB regions; the default) or "packed" (one
    allocation per buffer)."""

    def __init__(self, wl, dev, optimistic=False, placement="regions", whole=True, max_grad_norm=0.0,
                 n_regions=0):
        import zero_dp_partitioned_amd as zdp
        from zero_dp_partitioned_amd import layout
        from workloads import derive_seed, fill_normal_, torch_dtype

        self.wl = wl
        self.groups = []
        self.shard = 0
        self.optimistic = optimistic and wl.dynamic_loss_scale
        needs_norm = wl.dynamic_loss_scale or max_grad_norm > 0
        pipeline = ("optimistic" if self.optimistic else "checked") if needs_norm else "fused"
        self.pipeline = pipeline
        shards = []
        for spec in wl.groups:
            psi = sum(spec.numels)
            segs, _ = zdp.partition(psi, wl.n_d)
            shards.append((psi, *segs[wl.rank]))
        table = placement == "regions" and wl.n_d <= layout.INLINE_COPIES
        # with one copy the checked pipeline scans it instead of writing an average
        spec_pipeline = "fused" if pipeline == "checked" and wl.n_d == 1 else pipeline
        specs = layout.step_specs(shards, wl.n_d, torch_dtype(wl.grad_dt), torch_dtype(wl.param_dt),
                                  spec_pipeline, table)
        buf, self.placement = layout.allocate(specs, dev, placement, whole=whole, n_regions=n_regions)
        self.arena, self.free = buf.get("arena"), buf.get("free", [])   # for the copy ceiling
        for gi, (spec, (psi, off, n)) in enumerate(zip(wl.groups, shards)):
            master = buf[(gi, "master")][:n]
            fill_normal_(master, 0.02, derive_seed(wl.key, gi, "master"))
            flat = buf[(gi, "flat")][:psi]
            fill_normal_(flat, 0.02, derive_seed(wl.key, gi, "flat"))
            flat[off:off + n].copy_(master)
            reps = layout.copies_of(buf, gi, wl.n_d, n)
            for r, t in enumerate(reps):
                fill_normal_(t, 1e-3, derive_seed(wl.key, gi, "grad", 0, r), scale=wl.loss_scale)
            alt = {}
            if self.optimistic:
                alt = {name: buf[(gi, name)][:n] for name in ("master_alt", "exp_avg_alt", "exp_avg_sq_alt")}
            m, v = buf[(gi, "exp_avg")][:n].zero_(), buf[(gi, "exp_avg_sq")][:n].zero_()
            self.groups.append(zdp.Group(
                master=master, exp_avg=m, exp_avg_sq=v,
                replicas=reps, flat_param=flat, param_offset=off, lr=wl.lr, beta1=wl.beta1,
                beta2=wl.beta2, eps=wl.eps, weight_decay=spec.weight_decay, **alt))
            self.shard += n
        self.ws = zdp.new_workspace(len(self.groups))
        self.state = zdp.new_state(wl.loss_scale)
        self.policy = (zdp.policy(wl.dynamic_loss_scale, optimistic=self.optimistic, max_grad_norm=max_grad_norm)
                       if needs_norm else None)
        if spec_pipeline == "checked":
            self.avg = [buf[(gi, "avg")][:g.master.numel()] for gi, g in enumerate(self.groups)]

    def step(self):
        import zero_dp_partitioned_amd as zdp
        if self.policy is None or self.optimistic:
            zdp.adam_step(self.groups, self.ws, self.state, self.policy)
            return
        # checked pipeline (dynamic scale or clipping): norm / overflow verdict, then the update
        if self.wl.n_d == 1:
            # a single copy: scan it for the norm, then the update reads it again
            zdp.grad_norm_overflow([g.replicas[0] for g in self.groups], self.ws, len(self.groups), self.state,
                                   self.policy)
            zdp.adam_step(self.groups, self.ws, self.state, self.policy)
            return
        for gi, g in enumerate(self.groups):
            zdp.reduce_grad_segment(g.replicas, self.avg[gi], self.ws, gi, self.state)
        zdp.grad_norm_overflow(None, self.ws, len(self.groups), self.state, self.policy)
        reps = [g.replicas for g in self.groups]
        for gi, g in enumerate(self.groups):
            g.replicas, g.avg = None, self.avg[gi]
        try:
            zdp.adam_step(self.groups, self.ws, self.state, self.policy)
        finally:
            for gi, g in enumerate(self.groups):
                g.replicas, g.avg = reps[gi], None


# what one step launches, per pipeline (the events bracket all of it)
STEP_KERNELS = {
    "fused": "adam_kernel (average, partials, Adam, writeback) + fold + 1-block finalize",
    "checked": "reduce_kernel or scan_kernel (average / norm partials) + fold + finalize, then adam_kernel "
               "+ commit",
    "optimistic": "adam_kernel (into the second state set) + fold + finalize + restore (+ second pass when "
                  "clipping)",
}

CPU_CHUNK = 1 << 24


def cgroup_cpus():
    """CPUs this process may use by its cgroup's CPU quota (cgroup v2
    cpu.max, else v1 cfs_quota_us / cfs_period_us), or None when unlimited."""
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if quota != "max":
            return max(1, int(int(quota) // int(period)))
        return None
    except (OSError, ValueError):
        pass
    try:
        quota = int(open("/sys/fs/cgroup/cpu/cpu.cfs_quota_us").read())
        period = int(open("/sys/fs/cgroup/cpu/cpu.cfs_period_us").read())
        return max(1, quota // period) if quota > 0 and period > 0 else None
    except (OSError, ValueError):
        return None


def cpu_share():
    """The host CPUs the CPU baseline runs on: every CPU of this process's
    affinity mask, capped by the cgroup CPU quota when one is set and by an
    explicit OMP_NUM_THREADS. Returns (threads, description of the counts)."""
    affinity = len(os.sched_getaffinity(0))
    quota = cgroup_cpus()
    env = os.environ.get("OMP_NUM_THREADS", "")
    omp = int(env) if env.isdigit() and int(env) > 0 else None
    threads = min(x for x in (affinity, quota, omp) if x is not None)
    counts = {"affinity_cpus": affinity, "cgroup_quota_cpus": quota, "omp_num_threads": omp,
              "os_cpu_count": os.cpu_count()}
    return max(1, threads), counts


def cpu_baseline(setup, sample, single, args):
    """The CPU oracle as it stands, one step over the first `sample` elements
    of the first group's shard in fixed 2^24-element chunks (each chunk one
    oracle call) on a thread pool of the host's CPU share, and one step over
    the first `single` elements on one thread."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import oracle  # CPU oracle: used here only for the reported baseline

    wl = setup.wl
    g = setup.groups[0]
    k = min(sample, g.master.numel())
    k1 = min(single, k)
    odt = oracle.F16 if wl.grad_dt == "f16" else oracle.BF16
    reps = [r[:k].cpu().view(torch.int16).numpy().view(np.uint16) for r in g.replicas]
    master = g.master[:k].cpu().numpy()
    m, v, param = np.zeros(k, np.float32), np.zeros(k, np.float32), np.zeros(k, np.uint16)
    policy = oracle.Policy(skip_on_overflow=wl.dynamic_loss_scale)
    oracle.lib()

    def one(chunk):
        s, e = chunk
        og = oracle.Group(replicas=[r[s:e] for r in reps], grad_dt=odt, master=master[s:e], m=m[s:e],
                          v=v[s:e], param=param[s:e], param_dt=odt, lr=wl.lr, beta1=wl.beta1,
                          beta2=wl.beta2, eps=wl.eps, weight_decay=wl.groups[0].weight_decay)
        oracle.step([og], policy, oracle.State(loss_scale=wl.loss_scale))

    chunks = [(s, min(k, s + CPU_CHUNK)) for s in range(0, k, CPU_CHUNK)]
    threads, counts = cpu_share()
    log(args, f"cpu oracle: one step over {k} elements, {len(chunks)} chunks on {threads} threads "
              f"({counts}); one thread over {k1}")
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, chunks))
    dt = time.perf_counter() - t0
    t0 = time.perf_counter()
    one((0, k1))
    dt1 = time.perf_counter() - t0
    one_thread = k1 / dt1
    return {"value": k / dt, "unit": "params/s", "cores": threads, "kind": "oracle",
            "single_thread_value": one_thread, **counts,
            "sample": f"first {k} elements of the {wl.key} shard (N_d={wl.n_d}, group 0), one step, scalar C "
                      f"oracle over {len(chunks)} chunks of {CPU_CHUNK} elements on {threads} threads "
                      f"({dt:.1f} s); one thread over the first {k1} elements: {one_thread:.3g} params/s "
                      f"({dt1:.1f} s)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the partitioned step runs one rank on one GPU; --gpus {args.gpus} is not "
              f"supported (no collectives, no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    import torch

    import zero_dp_partitioned_amd as zdp
    from workloads import WORKLOADS

    zdp.load()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = WORKLOADS[args.workload]
    log(args, f"workload {wl.key}: {wl.title}")
    setup = Setup(wl, dev, optimistic=args.pipeline == "optimistic", placement=args.placement,
                  whole=args.arena == "whole", max_grad_norm=args.max_grad_norm, n_regions=args.regions)
    S = setup.shard
    bpp = bytes_per_param(wl.n_d)
    log(args, f"shard {S} params, {len(setup.groups)} group(s), {bpp} B/param, "
              f"{S * bpp / 1e9:.2f} GB per step")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        setup.step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        starts[k].record(stream)
        setup.step()
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    ev_mean = sum(ev_ms) / len(ev_ms)
    ms_per_step = wall * 1e3 / args.steps
    st = zdp.read_state(setup.state)
    log(args, f"steps {args.steps}: wall {ms_per_step:.3f} ms/step, events mean {ev_mean:.3f} "
              f"median {ev_ms[len(ev_ms) // 2]:.3f} min {ev_ms[0]:.3f} ms; state step {st['step']} "
              f"norm {st['grad_norm']:.6g} scale {st['loss_scale']}")
    value = S / (ms_per_step / 1e3)
    algo_bytes = S * bpp
    achieved = algo_bytes / (ev_mean / 1e3) / 1e9
    pipeline = setup.pipeline
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        key = wl.key if pipeline == "fused" else f"{wl.key}:{pipeline}"
        rec = json.load(open(TRAFFIC_FILE)).get(key)
        if rec and rec.get("kernel_source") == kernel_source_hash():
            traffic = rec.get("bytes_per_step")
    ceiling = copy_ceiling(setup)
    if ceiling:
        ceiling["achieved_frac"] = achieved / ceiling["gbps"]
        log(args, f"copy ceiling {ceiling['gbps']:.0f} GB/s; the step reaches {ceiling['achieved_frac']:.3f} of it")
    cpu = None
    if args.cpu_sample > 0:
        cpu = cpu_baseline(setup, args.cpu_sample, args.cpu_single, args)
    out = {
        "metric": "params updated/sec and achieved HBM GB/s (% peak) per sharded Adam step",
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.key, "shard_params": S, "n_d": wl.n_d, "rank": wl.rank,
                   "groups": len(setup.groups), "grad_dtype": wl.grad_dt, "param_dtype": wl.param_dt,
                   "loss_scale": wl.loss_scale, "dynamic_loss_scale": wl.dynamic_loss_scale,
                   "pipeline": pipeline, "max_grad_norm": args.max_grad_norm,
                   "bytes_per_param": bpp, **setup.placement},
        "gbps": achieved,
        "pct_peak": 100.0 * achieved / PEAK_HBM_GBPS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "kernel": STEP_KERNELS[pipeline] + ", HIP events around each step",
                     "kernel_ms": ev_mean, "algorithmic_bytes": algo_bytes},
        "cpu_baseline": cpu,
        "copy_ceiling": ceiling,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
