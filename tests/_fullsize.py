"""Element-by-element verification of full-size shards against the oracle.

Each coordinate's update depends only on that coordinate's gradient copies and
state, plus three whole-shard scalars (the overflow flag, the gradient norm and
the step count) [ZeRO reading notes, second part §3]. So a shard of billions of
elements is checked exactly, chunk by chunk, on the host:

1. pass A (only when the verdict needs the whole shard first: a dynamic loss
   scale or clipping): every chunk's gradient copies are staged device -> host,
   averaged by the oracle (kept), and their fp64 sum of squares and flag taken;
   the chunk sums are added in chunk order;
2. pass B: every chunk is stepped by the oracle from the state it holds for
   that chunk (its own copy, advanced call by call since the inputs were
   drawn) with the whole shard's norm and flag, and compared with the device's
   result for the same elements, staged device -> host.

Without a verdict (static scale, no clipping) the two passes are one: each
chunk's update does not depend on the other chunks, and the norm and flag are
still added over every chunk. The oracle's inputs are the harness's seeded
draws and the initial master and parameters, copied from the device where the
harness drew them; nothing the library computes is ever fed to the oracle.

Copies go through a pool of pinned host buffers on a side stream, so they
overlap the oracle's work on a thread pool of the host's CPU share.
"""
import os
import queue
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

STAGE_BYTES = 64 << 20          # bytes of one staged chunk (device -> host)


def chunk_for(n_d):
    """Elements per staged chunk for a group with n_d gradient copies: its
    copies (2 * n_d bytes per element) and its state and parameter (14 bytes)
    fit one staging buffer; a multiple of 4096."""
    c = STAGE_BYTES // (2 * n_d + 14) // 4096 * 4096
    return max(4096, c)


SAMPLE_CHUNK = 1 << 24         # elements per chunk of the fallback sample (host memory short)
SAMPLE_EVERY = 64              # the sample keeps every 64th such chunk


def host_bytes_available():
    """Host memory this process can still take: MemAvailable, capped by the
    room under the cgroup's memory limit when one is set (None if neither
    can be read)."""
    avail = None
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    avail = int(line.split()[1]) * 1024
    except OSError:
        pass
    for lim, cur in (("/sys/fs/cgroup/memory.max", "/sys/fs/cgroup/memory.current"),
                     ("/sys/fs/cgroup/memory/memory.limit_in_bytes", "/sys/fs/cgroup/memory/memory.usage_in_bytes")):
        try:
            with open(lim) as f:
                limit = f.read().strip()
            with open(cur) as f:
                used = int(f.read().strip())
        except (OSError, ValueError):
            continue
        if limit.isdigit():
            room = int(limit) - used
            avail = room if avail is None else min(avail, room)
        break
    return avail


def oracle_bytes(n, verdict_first):
    """Host bytes of the oracle's copy of n checked elements: fp32 master, m
    and v and the 16-bit parameters, plus the fp32 averages pass A keeps when
    the verdict comes first."""
    return n * (12 + 2 + (4 if verdict_first else 0))


def sample_ranges(n, boundaries, chunk=SAMPLE_CHUNK, every=SAMPLE_EVERY):
    """The fallback sample of a shard of n elements, as sorted disjoint
    [(start, end)]: every `every`-th chunk of `chunk` elements, the first and
    the last chunk, and every chunk holding one of `boundaries` (tensor or
    group boundaries, element offsets into the shard)."""
    if n <= 0:
        return []
    last = (n - 1) // chunk
    ids = set(range(0, last + 1, every)) | {0, last}
    ids |= {b // chunk for b in boundaries if 0 <= b < n}
    out = []
    for i in sorted(ids):
        s, e = i * chunk, min(n, (i + 1) * chunk)
        if out and out[-1][1] == s:
            out[-1] = (out[-1][0], e)
        else:
            out.append((s, e))
    return out


def plan_ranges(shards, verdict_first, workers, available):
    """What the oracle checks element by element in each shard: all of it,
    or, when its copy of the state would not fit in 80 % of the host memory
    still available (staging buffers included), the fallback sample.
    `shards` is [(n, boundaries)]; returns ([ranges per shard], message)."""
    need = sum(oracle_bytes(n, verdict_first) for n, _ in shards) + (workers + 4) * STAGE_BYTES
    full = [[(0, n)] if n else [] for n, _ in shards]
    if available is None or need <= 0.8 * available:
        return full, None
    ranges = [sample_ranges(n, b) for n, b in shards]
    kept = sum(e - s for r in ranges for s, e in r)
    total = sum(n for n, _ in shards)
    msg = (f"host memory short: every element needs {need / 2**30:.1f} GiB of host memory and "
           f"{available / 2**30:.1f} GiB is available, so only a chunk sample is compared element by "
           f"element ({kept} of {total} elements: every {SAMPLE_EVERY}th chunk of {SAMPLE_CHUNK}, the first "
           f"and last chunks and those holding tensor or group boundaries); norm and flag still cover "
           f"every element")
    return ranges, msg


def cpu_workers():
    """Threads for the oracle: the CPU share of this process (affinity mask,
    capped by OMP_NUM_THREADS when set)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


class Staged:
    """One pinned buffer holding copies of device tensors."""

    def __init__(self, stager, buf, layout, event):
        self.stager, self.buf, self.layout, self.event = stager, buf, layout, event

    def arrays(self):
        """numpy views of the staged tensors (waits for the copies)."""
        self.event.synchronize()
        host = self.buf.numpy()
        out = []
        for off, nb, dt in self.layout:
            a = host[off:off + nb]
            out.append(a.view(np.float32) if dt == torch.float32 else a.view(np.uint16))
        return out

    def release(self):
        self.stager.free.put(self.buf)


class Stager:
    """Device -> host copies through `count` pinned buffers of `nbytes`."""

    def __init__(self, count, nbytes):
        self.nbytes = nbytes
        self.free = queue.Queue()
        for _ in range(count):
            self.free.put(torch.empty(nbytes, dtype=torch.uint8, pin_memory=True))
        self.stream = torch.cuda.Stream()

    def fetch(self, tensors):
        """Enqueue copies of 1-D contiguous device tensors into a free buffer
        (waits for one); the work on the current stream comes first."""
        buf = self.free.get()
        layout, off = [], 0
        self.stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(self.stream):
            for t in tensors:
                nb = t.numel() * t.element_size()
                if off + nb > self.nbytes:
                    self.free.put(buf)
                    raise ValueError("staged tensors exceed the buffer")
                buf[off:off + nb].copy_(t.reshape(-1).view(torch.uint8), non_blocking=True)
                layout.append((off, nb, t.dtype))
                off += (nb + 255) // 256 * 256
            ev = torch.cuda.Event()
            ev.record(self.stream)
        return Staged(self, buf, layout, ev)


class HostStager:
    """The same interface over host tensors: copies at once. Lets the
    harness's logic run on the CPU (tests/test_fullsize_harness.py)."""

    def __init__(self):
        self.free = queue.Queue()

    def fetch(self, tensors):
        arrs = [t.reshape(-1).clone() for t in tensors]
        return _HostStaged(arrs)


class _HostStaged:
    def __init__(self, arrs):
        self.arrs = arrs

    def arrays(self):
        return [a.numpy() if a.dtype == torch.float32 else a.view(torch.int16).numpy().view(np.uint16)
                for a in self.arrs]

    def release(self):
        pass


def _same_state(a, b):
    """Oracle states equal in their step bookkeeping (NaN norms equal)."""
    return all(x == y or (x != x and y != y) for x, y in zip(vars(a).values(), vars(b).values()))


class GroupCheck:
    """The oracle's copy of one parameter group's shard over `ranges`
    ([(start, end)] in shard elements, sorted and disjoint), split into chunks
    of at most `chunk` elements, and the group's device tensors: `reps` (the N_d
    gradient copies), `flat` and `offset` (the 16-bit parameter vector and the
    shard's offset in it), and a function `state()` giving the (master, m, v)
    tensors that hold the current state on the device."""

    def __init__(self, n, reps, flat, offset, ranges, chunk, odt, pdt, lr, beta1, beta2, eps, weight_decay):
        self.n, self.reps, self.flat, self.offset = n, reps, flat, offset
        self.odt, self.pdt = odt, pdt
        self.hyper = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay)
        self.checked = []      # chunks compared element by element: [s, e)
        for s0, e0 in ranges:
            for s in range(s0, e0, chunk):
                self.checked.append((s, min(e0, s + chunk)))
        self.norm_only = []    # the rest of the shard: norm and flag only
        at = 0
        for s, e in self.checked + [(n, n)]:
            for u in range(at, s, chunk):
                self.norm_only.append((u, min(s, u + chunk)))
            at = max(at, e)
        self.host = {}         # (s, e) -> [master, m, v, param] of the oracle

    def elements(self):
        return sum(e - s for s, e in self.checked)


class FullCheck:
    """Element-by-element comparison of one device run (its groups as
    GroupCheck) with the oracle, call after call."""

    def __init__(self, groups, policy, loss_scale, workers=None, stager=None):
        self.groups = groups
        self.policy = policy
        self.ostate = oracle.State(loss_scale=loss_scale)
        self.workers = workers or min(16, cpu_workers())
        self.stager = stager or Stager(self.workers + 4, STAGE_BYTES)
        self.pool = ThreadPoolExecutor(self.workers)
        self.verdict_first = bool(policy.skip_on_overflow) or policy.max_grad_norm > 0

    def close(self):
        self.pool.shutdown(wait=True)

    # ------------------------------------------------------------------
    def _run(self, items, fetch, work):
        """For each item: stage fetch(item) and run work(item, arrays) on the
        pool; results in item order. The first failure stops the submission."""
        futs = []
        for it in items:
            if any(f.done() and f.exception() for f in futs[-self.workers:]):
                break
            st = self.stager.fetch(fetch(it))

            def job(it=it, st=st):
                try:
                    return work(it, st.arrays())
                finally:
                    st.release()
            futs.append(self.pool.submit(job))
        return [f.result() for f in futs]

    def load_initial(self):
        """The oracle's starting state for the checked chunks: the initial
        master and parameter slice as the harness drew them on the device,
        m = v = 0."""
        items = [(g, s, e) for g in self.groups for s, e in g.checked]

        def fetch(it):
            g, s, e = it
            return [g.state()[0][s:e], g.flat[g.offset + s:g.offset + e]]

        def work(it, arrs):
            g, s, e = it
            g.host[(s, e)] = [arrs[0].copy(), np.zeros(e - s, np.float32), np.zeros(e - s, np.float32),
                              arrs[1].copy()]
        self._run(items, fetch, work)

    # ------------------------------------------------------------------
    def _ogroup(self, g, s, e):
        master, m, v, param = g.host[(s, e)]
        return oracle.Group(replicas=None, grad_dt=g.odt, master=master, m=m, v=v, param=param,
                            param_dt=g.pdt, **g.hyper)

    def step_and_compare(self, tag, bar, gpu_state):
        """Advance the oracle by one call and compare every checked element
        with the device (whose state dict is `gpu_state`, read after the
        call). Returns the oracle's state."""
        pre = self.ostate
        inv = oracle.inv_scale_of(pre.loss_scale)
        odt_of = {id(g): g.odt for g in self.groups}
        avgs = {}
        sums = []   # (n2, flag) in (group, chunk) order over the whole shard

        def avg_items(g, chunks, keep):
            return [(g, s, e, keep) for s, e in chunks]

        def fetch_grads(it):
            g, s, e, _ = it
            return [r[s:e] for r in g.reps]

        def work_avg(it, arrs):
            g, s, e, keep = it
            a = oracle.average(arrs, odt_of[id(g)])
            n2, f = oracle.norm_overflow(a, inv)
            if keep:
                avgs[(id(g), s, e)] = a
            return s, n2, f

        def compare(g, s, e, got, st_after):
            master, m, v, param = g.host[(s, e)]
            where = f"{tag} elements [{s}, {e})"
            bar.state32(got[0], master, f"{where} master", "master")
            bar.state32(got[1], m, f"{where} exp_avg", "m")
            bar.state32(got[2], v, f"{where} exp_avg_sq", "v")
            bar.param16(got[3], param, f"{where} param")

        def fetch_state(it):
            g, s, e = it[:3]
            master, m, v = g.state()
            return [master[s:e], m[s:e], v[s:e], g.flat[g.offset + s:g.offset + e]]

        if self.verdict_first:
            # pass A over every chunk of every group, in order
            for g in self.groups:
                items = sorted(avg_items(g, g.checked, True) + avg_items(g, g.norm_only, False),
                               key=lambda it: it[1])
                sums += [(n2, f) for _, n2, f in self._run(items, fetch_grads, work_avg)]
            n2_all = float(sum(x for x, _ in sums))
            flag_all = int(any(f for _, f in sums))
            bar.clip(tag, gpu_state["clip_coef"], self._clip_of(n2_all, flag_all),
                     applied=not (flag_all and self.policy.skip_on_overflow))

            def work_step(it, arrs):
                g, s, e = it
                st = oracle.State(**vars(pre))
                og = self._ogroup(g, s, e)
                oracle.step_from_average([og], [avgs.pop((id(g), s, e))], self.policy, st, n2_all, flag_all)
                compare(g, s, e, arrs, st)
                return st

            posts = []
            for g in self.groups:
                posts += self._run([(g, s, e) for s, e in g.checked], fetch_state, work_step)
        else:
            # one pass: average, norm sums and the update per chunk
            def fetch_both(it):
                g, s, e, with_state = it
                t = [r[s:e] for r in g.reps]
                if with_state:
                    master, m, v = g.state()
                    t += [master[s:e], m[s:e], v[s:e], g.flat[g.offset + s:g.offset + e]]
                return t

            def work_one(it, arrs):
                g, s, e, with_state = it
                nd = len(g.reps)
                a = oracle.average(arrs[:nd], g.odt)
                n2, f = oracle.norm_overflow(a, inv)
                if not with_state:
                    return s, n2, f, None
                st = oracle.State(**vars(pre))
                oracle.step_from_average([self._ogroup(g, s, e)], [a], self.policy, st, n2, f)
                compare(g, s, e, arrs[nd:], st)
                return s, n2, f, st

            posts = []
            for g in self.groups:
                items = sorted([(g, s, e, True) for s, e in g.checked] + [(g, s, e, False) for s, e in g.norm_only],
                               key=lambda it: it[1])
                for _, n2, f, st in self._run(items, fetch_both, work_one):
                    sums.append((n2, f))
                    if st is not None:
                        posts.append(st)
            n2_all = float(sum(x for x, _ in sums))
            flag_all = int(any(f for _, f in sums))
            for st in posts:      # the chunks' own norms do not enter a static-scale, unclipped update
                st.norm2, st.overflow = n2_all, flag_all
            bar.clip(tag, gpu_state["clip_coef"], self._clip_of(n2_all, flag_all), applied=True)
        if not posts:
            raise AssertionError(f"{tag}: no chunk was checked")
        if not all(_same_state(p, posts[0]) for p in posts):
            raise AssertionError(f"{tag}: the oracle's chunks disagree on the step's bookkeeping")
        post = posts[0]
        post.norm2, post.overflow = n2_all, flag_all
        self.ostate = post
        return post

    def _clip_of(self, n2, flag):
        """The oracle's clip multiplier for this norm and flag: its step over
        an empty group, which computes the verdict and changes nothing."""
        st = oracle.State(**vars(self.ostate))
        e = np.zeros(0, np.float32)
        og = oracle.Group(replicas=None, grad_dt=self.groups[0].odt, master=e, m=e.copy(), v=e.copy())
        oracle.step_from_average([og], [e.copy()], self.policy, st, n2, flag)
        return st.clip
