#!/usr/bin/env python3
"""KIVI flush benchmark on one MI355X: effective HBM GB/s of the whole path.

A step is one pass of every kernel of the path over one batch of synthetic
KV: quantize keys (per channel) and values (per token), dequantize both, and
the fused quantize->dequantize of both.  Default workload: the dequantize
round trip, BH = 32 x 8 KV heads, S = 4096, D = 128, fp16, 2-bit, groups of
32 tokens (keys) and 32 channels (values).

value = algorithmic bytes of the step (each input read once, each output
written once) / measured step time, with inputs resident in HBM; inputs
rotate over a pool of distinct tensors larger than the 256 MB MALL, and the
dequantizers read codes written two steps earlier (see make_steps), so no
kernel's input is served from a cache.  Per-kernel durations come from HIP events
recorded at each kernel's own dispatch (hipExtLaunchKernel, armed through
kivi_time_next_launch) over a second pass of K steps, after the timed
region: the markers HIP queues for such events cost a few microseconds per
launch, so the step itself is timed without them.  The dominant kernel's
achieved bandwidth is reported against MI355X's 8 TB/s peak.  The CPU
baseline is the plain C oracle timed on a bounded sample of the same workload,
on the host's threads (value) and on one thread.

Prints ONE JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_HBM_GBS = 8000.0
METRIC = ("effective HBM GB/s (and % of MI355X peak) for KIVI 2-bit K+V "
          "flush/dequant")
# The kernel sources behind each family of workloads: the traffic measured
# for a workload stays valid while these files are unchanged.
_COMMON = ["kivi_device.h", "kivi_launch.h", "kivi_rows.h", "kivi_key_split.h"]
KERNEL_SOURCES = {
    "flush": _COMMON + ["quant_keys.hip", "quant_values.hip", "dequant.hip",
                        "generic.hip"],
    "cache": _COMMON + ["quant_keys.hip", "quant_values.hip", "cache.hip"],
    "attend": _COMMON + ["attend.hip", "attend_mfma.hip"],
    "sink": _COMMON + ["sink.hip", "quant_keys.hip", "quant_values.hip"],
    "mixed": _COMMON + ["sink.hip", "rows.hip", "quant_keys.hip",
                        "quant_values.hip"],
}


def bytes_per_elem(op, bits, group, dtype_bytes=2):
    """Algorithmic bytes per element: input once, every output once.
    quant: x + codes + fp32 scale and zero per group."""
    codes = bits / 8.0
    params = 8.0 / group
    if op == "quant":
        return dtype_bytes + codes + params
    if op == "dequant":
        return codes + params + dtype_bytes
    if op == "fused":
        return dtype_bytes + codes + params + dtype_bytes
    raise ValueError(op)


def kernel_source_hash(family="flush"):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "kv_cache_quantization_kivi_amd",
                               "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, src_hash):
    """HBM bytes per launch measured with rocprofv3 counters (committed in
    profiles/), used only while the kernel sources are unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(f"{kernel}@{workload}")
    if not ent or ent.get("source_hash") != src_hash:
        return None
    return ent.get("hbm_bytes_per_launch")


N_CODE_SETS = 4   # rotating code/param sets (see make_steps)


PAIRED = {"quant_kv": ("quant_keys", "quant_values"),
          "quant_dequant_kv": ("quant_dequant_keys", "quant_dequant_values"),
          "dequant_kv": ("dequant_keys", "dequant_values")}


class Dispatches:
    """The library's kernel dispatches in the order the GPU runs them,
    counted with kivi_launch_count, so that a profiler's dispatch trace can
    be split into this run's phases: an eager launch dispatches once, a
    launch recorded into a graph under capture dispatches at every replay."""

    def __init__(self, K):
        self.K = K
        self.mark = K.kivi_launch_count()
        self.n = self.mark          # every earlier launch was eager

    def eager(self):
        c = self.K.kivi_launch_count()
        self.n += c - self.mark
        self.mark = c

    def captured(self):
        """Launches recorded into a graph since the last call: their number
        (nothing is dispatched)."""
        c = self.K.kivi_launch_count()
        k = c - self.mark
        self.mark = c
        return k

    def replayed(self, k):
        self.n += k


def launch_labels(K, calls):
    """Run calls = [(name, fn)] once, in order, and label every kernel they
    launch: a call that launches n kernels gives name, name#2, ... name#n
    (the first is the one its per-kernel timing arms)."""
    labels = []
    for name, fn in calls:
        c0 = K.kivi_launch_count()
        fn()
        n = K.kivi_launch_count() - c0
        labels += [name] + [f"{name}#{k}" for k in range(2, n + 1)]
    return labels


def profile_layout(before, timed, labels):
    return {"dispatches_before_timed": int(before),
            "timed_dispatches": int(timed), "step_launches": labels}


def launch_bound(args, step_bytes, launches):
    """Whether the timed steps are HIP graph replays: asked for, or (auto) a
    launch-bound step, under 16 MB of traffic per launch (a decode-time
    flush, one-token cache appends).  Longer launches are issued eagerly: the
    host then stays ahead of the GPU, and a replay costs several
    microseconds more than it saves (a 2048-token cache append: 27.4 us a
    step eagerly, 32.8 us replayed)."""
    if args.launch != "auto":
        return args.launch == "graphs"
    return step_bytes / max(1, launches) < 16e6


def call_intervals(torch, stream, step, n_calls, n_steps, base):
    """Per call of a step, its duration in each of n_steps more steps
    launched as in the timed region, with a plain event recorded on the
    launch stream before the step and after every call
    (step(i, mark) calls mark(j) after call j): the interval that ends with
    a call holds its kernels and the dispatch gap before them, back to back
    with the rest of the step, so a step's intervals add up to the step.
    Returns n_calls lists of milliseconds."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_calls + 1)]
          for _ in range(n_steps)]
    torch.cuda.synchronize()
    for i in range(n_steps):
        ev[i][0].record(stream)
        step(base + i, lambda j, i=i: ev[i][j + 1].record(stream))
    torch.cuda.synchronize()
    return [[ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(n_steps)]
            for j in range(n_calls)]


def make_steps(K, w, pool_inputs, torch, paired=False):
    """Pre-allocated outputs and the list of (name, op, bytes, launch fn)
    that make one step.  Every launch goes to torch's current stream and
    takes the step index i.

    Cache hygiene, so that every input byte of every kernel comes from HBM:
    the quantizers of step i read input set i % P and write code/param set
    (i + 2) % 4; the fused kernels read the other input set (i + 1) % P; the
    dequantizers read code set i % 4, written two steps (over 0.5 GB of
    plain stores) earlier, after the MALL (256 MB) has turned over.  Without
    this a dequantizer would read codes written microseconds before and
    still resident in the memory-side cache.
    """
    E = w.elems
    dev = pool_inputs[0][0].device
    P = len(pool_inputs)
    bits, gk, gv = w.bits, w.group_k, w.group_v
    NG = (w.S + gk - 1) // gk
    NGD = (w.D + gv - 1) // gv
    shp = (w.BH, w.S, w.D)
    dt = pool_inputs[0][0].dtype

    def qbufs(keys):
        c = torch.empty((w.BH, w.S, w.D * bits // 8), dtype=torch.uint8,
                        device=dev)
        p = (w.BH, NG, w.D) if keys else (w.BH, w.S, NGD)
        return (c, torch.empty(p, dtype=torch.float32, device=dev),
                torch.empty(p, dtype=torch.float32, device=dev))

    qk = [qbufs(True) for _ in range(N_CODE_SETS)]
    qv = [qbufs(False) for _ in range(N_CODE_SETS)]
    for s in range(N_CODE_SETS):   # every set holds real codes before timing
        K.kivi_quant_keys(pool_inputs[s % P][0], bits, gk, *qk[s])
        K.kivi_quant_values(pool_inputs[s % P][1], bits, gv, *qv[s])
    fk, fv = qbufs(True), qbufs(False)
    dk = torch.empty(shp, dtype=dt, device=dev)
    dv = torch.empty(shp, dtype=dt, device=dev)
    rk = torch.empty(shp, dtype=dt, device=dev)
    rv = torch.empty(shp, dtype=dt, device=dev)

    def ws(i):
        return (i + 2) % N_CODE_SETS

    def rs(i):
        return i % N_CODE_SETS

    steps = [
        ("quant_keys", "quant", gk,
         lambda i: K.kivi_quant_keys(pool_inputs[i % P][0], bits, gk,
                                     *qk[ws(i)])),
        ("quant_values", "quant", gv,
         lambda i: K.kivi_quant_values(pool_inputs[i % P][1], bits, gv,
                                       *qv[ws(i)])),
    ]
    if w.name in ("tiny", "decode", "roundtrip"):
        steps += [
            ("quant_dequant_keys", "fused", gk,
             lambda i: K.kivi_quant_dequant_keys(
                 pool_inputs[(i + 1) % P][0], bits, gk, True, rk, *fk)),
            ("quant_dequant_values", "fused", gv,
             lambda i: K.kivi_quant_dequant_values(
                 pool_inputs[(i + 1) % P][1], bits, gv, True, rv, *fv)),
            ("dequant_keys", "dequant", gk,
             lambda i: K.kivi_dequant_keys(*qk[rs(i)], bits, gk, out_dtype=dt,
                                           out=dk)),
            ("dequant_values", "dequant", gv,
             lambda i: K.kivi_dequant_values(*qv[rs(i)], bits, gv,
                                             out_dtype=dt, out=dv)),
        ]
    out = []
    for name, op, g, fn in steps:
        out.append((name, op, bytes_per_elem(op, bits, g) * E, fn))
    if not paired:
        return out
    # the same work through the K+V calls: one launch each at these sizes
    kv = [
        ("quant_kv", lambda i: K.kivi_quant_kv(
            pool_inputs[i % P][0], pool_inputs[i % P][1], bits, gk, gv,
            qk[ws(i)], qv[ws(i)])),
        ("quant_dequant_kv", lambda i: K.kivi_quant_dequant_kv(
            pool_inputs[(i + 1) % P][0], pool_inputs[(i + 1) % P][1], bits, gk,
            gv, True, rk, rv, fk, fv)),
        ("dequant_kv", lambda i: K.kivi_dequant_kv(
            qk[rs(i)], qv[rs(i)], bits, gk, gv, out_dtype=dt, k_out=dk,
            v_out=dv)),
    ]
    byts = {name: b for name, _, b, _ in out}
    ops = {name: op for name, op, _, _ in out}
    return [(name, ops[PAIRED[name][0]], sum(byts[n] for n in PAIRED[name]), fn)
            for name, fn in kv if PAIRED[name][0] in byts]


def _oracle_step(O, w, k, v, names):
    """Every row of the step on one block of bh slices, through the oracle as
    it stands (the fused row is its quantize followed by its dequantize)."""
    ck = cv = None
    names = [n for name in names for n in PAIRED.get(name, (name,))]
    for name in names:
        if name == "quant_keys":
            ck = O.quant_keys(k, w.dtype, w.bits, w.group_k)
        elif name == "quant_values":
            cv = O.quant_values(v, w.dtype, w.bits, w.group_v)
        elif name == "dequant_keys":
            O.dequant_keys(*ck, k.shape, w.bits, w.group_k, w.dtype)
        elif name == "dequant_values":
            O.dequant_values(*cv, v.shape, w.bits, w.group_v, w.dtype)
        elif name == "quant_dequant_keys":
            q = O.quant_keys(k, w.dtype, w.bits, w.group_k)
            O.dequant_keys(*q, k.shape, w.bits, w.group_k, w.dtype)
        elif name == "quant_dequant_values":
            q = O.quant_values(v, w.dtype, w.bits, w.group_v)
            O.dequant_values(*q, v.shape, w.bits, w.group_v, w.dtype)


def cpu_baseline(w, n_bh, steps_desc, threads):
    """The oracle as it stands on n_bh slices of the same workload, timed
    twice: on one thread, then on `threads` threads that each run the whole
    step over a contiguous block of the slices (the oracle's C calls release
    the GIL, so the blocks run in parallel)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    O = oracle.default()
    bhs = list(range(n_bh))
    k = W.gen_tensor(w, "K", bhs)
    v = W.gen_tensor(w, "V", bhs)
    E = k.size
    names = [s[0] for s in steps_desc]
    byts = sum(b / w.elems * E for _, _, b, _ in steps_desc)

    t0 = time.perf_counter()
    _oracle_step(O, w, k, v, names)
    dt1 = time.perf_counter() - t0

    threads = max(1, min(threads, n_bh))
    cuts = np.linspace(0, n_bh, threads + 1).astype(int)
    blocks = [(np.ascontiguousarray(k[a:b]), np.ascontiguousarray(v[a:b]))
              for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    with ThreadPoolExecutor(max_workers=len(blocks)) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda kv: _oracle_step(O, w, kv[0], kv[1], names),
                    blocks))
        dtn = time.perf_counter() - t0
    return {
        "value": round(byts / dtn / 1e9, 4),
        "unit": "GB/s",
        "cores": len(blocks),
        "kind": "oracle",
        "sample": (f"{n_bh} of {w.BH} (bh) slices of the same workload "
                   f"({E} elements per tensor), every row of the step: "
                   f"{dtn:.2f} s on {len(blocks)} threads (value); "
                   f"{dt1:.2f} s on 1 thread"),
        "single_thread_value": round(byts / dt1 / 1e9, 4),
    }


def calibrate_copy(torch, dev, mb, reps):
    """A plain copy of known size: reads and writes exactly n bytes per
    launch; its rocprofv3 FETCH_SIZE / WRITE_SIZE give the counter scale."""
    n = mb * 1000 * 1000
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    big = torch.empty(4 * n, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, fn, nbytes in (("copy", lambda: dst.copy_(src), 2 * n),
                             ("read_sum", lambda: src.view(torch.int32).sum(),
                              n)):
        for _ in range(3):
            big.fill_(0)          # evict the operands from the caches
            fn()
        ts = []
        for _ in range(reps):
            big.fill_(0)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        med = float(np.median(ts))
        res[name] = {"bytes_per_launch": nbytes, "median_us": round(med * 1e3, 2),
                     "gbs": round(nbytes / (med * 1e-3) / 1e9, 1)}
    print(json.dumps({"calibration": res, "size_bytes": n}), flush=True)


# --------------------------------------------------------------------------
# residual-window cache workloads (kivi_cache_append)
# --------------------------------------------------------------------------

def flush_plan(cw):
    """The appends of one step, as the cache's rule schedules them: per
    append (T before, Q before, n, tokens flushed F, tokens stored in the
    ring), per bh.  Q = G_k * floor((T - R) / G_k)."""
    def q_of(t):
        return cw.group_k * ((t - cw.R) // cw.group_k) if t >= cw.R else 0
    T, Q = cw.T0, q_of(cw.T0)
    plan = []
    for _ in range(cw.appends):
        Tn = T + cw.n
        Qn = max(q_of(Tn), Q)
        plan.append((T, Q, cw.n, Qn - Q, Tn - max(Qn, T)))
        T, Q = Tn, Qn
    return plan


def cache_flush_paired(cw, F):
    """Whether the library flushes F tokens of K and V in one launch (the
    one-launch rule of the K+V calls, include/kivi.h, with a cache flush's
    item bound of 4 * 65536)."""
    D8 = cw.D // 8
    g32 = cw.group_v // 32
    return (cw.BH * (F // cw.group_k) * D8 < 4 * 65536 and 64 % (D8 * 4) == 0
            and 16 < cw.group_k <= 32 and cw.group_v % 32 == 0
            and g32 & (g32 - 1) == 0)


def cache_bytes(cw, F, copy, keys_flush_only=False, flush_only=False):
    """Algorithmic bytes of one append: the F flushed tokens of K and V read
    once, their codes and params written once, and the tokens that stay
    unquantized read once and written once to the ring."""
    D = cw.D
    kf = F * D * 2 + F * D * cw.bits // 8 + (F // cw.group_k) * D * 8
    if keys_flush_only:
        return kf * cw.BH
    vf = F * D * 2 + F * D * cw.bits // 8 + F * (-(-D // cw.group_v)) * 8
    if flush_only:
        return (kf + vf) * cw.BH
    ring = 2 * copy * D * 2 * 2
    return (kf + vf + ring) * cw.BH


def cache_cpu_baseline(cw, threads, plan, step_bytes):
    """The oracle's cache (token-by-token scheduler) on a sample of whole bh
    slices: the same appends from the same starting state, timed on
    `threads` threads (a cache per contiguous block of slices) and on one."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    O = oracle.default()
    tw = cw.tokens()
    n_bh = min(cw.BH, max(1, threads))
    k = W.gen_tensor(tw, "K", range(n_bh))
    v = W.gen_tensor(tw, "V", range(n_bh))
    S_max = cw.T0 + cw.n * cw.appends
    pw = W.Workload(cw.name, cw.BH, max(cw.T0, 1), cw.D, cw.dtype, cw.bits,
                    cw.group_k, cw.group_v, cw.seed + 100, tw.key_kind,
                    tw.value_kind, cw.desc)
    pk = W.gen_tensor(pw, "K", range(n_bh))[:, :cw.T0]
    pv = W.gen_tensor(pw, "V", range(n_bh))[:, :cw.T0]

    def run(a, b, timed):
        c = O.cache(b - a, cw.D, S_max, cw.R, cw.group_k, cw.group_v,
                    cw.bits, cw.dtype)
        c.append(np.ascontiguousarray(pk[a:b]), np.ascontiguousarray(pv[a:b]))
        t0 = time.perf_counter()
        for i in range(cw.appends):
            sl = slice(i * cw.n, (i + 1) * cw.n)
            c.append(np.ascontiguousarray(k[a:b, sl]),
                     np.ascontiguousarray(v[a:b, sl]))
        return time.perf_counter() - t0

    dt1 = run(0, 1, True)
    cuts = np.linspace(0, n_bh, n_bh + 1).astype(int)
    with ThreadPoolExecutor(max_workers=n_bh) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda ab: run(ab[0], ab[1], True),
                    zip(cuts[:-1], cuts[1:])))
        dtn = time.perf_counter() - t0
    per_bh = step_bytes / cw.BH
    return {
        "value": round(per_bh * n_bh / dtn / 1e9, 4),
        "unit": "GB/s",
        "cores": n_bh,
        "kind": "oracle",
        "sample": (f"{n_bh} of {cw.BH} (bh) slices, one step ({cw.appends} "
                   f"append(s) of {cw.n} token(s) from T = {cw.T0}): "
                   f"{dtn:.3f} s on {n_bh} threads, one slice per thread "
                   f"(value); {dt1:.3f} s for one slice on 1 thread; the "
                   "cache's setup appends are not timed"),
        "single_thread_value": round(per_bh / dt1 / 1e9, 4),
    }


def cache_bench(args, cw, K, torch, dev):
    """One step = `appends` calls of kivi_cache_append on a cache reset to
    T0 tokens (counters only; the ring and the store keep real data from
    a setup append).  Launch-bound steps are one HIP graph replay."""
    tdt = torch.float16 if cw.dtype == W.FP16 else torch.bfloat16
    tw = cw.tokens()
    plan = flush_plan(cw)
    step_bytes = sum(cache_bytes(cw, F, cp) for _, _, _, F, cp in plan)
    S_max = cw.T0 + cw.n * cw.appends
    cache = K.KiviCache(cw.BH, cw.D, S_max, cw.R, cw.group_k, cw.group_v,
                        cw.bits, tdt, dev)
    if cw.T0:
        pw = W.Workload(cw.name, cw.BH, cw.T0, cw.D, cw.dtype, cw.bits,
                        cw.group_k, cw.group_v, cw.seed + 100, tw.key_kind,
                        tw.value_kind, cw.desc)
        pk = torch.from_numpy(W.gen_tensor(pw, "K").view(np.int16)).view(tdt)
        pv = torch.from_numpy(W.gen_tensor(pw, "V").view(np.int16)).view(tdt)
        for a in range(0, cw.T0, 2048):
            cache.append(pk[:, a:a + 2048].contiguous().to(dev),
                         pv[:, a:a + 2048].contiguous().to(dev))
    T0, Q0 = cache.T, cache.Q
    set_bytes = 2 * cw.BH * cw.n * cw.appends * cw.D * 2
    P = args.pool or max(2, min(64, int(np.ceil(1.0e9 / set_bytes))))
    pool = []
    for p in range(P):
        kv = []
        for tensor in ("K", "V"):
            x = torch.from_numpy(W.gen_tensor(tw, tensor, pool=p).view(
                np.int16)).view(tdt)
            kv.append([x[:, i * cw.n:(i + 1) * cw.n].contiguous().to(dev)
                       for i in range(cw.appends)])
        pool.append(kv)
    stream = torch.cuda.current_stream(dev)

    def step(i, arm=None):
        cache.c.T, cache.c.Q = T0, Q0
        ks, vs = pool[i % P]
        for a in range(cw.appends):
            if arm is not None:
                K.kivi_time_next_launch(*arm[a])
            cache.append(ks[a], vs[a])

    disp = Dispatches(K)
    cache.c.T, cache.c.Q = T0, Q0
    n_launch = []            # launches of each append (the first step)
    for a in range(cw.appends):
        c0 = K.kivi_launch_count()
        cache.append(pool[0][0][a], pool[0][1][a])
        n_launch.append(K.kivi_launch_count() - c0)

    def append_kind(a):
        """The per-kernel name of append a's first launch: the flush (of K
        and V together when it is one launch, and with the ring store too
        when that is the append's only launch), else the ring store."""
        F, cp = plan[a][3], plan[a][4]
        if not F:
            return "cache_ring_store"
        if not cache_flush_paired(cw, F):
            return "cache_flush_keys"
        return "cache_append_kv" if cp and n_launch[a] == 1 else "cache_flush_kv"

    labels = []
    for a in range(cw.appends):
        labels += [append_kind(a)] + [f"{append_kind(a)}#{k}"
                                      for k in range(2, n_launch[a] + 1)]
    for i in range(1, args.warmup):
        step(i)
    base = max(args.warmup, 1)
    torch.cuda.synchronize()
    use_graphs = launch_bound(args, step_bytes, len(labels))
    graphs = None
    disp.eager()
    if use_graphs:
        graphs = []
        cap = torch.cuda.Stream(device=dev)
        for ph in range(P):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(ph)
            graphs.append((g, disp.captured()))
            g.replay()
            disp.replayed(graphs[-1][1])
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    before = disp.n
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        if graphs is not None:
            g, k = graphs[(base + i) % P]
            g.replay()
            disp.replayed(k)
        else:
            step(base + i)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    disp.eager()
    layout = profile_layout(before, disp.n - before, labels)
    ms_per_step = start.elapsed_time(end) / args.steps

    # kernel durations: the first kernel of every append (the key flush when
    # the append flushes, else the ring store of keys and values), eagerly,
    # K more steps
    def pairs():
        ev = [(torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True))
              for _ in range(cw.appends)]
        for a, b in ev:
            a.record(stream)
            b.record(stream)
        return ev
    arms = [pairs() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(base + args.steps + i, arms[i])
    torch.cuda.synchronize()
    kinds = {}
    for a, (_, _, n, F, cp) in enumerate(plan):
        name = append_kind(a)
        b = (cache_bytes(cw, F, cp) if name == "cache_append_kv"
             else cache_bytes(cw, F, cp, flush_only=True)
             if name == "cache_flush_kv"
             else cache_bytes(cw, F, cp, keys_flush_only=True) if F
             else cw.BH * cp * cw.D * 2 * 2 * 2)
        d = [arms[i][a][0].elapsed_time(arms[i][a][1])
             for i in range(args.steps)]
        kinds.setdefault(name, (b, []))[1].extend(d)
    per_kernel = {}
    for name, (b, d) in kinds.items():
        avg = float(np.mean(d))
        per_kernel[name] = {
            "avg_us": round(avg * 1e3, 3),
            "median_us": round(float(np.median(d)) * 1e3, 3),
            "min_us": round(float(np.min(d)) * 1e3, 3),
            "max_us": round(float(np.max(d)) * 1e3, 3),
            "algorithmic_bytes": int(b),
            "gbs": round(b / (avg * 1e-3) / 1e9, 1),
        }
    dom = max(per_kernel, key=lambda n: per_kernel[n]["avg_us"])
    dk = per_kernel[dom]
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    tokens = cw.BH * cw.n * cw.appends
    result = {
        "metric": METRIC + " (residual-window cache append)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{cw.name}: {cw.desc}; step = {cw.appends} "
                         f"kivi_cache_append call(s) of {cw.n} token(s) x "
                         f"BH={cw.BH} from T={T0} (Q={Q0})"),
            "step_algorithmic_bytes": int(step_bytes),
            "tokens_per_step": tokens,
            "us_per_append": round(ms_per_step * 1e3 / cw.appends, 3),
            "input_pool": P,
            "launch": (f"one HIP graph replay per step ({P} phases)"
                       if graphs is not None else "eager"),
            "wall_s": round(t_wall, 4),
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "roofline": {
            "kernel": dom,
            "avg_us": dk["avg_us"],
            "bound": "hbm",
            "achieved": dk["gbs"],
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(dk["gbs"] / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(dom, cw.name, kernel_source_hash("cache")),
        },
        "per_kernel": per_kernel,
        "per_kernel_note": ("value: K steps with no per-launch events; "
                            "per_kernel: the first kernel of every append of "
                            "a second pass of K eager steps"),
        "kernel_source_hash": kernel_source_hash("cache"),
        "profile_layout": dict(layout, per_kernel_timing="first_launch"),
        "cpu_baseline": (None if args.no_cpu_baseline else
                         cache_cpu_baseline(cw, args.cpu_threads, plan,
                                            step_bytes)),
    }
    print(json.dumps(result), flush=True)


# --------------------------------------------------------------------------
# decode attention over the packed cache (kivi_cache_attend)
# --------------------------------------------------------------------------

def attend_bytes(aw, Q):
    """Algorithmic bytes of one attention call: the packed store of tokens
    [0, Q) (codes and params of K and V), the exact tokens [Q, T) of K and
    V, and the queries read once; the outputs written once."""
    D, T = aw.D, aw.T
    per_bh = (2 * Q * D * aw.bits // 8 + (Q // aw.group_k) * D * 8
              + Q * (-(-D // aw.group_v)) * 8 + 2 * (T - Q) * D * 2
              + aw.n_q * D * 2)
    out = aw.n_q * D * 2
    return (per_bh + out) * aw.BH, out * aw.BH


def attend_bench(args, aw, K, torch, dev):
    """One step = one kivi_cache_attend call; the caches rotate over a pool
    whose packed stores exceed the 256 MB MALL together."""
    tdt = torch.float16 if aw.dtype == W.FP16 else torch.bfloat16
    q_of = aw.group_k * ((aw.T - aw.R) // aw.group_k) if aw.T >= aw.R else 0
    step_bytes, out_bytes = attend_bytes(aw, q_of)
    P = args.pool or max(2, min(16, int(np.ceil(600e6 / step_bytes))))
    tw = aw.tokens()
    caches, qs = [], []
    for p in range(P):
        c = K.KiviCache(aw.BH, aw.D, aw.T, aw.R, aw.group_k, aw.group_v,
                        aw.bits, tdt, dev)
        kx = torch.from_numpy(W.gen_tensor(tw, "K", pool=p).view(np.int16)).view(tdt)
        vx = torch.from_numpy(W.gen_tensor(tw, "V", pool=p).view(np.int16)).view(tdt)
        for a in range(0, aw.T, 2048):
            c.append(kx[:, a:a + 2048].contiguous().to(dev),
                     vx[:, a:a + 2048].contiguous().to(dev))
        assert c.Q == q_of
        caches.append(c)
        r = np.random.default_rng([aw.seed, 77, p])
        qx = (r.standard_normal((aw.BH, aw.n_q, aw.D)) * 0.5).astype(np.float32)
        qs.append(torch.from_numpy(qx).to(tdt).to(dev))
    out = torch.empty((aw.BH, aw.n_q, aw.D), dtype=tdt, device=dev)
    work = torch.empty(max(16, caches[0].attend_work_bytes(aw.n_q)),
                       dtype=torch.uint8, device=dev)
    sm = 1.0 / float(np.sqrt(aw.D))
    stream = torch.cuda.current_stream(dev)

    def step(i):
        caches[i % P].attend(qs[i % P], sm, out=out, work=work)

    disp = Dispatches(K)
    labels = launch_labels(K, [("attend_chunks", lambda: step(0))])
    for i in range(1, args.warmup):
        step(i)
    base = max(args.warmup, 1)
    use_graphs = launch_bound(args, step_bytes, len(labels))
    graphs = None
    disp.eager()
    if use_graphs:
        graphs = []
        cap = torch.cuda.Stream(device=dev)
        for ph in range(P):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(ph)
            graphs.append((g, disp.captured()))
            g.replay()
            disp.replayed(graphs[-1][1])
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    before = disp.n
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        if graphs is not None:
            g, k = graphs[(base + i) % P]
            g.replay()
            disp.replayed(k)
        else:
            step(base + i)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    disp.eager()
    layout = profile_layout(before, disp.n - before, labels)
    ms_per_step = start.elapsed_time(end) / args.steps

    # the attention kernel proper (the first of the call's two launches)
    ev = [(torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a_, b_ in ev:
        a_.record(stream)
        b_.record(stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        K.kivi_time_next_launch(*ev[i])
        step(base + args.steps + i)
    torch.cuda.synchronize()
    d = [a_.elapsed_time(b_) for a_, b_ in ev]
    kb = step_bytes - out_bytes
    avg = float(np.mean(d))
    pk = {"attend_chunks": {
        "avg_us": round(avg * 1e3, 3),
        "median_us": round(float(np.median(d)) * 1e3, 3),
        "min_us": round(float(np.min(d)) * 1e3, 3),
        "max_us": round(float(np.max(d)) * 1e3, 3),
        "algorithmic_bytes": int(kb),
        "gbs": round(kb / (avg * 1e-3) / 1e9, 1)}}
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    fp16_bytes = aw.BH * (2 * aw.T * aw.D * 2 + 2 * aw.n_q * aw.D * 2)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        O = oracle.default()
        n_bh = min(aw.BH, 16)
        oc = O.cache(n_bh, aw.D, aw.T, aw.R, aw.group_k, aw.group_v,
                     aw.bits, aw.dtype)
        kx = W.gen_tensor(tw, "K", range(n_bh))
        vx = W.gen_tensor(tw, "V", range(n_bh))
        oc.append(kx, vx)
        qx = qs[0][:n_bh].cpu().view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        oc.attend(qx, sm)
        dt = time.perf_counter() - t0
        cpu = {"value": round(step_bytes / aw.BH * n_bh / dt / 1e9, 4),
               "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": (f"{n_bh} of {aw.BH} (bh) slices, one attention "
                          f"call: {dt:.3f} s on 1 thread (float64 numpy; the "
                          "cache's setup appends are not timed)")}
    result = {
        "metric": METRIC + " (decode attention over the packed cache)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{aw.name}: {aw.desc}; step = one "
                         "kivi_cache_attend call"),
            "step_algorithmic_bytes": int(step_bytes),
            "fp16_cache_bytes_same_attention": int(fp16_bytes),
            "us_per_call": round(ms_per_step * 1e3, 3),
            "input_pool": P,
            "launch": (f"one HIP graph replay per step ({P} phases)"
                       if graphs is not None else "eager"),
            "wall_s": round(t_wall, 4),
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "roofline": {
            "kernel": "attend_chunks",
            "avg_us": pk["attend_chunks"]["avg_us"],
            "bound": "hbm",
            "achieved": pk["attend_chunks"]["gbs"],
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(pk["attend_chunks"]["gbs"] / PEAK_HBM_GBS, 4),
            "traffic": load_traffic("attend_chunks", aw.name,
                                    kernel_source_hash("attend")),
        },
        "per_kernel": pk,
        "kernel_source_hash": kernel_source_hash("attend"),
        "profile_layout": dict(layout, per_kernel_timing="first_launch"),
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


# --------------------------------------------------------------------------
# KIVI-Sink over a prompt (kivi_sink_select, kivi_quant_keys_sink, ...)
# --------------------------------------------------------------------------

def sink_bytes(sw):
    """Algorithmic bytes of one KIVI-Sink pass, per kernel: the scores read
    every key once and write one fp32 per token; the selection reads the
    scores once; the key quantizer reads the keys again (the sinks must be
    known before any key group's min/max) and writes codes and params; the
    value quantizer is plain KIVI; the two gathers copy the sinks' K and V
    rows."""
    E = sw.B * sw.H * sw.S * sw.D
    tok = sw.B * sw.S * 4
    kq = E * bytes_per_elem("quant", sw.bits, sw.group_k)
    vq = E * bytes_per_elem("quant", sw.bits, sw.group_v)
    gather = sw.B * sw.H * sw.n_sink * sw.D * 2 * 2
    return {"sink_score": E * 2 + tok, "sink_select": tok,
            "quant_keys_sink": int(kq), "quant_values": int(vq),
            "sink_gather_k": gather, "sink_gather_v": gather}


def sink_bench(args, sw, K, torch, dev):
    """One step = the KIVI-Sink pass over one prompt: select the sinks,
    quantize the keys without them, quantize the values, keep the sinks' K
    and V rows.  Inputs rotate over a pool of prompts larger than the MALL."""
    tdt = torch.float16 if sw.dtype == W.FP16 else torch.bfloat16
    w = sw.tokens()
    B, H, S, D = sw.B, sw.H, sw.S, sw.D
    nb = sink_bytes(sw)
    step_bytes = sum(nb.values())
    P = args.pool or 2
    inputs = []
    for p in range(P):
        kv = []
        for tensor in ("K", "V"):
            x = W.gen_tensor(w, tensor, pool=p)
            kv.append(torch.from_numpy(x.view(np.int16)).view(tdt).to(dev)
                      .view(B, H, S, D))
        inputs.append(tuple(kv))
    kc, ks, kz = K.kivi_quant_keys_sink(inputs[0][0], torch.zeros(
        (B, sw.n_sink), dtype=torch.int32, device=dev), sw.bits, sw.group_k)
    vc, vs, vz = K.kivi_quant_values(inputs[0][1], sw.bits, sw.group_v)
    idx = torch.empty((B, sw.n_sink), dtype=torch.int32, device=dev)
    score = torch.empty((B, S), dtype=torch.float32, device=dev)
    k_keep = torch.empty((B, H, sw.n_sink, D), dtype=tdt, device=dev)
    v_keep = torch.empty_like(k_keep)
    stream = torch.cuda.current_stream(dev)
    names = ["sink_select", "quant_keys_sink", "quant_values", "sink_gather_k",
             "sink_gather_v"]
    call_bytes = dict(nb)
    call_bytes["sink_select"] = nb["sink_score"] + nb["sink_select"]

    calls = [
        lambda k, v: K.kivi_sink_select(k, sw.n_sink, score=score, idx=idx),
        lambda k, v: K.kivi_quant_keys_sink(k, idx, sw.bits, sw.group_k,
                                            codes=kc, scale=ks, zero=kz),
        lambda k, v: K.kivi_quant_values(v, sw.bits, sw.group_v, codes=vc,
                                         scale=vs, zero=vz),
        lambda k, v: K.kivi_sink_gather(k, idx, out=k_keep),
        lambda k, v: K.kivi_sink_gather(v, idx, out=v_keep),
    ]

    def step(i, mark=None):
        k, v = inputs[i % P]
        for a, fn in enumerate(calls):
            fn(k, v)
            if mark is not None:
                mark(a)

    disp = Dispatches(K)
    labels = launch_labels(K, [(n, lambda fn=fn: fn(*inputs[0]))
                               for n, fn in zip(names, calls)])
    for i in range(1, args.warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    base = max(args.warmup, 1)
    disp.eager()
    before = disp.n
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(base + i)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    disp.eager()
    layout = profile_layout(before, disp.n - before, labels)
    ms_per_step = start.elapsed_time(end) / args.steps

    # per call: its interval between plain events recorded between the
    # calls of K more back-to-back steps (call_intervals)
    pk = {}
    iv = call_intervals(torch, stream, step, len(calls), args.steps,
                        base + args.steps)
    for a, name in enumerate(names):
        d = iv[a]
        avg = float(np.mean(d))
        b = call_bytes[name]
        pk[name] = {"avg_us": round(avg * 1e3, 3),
                    "median_us": round(float(np.median(d)) * 1e3, 3),
                    "min_us": round(float(np.min(d)) * 1e3, 3),
                    "max_us": round(float(np.max(d)) * 1e3, 3),
                    "algorithmic_bytes": int(b),
                    "gbs": round(b / (avg * 1e-3) / 1e9, 1)}
    layout["per_kernel_timing"] = "calls"
    dom = max(pk, key=lambda n: pk[n]["avg_us"])
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        O = oracle.default()
        one = W.SinkWorkload(sw.name, 1, H, S, D, sw.dtype, sw.bits,
                             sw.group_k, sw.group_v, sw.n_sink, sw.seed,
                             sw.key_kind, sw.value_kind, sw.desc)
        kx = W.gen_tensor(w, "K", range(H))
        vx = W.gen_tensor(w, "V", range(H))
        t0 = time.perf_counter()
        sc = O.sink_scores(kx, sw.dtype, H)
        ix = O.sink_select(sc, sw.n_sink)
        O.quant_keys_sink(kx, sw.dtype, H, sw.bits, sw.group_k, ix)
        O.quant_values(vx, sw.dtype, sw.bits, sw.group_v)
        O.sink_gather(kx, H, ix)
        O.sink_gather(vx, H, ix)
        dt = time.perf_counter() - t0
        cpu = {"value": round(sum(sink_bytes(one).values()) / dt / 1e9, 4),
               "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": (f"1 of {B} sequences ({H} heads x {S} tokens), the "
                          f"whole pass: {dt:.2f} s on 1 thread")}
    result = {
        "metric": METRIC + " (KIVI-Sink pass)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{sw.name}: {sw.desc}; step = kivi_sink_select + "
                         "kivi_quant_keys_sink + kivi_quant_values + two "
                         "kivi_sink_gather calls"),
            "step_algorithmic_bytes": int(step_bytes),
            "input_pool": P,
            "launch": "eager",
            "wall_s": round(t_wall, 4),
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "roofline": {
            "kernel": dom,
            "avg_us": pk[dom]["avg_us"],
            "bound": "hbm",
            "achieved": pk[dom]["gbs"],
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(pk[dom]["gbs"] / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(dom, sw.name, kernel_source_hash("sink")),
        },
        "per_kernel": pk,
        "kernel_source_hash": kernel_source_hash("sink"),
        "profile_layout": layout,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


# --------------------------------------------------------------------------
# per-token mixed precision over a prompt
# --------------------------------------------------------------------------

def mixed_bytes(mw):
    """Algorithmic bytes of one mixed-precision round trip, per launch: the
    scores read every key once; the partition reads the scores and writes
    both position lists; each set's quantizer reads its rows and writes
    codes and params; each dequantizer reads them back and writes the rows."""
    BH, S, D = mw.B * mw.H, mw.S, mw.D
    E = BH * S * D
    out = {"key_scores": E * 2 + mw.B * S * 4, "partition": mw.B * S * 8}
    for name, n, bits in (("hi", mw.n_hi, mw.hi_bits),
                          ("lo", S - mw.n_hi, mw.lo_bits)):
        kp = BH * (-(-n // mw.group_k)) * D * 8
        vp = BH * n * (-(-D // mw.group_v)) * 8
        rows = BH * n * D
        out[f"quant_keys_{name}"] = rows * 2 + rows * bits // 8 + kp
        out[f"quant_values_{name}"] = rows * 2 + rows * bits // 8 + vp
        out[f"dequant_keys_{name}"] = rows * bits // 8 + kp + rows * 2
        out[f"dequant_values_{name}"] = rows * bits // 8 + vp + rows * 2
    return out


def mixed_bench(args, mw, K, torch, dev):
    """One step = the mixed-precision round trip over one prompt: key-norm
    scores, the partition, both sets of keys and values quantized, and both
    sets dequantized back into full tensors.  Inputs rotate over a pool of
    prompts larger than the MALL."""
    tdt = torch.float16 if mw.dtype == W.FP16 else torch.bfloat16
    w = mw.tokens()
    B, H, S, D = mw.B, mw.H, mw.S, mw.D
    nb = mixed_bytes(mw)
    step_bytes = sum(nb.values())
    P = args.pool or 2
    inputs = []
    for p in range(P):
        kv = []
        for tensor in ("K", "V"):
            x = W.gen_tensor(w, tensor, pool=p)
            kv.append(torch.from_numpy(x.view(np.int16)).view(tdt).to(dev)
                      .view(B, H, S, D))
        inputs.append(tuple(kv))
    score = K.kivi_key_scores(inputs[0][0])
    hi, lo = K.kivi_partition_top(score, mw.n_hi)
    sets = [("hi", hi, mw.hi_bits), ("lo", lo, mw.lo_bits)]
    bufs = {}
    for name, pos, bits in sets:
        bufs["k" + name] = K.kivi_quant_keys_rows(inputs[0][0], pos, bits, mw.group_k)
        bufs["v" + name] = K.kivi_quant_values_rows(inputs[0][1], pos, bits, mw.group_v)
    k_out = torch.empty((B, H, S, D), dtype=tdt, device=dev)
    v_out = torch.empty_like(k_out)
    stream = torch.cuda.current_stream(dev)
    calls = [("key_scores", lambda k, v: K.kivi_key_scores(k, score=score)),
             ("partition", lambda k, v: K.kivi_partition_top(
                 score, mw.n_hi, pos_hi=hi, pos_lo=lo))]
    for name, pos, bits in sets:
        kb, vb = bufs["k" + name], bufs["v" + name]
        calls.append((f"quant_keys_{name}", lambda k, v, pos=pos, bits=bits, kb=kb:
                      K.kivi_quant_keys_rows(k, pos, bits, mw.group_k, codes=kb[0],
                                             scale=kb[1], zero=kb[2])))
        calls.append((f"quant_values_{name}", lambda k, v, pos=pos, bits=bits, vb=vb:
                      K.kivi_quant_values_rows(v, pos, bits, mw.group_v, codes=vb[0],
                                               scale=vb[1], zero=vb[2])))
    for name, pos, bits in sets:
        kb, vb = bufs["k" + name], bufs["v" + name]
        calls.append((f"dequant_keys_{name}", lambda k, v, pos=pos, bits=bits, kb=kb:
                      K.kivi_dequant_keys_rows(*kb, pos, k_out, bits, mw.group_k)))
        calls.append((f"dequant_values_{name}", lambda k, v, pos=pos, bits=bits, vb=vb:
                      K.kivi_dequant_values_rows(*vb, pos, v_out, bits, mw.group_v)))

    def step(i, mark=None):
        k, v = inputs[i % P]
        for a, (_, fn) in enumerate(calls):
            fn(k, v)
            if mark is not None:
                mark(a)

    disp = Dispatches(K)
    labels = launch_labels(K, [(n, lambda fn=fn: fn(*inputs[0]))
                               for n, fn in calls])
    for i in range(1, args.warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    base = max(args.warmup, 1)
    disp.eager()
    before = disp.n
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(base + i)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    disp.eager()
    layout = profile_layout(before, disp.n - before, labels)
    ms_per_step = start.elapsed_time(end) / args.steps

    # per call: its interval between plain events recorded between the
    # calls of K more back-to-back steps (call_intervals)
    pk = {}
    iv = call_intervals(torch, stream, step, len(calls), args.steps,
                        base + args.steps)
    for a, (name, _) in enumerate(calls):
        d = iv[a]
        avg = float(np.mean(d))
        pk[name] = {"avg_us": round(avg * 1e3, 3),
                    "median_us": round(float(np.median(d)) * 1e3, 3),
                    "algorithmic_bytes": int(nb[name]),
                    "gbs": round(nb[name] / (avg * 1e-3) / 1e9, 1)}
    layout["per_kernel_timing"] = "calls"
    dom = max(pk, key=lambda n: pk[n]["avg_us"])
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        O = oracle.default()
        one = W.MixedWorkload(mw.name, 1, H, S, D, mw.dtype, mw.hi_bits,
                              mw.lo_bits, mw.group_k, mw.group_v,
                              mw.hi_fraction, mw.seed, mw.key_kind,
                              mw.value_kind, mw.desc)
        kx = W.gen_tensor(w, "K", range(H))
        vx = W.gen_tensor(w, "V", range(H))
        t0 = time.perf_counter()
        ohi, olo = O.partition_top(O.sink_scores(kx, mw.dtype, H), mw.n_hi)
        for pos, bits in ((ohi, mw.hi_bits), (olo, mw.lo_bits)):
            kq = O.quant_keys_rows(kx, mw.dtype, H, bits, mw.group_k, pos)
            vq = O.quant_values_rows(vx, mw.dtype, H, bits, mw.group_v, pos)
            O.dequant_keys_rows(*kq, kx.shape, H, bits, mw.group_k, pos, mw.dtype)
            O.dequant_values_rows(*vq, vx.shape, H, bits, mw.group_v, pos, mw.dtype)
        dt = time.perf_counter() - t0
        cpu = {"value": round(sum(mixed_bytes(one).values()) / dt / 1e9, 4),
               "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": (f"1 of {B} sequences ({H} heads x {S} tokens), the "
                          f"whole round trip: {dt:.2f} s on 1 thread")}
    result = {
        "metric": METRIC + " (per-token mixed precision round trip)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{mw.name}: {mw.desc}; step = key scores + "
                         "partition + 4 set quantizers + 4 set dequantizers"),
            "n_hi": mw.n_hi,
            "step_algorithmic_bytes": int(step_bytes),
            "input_pool": P,
            "launch": "eager",
            "wall_s": round(t_wall, 4),
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "roofline": {
            "kernel": dom,
            "avg_us": pk[dom]["avg_us"],
            "bound": "hbm",
            "achieved": pk[dom]["gbs"],
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(pk[dom]["gbs"] / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(dom, mw.name, kernel_source_hash("mixed")),
        },
        "per_kernel": pk,
        "kernel_source_hash": kernel_source_hash("mixed"),
        "profile_layout": layout,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


# --------------------------------------------------------------------------
# rocprofv3 summaries (profiles/): the recipe and the summarizers
# --------------------------------------------------------------------------

def profile_recipe(workload, repo="<repo>", out="<dir>"):
    """The commands behind a workload's profiles: a plain run, a
    kernel-trace run and one counter pass per counter, all of the same
    launch configuration as the default benchmark run; the counter scale
    comes from a plain device copy of known size (--calibrate-copy)."""
    b = f"python3 {repo}/bench.py --workload {workload} --no-cpu-baseline"
    return {
        "plain": f"{b} --steps 20 --warmup 3 > {out}/plain.json",
        "trace": (f"rocprofv3 --kernel-trace --stats -f csv -d {out}/trace "
                  f"-o bench -- {b} --steps 20 --warmup 3 > {out}/profiled.json"),
        "fetch": (f"rocprofv3 --pmc FETCH_SIZE -f csv -d {out}/pmc_fetch -o bench"
                  f" -- {b} --steps 2 --warmup 1 > {out}/fetch.json"),
        "write": (f"rocprofv3 --pmc WRITE_SIZE -f csv -d {out}/pmc_write -o bench"
                  f" -- {b} --steps 2 --warmup 1 > {out}/write.json"),
        "copy_fetch": (f"rocprofv3 --pmc FETCH_SIZE -f csv -d <copydir>/fetch -o "
                       f"copy -- python3 {repo}/bench.py --calibrate-copy 512 "
                       "--steps 3"),
        "copy_write": (f"rocprofv3 --pmc WRITE_SIZE -f csv -d <copydir>/write -o "
                       f"copy -- python3 {repo}/bench.py --calibrate-copy 512 "
                       "--steps 3"),
    }


def _json_line(path):
    """The benchmark's result line in a captured stdout."""
    found = None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                try:
                    d = json.loads(line)
                except ValueError:
                    continue
                if "metric" in d or "calibration" in d:
                    found = d
    if found is None:
        raise SystemExit(f"no result line in {path}")
    return found


def _one_csv(d, suffix):
    import glob
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if len(hits) != 1:
        raise SystemExit(f"expected one *{suffix} under {d}, found {hits}")
    return hits[0]


def _template(name):
    """The kernel's template signature without its parameter list."""
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def _library_dispatches(rows, value_of=None):
    """Per dispatch of a library kernel (name in namespace kivi), in the
    order the GPU ran them: (kernel name, start, end, value) where value
    comes from value_of(rows of that dispatch) (counter runs) or None.
    The order is the dispatch id's, the order of submission: every step
    runs on one stream, whose kernels run in that order, while the
    profiler's start timestamps of back-to-back kernels can land a few
    hundred nanoseconds out of order."""
    import collections
    by = collections.OrderedDict()
    for r in rows:
        if "kivi::" not in r["Kernel_Name"]:
            continue
        by.setdefault(r["Dispatch_Id"], []).append(r)
    out = []
    for rs in by.values():
        r0 = rs[0]
        out.append((int(r0["Dispatch_Id"]), r0["Kernel_Name"],
                    int(r0["Start_Timestamp"]), int(r0["End_Timestamp"]),
                    value_of(rs) if value_of else None))
    out.sort(key=lambda x: x[0])
    return [x[1:] for x in out]


def _timed(disp, layout):
    """The dispatches of the timed region, each with its step label."""
    a = layout["dispatches_before_timed"]
    n = layout["timed_dispatches"]
    labels = layout["step_launches"]
    if len(disp) < a + n or n % len(labels):
        raise SystemExit(f"trace holds {len(disp)} library dispatches; the "
                         f"layout asks for {a} + {n} ({len(labels)} a step)")
    sel = disp[a:a + n]
    return [(labels[j % len(labels)],) + d for j, d in enumerate(sel)]


def summarize_trace(d, workload):
    import csv
    prof = _json_line(os.path.join(d, "profiled.json"))
    plain = _json_line(os.path.join(d, "plain.json"))
    rows = list(csv.DictReader(open(_one_csv(os.path.join(d, "trace"),
                                             "kernel_trace.csv"))))
    disp = _library_dispatches(rows)
    timed = _timed(disp, prof["profile_layout"])
    per = {}
    for label, name, t0, t1, _ in timed:
        e = per.setdefault(label, {"template": _template(name), "d": []})
        if e["template"] != _template(name):
            raise SystemExit(f"label {label} maps to two kernels")
        e["d"].append((t1 - t0) / 1e3)
    lay = prof["profile_layout"]
    timing = lay.get("per_kernel_timing", "first_launch")
    per_call = {}          # call -> its launches' summed duration, per call
    call = -1
    for label, _, t0, t1, _ in timed:
        call += "#" not in label
        c = per_call.setdefault(label.split("#")[0], {})
        c[call] = c.get(call, 0.0) + (t1 - t0) / 1e3
    alld = {}
    for name, t0, t1, _ in disp:
        alld.setdefault(_template(name), []).append((t1 - t0) / 1e3)
    rec = profile_recipe(workload)
    fam = ("cache" if workload in W.CACHE_WORKLOADS else "attend"
           if workload in W.ATTEND_WORKLOADS else "sink"
           if workload in W.SINK_WORKLOADS else "mixed"
           if workload in W.MIXED_WORKLOADS else "flush")
    L = []
    L.append(f"# rocprofv3 kernel trace: {workload}\n")
    L.append(f"workload: {plain['config']['workload']}\n")
    L.append("commands (run from /tmp with TMPDIR=/tmp, one after the other "
             "on one GPU):")
    L.append(f"  {rec['plain']}")
    L.append(f"  {rec['trace']}")
    L.append(f"  python3 <repo>/bench.py --summarize-trace <dir> --workload "
             f"{workload}   (this summary)\n")
    L.append(f"kernel source hash (bench.py kernel_source_hash, family {fam}): "
             f"{kernel_source_hash(fam)}; profiled run's hash "
             f"{prof.get('kernel_source_hash')}\n")
    L.append(f"Timed region of the profiled run: library dispatches "
             f"{lay['dispatches_before_timed']} .. "
             f"{lay['dispatches_before_timed'] + lay['timed_dispatches'] - 1} "
             f"({prof['steps']} steps of {len(lay['step_launches'])} launches; "
             f"launch: {plain['config'].get('launch')}), per launch of a step:")
    pk_plain = plain.get("per_kernel", {})
    pk_prof = prof.get("per_kernel", {})
    L.append(f"{'launch':24s} {'n':>4s} {'rocprof avg us':>15s} {'min':>8s} "
             f"{'max':>8s} {'events, plain run':>18s}   template")
    for label, e in per.items():
        dd = e["d"]
        ev = pk_plain.get(label, {}).get("avg_us")
        L.append(f"{label:24s} {len(dd):4d} {np.mean(dd):15.2f} {min(dd):8.2f} "
                 f"{max(dd):8.2f} {ev if ev is not None else '-':>18}   "
                 f"{e['template']}")
    if timing == "calls":
        L.append("\nPer call (its launches summed), against the benchmark's "
                 "own per-call intervals (plain events between the calls of "
                 "back-to-back steps, each interval also holding the dispatch "
                 "gap before the call):")
        L.append(f"{'call':24s} {'rocprof avg us':>15s} {'intervals, plain':>17s}"
                 f" {'intervals, profiled':>20s}")
        for c, dd in per_call.items():
            a = pk_plain.get(c, {}).get("avg_us")
            b = pk_prof.get(c, {}).get("avg_us")
            L.append(f"{c:24s} {np.mean(list(dd.values())):15.2f} "
                     f"{a if a is not None else '-':>17} "
                     f"{b if b is not None else '-':>20}")
    L.append("\nEvery dispatch of the run (setup, warmup, timed region, "
             "per-kernel pass), for reference:")
    for t, dd in alld.items():
        L.append(f"  {len(dd):4d} x {np.mean(dd):9.2f} us avg   {t}")
    dom = plain["roofline"]["kernel"]
    b = pk_plain[dom]["algorithmic_bytes"]
    avg = (float(np.mean(list(per_call[dom].values()))) if timing == "calls"
           else float(np.mean(per[dom]["d"])))
    gbs = b / (avg * 1e-6) / 1e9
    L.append(f"\ndominant kernel {dom}: {b} algorithmic bytes / {avg:.2f} us "
             f"(rocprof, timed region) = {gbs:.1f} GB/s, frac {gbs / PEAK_HBM_GBS:.4f}")
    L.append(f"plain run: value {plain['value']} GB/s ({plain['pct_of_peak']}% "
             f"of 8 TB/s), {plain['ms_per_step'] * 1e3:.1f} us per step; "
             f"roofline {dom} {plain['roofline']['avg_us']} us by events, "
             f"{plain['roofline']['achieved']} GB/s, frac "
             f"{plain['roofline']['frac']} ({100 * (plain['roofline']['avg_us'] / avg - 1):+.1f}% "
             f"against rocprof)")
    L.append(f"profiled run: value {prof['value']} GB/s, "
             f"{prof['ms_per_step'] * 1e3:.1f} us per step; roofline {dom} "
             f"{prof['roofline']['avg_us']} us, frac {prof['roofline']['frac']} "
             f"({100 * (prof['roofline']['avg_us'] / avg - 1):+.1f}% against "
             f"rocprof in the same run"
             + ("" if timing == "calls" else
                "; under the profiler its dispatch interception falls between "
                "the armed events and the kernel") + ")")
    L.append(f"per-kernel timing: {timing} ("
             + ("intervals between plain events between the calls of "
                "back-to-back steps" if timing == "calls" else
                "HIP events recorded at each kernel's own dispatch, in an "
                "eager pass after the timed region") + ")")
    print("\n".join(L))


def summarize_traffic(d, workload, copy_dir, path=None):
    """HBM bytes per launch from the FETCH_SIZE and WRITE_SIZE passes, over
    the timed region's dispatches, scaled by the same counters on a plain
    copy of known size; prints the summary and updates the traffic record
    at path (default profiles/traffic.json)."""
    import csv

    def value(rs):
        return sum(float(r["Counter_Value"]) for r in rs)

    def counter(sub, js):
        prof = _json_line(os.path.join(d, js))
        rows = list(csv.DictReader(open(_one_csv(os.path.join(d, sub),
                                                 "counter_collection.csv"))))
        lay = prof["profile_layout"]
        timed = _timed(_library_dispatches(rows, value), lay)
        calls = lay.get("per_kernel_timing") == "calls"
        per = {}
        call = -1
        for idx, (label, name, _, _, v) in enumerate(timed):
            # per call (its launches summed: name, name#2, ...) where the
            # benchmark times calls, else per dispatch; a label that recurs
            # in a step (a ring store per decode token) averages over its
            # calls or launches
            call += "#" not in label
            key = label.split("#")[0] if calls else label
            acc = per.setdefault(key, {})
            slot = call if calls else idx
            acc[slot] = acc.get(slot, 0.0) + v
        return prof, {k: float(np.mean(list(v.values()))) for k, v in per.items()}

    def copy_scale(sub, per_launch):
        rows = list(csv.DictReader(open(_one_csv(os.path.join(copy_dir, sub),
                                                 "counter_collection.csv"))))
        calib = _json_line(os.path.join(copy_dir, sub + ".json"))
        n = calib["size_bytes"] * per_launch
        vals = {}
        for r in rows:
            if "copyBuffer" in r["Kernel_Name"]:
                vals.setdefault(r["Dispatch_Id"], 0.0)
                vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
        kib = float(np.median(list(vals.values())))
        return n / (kib * 1024.0)

    prof, fetch = counter("pmc_fetch", "fetch.json")
    _, write = counter("pmc_write", "write.json")
    fs = copy_scale("fetch", 1)
    wsc = copy_scale("write", 1)
    fam = ("cache" if workload in W.CACHE_WORKLOADS else "attend"
           if workload in W.ATTEND_WORKLOADS else "sink"
           if workload in W.SINK_WORKLOADS else "mixed"
           if workload in W.MIXED_WORKLOADS else "flush")
    h = kernel_source_hash(fam)
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    rec = profile_recipe(workload)
    L = [f"# HBM traffic per launch from rocprofv3 counters: {workload}\n",
         f"workload: {prof['config']['workload']}\n",
         "commands (run from /tmp with TMPDIR=/tmp), one counter per pass:",
         f"  {rec['fetch']}", f"  {rec['write']}", f"  {rec['copy_fetch']}",
         f"  {rec['copy_write']}",
         f"  python3 <repo>/bench.py --summarize-traffic <dir> --copy-dir "
         f"<copydir> --workload {workload}   (this summary)\n",
         f"Scale from a plain device copy of 512e6 bytes "
         f"(__amd_rocclr_copyBuffer): bytes = FETCH_SIZE KiB * 1024 * "
         f"{fs:.4f}; WRITE_SIZE KiB * 1024 * {wsc:.4f}\n",
         f"kernel source hash (family {fam}): {h}\n",
         "averages over the timed region's dispatches, "
         + ("per call of a step (its launches summed):"
            if prof["profile_layout"].get("per_kernel_timing") == "calls"
            else "per launch:"),
         f"{'launch':24s} {'FETCH KiB':>11s} {'WRITE KiB':>11s} "
         f"{'read MB':>9s} {'write MB':>9s} {'HBM MB':>9s} {'alg MB':>9s} "
         f"{'HBM/alg':>8s}"]
    pk = prof.get("per_kernel", {})
    for label in fetch:
        rb = fetch[label] * 1024 * fs
        wb = write.get(label, 0.0) * 1024 * wsc
        alg = pk.get(label, {}).get("algorithmic_bytes")
        L.append(f"{label:24s} {fetch[label]:11.0f} {write.get(label, 0):11.0f} "
                 f"{rb / 1e6:9.2f} {wb / 1e6:9.2f} {(rb + wb) / 1e6:9.2f} "
                 + (f"{alg / 1e6:9.2f} {(rb + wb) / alg:8.3f}" if alg else
                    f"{'-':>9s} {'-':>8s}"))
        if alg:
            data[f"{label}@{workload}"] = {
                "source_hash": h, "hbm_bytes_per_launch": int(rb + wb),
                "fetch_bytes": int(rb), "write_bytes": int(wb),
                "algorithmic_bytes": int(alg), "fetch_scale": round(fs, 4),
                "write_scale": round(wsc, 4)}
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print("\n".join(L))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="roundtrip",
                    choices=sorted(W.WORKLOADS) + sorted(W.CACHE_WORKLOADS)
                    + sorted(W.ATTEND_WORKLOADS) + sorted(W.SINK_WORKLOADS)
                    + sorted(W.MIXED_WORKLOADS))
    ap.add_argument("--pool", type=int, default=0,
                    help="distinct input sets (0: enough to exceed 1 GB)")
    ap.add_argument("--cpu-sample-bh", type=int, default=0,
                    help="bh slices of the CPU-baseline sample (0: enough "
                         "for about 2^27 elements per tensor)")
    ap.add_argument("--cpu-threads", type=int,
                    default=min(16, os.cpu_count() or 1),
                    help="threads of the multi-threaded oracle timing")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="instead of the benchmark, time a plain device copy "
                         "of MB megabytes (the reference kernel used to scale "
                         "rocprofv3 byte counters) and a plain read (sum)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--single-calls", action="store_true",
                    help="decode/tiny: time the separate key and value calls "
                         "instead of the K+V calls")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print the kernel-trace summary of a profiled run "
                         "(DIR holds plain.json, profiled.json and trace/; "
                         "see profile_recipe)")
    ap.add_argument("--summarize-traffic", metavar="DIR",
                    help="print the HBM traffic summary of the counter runs "
                         "in DIR and update profiles/traffic.json")
    ap.add_argument("--copy-dir", metavar="DIR",
                    help="the copy-calibration counter runs (fetch/, write/, "
                         "fetch.json, write.json)")
    ap.add_argument("--traffic-json", metavar="PATH", default=None,
                    help="the traffic record --summarize-traffic updates "
                         "(default profiles/traffic.json)")
    ap.add_argument("--launch", choices=("auto", "graphs", "eager"),
                    default="auto",
                    help="timed steps as HIP graph replays or eager launches; "
                         "auto: graphs for launch-bound steps (under 16 MB "
                         "of traffic per launch), eager otherwise (a replay "
                         "costs more than a launch it does not hide)")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.workload)
        return
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic, args.workload, args.copy_dir,
                          args.traffic_json)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus},"
              f" WORLD_SIZE {world}); the KIVI flush needs no collectives: "
              "each GPU quantizes its own heads, so the figure for N GPUs is "
              "N times the one-GPU figure and is not measured here.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_quantization_kivi_amd as K

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(torch, dev, args.calibrate_copy, args.steps)
        return
    if args.workload in W.ATTEND_WORKLOADS:
        attend_bench(args, W.ATTEND_WORKLOADS[args.workload], K, torch, dev)
        return
    if args.workload in W.CACHE_WORKLOADS:
        cache_bench(args, W.CACHE_WORKLOADS[args.workload], K, torch, dev)
        return
    if args.workload in W.SINK_WORKLOADS:
        sink_bench(args, W.SINK_WORKLOADS[args.workload], K, torch, dev)
        return
    if args.workload in W.MIXED_WORKLOADS:
        mixed_bench(args, W.MIXED_WORKLOADS[args.workload], K, torch, dev)
        return
    w = W.WORKLOADS[args.workload]
    tdt = torch.float16 if w.dtype == W.FP16 else torch.bfloat16

    in_bytes = 2 * w.elems * 2
    pool = args.pool or max(2, int(np.ceil(1.0e9 / in_bytes)))
    if pool % 2:
        pool += 1   # fused kernels read the set the quantizers do not
    pool = min(pool, 64)
    inputs = []
    for p in range(pool):
        kv = []
        for tensor in ("K", "V"):
            x = W.gen_tensor(w, tensor, pool=p)
            kv.append(torch.from_numpy(x.view(np.int16)).view(tdt).to(dev))
        inputs.append(tuple(kv))

    # decode-size flushes go through the K+V calls (one launch per pair of
    # rows); --single-calls times the separate key and value calls instead
    paired = w.name in ("tiny", "decode") and not args.single_calls
    steps = make_steps(K, w, inputs, torch, paired)
    step_bytes = sum(s[2] for s in steps)
    stream = torch.cuda.current_stream(dev)

    disp = Dispatches(K)
    labels = launch_labels(K, [(name, lambda fn=fn: fn(0))
                               for name, _, _, fn in steps])
    for i in range(1, args.warmup):
        for _, _, _, fn in steps:
            fn(i)
    torch.cuda.synchronize()

    def stats(name, op, b, d):
        avg = float(np.mean(d))
        return {
            "avg_us": round(avg * 1e3, 3),
            "median_us": round(float(np.median(d)) * 1e3, 3),
            "min_us": round(float(np.min(d)) * 1e3, 3),
            "max_us": round(float(np.max(d)) * 1e3, 3),
            "algorithmic_bytes": int(b),
            "gbs": round(b / (avg * 1e-3) / 1e9, 1),
        }

    def event_pairs(n):
        ev = [(torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:          # torch creates its events on first record
            a.record(stream)
            b.record(stream)
        return ev

    # Pass 1, the timed region: exactly K steps between two events on the
    # launch stream, with nothing else in the queue.  A launch-bound step
    # (a decode-time flush) is one HIP graph replay: the step's launches
    # depend only on the step index modulo `period` (input sets and code
    # sets rotate), so one graph per phase is captured once, before timing,
    # and replayed in order; kernels and arguments are exactly those of the
    # eager calls.
    period = int(np.lcm(pool, N_CODE_SETS))
    use_graphs = launch_bound(args, step_bytes, len(labels))
    graphs = None
    disp.eager()
    if use_graphs:
        graphs = []
        cap = torch.cuda.Stream(device=dev)
        for ph in range(period):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for _, _, _, fn in steps:
                    fn(ph)
            graphs.append((g, disp.captured()))
        for g, k in graphs:           # first replays happen outside the timing
            g.replay()
            disp.replayed(k)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    base = max(args.warmup, 1)
    torch.cuda.synchronize()
    before = disp.n
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        if graphs is not None:
            g, k = graphs[(base + i) % period]
            g.replay()
            disp.replayed(k)
        else:
            for _, _, _, fn in steps:
                fn(base + i)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    disp.eager()
    layout = profile_layout(before, disp.n - before, labels)
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    # Pass 2, kernel durations, over K more steps.  Steps timed eagerly (the
    # HBM-bound workloads) are launched exactly as in the timed region, with
    # a plain event between calls (call_intervals): each kernel's interval
    # is its share of a back-to-back step, including the write-back of the
    # kernel before it that it competes with, so the intervals add up to the
    # step and agree with a profiler's durations of the timed region.
    # Launch-bound steps (graph replays in the timed region) would count the
    # host's launch gaps that way, so there every launch records its own
    # start/stop pair at its dispatch instead (kivi_time_next_launch,
    # hipExtLaunchKernel): the kernel alone.  The dominant kernel (longest
    # average) gives the roofline.
    n_k = len(steps)
    base = max(args.warmup, 1) + args.steps
    per_kernel = {}
    if graphs is None:
        def timed_step(i, mark):
            for jj, (_, _, _, fn) in enumerate(steps):
                fn(i)
                mark(jj)

        iv = call_intervals(torch, stream, timed_step, n_k, args.steps, base)
        for jj, (name, op, b, _) in enumerate(steps):
            per_kernel[name] = stats(name, op, b, iv[jj])
        timing = "calls"
    else:
        kev = [event_pairs(n_k) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            for jj, (_, _, _, fn) in enumerate(steps):
                K.kivi_time_next_launch(*kev[i][jj])
                fn(base + i)
        torch.cuda.synchronize()
        for jj, (name, op, b, _) in enumerate(steps):
            d = [kev[i][jj][0].elapsed_time(kev[i][jj][1])
                 for i in range(args.steps)]
            per_kernel[name] = stats(name, op, b, d)
        timing = "first_launch"
    layout["per_kernel_timing"] = timing
    dom = max(per_kernel, key=lambda n: per_kernel[n]["avg_us"])
    dk = per_kernel[dom]

    src_hash = kernel_source_hash()
    traffic = load_traffic(dom, w.name, src_hash)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name}: {w.desc}; K and V [BH={w.BH}, S={w.S}, "
                         f"D={w.D}] {'fp16' if w.dtype == 0 else 'bf16'}, "
                         f"bits={w.bits}, key group={w.group_k} tokens, "
                         f"value group={w.group_v} channels; step = "
                         + " + ".join(s[0] for s in steps)),
            "step_algorithmic_bytes": int(step_bytes),
            "input_pool": pool,
            "launch": (f"one HIP graph replay per step ({period} phases)"
                       if use_graphs else "eager"),
            "wall_s": round(t_wall, 4),
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "roofline": {
            "kernel": dom,
            "avg_us": dk["avg_us"],
            "bound": "hbm",
            "achieved": dk["gbs"],
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(dk["gbs"] / PEAK_HBM_GBS, 4),
            "traffic": traffic,
        },
        "per_kernel": per_kernel,
        "per_kernel_note": ("value: K steps with no per-launch events; "
                            "per_kernel and roofline: a second pass of K "
                            "steps, " + (
                                "each call's interval between plain events "
                                "recorded between the calls of back-to-back "
                                "steps" if timing == "calls" else
                                "every launch timed by HIP events at its own "
                                "dispatch")),
        "kernel_source_hash": src_hash,
        "profile_layout": layout,
    }
    if not args.no_cpu_baseline:
        n_bh = args.cpu_sample_bh or max(1, (1 << 27) // (w.S * w.D))
        n_bh = min(n_bh, w.BH)
        result["cpu_baseline"] = cpu_baseline(w, n_bh, steps,
                                              args.cpu_threads)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
