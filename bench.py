"""Throughput of the fused per-shard ZeRO Adam step on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
shard plan, gather of the P rank-local gradient slices, rank-order fp32
mean, Adam moments with bias correction, fp32 master update and the
16-bit working-copy write-back.  Default workload: the 7.5B-parameter model
at P=64, rank 63's shard (M = 117,187,500), fp16 gradients.

Other workloads (--workload): the two parameter-list shapes go through the
multi-tensor chunk table (zs_fused_shard_step_multi, one launch per step);
the all-shard workloads (full-N gradient buffers) run one zs_fused_shard_step
launch per shard, P launches per step.

Prints ONE JSON line on stdout.  Inputs are resident in HBM before the timed
region; the timed region is K back-to-back steps between two device
synchronisations, timed with HIP events on the stream the kernel runs on.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "shard elements/s and achieved HBM GB/s (% of MI355X peak), fused shard Adam"
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "adam_zs_shard_amd", "csrc")
# the step's device code and launch logic (not the host offload or the probes)
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in (
    "zs_device.h", "zs_fused.h", "zs_fused_f16.hip", "zs_fused_bf16.hip", "zs_table.hip",
    "zs_unfused.hip", "zs_common.hip", "zs_internal.h", "zs_capi.cpp")]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, form: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    there are none for this workload and update form, or the kernel sources
    changed since."""
    try:
        with open(COUNTERS_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    rec = data.get(workload)
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    if rec.get("form", "standard") != form:
        return None
    return rec.get("hbm_bytes_per_launch")


def _time_steps(run_step, steps: int, warmup: int, stream):
    import torch

    for i in range(warmup):
        run_step(i)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(steps):
        run_step(warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    return ev0.elapsed_time(ev1) / steps, wall


def cpu_baseline(gdt: str, pdt: str, grads_host, w, m, v, threads: int, form: str):
    """The oracle, as it stands, on a contiguous sample of the same shard,
    split over `threads` host threads (elements are independent)."""
    import numpy as np

    import oracle

    n = w.size
    bounds = np.linspace(0, n, threads + 1).astype(np.int64)
    param = np.empty(n, np.uint16)

    def run(a, b):
        oracle.step_elems(gdt, [g[a:b] for g in grads_host], w[a:b], m[a:b], v[a:b], pdt,
                          1e-3, 0.9, 0.999, 1e-8, 1, form, param=param[a:b])

    ths = [threading.Thread(target=run, args=(int(bounds[i]), int(bounds[i + 1])))
           for i in range(threads)]
    t0 = time.perf_counter()
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    return time.perf_counter() - t0


def host_threads() -> int:
    """The host CPUs this process may use: its affinity mask, capped by
    OMP_NUM_THREADS when that is set (the CPU share a GPU host gives one
    GPU's jobs)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return max(1, min(n, cap) if cap > 0 else n)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def _state(wl, w):
    """(m, v) for the workload's form: None where the form uses no such state."""
    import torch

    from adam_zs_shard_amd import zshard as z

    f = z.FORMS[wl.form]
    m = torch.zeros_like(w) if f != z.ZS_SGD else None
    v = torch.zeros_like(w) if f in (z.ZS_ADAM_STANDARD, z.ZS_ADAM_PAGE1_LITERAL) else None
    return m, v


def _bytes_per_elem(wl):
    from adam_zs_shard_amd import zshard as z

    return 2 * wl.p + z.BYTES_PER_ELEM[z.FORMS[wl.form]]


def _single_setup(args):
    """Inputs of one shard of a single-tensor workload, resident in HBM: P
    separate gradient slices, the fp32 state and the working copy."""
    import torch

    from adam_zs_shard_amd import zshard as z
    from zs_synth import WORKLOADS, seed_for
    from zs_synth.gen import normal

    wl = WORKLOADS[args.workload]
    k = wl.shards[-1]
    M, s, e = z.zs_plan_shards(wl.n, wl.p)
    L = e[k] - s[k]
    dev = "cuda"
    td = {"f16": torch.float16, "bf16": torch.bfloat16}
    print(f"[bench] {wl.name}: N={wl.n} P={wl.p} k={k} L={L}", file=sys.stderr, flush=True)
    grads = [normal(L, wl.grad_std, seed_for(20261202, r, 1, 1, k), td[wl.grad_dtype], dev)
             for r in range(wl.p)]
    w = normal(L, wl.w_std, seed_for(20261202, -1, 0, 2, k), torch.float32, dev)
    m, v = _state(wl, w)
    if wl.param_layout == "full":
        param = torch.empty(wl.n, dtype=td[wl.param_dtype], device=dev)
        pbase = 0
    else:
        param = torch.empty(L, dtype=td[wl.param_dtype], device=dev)
        pbase = s[k]
    assert wl.grad_layout == "slice"
    torch.cuda.synchronize()
    return dict(wl=wl, k=k, L=L, s=s, grads=grads, w=w, m=m, v=v, param=param, pbase=pbase,
                gbase=s[k], stream=torch.cuda.current_stream())


def bench_single(args):
    """Fused single-tensor step on one shard with P separate gradient slices."""
    from adam_zs_shard_amd import zshard as z

    x = _single_setup(args)
    wl, k, L = x["wl"], x["k"], x["L"]
    grads, w, m, v, param, stream = x["grads"], x["w"], x["m"], x["v"], x["param"], x["stream"]

    def step(i):
        z.zs_fused_shard_step(wl.n, wl.p, k, grads, w, m, v, param,
                              z.hparams(wl.lr, wl.beta1, wl.beta2, wl.eps, i + 1, wl.form),
                              grad_base=x["gbase"], param_base=x["pbase"],
                              stream=stream.cuda_stream)

    ms, wall = _time_steps(step, args.steps, args.warmup, stream)
    cpu = None if args.no_cpu_baseline else _cpu_leg(args, wl, grads, w, m, v, f"shard {k}")
    return dict(wl=wl, k=k, elems=L, ms=ms, wall=wall, bytes_per_elem=_bytes_per_elem(wl),
                launches=1, launch_elems=L, cpu=cpu)


def bench_unfused(args):
    """The unfused pair on the same shard: zs_reduce_scatter_mean_local stores
    the fp32 rank-order mean (2P + 4 B/element), then zs_adam_step reads it
    (the form's bytes + 4).  Each kernel is also timed alone; the roofline
    entry is the mean kernel's, which moves most of the bytes."""
    import torch

    from adam_zs_shard_amd import zshard as z

    x = _single_setup(args)
    wl, k, L = x["wl"], x["k"], x["L"]
    grads, w, m, v, param, stream = x["grads"], x["w"], x["m"], x["v"], x["param"], x["stream"]
    gmean = torch.empty(L, dtype=torch.float32, device="cuda")
    pslice = param.narrow(0, x["s"][k], L) if wl.param_layout == "full" else param
    st = stream.cuda_stream

    def mean(i):
        z.zs_reduce_scatter_mean_local(grads, wl.n, wl.p, k, gmean, grad_base=x["gbase"],
                                       stream=st)

    def adam(i):
        z.zs_adam_step(gmean, w, m, v, pslice, L,
                       z.hparams(wl.lr, wl.beta1, wl.beta2, wl.eps, i + 1, wl.form), stream=st)

    def pair(i):
        mean(i)
        adam(i)

    ms, wall = _time_steps(pair, args.steps, args.warmup, stream)
    ms_mean, _ = _time_steps(mean, args.steps, args.warmup, stream)
    ms_adam, _ = _time_steps(adam, args.steps, args.warmup, stream)
    b_mean = 2 * wl.p + 4
    b_adam = z.BYTES_PER_ELEM[z.FORMS[wl.form]] + 4
    cpu = None if args.no_cpu_baseline else _cpu_leg(args, wl, grads, w, m, v, f"shard {k}")
    return dict(wl=wl, k=k, elems=L, ms=ms, wall=wall, bytes_per_elem=b_mean + b_adam,
                launches=2, launch_elems=L, cpu=cpu,
                dominant=dict(name="mean_kernel", ms=ms_mean, bytes_per_elem=b_mean),
                extra={"path": "unfused (zs_reduce_scatter_mean_local + zs_adam_step)",
                       "mean_kernel_ms": ms_mean, "adam_kernel_ms": ms_adam,
                       "adam_kernel_gbs": b_adam * L / (ms_adam / 1e3) / 1e9})


def _cpu_leg(args, wl, grads, w, m, v, label):
    """The oracle on a contiguous sample of one shard's elements: once on all
    the host threads this process may use, once on one thread (an eighth of
    the sample)."""
    import numpy as np
    import torch

    L = w.numel()
    S = min(L, args.cpu_sample)
    a0 = (L - S) // 2
    gh = [g[a0:a0 + S].view(torch.int16).cpu().numpy().view(np.uint16) for g in grads]
    wh = w[a0:a0 + S].cpu().numpy().copy()
    mh = m[a0:a0 + S].cpu().numpy().copy() if m is not None else np.zeros(S, np.float32)
    vh = v[a0:a0 + S].cpu().numpy().copy() if v is not None else np.zeros(S, np.float32)
    thr = host_threads()
    secs = cpu_baseline(wl.grad_dtype, wl.param_dtype, gh, wh, mh, vh, thr, wl.form)
    S1 = max(1, S // 8)
    secs1 = cpu_baseline(wl.grad_dtype, wl.param_dtype, [g[:S1] for g in gh], wh[:S1].copy(),
                         mh[:S1].copy(), vh[:S1].copy(), 1, wl.form)
    try:
        visible = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        visible = os.cpu_count() or 1
    return {"value": S / secs, "unit": "elements/s", "cores": thr, "kind": "oracle",
            "sample": f"{S} contiguous elements from the middle of {label} ({wl.p} ranks), one "
                      f"step, {secs:.2f} s wall on {thr} threads; one thread: the first {S1} "
                      f"of them, {secs1:.2f} s",
            "one_thread": S1 / secs1, "cpu_model": cpu_model(), "cpus_visible": visible,
            "os_cpu_count": os.cpu_count()}


def bench_multi(args):
    """Multi-tensor step of one shard of a parameter list, through the chunk table."""
    import torch

    from adam_zs_shard_amd import zshard as z
    from zs_synth import WORKLOADS, make

    wl = WORKLOADS[args.workload]
    k = wl.shards[0] if args.shard is None else args.shard
    numel = [n for _, n in wl.tensors]
    M, s, e = z.zs_plan_shards(wl.n, wl.p)
    L = e[k] - s[k]
    dev = "cuda"
    td = {"f16": torch.float16, "bf16": torch.bfloat16}
    if args.chunk <= 0:  # the library's chunk rule for this shard
        npieces = len(z.zs_plan_chunks(numel, wl.p, k, 8)[0])
        args.chunk = z.zs_mt_chunk_elems(L, npieces)
    pieces, nchunks = z.zs_plan_chunks(numel, wl.p, k, args.chunk)
    print(f"[bench] {wl.name}: N={wl.n} P={wl.p} k={k} L={L} pieces={len(pieces)} "
          f"chunks={nchunks} chunk_elems={args.chunk}", file=sys.stderr, flush=True)
    grads = [make.normal_grad(wl, r, 1, L, dev, stream=k) for r in range(wl.p)]
    w = make.initial_w(wl, k, L, dev)
    m, v = _state(wl, w)
    params = {}
    for (t, _, _, _) in pieces:
        if t not in params:
            params[t] = torch.empty(numel[t], dtype=td[wl.param_dtype], device=dev)
    def at(x, off):
        return None if x is None else x.data_ptr() + off

    ptrs = [dict(w=at(w, 4 * so), m=at(m, 4 * so), v=at(v, 4 * so),
                 param=params[t].data_ptr() + 2 * to, grads=[g.data_ptr() + 2 * so for g in grads])
            for (t, to, so, ln) in pieces]
    stream = torch.cuda.current_stream()
    # one table for the whole shard, or (--bucket-elems) one per bucket of
    # consecutive pieces holding at least that many elements (zs_plan_buckets),
    # each with the chunk length the library gives for the bucket on its own
    if args.bucket_elems > 0:
        of, nb = z.zs_plan_buckets(pieces, args.bucket_elems)
        groups = [[i for i in range(len(pieces)) if of[i] == b] for b in range(nb)]
    else:
        groups = [list(range(len(pieces)))]
    tables, keep = [], []
    for g in groups:
        sub = [pieces[i] for i in g]
        chunk = args.chunk
        if len(groups) > 1:
            chunk = z.zs_mt_chunk_elems(sum(pc[3] for pc in sub), 1)
        nch = sum((ln + chunk - 1) // chunk for (_, _, _, ln) in sub)
        nb = z.zs_mt_workspace_bytes(len(sub), nch, wl.p)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        keep.append(ws)
        tables.append(z.zs_mt_upload(sub, [ptrs[i] for i in g], wl.p, wl.grad_dtype,
                                     wl.param_dtype, chunk, ws, nb, stream=stream.cuda_stream))
    torch.cuda.synchronize()

    if args.graph:
        # captured once and replayed: the step constants come from a device
        # step table that a one-thread kernel in the graph advances
        nsteps = args.warmup + args.steps + 1
        nbytes = z.zs_step_table_bytes(nsteps)
        st_buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        keep.append(st_buf)
        steps = z.zs_step_table_init(z.hparams(wl.lr, wl.beta1, wl.beta2, wl.eps, 1, wl.form),
                                     wl.p, nsteps, st_buf, nbytes, stream=stream.cuda_stream)

        def launches_dev(st):
            for tb in tables:
                z.zs_fused_shard_step_multi_dev(tb, steps, stream=st)
            z.zs_step_table_advance(steps, stream=st)

        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph):
                launches_dev(torch.cuda.current_stream().cuda_stream)
        stream.wait_stream(side)
        torch.cuda.synchronize()

        def step(i):
            graph.replay()
    else:
        def step(i):
            hp = z.hparams(wl.lr, wl.beta1, wl.beta2, wl.eps, i + 1, wl.form)
            for tb in tables:
                z.zs_fused_shard_step_multi(tb, hp, stream=stream.cuda_stream)

    ms, wall = _time_steps(step, args.steps, args.warmup, stream)
    cpu = None if args.no_cpu_baseline else _cpu_leg(args, wl, grads, w, m, v, f"shard {k}")
    return dict(wl=wl, k=k, elems=L, ms=ms, wall=wall, bytes_per_elem=_bytes_per_elem(wl),
                launches=len(tables), launch_elems=L / len(tables), cpu=cpu,
                extra={"pieces": len(pieces), "chunks": nchunks, "chunk_elems": args.chunk,
                       "launches_per_step": len(tables), "graph": bool(args.graph)})


def bench_all_shards(args):
    """One step of every shard of a model with full-N gradient buffers: P launches."""
    import torch

    from adam_zs_shard_amd import zshard as z
    from zs_synth import WORKLOADS, make

    wl = WORKLOADS[args.workload]
    M, s, e = z.zs_plan_shards(wl.n, wl.p)
    dev = "cuda"
    td = {"f16": torch.float16, "bf16": torch.bfloat16}
    print(f"[bench] {wl.name}: N={wl.n} P={wl.p}, all {wl.p} shards per step",
          file=sys.stderr, flush=True)
    if wl.grad_kind == "edge":
        zero = make.edge_zero_mask(wl, wl.n, dev)
        grads = [make.edge_grad(wl, r, 1, wl.n, zero, s, e, dev) for r in range(wl.p)]
        del zero
    else:
        grads = [make.normal_grad(wl, r, 1, wl.n, dev) for r in range(wl.p)]
    states = []
    for k in range(wl.p):
        w = make.initial_w(wl, k, e[k] - s[k], dev)
        states.append((w,) + _state(wl, w))
    param = torch.empty(wl.n, dtype=td[wl.param_dtype], device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(i):
        hp = z.hparams(wl.lr, wl.beta1, wl.beta2, wl.eps, i + 1, wl.form)
        for k in range(wl.p):
            w, m, v = states[k]
            z.zs_fused_shard_step(wl.n, wl.p, k, grads, w, m, v, param, hp,
                                  stream=stream.cuda_stream)

    ms, wall = _time_steps(step, args.steps, args.warmup, stream)
    k0 = wl.p - 1
    cpu = None
    if not args.no_cpu_baseline:
        w, m, v = states[k0]
        cpu = _cpu_leg(args, wl, [g[s[k0]:e[k0]] for g in grads], w, m, v, f"shard {k0}")
    return dict(wl=wl, k=None, elems=wl.n, ms=ms, wall=wall, bytes_per_elem=_bytes_per_elem(wl),
                launches=wl.p, launch_elems=wl.n / wl.p, cpu=cpu,
                extra={"launches_per_step": wl.p})


def bench_cpu_offload(args):
    """The optimizer-offload update of one shard on the host CPU: the shard's
    16-bit gradient, fp32 w/m/v and the 16-bit copy all in host memory; the
    roofline is host memory bandwidth, taken from a multithreaded in-place
    pass over 2 GiB timed in the same run."""
    import numpy as np
    import torch

    from adam_zs_shard_amd import zshard as z
    from zs_synth import WORKLOADS, make

    wl = WORKLOADS[args.workload]
    k = wl.shards[-1]
    M, s, e = z.zs_plan_shards(wl.n, wl.p)
    L = e[k] - s[k]
    thr = host_threads()
    torch.set_num_threads(thr)
    print(f"[bench] cpu offload {wl.name}: shard {k}, {L} elements, {thr} threads, form {wl.form}",
          file=sys.stderr, flush=True)
    g = make.normal_grad(wl, 0, 1, L, "cpu", stream=k).view(torch.int16).numpy().view(np.uint16)
    w = make.initial_w(wl, k, L, "cpu").numpy().copy()
    f = z.FORMS[wl.form]
    m = np.zeros(L, np.float32) if f != z.ZS_SGD else None
    v = np.zeros(L, np.float32) if f in (z.ZS_ADAM_STANDARD, z.ZS_ADAM_PAGE1_LITERAL) else None
    par = np.empty(L, np.uint16)
    gdt = wl.grad_dtype

    def step(i):
        z.zs_cpu_adam_step(g, gdt, w, m, v, par, wl.param_dtype, L,
                           z.hparams(wl.lr, wl.beta1, wl.beta2, wl.eps, i + 1, wl.form),
                           threads=thr)

    for i in range(args.warmup):
        step(i)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    sec = (time.perf_counter() - t0) / args.steps
    per_elem = 2 + z.BYTES_PER_ELEM[f]   # 2 (16-bit gradient) + state + 2 (16-bit copy)
    gbs = per_elem * L / sec / 1e9
    # host ceiling: a multithreaded in-place scale of 2 GiB by exactly 1.0, the
    # same read-modify-write streaming pattern as the update
    buf = torch.ones(1 << 29)
    buf.mul_(1.0)
    t0 = time.perf_counter()
    for _ in range(5):
        buf.mul_(1.0)
    copy_gbs = 2 * buf.numel() * 4 / ((time.perf_counter() - t0) / 5) / 1e9
    print(json.dumps({
        "metric": "shard elements/s and achieved host-memory GB/s, optimizer-offload update on "
                  "the host CPU",
        "value": L / sec, "unit": "elements/s", "n_gpus": 0, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": sec * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "shard": k, "elems_per_step": L,
                   "grad_dtype": wl.grad_dtype, "param_dtype": wl.param_dtype,
                   "adam_form": wl.form, "threads": thr},
        "roofline": {"bound": "host_dram", "achieved": gbs, "peak": copy_gbs, "unit": "GB/s",
                     "frac": gbs / copy_gbs, "traffic": None, "bytes_per_element": per_elem,
                     "peak_source": f"in-place scale of 2 GiB (torch, {thr} threads), "
                                    "this run"},
    }), flush=True)


def bench_offload(args):
    """The optimizer offload of one shard on one GPU (zs_offload_step): GPU
    rank mean rounded to 16 bits, bucket by bucket, copied to pinned host
    memory; the update on the host CPU; the 16-bit parameters copied back.
    Timed per step with the plain schedule and with the delayed parameter
    update (the update of step t-1's gradient overlapping the GPU mean and
    copy of step t's), next to each part timed alone."""
    import numpy as np
    import torch

    from adam_zs_shard_amd import zshard as z
    from zs_synth import WORKLOADS, seed_for
    from zs_synth.gen import normal

    wl = WORKLOADS[args.workload]
    k = wl.shards[-1]
    M, s, e = z.zs_plan_shards(wl.n, wl.p)
    L = e[k] - s[k]
    thr = host_threads()
    bucket = args.bucket_elems if args.bucket_elems > 0 else 1 << 23
    td = {"f16": torch.float16, "bf16": torch.bfloat16}
    dt = td[wl.grad_dtype]
    print(f"[bench] offload {wl.name}: shard {k}, {L} elements, P={wl.p}, buckets of {bucket}, "
          f"{thr} threads", file=sys.stderr, flush=True)
    grads = [normal(L, wl.grad_std, seed_for(20261202, r, 1, 1, k), dt, "cuda")
             for r in range(wl.p)]
    param = torch.empty(L, dtype=td[wl.param_dtype], device="cuda")
    g16_dev = torch.empty(L, dtype=dt, device="cuda")
    partial = torch.empty(L, device="cuda") if wl.p > z.ZS_KERNARG_P else None
    pin = dict(pin_memory=True)
    g16_host = [torch.empty(L, dtype=dt, **pin) for _ in range(2)]
    w = torch.empty(L, **pin)
    w.copy_(normal(L, wl.w_std, seed_for(20261202, -1, 0, 2, k)))
    f = z.FORMS[wl.form]
    m = torch.zeros(L, **pin) if f != z.ZS_SGD else None
    v = torch.zeros(L, **pin) if f in (z.ZS_ADAM_STANDARD, z.ZS_ADAM_PAGE1_LITERAL) else None
    param_host = torch.empty(L, dtype=td[wl.param_dtype], **pin)
    cs = torch.cuda.current_stream()
    d2h, h2d = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    count = [0]

    def step(mode, slot):
        count[0] += 1
        hp = z.hparams(wl.lr, wl.beta1, wl.beta2, wl.eps, count[0], wl.form)
        z.zs_offload_step(wl.n, wl.p, k, grads, param, g16_dev, g16_host, w, m, v, param_host,
                          hp, mode, slot, grad_base=s[k], param_base=s[k], partial=partial,
                          bucket_elems=bucket, threads=thr, compute_stream=cs, d2h_stream=d2h,
                          h2d_stream=h2d)

    def timed(fn, n):
        t0 = time.perf_counter()
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    for i in range(args.warmup):
        step(z.ZS_OFFLOAD_PLAIN, 0)
    plain = timed(lambda i: step(z.ZS_OFFLOAD_PLAIN, 0), args.steps)
    step(z.ZS_OFFLOAD_RECEIVE, 0)
    delayed = timed(lambda i: step(z.ZS_OFFLOAD_DELAYED, (i + 1) % 2), args.steps)
    # the parts alone
    hp1 = z.hparams(wl.lr, wl.beta1, wl.beta2, wl.eps, 1, wl.form)
    mean_t = timed(lambda i: z.zs_reduce_scatter_mean_local16(grads, wl.n, wl.p, k, g16_dev,
                                                              grad_base=s[k], partial=partial),
                   args.steps)
    d2h_t = timed(lambda i: g16_host[0].copy_(g16_dev, non_blocking=True), args.steps)
    cpu_t = timed(lambda i: z.zs_cpu_adam_step(g16_host[0], wl.grad_dtype, w, m, v, param_host,
                                               wl.param_dtype, L, hp1, threads=thr), args.steps)
    h2d_t = timed(lambda i: param.copy_(param_host, non_blocking=True), args.steps)
    parts = mean_t + d2h_t + cpu_t + h2d_t
    print(json.dumps({
        "metric": "shard elements/s, optimizer offload on one GPU (GPU mean -> host update -> "
                  "parameters back)",
        "value": L / delayed, "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": delayed * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "shard": k, "elems_per_step": L, "ranks": wl.p,
                   "grad_dtype": wl.grad_dtype, "param_dtype": wl.param_dtype,
                   "adam_form": wl.form, "bucket_elems": bucket, "cpu_threads": thr,
                   "cpu_model": cpu_model()},
        "offload": {"plain_ms": plain * 1e3, "delayed_ms": delayed * 1e3,
                    "parts_ms": {"gpu_mean16": mean_t * 1e3, "d2h": d2h_t * 1e3,
                                 "cpu_update": cpu_t * 1e3, "h2d": h2d_t * 1e3},
                    "sum_of_parts_ms": parts * 1e3,
                    "d2h_gbs": 2 * L / d2h_t / 1e9, "h2d_gbs": 2 * L / h2d_t / 1e9,
                    "cpu_update_gbs": (2 + z.BYTES_PER_ELEM[f]) * L / cpu_t / 1e9},
    }), flush=True)


def copy_probe(nbytes: int = 1 << 31, reps: int = 10):
    """A plain device copy of known size (torch's copy kernel), used to
    calibrate rocprofv3's FETCH_SIZE / WRITE_SIZE counters: each dispatch
    reads and writes exactly `nbytes`."""
    import torch

    src = torch.ones(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes,
                      "dispatches": reps, "seconds_per_copy": dt,
                      "gbs_read_plus_write": 2 * nbytes / dt / 1e9}), flush=True)


def ceiling(args):
    """HBM ceilings of this part from the stream probes: for each mix, the
    best of several grid sizes (10 timed launches each after 2 warm-ups, HIP
    events on the probe's stream); every launch moves about 6 GB."""
    import ctypes as C

    import torch

    from adam_zs_shard_amd import _build

    if not os.path.exists(_build.PROBE_PATH):
        raise RuntimeError(f"{_build.PROBE_PATH} is not built; run __graft_entry__.build()")
    P = C.CDLL(_build.PROBE_PATH)
    P.zsp_stream.argtypes = [C.c_int32, C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_int32,
                             C.c_void_p, C.c_void_p]
    P.zsp_stream.restype = C.c_int32
    P.zsp_streams.argtypes = [C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32)]
    P.zsp_streams.restype = C.c_int32
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    mixes = [("read", 0, None), ("copy", 1, None), ("mix_10_1", 4, 154), ("mix_22_7", 3, 58),
             ("mix_2_1", 2, 42), ("phased_read", 5, None), ("phased_copy", 6, None),
             ("phased_10_1", 9, 154), ("phased_22_7", 8, 58), ("phased_2_1", 7, 42),
             ("read_1x16", 10, None), ("read_2x8", 11, None), ("read_4x8", 12, None),
             ("read_8x8", 13, None), ("read_1x32", 14, None)]
    out = {}
    for name, mix, bpe in mixes:
        nr, nw = C.c_int32(), C.c_int32()
        assert P.zsp_streams(mix, C.byref(nr), C.byref(nw)) == 0
        nstreams = nr.value + nw.value
        sb = (6_000_000_000 // nstreams) // (1 << 20) * (1 << 20)
        nvec = sb // 16
        src = torch.empty(nr.value * sb, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty(max(nw.value, 1) * sb if nw.value else 16, dtype=torch.uint8,
                          device="cuda")
        moved = 16 * nvec * nstreams
        best, sweep = None, {}
        for per_cu in ((1,) if name.startswith("phased") else (1, 2, 4, 8)):
            grid = ncu * per_cu

            def launch():
                rc = P.zsp_stream(mix, src.data_ptr(), dst.data_ptr() if nw.value else None, sb,
                                  nvec, grid, sink.data_ptr(), stream.cuda_stream)
                assert rc == 0, f"probe {name} failed ({rc})"

            for _ in range(2):
                launch()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            gbs = moved / (ms / 1e3) / 1e9
            sweep[f"{per_cu}_per_cu"] = round(gbs, 1)
            if best is None or gbs > best[0]:
                best = (gbs, per_cu, ms)
        out[name] = {"streams_read": nr.value, "streams_written": nw.value,
                     "bytes_per_launch": moved, "best_gbs": round(best[0], 1),
                     "best_frac_of_8tbs": round(best[0] / HBM_PEAK_GBS, 4),
                     "best_workgroups_per_cu": best[1], "best_ms": round(best[2], 4),
                     "gbs_by_workgroups_per_cu": sweep, "step_bytes_per_element": bpe}
        print(f"[ceiling] {name}: {best[0]:.0f} GB/s ({best[1]} workgroups per CU)",
              file=sys.stderr, flush=True)
        del src, dst
        torch.cuda.empty_cache()
    # the fused step's read phase alone, in its own pattern: the 64 rank
    # slices of the 7.5B-parameter shard (fp16), whole chunks only
    P.zsp_step_reads.argtypes = [C.POINTER(C.c_void_p), C.c_int32, C.c_int64, C.c_int32,
                                 C.c_void_p, C.c_void_p]
    P.zsp_step_reads.restype = C.c_int32
    from adam_zs_shard_amd import zshard as z
    from zs_synth import WORKLOADS

    wl = WORKLOADS["zero_7p5b_p64"]
    M, _, _ = z.zs_plan_shards(wl.n, wl.p)
    ranks = [torch.empty(M, dtype=torch.float16, device="cuda").normal_(0.0, 1e-3)
             for _ in range(wl.p)]
    arr = (C.c_void_p * wl.p)(*[g.data_ptr() for g in ranks])
    chunk = 28 * 256 * 8
    moved = (M // chunk) * chunk * 2 * wl.p

    P.zsp_step_reads_paced.argtypes = [C.POINTER(C.c_void_p), C.c_int32, C.c_int64, C.c_int32,
                                       C.c_int32, C.c_void_p, C.c_void_p]
    P.zsp_step_reads_paced.restype = C.c_int32
    # plain, and paced like the library's whole-chunk kernels (a soft barrier
    # every 2 rounds, the pacing of its read-only mean kernel)
    for name, pace in (("step_reads_p64", 0), ("step_reads_p64_paced", 2)):
        def launch_reads(pace=pace):
            if pace:
                rc = P.zsp_step_reads_paced(arr, wl.p, M, ncu, pace, sink.data_ptr(),
                                            stream.cuda_stream)
            else:
                rc = P.zsp_step_reads(arr, wl.p, M, ncu, sink.data_ptr(), stream.cuda_stream)
            assert rc == 0, f"probe {name} failed ({rc})"

        for _ in range(2):
            launch_reads()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            launch_reads()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        gbs = moved / (ms / 1e3) / 1e9
        out[name] = {"streams_read": wl.p, "streams_written": 0, "bytes_per_launch": moved,
                     "best_gbs": round(gbs, 1), "best_frac_of_8tbs": round(gbs / HBM_PEAK_GBS, 4),
                     "best_workgroups_per_cu": 1, "best_ms": round(ms, 4),
                     "gbs_by_workgroups_per_cu": {"1_per_cu": round(gbs, 1)},
                     "step_bytes_per_element": None, "soft_barrier_every_rounds": pace or None}
        print(f"[ceiling] {name}: {gbs:.0f} GB/s ({ms:.3f} ms)", file=sys.stderr, flush=True)
    del ranks
    torch.cuda.empty_cache()
    print(json.dumps({"ceiling": out, "peak_gbs": HBM_PEAK_GBS, "cus": ncu}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="zero_7p5b_p64")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=1 << 25)
    ap.add_argument("--form", default=None,
                    choices=["standard", "page1_literal", "sgd", "sgd_momentum"],
                    help="override the workload's update form (bytes per element follow it)")
    ap.add_argument("--dtype", default=None, choices=["f16", "bf16"],
                    help="override the workload's gradient and working-copy dtype")
    ap.add_argument("--unfused", action="store_true",
                    help="single-tensor workloads: time the unfused pair (stored fp32 mean, "
                         "then the separate update) instead of the fused step")
    ap.add_argument("--chunk", type=int, default=0,
                    help="chunk-table chunk length in elements (multi-tensor workloads); 0 picks "
                         "one whole kernel chunk (57,344), or for shards under two of those per "
                         "CU, the shard's per-CU share (a quarter of it when the shard spans "
                         "several tensors), rounded up to 2,048")
    ap.add_argument("--shard", type=int, default=None,
                    help="chunk-table workloads: the rank k whose shard is timed")
    ap.add_argument("--bucket-elems", type=int, default=0,
                    help="chunk-table workloads: one launch per bucket of consecutive pieces "
                         "holding at least this many elements (0: one launch per step)")
    ap.add_argument("--graph", action="store_true",
                    help="chunk-table workloads: capture the step's launches in a HIP graph once "
                         "(step constants read from a device step table) and time its replays")
    ap.add_argument("--ceiling", action="store_true",
                    help="time only the bandwidth probes (libzsprobe): pure reads, a copy, and "
                         "the read:write mixes of 154, 58 and 42 bytes per element")
    ap.add_argument("--cpu-offload", action="store_true",
                    help="time the host-CPU offload update (zs_cpu_adam_step) of the "
                         "workload's shard instead of the GPU step; no GPU needed")
    ap.add_argument("--offload", action="store_true",
                    help="time the optimizer offload on one GPU (zs_offload_step), plain and "
                         "with the delayed parameter update, next to its parts")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 2 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the shard step runs on one device and this "
              f"build has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    from adam_zs_shard_amd import zshard as z
    from zs_synth import WORKLOADS

    if args.workload not in WORKLOADS:
        print(f"unknown workload {args.workload}; one of {sorted(WORKLOADS)}", file=sys.stderr)
        sys.exit(2)
    wl0 = WORKLOADS[args.workload]
    if args.unfused and (wl0.param_layout == "tensors" or wl0.grad_layout != "slice"):
        print("--unfused times single-tensor workloads with slice gradients", file=sys.stderr)
        sys.exit(2)
    if args.form is not None or args.dtype is not None:
        import dataclasses

        wl = WORKLOADS[args.workload]
        WORKLOADS[args.workload] = dataclasses.replace(
            wl, form=args.form or wl.form, grad_dtype=args.dtype or wl.grad_dtype,
            param_dtype=args.dtype or wl.param_dtype)
    if args.cpu_offload:
        z.lib()  # fails loudly if the library is not built
        bench_cpu_offload(args)
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe()
        return
    if args.ceiling:
        ceiling(args)
        return
    if args.offload:
        z.lib()
        bench_offload(args)
        return

    z.lib()  # fails loudly if the HIP library is not built
    wlx = WORKLOADS[args.workload]
    if args.unfused:
        r = bench_unfused(args)
    elif wlx.param_layout == "tensors":
        r = bench_multi(args)
    elif wlx.grad_layout == "full":
        r = bench_all_shards(args)
    else:
        r = bench_single(args)
    wl = r["wl"]
    ms = r["ms"]
    elems_per_s = r["elems"] / (ms / 1e3)
    dom = r.get("dominant")
    if dom is None:  # every launch of the step is the same kernel on equal work
        launch_ms = ms / r["launches"]
        alg_bytes = r["bytes_per_elem"] * r["launch_elems"]
        gbs = alg_bytes / (launch_ms / 1e3) / 1e9
        k_gbs = gbs
        # the stored counters were taken at the workload's own dtypes
        traffic = measured_traffic(wl.name, wl.form) if args.dtype is None else None
    else:  # different kernels: the step's rate, and the dominant kernel's roofline
        gbs = r["bytes_per_elem"] * r["elems"] / (ms / 1e3) / 1e9
        launch_ms = dom["ms"]
        alg_bytes = dom["bytes_per_elem"] * r["launch_elems"]
        k_gbs = alg_bytes / (launch_ms / 1e3) / 1e9
        traffic = None
    out = {
        "metric": METRIC,
        "value": elems_per_s,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": dict({"workload": wl.name, "n_params": wl.n, "ranks": wl.p,
                        "shard": r["k"] if r["k"] is not None else "all",
                        "elems_per_step": r["elems"], "grad_dtype": wl.grad_dtype,
                        "param_dtype": wl.param_dtype, "adam_form": wl.form},
                       **r.get("extra", {})),
        "hbm_gbs": gbs,
        "pct_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "achieved": k_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": k_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "bytes_per_element": dom["bytes_per_elem"] if dom else r["bytes_per_elem"],
                     "kernel_ms": launch_ms},
        "cpu_baseline": r["cpu"],
        "wall_s_timed": r["wall"],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
