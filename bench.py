"""MoE layer forward throughput on one MI355X, Quartz shape.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload quartz] [--no-cpu]

One step is one call of moe_layer_forward (router GEMM, top-k, scan, rank,
fused gate/up grouped GEMM, down grouped GEMM, combine) over one batch of
synthetic inputs already resident in device memory. Prints one JSON line.
For bf16 dense layers the line also carries the training pair under
"backward": the forward that keeps its gate and up products, the
moe_layer_backward call after it, forward + backward tokens/s, and the
backward products' TFLOP/s; and under "fp8" the same layer with fp8 (E4M3)
expert weights (moe_quantize_fp8), its step time and expert-GEMM rates.

Per-kernel durations come from HIP events that the library records on the
launch stream between its kernels (moe_layer_forward_timed); the dominant
kernel's roofline is its algorithmic FLOPs per launch over its mean duration.
The CPU baseline is the float64 oracle timed over the workload's tokens on
the host cores (worker processes, before the GPU is used). The streaming
stages are also timed alone from a cold cache through the stage entry points.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="quartz")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the layer backward")
    ap.add_argument("--no-fp8", action="store_true", help="skip timing the fp8-expert layer")
    ap.add_argument("--no-clock", action="store_true",
                    help="do not sample the shader clock with rocm-smi (use under a profiler)")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the workload the CPU oracle processes (0: all of them)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the workload's token count T (e.g. decode-sized batches)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="also time the platform BLAS (torch.bmm / matmul, hipBLASLt) on "
                         "uniform stand-ins for the workload's expert products, for context")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the layer, run 3 plain device copies of this many MiB "
                         "(calibrates the HBM byte counters of a profiler run)")
    return ap.parse_args()


def copy_calibration(mib: int):
    """Three launches of a plain elementwise copy (y = x * 1) of `mib` MiB of
    float32: each reads and writes exactly mib MiB."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, device="cuda:0", dtype=torch.float32)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                      "launches": 3}))


def algorithmic(wl, rows):
    """Algorithmic FLOPs and bytes of each stage for `rows` dispatched rows."""
    T, d, E, k, S, F, r = wl.T, wl.hidden, wl.n_routed, wl.top_k, wl.n_shared, wl.ffn, wl.rank
    b = 2 if wl.dtype in ("bf16", "fp8") else 4
    if r == 0:
        gate_up = 4.0 * d * F * rows
        down = 2.0 * d * F * rows
    else:
        gate_up = rows * 2.0 * 2 * (d * r + r * F)
        down = rows * 2.0 * (F * r + r * d)
    return dict(
        router_flops=2.0 * T * d * E,
        gate_up_flops=gate_up,
        down_flops=down,
        shared_gate_up_flops=4.0 * d * F * S * T,
        shared_down_flops=2.0 * d * F * S * T,
        route_bytes=T * d * b + d * E * b + T * E * 4,
        topk_bytes=T * E * 4 + 8 * T * k,
        combine_bytes=rows * d * 4 + (T * d * 4 if S > 0 else 0) + T * d * 4 + 8 * T * k,
    )


def backward_flops(wl, rows):
    """Algorithmic FLOPs of the layer backward's products for `rows` dispatched
    rows, with the forward's gate and up products saved: dh = dy W_down^T, the
    input-gradient products (experts and router) and the weight-gradient
    products (experts and router)."""
    T, d, E, S, F = wl.T, wl.hidden, wl.n_routed, wl.n_shared, wl.ffn
    ex = rows + S * T
    return dict(dh_gemm=2.0 * d * F * ex, dgrad_gemm=4.0 * d * F * ex + 2.0 * d * E * T,
                wgrad_gemm=6.0 * d * F * ex + 2.0 * d * E * T)


def lowrank_backward_work(wl, rows, used):
    """Algorithmic FLOPs and HBM bytes of each product kernel of the rank-r
    experts' backward, for `rows` dispatched rows and `used` experts with
    rows: each operand read once, each result written once (bf16 operands and
    factors, fp32 products and gradients)."""
    T, d, E, F, r = wl.T, wl.hidden, wl.n_routed, wl.ffn, wl.rank
    R, fac = rows, used * r * 2            # one factor column set of `used` experts, bf16
    flops = dict(lr_in_gemm=6.0 * R * d * r, lr_ab_gemm=4.0 * R * r * F,
                 lr_ud_gemm=2.0 * R * F * r, lr_dh_gemm=2.0 * R * r * F,
                 lr_dz_gemm=4.0 * R * F * r, dgrad_gemm=4.0 * R * r * d + 2.0 * T * E * d,
                 wgrad_gemm=4.0 * R * d * r + 6.0 * R * F * r,
                 wgrad_gemm2=2.0 * R * d * r + 2.0 * d * E * T)
    nbytes = dict(
        lr_in_gemm=4 * R * d + 3 * d * fac + 12 * R * r,
        lr_ab_gemm=4 * R * r + 2 * F * fac + 8 * R * F,
        lr_ud_gemm=2 * R * F + F * fac + 4 * R * r,
        lr_dh_gemm=2 * R * r + F * fac + 8 * R * F + 4 * R * F,
        lr_dz_gemm=4 * R * F + 2 * F * fac + 8 * R * r,
        dgrad_gemm=4 * R * r + 2 * d * fac + 4 * R * d + 2 * T * E + 2 * d * E + 4 * T * d,
        wgrad_gemm=(2 * R * d + 2 * R * r + 2 * R * F + 2 * R * r + 4 * R * F + 4 * R * r +
                    2 * R * d + 2 * R * r + 4 * E * r * (2 * d + 3 * F)),
        wgrad_gemm2=2 * R * d + 2 * R * r + 4 * E * d * r + 2 * T * d + 2 * T * E + 4 * d * E)
    return flops, nbytes


def blas_reference(wl, steps):
    """The platform BLAS (torch.bmm and matmul, i.e. hipBLASLt) on uniform stand-ins for the
    dense expert products of this workload: every routed expert given T k / E rows, the
    gate and up products as one [rows, d] x [d, 2F] product per expert, the down product
    [rows, F] x [F, d] with a bf16 output, the shared experts as one product over all T
    tokens (K = S F for down). Context only: no gather, no ragged groups, no fused
    epilogue, no fp32 output. Also an 8192^3 product, the library's ceiling."""
    import torch

    T, d, E, k, S, F = wl.T, wl.hidden, wl.n_routed, wl.top_k, wl.n_shared, wl.ffn
    dev, bf = "cuda", torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(0)

    def rnd(*shape):
        return torch.randn(*shape, device=dev, dtype=bf, generator=g).contiguous()

    def us_of(fn, n):
        for _ in range(max(2, n // 5)):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    rows = max(1, T * k // E)
    out = {"rows_per_expert": rows}
    parts = {"gate_up": [(rnd(E, rows, d), rnd(E, d, 2 * F))],
             "down": [(rnd(E, rows, F), rnd(E, F, d))]}
    if S:
        parts["gate_up"].append((rnd(T, d), rnd(d, S * 2 * F)))
        parts["down"].append((rnd(T, S * F), rnd(S * F, d)))
    for name, prods in parts.items():
        us = flops = 0.0
        for a, b in prods:
            us += us_of(lambda a=a, b=b: torch.matmul(a, b), steps)
            flops += 2.0 * a.numel() * b.shape[-1]
        out[name] = {"us": us, "tflops": flops / (us * 1e-6) / 1e12,
                     "frac_of_bf16_peak": flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS}
    n = 8192
    a, b = rnd(n, n), rnd(n, n)
    us = us_of(lambda: torch.matmul(a, b), 20)
    out["square_8192"] = {"us": us, "tflops": 2.0 * n ** 3 / (us * 1e-6) / 1e12,
                          "frac_of_bf16_peak": 2.0 * n ** 3 / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS}
    return out


def time_backward(wl, cfg, x, w, steps, warmup, stream):
    """The training pair: mean time of moe_layer_forward keeping its gate and
    up products (saved_ab), and of moe_layer_backward after it (reading that
    forward's workspace and products), with the backward's per-kernel
    durations from the library's events."""
    import numpy as np
    import torch

    from fine_grained_mixture_amd import _lib, synth
    from fine_grained_mixture_amd.layer import (allocate_backward_workspace, allocate_grads,
                                                allocate_outputs, allocate_workspace)

    dev = x.device
    dy = torch.from_numpy(synth.make_upstream(wl)).to(dev)
    out = allocate_outputs(cfg, wl.T, dev, saved_ab=wl.rank == 0)
    ws = allocate_workspace(cfg, wl.T, dev)
    g = allocate_grads(cfg, wl.T, dev)
    bws = allocate_backward_workspace(cfg, wl.T, dev)

    def fstep():
        _lib.moe_layer_forward(cfg, wl.T, x.data_ptr(), w.struct, out.struct, ws.data_ptr(),
                               ws.numel(), stream)

    for _ in range(warmup):
        fstep()
    torch.cuda.synchronize()
    f0 = torch.cuda.Event(enable_timing=True)
    f1 = torch.cuda.Event(enable_timing=True)
    f0.record()
    for _ in range(steps):
        fstep()
    f1.record()
    torch.cuda.synchronize()
    fwd_ms = f0.elapsed_time(f1) / steps

    def bstep(events=None):
        a = (cfg, wl.T, x.data_ptr(), w.struct, out.struct, dy.data_ptr(), 1.0, g.struct,
             ws.data_ptr(), ws.numel(), bws.data_ptr(), bws.numel(), stream)
        if events is None:
            _lib.moe_layer_backward(*a)
            return 0
        return _lib.moe_layer_backward_timed(*a, [e.cuda_event for e in events])

    for _ in range(warmup):
        bstep()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        bstep()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    n_ev = 64
    sets = []
    for _ in range(steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        for e in evs:
            e.record()
        sets.append(evs)
    torch.cuda.synchronize()
    n_k = 0
    for evs in sets:
        n_k = bstep(evs)
    torch.cuda.synchronize()
    names = [_lib.moe_stage_name(i) for i in range(min(n_k, n_ev // 2))]
    dur = {n: [] for n in names}
    for evs in sets:
        for i, n in enumerate(names):
            dur[n].append(evs[2 * i].elapsed_time(evs[2 * i + 1]) * 1e3)
    return fwd_ms, ms, {n: float(np.mean(v)) for n, v in dur.items()}


def per_call_ms(step, n, flush=None):
    """Each call timed alone between two events on the launch stream, after
    `flush` when given: (p10, median, p90) in ms and, for timed steps, the
    per-stage medians in us."""
    import numpy as np
    import torch

    calls = []
    for _ in range(n):
        if flush is not None:
            flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        calls.append((e0, e1))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in calls])
    return [float(np.percentile(ms, q)) for q in (10, 50, 90)]


def clock_sampler(path, seconds):
    """Child process: once `path`.go exists, append one `rocm-smi
    --showclocks --json` reading per line (with its time) to `path` until
    `seconds` pass or the parent exits. It is started before the parent
    touches the GPU and never uses it."""
    import subprocess

    parent = os.getppid()
    end = time.time() + seconds
    # idle until the parent's clock window opens, so the timed steps run
    # without the tool beside them
    while not os.path.exists(path + ".go"):
        if time.time() >= end or os.getppid() != parent:
            return
        time.sleep(0.05)
    with open(path, "w") as f:
        while time.time() < end and os.getppid() == parent:
            try:
                r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                                   text=True, timeout=20)
                f.write(json.dumps({"t": time.time(), "out": r.stdout}) + "\n")
                f.flush()
            except Exception:      # no tool or a time-out: nothing to record
                return
            time.sleep(0.1)


def start_clock_sampler():
    import subprocess
    import tempfile

    fd, path = tempfile.mkstemp(prefix="moe_clock_", suffix=".jsonl")
    os.close(fd)
    proc = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--clock-sampler", path],
                            stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return proc, path


def clock_during(step, sampler, seconds=3.0):
    """Median shader clock of the sampler's readings taken while the layer
    runs back to back for `seconds`; None where there are none."""
    import numpy as np
    import torch

    res = {"sclk_mhz": None, "samples": 0,
           "source": "rocm-smi (a process started before the GPU was used) during back-to-back calls"}
    if sampler is None:
        return res
    proc, path = sampler
    open(path + ".go", "w").close()
    t0 = time.time()
    while time.time() - t0 < seconds:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    t1 = time.time()
    proc.terminate()
    proc.wait(timeout=30)
    vals = []
    with open(path) as f:
        for line in f:
            try:
                rec = json.loads(line)
                if not (t0 <= rec["t"] <= t1):
                    continue
                card = next(iter(json.loads(rec["out"]).values()))
                for key, val in card.items():
                    m = re.search(r"([0-9]+(?:\.[0-9]+)?)", str(val))
                    if m and "sclk" in key.lower() and "level" not in key.lower():
                        vals.append(float(m.group(1)))
                        break
            except (ValueError, KeyError, StopIteration, AttributeError):
                continue
    for f in (path, path + ".go"):
        if os.path.exists(f):
            os.unlink(f)
    if vals:
        res["sclk_mhz"] = float(np.median(vals))
        res["samples"] = len(vals)
    return res


def lowrank_expert_bytes(wl, fp8):
    """Bytes of one low-rank expert's parameters: six factors of (d + F) r
    values in total ((2d + F) r for U, (2F + d) r for V), 3r bf16 s values and,
    with fp8 factors, one fp32 scale per column of U and per row of V."""
    d, F, r = wl.hidden, wl.ffn, wl.rank
    n = 3 * (d + F) * r
    if not fp8:
        return 2 * (n + 3 * r)
    return n + 2 * 3 * r + 4 * (3 * r + 2 * F + d)


def time_fp8(wl, inp, x, steps, warmup, stream):
    """The same layer with fp8 (E4M3) expert weights: mean step time and the
    per-kernel durations from the library's events."""
    import numpy as np
    import torch

    from fine_grained_mixture_amd import _lib
    from fine_grained_mixture_amd.layer import (DeviceWeights, allocate_outputs,
                                                allocate_workspace, config_from_workload)

    wl8 = wl.replace(dtype="fp8")
    cfg = config_from_workload(wl8)
    w = DeviceWeights.from_numpy(inp, cfg, x.device)
    out = allocate_outputs(cfg, wl.T, x.device)
    ws = allocate_workspace(cfg, wl.T, x.device)

    def step(events=None):
        if events is None:
            _lib.moe_layer_forward(cfg, wl.T, x.data_ptr(), w.struct, out.struct, ws.data_ptr(),
                                   ws.numel(), stream)
            return 0
        return _lib.moe_layer_forward_timed(cfg, wl.T, x.data_ptr(), w.struct, out.struct,
                                            ws.data_ptr(), ws.numel(), stream,
                                            [e.cuda_event for e in events])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    sets = []
    for _ in range(steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(32)]
        for e in evs:
            e.record()
        sets.append(evs)
    torch.cuda.synchronize()
    n_k = 0
    for evs in sets:
        n_k = step(evs)
    torch.cuda.synchronize()
    names = [_lib.moe_stage_name(i) for i in range(n_k)]
    dur = {n: [] for n in names}
    for evs in sets:
        for i, n in enumerate(names):
            dur[n].append(evs[2 * i].elapsed_time(evs[2 * i + 1]) * 1e3)
    return ms, {n: float(np.mean(v)) for n, v in dur.items()}


def traffic_from_profile(kernel_src: str, summary: str = "gate_up_gemm_quartz_counters.md"):
    """HBM bytes per launch of a dominant kernel from its committed counter
    summary, if it was taken from the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source sha256:\s*([0-9a-f]{64})", text)
    t = re.search(r"hbm bytes per launch:\s*([0-9.eE+]+)", text)
    if not m or not t:
        return None
    cur = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    return float(t.group(1)) if m.group(1) == cur else None


# the CPU baseline's worker processes share these (inherited by fork)
_CPU_JOB = {}
# worker processes at most: the host share that goes with one GPU
MAX_CPU_WORKERS = 16


def _oracle_shard(tokens):
    """One worker: the oracle's layer forward for its share of the tokens
    (routing and dispatch over the whole batch, as capacity needs), one BLAS
    thread; returns its own wall time."""
    from threadpoolctl import threadpool_limits

    import oracle
    job = _CPU_JOB
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.layer_forward(job["inp"]["x"], job["inp"], job["spec"], tokens=tokens)
        return time.perf_counter() - t0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, inp, n_tokens):
    """The float64 oracle (the token loop as it stands) over the workload's
    tokens, split evenly over worker processes, one per usable host core (at
    most MAX_CPU_WORKERS), each with one BLAS thread. Runs before this process
    touches the GPU; the workers are forked and never use it."""
    import multiprocessing as mp

    import numpy as np

    import oracle
    n = wl.T if n_tokens <= 0 else min(n_tokens, wl.T)
    spec = oracle.LayerSpec(hidden=wl.hidden, n_routed=wl.n_routed, top_k=wl.top_k,
                            n_shared=wl.n_shared, ffn=wl.ffn, rank=wl.rank, score=wl.score,
                            renorm=bool(wl.renorm), capacity=wl.capacity,
                            aux_coef=wl.aux_coef, bf16=wl.dtype in ("bf16", "fp8"),
                            fp8=wl.dtype == "fp8")
    _CPU_JOB.update(inp=inp, spec=spec)
    workers = max(1, min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS))
    shards = [a for a in np.array_split(np.arange(n), workers) if len(a)]
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ.setdefault(var, "1")
    with mp.get_context("fork").Pool(len(shards)) as pool:
        pool.map(int, range(len(shards)))             # workers up before the clock starts
        t0 = time.perf_counter()
        per = pool.map(_oracle_shard, shards)
        dt = time.perf_counter() - t0
    _CPU_JOB.clear()
    return {"value": n / dt, "unit": "tokens/s", "cores": len(shards), "kind": "oracle",
            "cpu_model": cpu_model(), "wall_s": dt,
            "sample": f"{n} of the {wl.T} tokens of the same inputs, split over "
                      f"{len(shards)} worker processes (one BLAS thread each; routing and "
                      f"dispatch over all tokens in every worker, y for its share); "
                      f"float64 NumPy token loop; slowest worker {max(per):.1f} s"}


def run_metadata(wl):
    """What identifies the run: the sources' hash, the git commit when the
    tree has one, the seeds of the synthetic inputs."""
    import subprocess
    h = hashlib.sha256()
    src_dirs = [os.path.join(ROOT, "fine_grained_mixture_amd", "csrc"), os.path.join(ROOT, "include")]
    for dname in src_dirs:
        for name in sorted(os.listdir(dname)):
            if name.endswith((".hip", ".cpp", ".h")):
                h.update(name.encode())
                h.update(open(os.path.join(dname, name), "rb").read())
    h.update(open(os.path.abspath(__file__), "rb").read())
    try:
        sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                             text=True, timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        sha = None
    sha_from = "git" if sha else None
    if not sha:
        # a copy of the tree without its history: the commit recorded when the
        # library was built, if its sources are the ones here
        from fine_grained_mixture_amd import build as _build
        try:
            with open(_build.INFO) as f:
                info = json.load(f)
            if info.get("source_sha256") == _build.source_digest() and info.get("git_sha"):
                sha = info["git_sha"]
                sha_from = ("build (sources modified since that commit)"
                            if info.get("sources_modified_since_commit") else "build")
        except (OSError, ValueError):
            pass
    return {"source_sha256": h.hexdigest(), "git_sha": sha, "git_sha_from": sha_from,
            "input_seed": wl.seed, "upstream_seed": wl.seed + 1000,
            "date_utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime())}


def cold_stages(wl, cfg, x, w, steps, stream):
    """The streaming stages alone, each call after a 512 MiB write (twice the
    Infinity Cache) so that their operands come from HBM, through the stage
    entry points: moe_permute gathering x_perm, and moe_combine. The gather's
    time is the median of moe_permute with x_perm less the median without it
    (the rank alone), both cold. Returns medians and HBM rates."""
    import numpy as np
    import torch

    from fine_grained_mixture_amd import _lib
    from fine_grained_mixture_amd.layer import allocate_outputs, allocate_workspace

    T, d, k = wl.T, wl.hidden, wl.top_k
    dev = x.device
    out = allocate_outputs(cfg, T, dev)
    ws = allocate_workspace(cfg, T, dev)
    _lib.moe_layer_forward(cfg, T, x.data_ptr(), w.struct, out.struct, ws.data_ptr(), ws.numel(),
                           stream)
    R = _lib.moe_max_rows(cfg, T)
    x_perm = torch.empty((max(R, 1), d), dtype=x.dtype, device=dev)
    torch.cuda.synchronize()
    rows = int(out["offsets"][-1].item())
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    fill = [0]

    def flush():
        fill[0] ^= 1
        flush_buf.fill_(fill[0])

    def permute(xp):
        return lambda: _lib.moe_permute(cfg, T, x.data_ptr(), out.struct, xp, ws.data_ptr(),
                                        ws.numel(), stream)

    yr_off, _ = _lib.moe_workspace_region(cfg, T, _lib.MOE_WS_Y_ROUTED)
    ys_off, ys_n = _lib.moe_workspace_region(cfg, T, _lib.MOE_WS_Y_SHARED)
    base = ws.data_ptr()

    def combine():
        _lib.moe_combine(cfg, T, base + yr_off, base + ys_off if ys_n else None, out.struct,
                         stream)

    b = x.element_size()
    rank_ms = per_call_ms(permute(None), steps, flush)[1]
    perm_ms = per_call_ms(permute(x_perm.data_ptr()), steps, flush)[1]
    comb_ms = per_call_ms(combine, steps, flush)[1]
    del flush_buf
    gather_bytes = T * d * b + rows * d * b + 4 * rows
    combine_bytes = rows * d * 4 + (T * d * 4 if wl.n_shared else 0) + T * d * 4 + 8 * T * k
    gather_us = max(perm_ms - rank_ms, 1e-6) * 1e3
    comb_us = comb_ms * 1e3
    res = {"protocol": "each call after a 512 MiB device write; medians of the calls",
           "permute_rank_only_us": rank_ms * 1e3, "permute_with_gather_us": perm_ms * 1e3,
           "gather_us": gather_us, "gather_bytes": gather_bytes,
           "gather_gbs": gather_bytes / (gather_us * 1e-6) / 1e9,
           "combine_us": comb_us, "combine_bytes": combine_bytes,
           "combine_gbs": combine_bytes / (comb_us * 1e-6) / 1e9}
    res["gather_frac_of_hbm_peak"] = res["gather_gbs"] / PEAK_HBM_GBS
    res["combine_frac_of_hbm_peak"] = res["combine_gbs"] / PEAK_HBM_GBS
    return res


def main():
    if len(sys.argv) == 3 and sys.argv[1] == "--clock-sampler":
        clock_sampler(sys.argv[2], 300)
        return
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this MoE layer build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_mib > 0:
        copy_calibration(args.copy_mib)
        return
    from fine_grained_mixture_amd import synth

    wl = synth.WORKLOADS[args.workload]
    if args.tokens > 0:
        wl = wl.replace(T=args.tokens)
    inp = synth.make_inputs(wl)
    # the CPU baseline's forked workers and the clock sampler start before
    # anything here uses the GPU
    cpu = None if args.no_cpu else cpu_baseline(wl, inp, args.cpu_tokens)
    sampler = None if args.no_clock else start_clock_sampler()
    import numpy as np
    import torch

    from fine_grained_mixture_amd import _lib
    from fine_grained_mixture_amd.layer import (DeviceWeights, allocate_outputs,
                                                allocate_workspace, config_from_workload,
                                                current_stream)

    cfg = config_from_workload(wl)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if wl.dtype in ("bf16", "fp8") else torch.float32
    x = torch.from_numpy(inp["x"]).to(device=dev, dtype=dt)
    w = DeviceWeights.from_numpy(inp, cfg, dev)
    out = allocate_outputs(cfg, wl.T, dev)
    ws = allocate_workspace(cfg, wl.T, dev)
    stream = current_stream()

    def step(events=None):
        if events is None:
            _lib.moe_layer_forward(cfg, wl.T, x.data_ptr(), w.struct, out.struct, ws.data_ptr(),
                                   ws.numel(), stream)
            return 0
        return _lib.moe_layer_forward_timed(cfg, wl.T, x.data_ptr(), w.struct, out.struct,
                                            ws.data_ptr(), ws.numel(), stream,
                                            [e.cuda_event for e in events])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole-layer steps back to back
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps

    # per-kernel durations: the same steps with a start and an end event
    # around every kernel, on the stream it runs on
    n_ev = 32
    ev_sets = []
    for _ in range(args.steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        for e in evs:
            e.record()          # materialise the underlying hipEvent
        ev_sets.append(evs)
    torch.cuda.synchronize()
    n_k = 0
    for evs in ev_sets:
        n_k = step(evs)
    torch.cuda.synchronize()
    names = [_lib.moe_stage_name(i) for i in range(min(n_k, n_ev // 2))]
    dur = {n: [] for n in names}
    for evs in ev_sets:
        for i, n in enumerate(names):
            dur[n].append(evs[2 * i].elapsed_time(evs[2 * i + 1]) * 1e3)   # us
    stage_us = {n: float(np.mean(v)) for n, v in dur.items()}
    stage_us_med = {n: float(np.median(v)) for n, v in dur.items()}

    # distribution of single calls, warm and after evicting the caches (a
    # 512 MiB write, twice the 256 MiB Infinity Cache, before each call)
    warm_p = per_call_ms(step, args.steps)
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    fill = [0]

    def flush():
        fill[0] ^= 1
        flush_buf.fill_(fill[0])

    cold_p = per_call_ms(step, args.steps, flush)
    del flush_buf
    clk = clock_during(step, sampler)
    cold = cold_stages(wl, cfg, x, w, args.steps, stream)

    rows = int(out["offsets"][-1].item())
    alg = algorithmic(wl, rows)

    def full_shape(name):
        return wl.name == name and wl.T == synth.WORKLOADS[name].T
    kernel_src = os.path.join(ROOT, "fine_grained_mixture_amd", "csrc", "gemm_big.hip")
    # every expert GEMM stage present and its algorithmic FLOPs
    gemm_stages = {"gate_up_gemm": alg["gate_up_flops"], "down_gemm": alg["down_flops"],
                   "lowrank_experts": alg["gate_up_flops"] + alg["down_flops"],
                   "shared_gate_up_gemm": alg["shared_gate_up_flops"],
                   "shared_down_gemm": alg["shared_down_flops"]}
    if "shared_gate_up_gemm" not in stage_us:
        # the shared experts run inside the routed launches
        gemm_stages["gate_up_gemm"] += alg["shared_gate_up_flops"]
        gemm_stages["down_gemm"] += alg["shared_down_flops"]
    present = {n: f for n, f in gemm_stages.items() if n in stage_us}
    expert_tflops = sum(present.values()) / (sum(stage_us[n] for n in present) * 1e-6) / 1e12
    if wl.rank == 0 and wl.dtype == "bf16":
        # dominant kernel: the fused gate/up grouped GEMM of the routed experts
        # (MFMA bound)
        dom = "gate_up_gemm"
        gu_us = stage_us["gate_up_gemm"]
        achieved = gemm_stages["gate_up_gemm"] / (gu_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                # the counters were taken at the Quartz shape
                "traffic": traffic_from_profile(kernel_src) if full_shape("quartz") else None}
    elif wl.rank > 0:
        # dominant kernel: the fused low-rank experts, bound by streaming the
        # factor weights of every expert that received rows
        dom = "lowrank_experts"
        us = stage_us[dom]
        kept = out["kept"].cpu().numpy()
        used = int((kept > 0).sum())
        wbytes = used * lowrank_expert_bytes(wl, fp8=False)
        io = rows * wl.hidden * 2 + rows * wl.hidden * 4
        achieved = (wbytes + io) / (us * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                "traffic": traffic_from_profile(
                    os.path.join(ROOT, "fine_grained_mixture_amd", "csrc", "lowrank.hip"),
                    "lowrank_experts_dormouse_counters.md") if full_shape("dormouse") else None,
                "algorithmic_bytes": wbytes + io}
    else:
        dom = "gate_up_gemm"
        gu_us = stage_us["gate_up_gemm"]
        achieved = gemm_stages["gate_up_gemm"] / (gu_us * 1e-6) / 1e12
        roof = {"bound": "alu", "kernel": dom, "achieved": achieved, "peak": 157.3,
                "unit": "TFLOP/s", "frac": achieved / 157.3, "traffic": None}
    # every stage against its own bound: MFMA for the products, HBM for the
    # streaming stages (algorithmic FLOPs or bytes over the event-timed mean);
    # scan and rank are latency-bound and carry no roofline
    peak_mm = PEAK_BF16_TFLOPS if wl.dtype != "f32" else 157.3
    stage_work = {"router_gemm": ("mfma", alg["router_flops"]),
                  "route": ("hbm", alg["route_bytes"] + 8 * wl.T * wl.top_k),
                  "route_scan_rank": ("hbm", alg["route_bytes"] + 8 * wl.T * wl.top_k),
                  "topk": ("hbm", alg["topk_bytes"]),
                  "combine": ("hbm", alg["combine_bytes"])}
    stage_work.update({n: ("mfma", f) for n, f in gemm_stages.items() if n != "lowrank_experts"})
    if wl.rank > 0:
        stage_work["lowrank_experts"] = ("hbm", roof["algorithmic_bytes"])
    stage_roof = {}
    for n, (bound, work) in stage_work.items():
        if n not in stage_us or stage_us[n] <= 0:
            continue
        if bound == "mfma":
            ach = work / (stage_us[n] * 1e-6) / 1e12
            stage_roof[n] = {"bound": "mfma" if wl.dtype != "f32" else "alu", "achieved": ach,
                             "unit": "TFLOP/s", "frac": ach / peak_mm}
        else:
            ach = work / (stage_us[n] * 1e-6) / 1e9
            stage_roof[n] = {"bound": "hbm", "achieved": ach, "unit": "GB/s",
                             "frac": ach / PEAK_HBM_GBS}

    result = {
        "metric": "MoE layer fwd tokens/s + expert-GEMM TFLOP/s (% MFMA peak), Quartz shape",
        "value": wl.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}-shape MoE layer forward"
                   + (f", T={wl.T}" if args.tokens > 0 else ""), "tokens": wl.T,
                   "hidden": wl.hidden, "routed_experts": wl.n_routed, "top_k": wl.top_k,
                   "shared_experts": wl.n_shared, "expert_ffn": wl.ffn, "rank": wl.rank,
                   "score": wl.score, "capacity": wl.capacity, "rows": rows,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "expert_gemm_tflops": expert_tflops,
        "expert_gemm_frac_of_peak": expert_tflops / PEAK_BF16_TFLOPS,
        "stage_us_mean": stage_us,
        "stage_us_median": stage_us_med,
        "call_ms_p10_p50_p90": warm_p,
        "cold_call_ms_p10_p50_p90": cold_p,
        "cold_stages": cold,
        "clock": clk,
        "stage_roofline": stage_roof,
        "combine_gbs": alg["combine_bytes"] / (stage_us["combine"] * 1e-6) / 1e9,
        "layer_flops": alg["router_flops"] + alg["gate_up_flops"] + alg["down_flops"]
        + alg["shared_gate_up_flops"] + alg["shared_down_flops"],
        "wall_s_timed_region": wall,
        "run": run_metadata(wl),
    }
    if wl.score == "sigmoid":
        # loss-free balancing step on this call's counts (the bias is restored)
        sb = w.t["select_bias"]
        saved = sb.clone()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            _lib.moe_bias_update(cfg, wl.T, out["counts"].data_ptr(), sb.data_ptr(), 1e-3, stream)
        e1.record()
        torch.cuda.synchronize()
        result["bias_update_us"] = e0.elapsed_time(e1) * 1e3 / args.steps
        sb.copy_(saved)
    if ((wl.dtype == "bf16" and wl.n_routed % 8 == 0) or wl.dtype == "f32") and wl.rank == 0 \
            and not args.no_backward:
        fms, bms, bst = time_backward(wl, cfg, x, w, args.steps, args.warmup, stream)
        bfl = backward_flops(wl, rows)
        gemm = {n: f for n, f in bfl.items() if n in bst}
        bwd = {"ms_per_step": bms, "tokens_per_s": wl.T / (bms * 1e-3),
               "forward_saving_products_ms": fms,
               "fwd_plus_bwd_tokens_per_s": wl.T / ((bms + fms) * 1e-3),
               "flops": sum(bfl.values()),
               "gemm_tflops": sum(gemm.values()) / (sum(bst[n] for n in gemm) * 1e-6) / 1e12,
               "stage_us_mean": bst}
        for n, f in gemm.items():
            bwd[n + "_tflops"] = f / (bst[n] * 1e-6) / 1e12
        result["backward"] = bwd
    if wl.dtype == "bf16" and wl.rank > 0 and not args.no_fp8:
        # low-rank experts with fp8 factors: the same HBM-bound kernel streams
        # half the weight bytes
        fms8, st8 = time_fp8(wl, inp, x, args.steps, args.warmup, stream)
        us8 = st8["lowrank_experts"]
        b8 = used * lowrank_expert_bytes(wl, fp8=True) + io
        result["fp8"] = {
            "ms_per_step": fms8, "tokens_per_s": wl.T / (fms8 * 1e-3), "stage_us_mean": st8,
            "lowrank_experts_algorithmic_bytes": b8,
            "lowrank_experts_gbs": b8 / (us8 * 1e-6) / 1e9,
            "lowrank_experts_frac_of_hbm_peak": b8 / (us8 * 1e-6) / 1e9 / PEAK_HBM_GBS,
        }
    if (wl.dtype == "bf16" and wl.rank in (32, 64) and wl.n_shared == 0 and wl.n_routed % 8 == 0
            and not args.no_backward):
        # rank-r experts: the backward recomputes the forward chain per row
        fms, bms, bst = time_backward(wl, cfg, x, w, args.steps, args.warmup, stream)
        used = int((out["kept"].cpu().numpy() > 0).sum())
        bfl, bby = lowrank_backward_work(wl, rows, used)
        bwd = {"ms_per_step": bms, "tokens_per_s": wl.T / (bms * 1e-3),
               "forward_ms": fms, "fwd_plus_bwd_tokens_per_s": wl.T / ((bms + fms) * 1e-3),
               "flops": sum(bfl.values()), "product_bytes": sum(bby.values()),
               "stage_us_mean": bst}
        for n in bfl:
            if n in bst:
                bwd[n + "_tflops"] = bfl[n] / (bst[n] * 1e-6) / 1e12
                bwd[n + "_gbs"] = bby[n] / (bst[n] * 1e-6) / 1e9
        result["backward"] = bwd
    if wl.dtype == "bf16" and wl.rank == 0 and not args.no_fp8:
        fms8, st8 = time_fp8(wl, inp, x, args.steps, args.warmup, stream)
        gu8 = alg["gate_up_flops"] + alg["shared_gate_up_flops"]
        dn8 = alg["down_flops"] + alg["shared_down_flops"]
        result["fp8"] = {
            "ms_per_step": fms8, "tokens_per_s": wl.T / (fms8 * 1e-3), "stage_us_mean": st8,
            "gate_up_tflops": gu8 / (st8["gate_up_gemm"] * 1e-6) / 1e12,
            "gate_up_frac_of_fp8_peak": gu8 / (st8["gate_up_gemm"] * 1e-6) / 1e12 / PEAK_FP8_TFLOPS,
            "expert_gemm_tflops": (gu8 + dn8) / ((st8["gate_up_gemm"] + st8["down_gemm"]) * 1e-6)
            / 1e12,
        }
    if args.blas_reference and wl.dtype == "bf16" and wl.rank == 0:
        result["blas_reference"] = blas_reference(wl, args.steps)
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result))


if __name__ == "__main__":
    main()
