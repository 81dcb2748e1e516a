"""Throughput of the fused SSIM loss, forward + backward, on one MI355X.

One step = one forward + backward of the chosen design (--design) on one batch
of synthetic images already resident in HBM, through the C ABI on torch's
current stream:
  one-pass  : ssim_loss_and_grad (loss and both gradients in one launch;
              the default)
  saved     : ssim_forward (training mode: loss + saved maps), then
              ssim_backward (both image gradients)
  recompute : ssim_forward (inference: loss only), then
              ssim_backward_recompute (both gradients, no maps)
  one-pass-ref : ssim_loss_and_grad_ref (a fixed reference whose statistics
              were cached outside the step; grad_img1 only)
  one-pass-x : ssim_loss_and_grad with grad_img2 NULL (a kernel that forms
              grad_img1 alone, as when only the render is differentiable)

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--dtype float32|float16|bfloat16] [--design NAME]
                    [--no-all-kernels] [--no-cpu]

Prints one JSON line: metric Mpix/s (pixels = N*H*W per step, wall clock over
K steps), the roofline of the dominant kernel (algorithmic bytes per launch /
average launch time from HIP events around K back-to-back launches of that
kernel on the stream it runs on), every design's step time from its kernels'
times (unless --no-all-kernels), the fp64 CPU oracle's throughput on a
bounded sample of the same workload and the parity of the timed step against
it.  Volume workloads (vol-*) time ssim3d_forward + ssim3d_backward instead.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published (256 CUs, 2.4 GHz)
PAGES_MPIX_S = 1920 * 1080 / 7.2e-3 / 1e6  # the pages' 7.2 ms fwd+bwd at 1080p (RDNA4 R9700)
CSRC = os.path.join(ROOT, "ssim_loss_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="1080p-valid")
    ap.add_argument("--dtype", default="float32", choices=["float32", "float16", "bfloat16"],
                    help="storage type of images and gradients (arithmetic is fp32)")
    ap.add_argument("--design", default="one-pass",
                    choices=["saved", "recompute", "one-pass", "one-pass-ref", "one-pass-x"],
                    help="saved: forward saves the statistics, backward reads them; "
                         "recompute: loss-only forward, backward recomputes the statistics; "
                         "one-pass: loss and gradients in one launch; "
                         "one-pass-ref: the same with the reference's statistics cached and "
                         "only the first image's gradient; "
                         "one-pass-x: one launch forming the first image's gradient alone")
    ap.add_argument("--all-kernels", action=argparse.BooleanOptionalAction, default=True,
                    help="after the timed steps, also time the kernels of the other designs "
                         "(reported under 'designs'; on by default)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other configurations (1080p-same, 4k-batch8) a default "
                         "1080p-valid run also times (profile passes skip them, so that every "
                         "dispatch of a kernel in the run has the workload's size)")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra steps timed with a cache flush before each (0 = skip)")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="before the warmup steps, run untimed steps for at least this long "
                         "(an idle GPU needs some milliseconds of load to reach its clock)")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB 3 times (counter calibration)")
    ap.add_argument("--profile", metavar="OUTDIR", default=None,
                    help="run the rocprofv3 passes for --workload / --dtype (kernel trace, "
                         "FETCH_SIZE, WRITE_SIZE, three SQ/GRBM counter groups), each a child "
                         "process under its own time limit, writing under OUTDIR, then "
                         "summarize them into profiles/")
    ap.add_argument("--summarize", metavar="OUTDIR", default=None,
                    help="only summarize the rocprofv3 CSVs a --profile run left under OUTDIR")
    return ap.parse_args()


def settle(step, ms):
    """Untimed steps until at least `ms` milliseconds of them have run: a GPU
    that sat idle (while the host built the inputs) takes several milliseconds
    of load to reach its clock, longer than a few dozen short warmup steps
    last.  Synchronised every 10 steps, so the host never queues far ahead.
    Returns the number of steps run."""
    import torch

    n = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        n += 10
    return n


_CODE_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"', re.S)


def source_hash() -> str:
    """Hash of the library's code (every file under csrc/ and include/, in
    name order), with comments dropped and white space collapsed: counters
    taken from a kernel stay valid across edits that do not change its code."""
    h = hashlib.sha256()
    inc = os.path.join(ROOT, "include")
    paths = [os.path.join(CSRC, n) for n in sorted(os.listdir(CSRC))]
    paths += [os.path.join(inc, n) for n in sorted(os.listdir(inc))]
    for path in paths:
        name = os.path.basename(path)
        with open(path, encoding="utf-8") as f:
            src = f.read()
        code = _CODE_TOKENS.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", src)
        h.update(name.encode() + b"\0" + " ".join(code.split()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(shape, padding, eb=4):
    """Compulsory HBM bytes per launch of each kernel (saved-maps design), for
    images and gradients of eb bytes per element: forward reads x, y (2 eb per
    input element) and writes four fp32 maps (16 B per map entry); backward
    reads the maps (16 B per entry), x and y (2 eb per element) and writes
    both gradients (2 eb per element).  The recomputing kernels read x, y and
    write both gradients (4 eb per element); the inference forward reads x, y.
    With a cached reference: x, y and the cached map (4 B per map entry) in,
    grad_x out; forming that map reads y and writes it.  One launch forming
    grad_x alone: x, y in, grad_x out (3 eb per element)."""
    N, C, H, W = shape
    Ho, Wo = (H - 10, W - 10) if padding == "valid" else (H, W)
    e_in = N * C * H * W
    e_out = N * C * Ho * Wo
    return {"ssim_forward": 2 * eb * e_in + 16 * e_out,
            "ssim_backward": 16 * e_out + 4 * eb * e_in,
            "ssim_forward(inference)": 2 * eb * e_in,
            "ssim_backward_recompute": 4 * eb * e_in,
            "ssim_loss_and_grad": 4 * eb * e_in,
            "ssim_loss_and_grad_ref": 3 * eb * e_in + 4 * e_out,
            "ssim_loss_and_grad(grad_x)": 3 * eb * e_in,
            "ssim_reference_stats": eb * e_in + 4 * e_out}


def algorithmic_flops(shape, padding):
    """fp32 operations per launch of each kernel (a fused multiply-add counts
    2), from the arithmetic of the method in the kernels' basis: per image
    element 5 for the products x', y', x - y, (x - y)^2, x'y'; per blurred
    quantity and output, 21 per separable pass (one multiply, ten FMAs) in
    each direction; per map entry 17 for the SSIM terms, 5 for 1 - S and its
    sum, 25 for the four loss partials; per image element 13 for the chain
    rule.  Four quantities are blurred forward (to map entries) and four
    partials backward (to image elements)."""
    N, C, H, W = shape
    Ho, Wo = (H - 10, W - 10) if padding == "valid" else (H, W)
    e_in = N * C * H * W
    e_out = N * C * Ho * Wo
    blur = 4 * 2 * 21
    fwd = 5 * e_in + (blur + 17 + 5) * e_out
    bwd_from_stats = (17 + 25) * e_out + (blur + 13) * e_in
    recompute = 5 * e_in + (blur + 17 + 25) * e_out + (blur + 13) * e_in
    blur3 = 3 * 2 * 21  # three quantities
    ref_step = 5 * e_in + (blur3 + 17 + 5 + 25) * e_out + (blur3 + 7) * e_in
    # grad_x alone: all four quantities forward, three partials backward
    x_step = 5 * e_in + (blur + 17 + 5 + 25) * e_out + (blur3 + 7) * e_in
    return {"ssim_forward": fwd, "ssim_forward(inference)": fwd,
            "ssim_backward": bwd_from_stats, "ssim_backward_recompute": recompute,
            "ssim_loss_and_grad": recompute + 5 * e_out, "ssim_loss_and_grad_ref": ref_step,
            "ssim_loss_and_grad(grad_x)": x_step}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_threads():
    """(cores this process may run on, threads the oracle uses, OMP_NUM_THREADS
    or None): every core of the affinity mask, unless OMP_NUM_THREADS sets a
    smaller share of the host (a GPU machine gives each GPU a share of its
    cores)."""
    try:
        ncores = len(os.sched_getaffinity(0))
    except AttributeError:
        ncores = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS")
    try:
        omp = int(omp) if omp else None
    except ValueError:
        omp = None
    threads = max(1, min(ncores, omp) if omp else ncores)
    return ncores, threads, omp


def cpu_baseline(x, y, padding, pixels_per_image_batch, dloss):
    """The fp64 oracle, as it stands, on the host cores: whole forward +
    gradient of the same workload, repeated until about 10 s have passed
    (at most 200 times); then one image plane on a single thread.  Returns
    the baseline record and the oracle's last (loss, grad_x, grad_y)."""
    import oracle

    ncores, threads, omp = host_threads()
    oracle.set_threads(threads)
    reps, t0 = 0, time.perf_counter()
    while True:
        res = oracle.ssim_loss(x, y, padding, dloss=dloss)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or reps >= 200:
            break
    # one (n, c) plane on one thread: a pixel of the batch has C planes
    C = x.shape[1]
    oracle.set_threads(1)
    t1 = time.perf_counter()
    oracle.ssim_loss(x[:1, :1], y[:1, :1], padding, dloss=dloss)
    el1 = time.perf_counter() - t1
    oracle.set_threads(threads)
    plane_pixels = x.shape[2] * x.shape[3]
    record = {
        "value": round(reps * pixels_per_image_batch / el / 1e6, 3),
        "unit": "Mpix/s",
        "cores": threads,
        "affinity_cores": ncores,
        "host_cpus": os.cpu_count(),
        "omp_num_threads": omp,
        "kind": "oracle",
        "sample": f"{reps} x whole forward+gradient of the benchmark batch "
                  f"({x.shape}, {padding}) in {el:.1f} s",
        "single_thread": {"value": round(plane_pixels / C / el1 / 1e6, 3), "unit": "Mpix/s",
                          "sample": f"one {x.shape[2]}x{x.shape[3]} plane in {el1:.2f} s"},
        "cpu_model": cpu_model(),
    }
    return record, res


def volume_algorithmic(shape, padding, eb):
    """Compulsory HBM bytes and fp32 operations per launch of the volume
    kernels (forward saves the four loss partials, 16 B per map voxel;
    backward reads them, reads both volumes and writes both gradients).
    Operations as for the images, with three 21-operation passes per blurred
    quantity instead of two."""
    N, C, D, H, W = shape
    sh = 10 if padding == "valid" else 0
    e_in = N * C * D * H * W
    e_out = N * C * (D - sh) * (H - sh) * (W - sh)
    blur = 4 * 3 * 21
    by = {"ssim3d_forward": 2 * eb * e_in + 16 * e_out,
          "ssim3d_backward": 16 * e_out + 4 * eb * e_in,
          "ssim3d_forward(inference)": 2 * eb * e_in}
    fl = {"ssim3d_forward": 5 * e_in + (blur + 17 + 5 + 25) * e_out,
          "ssim3d_backward": blur * e_in + 13 * e_in,
          "ssim3d_forward(inference)": 5 * e_in + (blur + 17 + 5) * e_out}
    return by, fl


def measured_traffic(args, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a copy kernel of known
    size), or None when there is none for this workload and dtype or it was
    taken from another version of the kernel sources."""
    tag = args.workload if args.dtype == "float32" else f"{args.workload}-{args.dtype}"
    path = os.path.join(PROFILES, f"hbm_traffic_{tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    if (tr.get("source_sha256_16") == source_hash() and tr.get("workload") == args.workload
            and tr.get("dtype", "float32") == args.dtype):
        return tr.get("bytes_per_launch", {}).get(kernel)
    return None


def copy_calibration(mib, dev):
    """A plain device copy of known size, for scaling the HBM counters."""
    import torch

    a = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def bench_volume(args, w, x, y):
    """Volumes: one step = ssim3d_forward (training: loss + saved partials)
    then ssim3d_backward (both gradients).  Mvox/s = N*D*H*W per step."""
    import torch

    import ssim_loss_amd as S

    N, C, D, H, W = x.shape
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdtype = getattr(torch, args.dtype)
    eb = torch.empty((), dtype=tdtype).element_size()
    t1 = torch.from_numpy(x).to(dev).to(tdtype).contiguous()
    t2 = torch.from_numpy(y).to(dev).to(tdtype).contiguous()
    loss = torch.empty((), dtype=torch.float32, device=dev)
    maps = S.alloc_saved_maps3d(t1, w.padding)
    ws = S.workspace_for(dev)
    dloss = torch.tensor(0.8, dtype=torch.float32, device=dev)
    g1 = torch.empty_like(t1)
    g2 = torch.empty_like(t2)
    fwd = lambda: S.ssim3d_forward(t1, t2, w.padding, loss, maps, ws)
    bwd = lambda: S.ssim3d_backward(dloss, t1, t2, w.padding, maps, g1, g2)
    def vstep():
        fwd()
        bwd()

    n_settle = settle(vstep, args.settle_ms)
    for _ in range(args.warmup):
        vstep()
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for _ in range(K):
        vstep()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    mvox = N * D * H * W / 1e6

    def per_launch_ms(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    kern = {"ssim3d_forward": per_launch_ms(fwd), "ssim3d_backward": per_launch_ms(bwd),
            "ssim3d_forward(inference)":
                per_launch_ms(lambda: S.ssim3d_forward(t1, t2, w.padding, loss, None, ws))}
    if args.copy_calib > 0:
        copy_calibration(args.copy_calib, dev)
    by, fl = volume_algorithmic(x.shape, w.padding, eb)
    dom = max(("ssim3d_forward", "ssim3d_backward"), key=lambda k: kern[k])
    gbs = by[dom] / (kern[dom] * 1e-3) / 1e9
    tfs = fl[dom] / (kern[dom] * 1e-3) / 1e12
    out = {
        "metric": "Mvox/s fused 3-D SSIM fwd+bwd (volumes)",
        "value": round(mvox * K / elapsed, 1),
        "unit": "Mvox/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": n_settle},
        "ms_per_step": round(elapsed * 1e3 / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"float32": "f32", "float16": "f16 I/O, f32 math",
                  "bfloat16": "bf16 I/O, f32 math"}[args.dtype],
        "data": "synthetic",
        "config": {"workload": args.workload, "shape": list(x.shape), "padding": w.padding,
                   "design": "saved partials"},
        # the volume kernels are bound by neither roofline (LDS and latency);
        # the nearer of the two is HBM, and the ALU position goes beside it
        "roofline": {"bound": "hbm", "kernel": dom,
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args, dom), "algorithmic_bytes": by[dom],
                     "alu": {"achieved": round(tfs, 2), "peak": FP32_VECTOR_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tfs / FP32_VECTOR_PEAK_TFLOPS, 4),
                             "algorithmic_flops": fl[dom]}},
        "kernels_ms": {k: round(v, 5) for k, v in kern.items()},
        "loss": float(loss.item()),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def events_ms(fn, reps, warm=3):
    """Average milliseconds per call of fn over reps calls back to back,
    between two HIP events on torch's current stream (the stream the library
    launches on)."""
    import torch

    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def roofline_fracs(shape, padding, kernel, ms, eb=4):
    """The kernel's algorithmic fp32 rate and HBM rate per launch of ms
    milliseconds, as fractions of the published peaks."""
    tf = algorithmic_flops(shape, padding)[kernel] / (ms * 1e-3) / 1e12
    gbs = algorithmic_bytes(shape, padding, eb)[kernel] / (ms * 1e-3) / 1e9
    return {"alu": {"achieved": round(tf, 2), "unit": "TFLOP/s",
                    "frac": round(tf / FP32_VECTOR_PEAK_TFLOPS, 4)},
            "hbm": {"achieved": round(gbs, 1), "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def one_launch_record(t1, t2, padding, ws, reps):
    """The one-launch step (ssim_loss_and_grad, both gradients) on resident
    images: per-launch time from HIP events, Mpix/s and both roofline
    fractions."""
    import torch

    import ssim_loss_amd as S

    N, C, H, W = t1.shape
    loss = torch.empty((), dtype=torch.float32, device=t1.device)
    dl = torch.tensor(0.8, dtype=torch.float32, device=t1.device)
    g1, g2 = torch.empty_like(t1), torch.empty_like(t2)
    f = lambda: S.ssim_loss_and_grad(t1, t2, padding, dl, loss, ws, g1, g2)
    settle(f, 200.0)
    ms = events_ms(f, reps)
    rec = {"shape": [N, C, H, W], "padding": padding, "launches": reps,
           "ms_per_launch": round(ms, 5), "mpix_per_s": round(N * H * W / (ms * 1e-3) / 1e6, 1)}
    rec.update(roofline_fracs((N, C, H, W), padding, "ssim_loss_and_grad", ms))
    return rec


def autograd_record(t1, t2, padding, reps, both=True):
    """ssim_loss(img1, img2).backward() with both images requiring gradients
    (or img1 alone, as for a render against a fixed ground truth), timed
    three ways: the step as the GPU queue sees it (HIP events around reps
    steps), the host's time to issue a step (autograd engine and binding; no
    synchronisation inside the loop) and the GPU time of the step's launches
    alone, back to back without autograd."""
    import torch

    import ssim_loss_amd as S

    a1 = t1.detach().clone().requires_grad_(True)
    a2 = t2.detach().clone().requires_grad_(both)
    early = 4 * t1.nbytes <= S.EARLY_GRADIENT_BYTES

    def step():
        a1.grad = None
        a2.grad = None
        S.ssim_loss(a1, a2, padding).backward()

    settle(step, 200.0)
    step_ms = events_ms(step, reps)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for _ in range(reps):
        step()
    host_ms = (time.perf_counter() - h0) * 1e3 / reps
    torch.cuda.synchronize()
    dev = t1.device
    ws = S.workspace_for(dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    dl = torch.ones((), dtype=torch.float32, device=dev)
    if early:
        gbuf = torch.empty((2 if both else 1,) + tuple(t1.shape), dtype=torch.float32, device=dev)

        def kernels():
            S.ssim_loss_and_grad(t1, t2, padding, dl, loss, ws, gbuf[0], gbuf[1] if both else None)
            S.ssim_grad_scale(dl, gbuf, gbuf)

        launches = ("ssim_loss_and_grad (upstream gradient 1) + one ssim_grad_scale over "
                    + ("both" if both else "grad_img1"))
    else:
        g1, g2 = torch.empty_like(t1), (torch.empty_like(t2) if both else None)

        def kernels():
            S.ssim_forward(t1, t2, padding, loss, None, ws)
            S.ssim_backward_recompute(dl, t1, t2, padding, g1, g2)

        launches = "ssim_forward (inference) + ssim_backward_recompute"
    gpu_ms = events_ms(kernels, reps)
    N, C, H, W = t1.shape
    return {"ms_per_step": round(step_ms, 5), "mpix_per_s": round(N * H * W / (step_ms * 1e-3) / 1e6, 1),
            "host_ms_per_step": round(host_ms, 5), "gpu_ms_per_step": round(gpu_ms, 5),
            "gradients": "both" if both else "grad_img1", "launches": launches, "steps": reps}


# ---------------------------------------------------------------------------
# rocprofv3 passes and their summaries (profiles/)

# The library's kernels by entry point: (kernel-name prefix without the image
# type, entry point).  Stream and unaligned variants count for their entry.
KERNEL_ENTRY = [
    ("ssim_loss_grad_ref", "ssim_loss_and_grad_ref"),
    ("ssim_loss_grad_x", "ssim_loss_and_grad(grad_x)"),
    ("ssim_loss_grad_y", "ssim_loss_and_grad(grad_y)"),
    ("ssim_bwd_recompute_x", "ssim_backward_recompute(grad_x)"),
    ("ssim_bwd_recompute_y", "ssim_backward_recompute(grad_y)"),
    ("ssim_loss_grad", "ssim_loss_and_grad"),
    ("ssim_bwd_recompute", "ssim_backward_recompute"),
    ("ssim_bwd", "ssim_backward"),
    ("ssim_fwd_train", "ssim_forward"),
    ("ssim_fwd_infer", "ssim_forward(inference)"),
    ("ssim_ref_stats", "ssim_reference_stats"),
    ("ssim3d_fwd_train", "ssim3d_forward"),
    ("ssim3d_fwd_infer", "ssim3d_forward(inference)"),
    ("ssim3d_bwd", "ssim3d_backward"),
    ("ssim_grad_scale", "ssim_grad_scale"),
]
SQ_GROUPS = {
    "sq_a": "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_VALU_FMA_F32 SQ_INSTS_LDS SQ_INSTS_SALU "
            "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_ACTIVE_INST_VALU",
    "sq_b": "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS "
            "SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_LDS",
    "sq_c": "GRBM_GUI_ACTIVE GRBM_COUNT SQ_INSTS_VALU SQ_WAVES",
}


def kernel_entry(name):
    """The entry point a kernel name belongs to, or None (other kernels)."""
    m = re.search(r"(ssim(?:3d)?_\w*?kernel)", name)
    if not m:
        return None
    base = m.group(1)
    for prefix, entry in KERNEL_ENTRY:
        if base.startswith(prefix):
            rest = base[len(prefix):]
            # the next prefix down is a longer name (ssim_bwd vs ssim_bwd_recompute)
            if prefix == "ssim_bwd" and rest.startswith("_recompute"):
                continue
            if prefix == "ssim_loss_grad" and rest.startswith("_ref"):
                continue
            return entry
    return None


def profile_passes(workload, dtype, outdir):
    """The rocprofv3 command lines of a profile of one workload (each run from
    the repository root): the kernel trace of the whole bench (every design's
    kernels) and one counter pass per group, on a short run with a 512 MiB
    calibration copy."""
    bench = ["python3", "bench.py", "--workload", workload, "--dtype", dtype, "--no-cpu",
             "--no-workloads", "--cold-steps", "0"]
    short = bench + ["--steps", "20", "--warmup", "3", "--settle-ms", "50"]
    passes = {"trace": (300, ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv",
                              "-d", f"{outdir}/trace", "-o", "run", "--"]
                        + bench + ["--steps", "300", "--warmup", "10"])}
    pmc = {"fetch": "FETCH_SIZE", "write": "WRITE_SIZE", **SQ_GROUPS}
    for key, counters in pmc.items():
        passes[key] = (120, ["rocprofv3", "--pmc", *counters.split(), "--output-format", "csv",
                             "-d", f"{outdir}/{key}", "-o", "p", "--"]
                       + short + ["--copy-calib", "512"])
    return passes


def run_profile(workload, dtype, outdir):
    """Every pass of profile_passes, in order, each a child process under its
    own kill-on-expiry time limit; stops at the first pass that fails.  The
    bench line each pass prints goes to <outdir>/<pass>.log."""
    import subprocess

    os.makedirs(outdir, exist_ok=True)
    for key, (limit, cmd) in profile_passes(workload, dtype, outdir).items():
        print(f"[profile] {workload} {dtype} pass {key}: {' '.join(cmd)}", flush=True)
        with open(os.path.join(outdir, f"{key}.log"), "w") as log:
            rc = subprocess.run(["timeout", "-s", "KILL", str(limit), *cmd], cwd=ROOT, stdout=log,
                                stderr=subprocess.STDOUT).returncode
        # (rocprofv3 itself may end with a segmentation fault after the program's
        # results are whole; the summary checks for them)
        print(f"[profile] pass {key} exit {rc}", flush=True)
        if rc not in (0, 139, -11):
            return rc
    return 0


def _csv_rows(outdir, key, suffix):
    import csv
    import glob

    rows = []
    for path in sorted(glob.glob(os.path.join(outdir, key, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _bench_line(outdir, key):
    path = os.path.join(outdir, f"{key}.log")
    if not os.path.exists(path):
        return None
    for line in reversed(open(path).read().splitlines()):
        if line.startswith("{"):
            try:
                return json.loads(line)
            except ValueError:
                return None
    return None


def _counter_dispatches(outdir, key):
    """Per kernel name: {counter: {dispatch: value}}, from one --pmc pass."""
    acc = {}
    for r in _csv_rows(outdir, key, "counter_collection.csv"):
        name = r.get("Kernel_Name", "")
        cnt = r.get("Counter_Name", "")
        try:
            val = float(r.get("Counter_Value", "nan"))
        except ValueError:
            continue
        disp = r.get("Dispatch_Id", "")
        acc.setdefault(name, {}).setdefault(cnt, {})
        # a dispatch's value may come in several rows (per XCD or SE): sum them
        acc[name][cnt][disp] = acc[name][cnt].get(disp, 0.0) + val
    return acc


def _counter_means(outdir, key):
    """Per kernel name: {counter: mean per dispatch}, from one --pmc pass."""
    return {n: {c: sum(d.values()) / len(d) for c, d in cs.items()}
            for n, cs in _counter_dispatches(outdir, key).items()}


def _per_entry(means):
    """Counter means by entry point (the dispatch-weighted mean over its
    kernel variants present in the run; one variant runs per workload)."""
    out = {}
    for name, cs in means.items():
        e = kernel_entry(name)
        if e is not None:
            out.setdefault(e, cs)
    return out


def summarize_profile(workload, dtype, outdir, profiles_dir=PROFILES):
    """Writes profiles/ssim_kernels_<tag>_kernel_trace.md, hbm_traffic_<tag>.json
    and sq_counters_<tag>.json (+ .md) from a --profile run's CSVs, tag =
    workload, with -<dtype> for half types.  FETCH_SIZE and WRITE_SIZE are
    scaled by what they read for the 512 MiB calibration copy."""
    tag = workload if dtype == "float32" else f"{workload}-{dtype}"
    sha = source_hash()
    passes = profile_passes(workload, dtype, "OUT")
    cmd = lambda key: " ".join(passes[key][1]).replace("OUT", os.path.relpath(outdir, ROOT))
    os.makedirs(profiles_dir, exist_ok=True)

    # kernel trace
    stats = _csv_rows(outdir, "trace", "kernel_stats.csv")
    trace = _csv_rows(outdir, "trace", "kernel_trace.csv")
    lines = [f"# rocprofv3 kernel trace: {workload} ({dtype} images)", "",
             "Command (from the repository root, on the MI355X):", "", "```", cmd("trace"), "```",
             "", f"Library code sha256[:16] (ssim_loss_amd/csrc and include, comments dropped): "
             f"`{sha}`", "", "| kernel | entry point | calls | average (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|---|"]
    for r in stats:
        name = r.get("Name", r.get("Kernel_Name", ""))
        try:
            calls = int(r["Calls"])
            avg, mn, mx = (float(r[k]) / 1e3 for k in ("AverageNs", "MinNs", "MaxNs"))
            share = float(r.get("Percentage", "nan"))
        except (KeyError, ValueError):
            continue
        lines.append(f"| {name[:60]} | {kernel_entry(name) or '-'} | {calls} | {avg:.2f} | "
                     f"{mn:.2f} | {mx:.2f} | {share:.1f}% |")
    # runs of one kernel launched back to back (bench times each entry point's
    # launches between HIP events after the timed steps)
    runs = []
    for r in sorted(trace, key=lambda r: int(r.get("Start_Timestamp", 0))):
        name = r.get("Kernel_Name", "")
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if runs and runs[-1][0] == name:
            runs[-1][1].append(dur)
        else:
            runs.append([name, [dur]])
    lines += ["", "The same dispatches as runs of one kernel launched back to back, in launch order "
              "(runs of fewer than 6 left out):", "", "| order | kernel | launches | average (us) | "
              "median (us) |", "|---|---|---|---|---|"]
    k = 0
    for name, durs in runs:
        if len(durs) < 6:
            continue
        k += 1
        durs = sorted(durs)
        lines.append(f"| {k} | {kernel_entry(name) or name[:40]} | {len(durs)} | "
                     f"{sum(durs) / len(durs):.2f} | {durs[len(durs) // 2]:.2f} |")
    line = _bench_line(outdir, "trace")
    if line:
        lines += ["", "The bench line printed by the profiled run: "
                  f"{line.get('value')} {line.get('unit')}, {line.get('ms_per_step', 0) * 1e3:.2f} us "
                  f"per step; kernels_ms " + ", ".join(f"{k} {v * 1e3:.2f} us" for k, v in
                                                       line.get("kernels_ms", {}).items()) + "."]
    with open(os.path.join(profiles_dir, f"ssim_kernels_{tag}_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # HBM traffic
    fetch = _counter_means(outdir, "fetch")
    write = _counter_means(outdir, "write")

    # the calibration copies: copy_calibration's three device copies, the last
    # three large copy dispatches of the run (earlier ones stage the inputs
    # from the host and can be larger; the small ones move scalars)
    def calib(key, cnt):
        disp = sorted((int(i), v) for n, cs in _counter_dispatches(outdir, key).items()
                      if "copy" in n.lower() for i, v in cs.get(cnt, {}).items())
        big = [v for _, v in disp if v >= 1024.0]
        return sorted(big[-3:])[len(big[-3:]) // 2] if len(big) >= 3 else None

    f_cal, w_cal = calib("fetch", "FETCH_SIZE"), calib("write", "WRITE_SIZE")
    traffic = None
    if f_cal and w_cal:
        fs, wsc = 524288.0 / f_cal, 524288.0 / w_cal
        fe, we = _per_entry(fetch), _per_entry(write)
        detail = {e: {"read_bytes": int(fe[e]["FETCH_SIZE"] * 1024 * fs),
                      "write_bytes": int(we[e]["WRITE_SIZE"] * 1024 * wsc)}
                  for e in fe if e in we and "FETCH_SIZE" in fe[e] and "WRITE_SIZE" in we[e]}
        traffic = {"workload": workload, "dtype": dtype, "source_sha256_16": sha,
                   "fetch_scale": round(fs, 4), "write_scale": round(wsc, 4),
                   "calibration": f"torch copy of 512 MiB: FETCH_SIZE {f_cal:.0f} KiB, WRITE_SIZE "
                                  f"{w_cal:.0f} KiB per dispatch",
                   "commands": [cmd("fetch"), cmd("write")],
                   "bytes_per_launch": {e: d["read_bytes"] + d["write_bytes"] for e, d in detail.items()},
                   "detail": detail}
        with open(os.path.join(profiles_dir, f"hbm_traffic_{tag}.json"), "w") as f:
            json.dump(traffic, f, indent=1)
        from ssim_loss_amd.inputs import WORKLOADS

        w = WORKLOADS[workload]
        eb = 4 if dtype == "float32" else 2
        algo = (volume_algorithmic(w.shape, w.padding, eb)[0] if len(w.shape) == 5
                else algorithmic_bytes(w.shape, w.padding, eb))
        md = [f"# HBM traffic per launch (rocprofv3 --pmc): {workload}, {dtype} images", "",
              "Commands:", "", "```", cmd("fetch"), cmd("write"), "```", "",
              f"Library code sha256[:16]: `{sha}`", "",
              f"Calibration: a torch device copy of 512 MiB in the same process reads FETCH_SIZE = "
              f"{f_cal:.0f} KiB and WRITE_SIZE = {w_cal:.0f} KiB per dispatch, so FETCH_SIZE is "
              f"scaled by {fs:.3f} and WRITE_SIZE by {wsc:.3f}.", "",
              "| kernel | read MB | write MB | traffic MB | algorithmic MB | traffic / algorithmic |",
              "|---|---|---|---|---|---|"]
        for e, d in detail.items():
            tot = d["read_bytes"] + d["write_bytes"]
            a = algo.get(e)
            md.append(f"| {e} | {d['read_bytes'] / 1e6:.1f} | {d['write_bytes'] / 1e6:.1f} | "
                      f"{tot / 1e6:.1f} | {'-' if a is None else f'{a / 1e6:.1f}'} | "
                      f"{'-' if not a else f'{tot / a:.3f}'} |")
        with open(os.path.join(profiles_dir, f"ssim_kernels_{tag}_hbm_traffic.md"), "w") as f:
            f.write("\n".join(md) + "\n")

    # SQ / GRBM counters
    sq = {}
    for key in SQ_GROUPS:
        for e, cs in _per_entry(_counter_means(outdir, key)).items():
            sq.setdefault(e, {}).update(cs)
    kernel_us = {}
    for r in stats:
        e = kernel_entry(r.get("Name", ""))
        if e is not None:
            kernel_us.setdefault(e, float(r["AverageNs"]) / 1e3)
    derived = {}
    for e, c in sq.items():
        d = {}
        g = lambda k: c.get(k)
        if g("SQ_INSTS_VALU") and g("SQ_WAVES"):
            d["valu_insts_per_wave"] = round(g("SQ_INSTS_VALU") / g("SQ_WAVES"), 1)
        if g("SQ_ACTIVE_INST_VALU") and g("SQ_WAVE_CYCLES"):
            d["valu_active_share_of_wave_cycles"] = round(g("SQ_ACTIVE_INST_VALU") / g("SQ_WAVE_CYCLES"), 4)
        if g("SQ_LDS_BANK_CONFLICT") is not None and g("SQ_LDS_IDX_ACTIVE"):
            d["lds_bank_conflict_share_of_lds_active"] = round(g("SQ_LDS_BANK_CONFLICT") / g("SQ_LDS_IDX_ACTIVE"), 4)
        if g("SQ_WAIT_INST_ANY") and g("SQ_WAVE_CYCLES"):
            d["wait_share_of_wave_cycles"] = round(g("SQ_WAIT_INST_ANY") / g("SQ_WAVE_CYCLES"), 4)
        if g("SQ_WAIT_INST_LDS") and g("SQ_WAVE_CYCLES"):
            d["lds_wait_share_of_wave_cycles"] = round(g("SQ_WAIT_INST_LDS") / g("SQ_WAVE_CYCLES"), 4)
        if g("SQ_INSTS_VALU_FMA_F32") and g("SQ_INSTS_VALU"):
            d["fma_f32_share_of_valu"] = round(g("SQ_INSTS_VALU_FMA_F32") / g("SQ_INSTS_VALU"), 4)
        us = kernel_us.get(e)
        if us and g("GRBM_GUI_ACTIVE"):
            ghz = g("GRBM_GUI_ACTIVE") / 8 / (us * 1e3)
            d["clock_ghz"] = round(ghz, 3)
            if g("SQ_INSTS_VALU"):
                d["valu_insts_per_cu_per_cycle"] = round(g("SQ_INSTS_VALU") / 256 / (us * 1e3 * ghz), 3)
        if us and g("SQ_INSTS_VALU"):
            d["valu_insts_per_cu_per_ns"] = round(g("SQ_INSTS_VALU") / 256 / (us * 1e3), 3)
        if us and traffic and e in traffic["bytes_per_launch"]:
            d["counter_gbs"] = round(traffic["bytes_per_launch"][e] / (us * 1e-6) / 1e9, 1)
        if us:
            d["trace_avg_us"] = round(us, 2)
        derived[e] = d
    sqrec = {"workload": workload, "dtype": dtype, "source_sha256_16": sha,
             "commands": [cmd(k) for k in SQ_GROUPS], "counters": sq, "derived": derived}
    with open(os.path.join(profiles_dir, f"sq_counters_{tag}.json"), "w") as f:
        json.dump(sqrec, f, indent=1)
    md = [f"# SQ and GRBM counters per launch (rocprofv3 --pmc): {workload}, {dtype} images", "",
          "Commands (each pass in a run of its own, under `timeout -s KILL 120`):", "", "```",
          *[cmd(k) for k in SQ_GROUPS], "```", "",
          f"Library code sha256[:16]: `{sha}`. Each counter is the per-dispatch value summed over "
          "the chip, averaged over the dispatches of the run; SQ_WAVE_CYCLES, SQ_ACTIVE_INST_* and "
          "SQ_WAIT_INST_* count in one unit, so only their ratios are used; GRBM_GUI_ACTIVE / 8 / "
          "(the kernel's trace average) gives the clock the launch ran at.", ""]
    for e, d in derived.items():
        md.append(f"- **{e}**: " + ", ".join(f"{k} {v}" for k, v in d.items()))
    with open(os.path.join(profiles_dir, f"ssim_kernels_{tag}_sq_counters.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(f"[summarize] wrote profiles for {tag} (source {sha})", flush=True)


def committed_counters(args, kernel):
    """The dominant kernel's derived counter figures from the committed
    profiles/sq_counters_<tag>.json, or None when there is none for this
    workload and dtype or it belongs to other kernel sources."""
    tag = args.workload if args.dtype == "float32" else f"{args.workload}-{args.dtype}"
    path = os.path.join(PROFILES, f"sq_counters_{tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash():
        return None
    return rec.get("derived", {}).get(kernel)


DESIGNS = {
    # design: the launches of one step
    "saved": ("ssim_forward", "ssim_backward"),
    "recompute": ("ssim_forward(inference)", "ssim_backward_recompute"),
    "one-pass": ("ssim_loss_and_grad",),
    # a fixed reference with its statistics cached (computed once, outside
    # the step), only the first image's gradient
    "one-pass-ref": ("ssim_loss_and_grad_ref",),
    # only the first image's gradient (the second pointer NULL)
    "one-pass-x": ("ssim_loss_and_grad(grad_x)",),
}


def main():
    args = parse()
    if args.summarize or args.profile:
        outdir = os.path.abspath(args.summarize or args.profile)
        if args.profile:
            rc = run_profile(args.workload, args.dtype, outdir)
            if rc != 0:
                sys.exit(rc)
        summarize_profile(args.workload, args.dtype, outdir)
        return
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by image planes with one scalar all-reduce, which is not built",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import ssim_loss_amd as S
    from ssim_loss_amd.inputs import WORKLOADS, make_workload

    w = WORKLOADS[args.workload]
    x, y = make_workload(args.workload)
    if x.ndim == 5:
        return bench_volume(args, w, x, y)
    N, C, H, W = x.shape
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdtype = getattr(torch, args.dtype)
    eb = torch.empty((), dtype=tdtype).element_size()
    t1 = torch.from_numpy(x).to(dev).to(tdtype).contiguous()
    t2 = torch.from_numpy(y).to(dev).to(tdtype).contiguous()
    loss = torch.empty((), dtype=torch.float32, device=dev)
    maps = S.alloc_saved_maps(t1, w.padding) if args.design == "saved" or args.all_kernels else None
    ws = S.workspace_for(dev)
    dloss = torch.tensor(0.8, dtype=torch.float32, device=dev)  # as under a weighted loss
    g1 = torch.empty_like(t1)
    g2 = torch.empty_like(t2)
    ref = (S.reference_stats(t2, w.padding)
           if args.design == "one-pass-ref" or args.all_kernels else None)
    torch.cuda.synchronize()

    launches = {
        "ssim_forward": lambda: S.ssim_forward(t1, t2, w.padding, loss, maps, ws),
        "ssim_backward": lambda: S.ssim_backward(dloss, t1, t2, w.padding, maps, g1, g2),
        "ssim_forward(inference)": lambda: S.ssim_forward(t1, t2, w.padding, loss, None, ws),
        "ssim_backward_recompute":
            lambda: S.ssim_backward_recompute(dloss, t1, t2, w.padding, g1, g2),
        "ssim_loss_and_grad":
            lambda: S.ssim_loss_and_grad(t1, t2, w.padding, dloss, loss, ws, g1, g2),
        "ssim_loss_and_grad_ref":
            lambda: S.ssim_loss_and_grad_ref(t1, t2, ref, w.padding, dloss, loss, ws, g1),
        "ssim_loss_and_grad(grad_x)":
            lambda: S.ssim_loss_and_grad(t1, t2, w.padding, dloss, loss, ws, g1, None),
    }
    step_launches = [launches[k] for k in DESIGNS[args.design]]

    def step():
        for f in step_launches:
            f()

    n_settle = settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the step: K passes of the design's launches, wall clock between two
    # synchronisations
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / K
    mpix = N * H * W / 1e6
    value = mpix * K / elapsed

    # per-kernel launch time: K launches of one kernel back to back between two
    # HIP events on the stream the kernels run on (torch's current stream)
    def per_launch_ms(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    timed = [k for k in launches if (maps is not None or k not in ("ssim_forward", "ssim_backward"))
             and (ref is not None or k != "ssim_loss_and_grad_ref")
             and (args.all_kernels or k in DESIGNS[args.design])]
    kern = {k: per_launch_ms(launches[k]) for k in timed}

    # the autograd path (ssim_loss(...).backward(), both gradients) at this
    # size; the default run adds the 4K batch below
    autograd = None
    if args.all_kernels and args.dtype == "float32":
        autograd = {args.workload: autograd_record(t1, t2, w.padding, min(K, 500)),
                    f"{args.workload}, grad_img1 only":
                        autograd_record(t1, t2, w.padding, min(K, 500), both=False)}

    # cold: flush the 256 MB last-level cache before each step (outside the events)
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        times = []
        for _ in range(args.cold_steps):
            flush.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        del flush
        cms = sum(times) / len(times)
        cold = {"ms_per_step": round(cms, 5), "mpix_per_s": round(mpix / (cms * 1e-3), 1)}

    if args.copy_calib > 0:
        copy_calibration(args.copy_calib, dev)

    # a plain device copy moving the dominant kernel's algorithmic bytes
    # (half read, half written), for the HBM fraction against what a copy of
    # that size reaches on this device
    def copy_gbs(nbytes):
        n = max(1, int(nbytes // 8))
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record()
        for _ in range(reps):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        return 8.0 * n / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9

    alg = algorithmic_bytes((N, C, H, W), w.padding, eb)
    flops = algorithmic_flops((N, C, H, W), w.padding)
    dom = max(DESIGNS[args.design], key=lambda k: kern[k])
    achieved = alg[dom] / (kern[dom] * 1e-3) / 1e9
    # (not in counter runs: the calibration copy must be the only large copy)
    cgbs = copy_gbs(alg[dom]) if args.copy_calib == 0 else None
    achieved_tf = flops[dom] / (kern[dom] * 1e-3) / 1e12
    # the bound of the dominant kernel: the resource it uses the larger
    # fraction of (the saved-maps kernels stream HBM; the recomputing ones
    # are arithmetic-heavy)
    alu_bound = achieved_tf / FP32_VECTOR_PEAK_TFLOPS > achieved / HBM_PEAK_GBS

    # HBM bytes per launch measured by rocprofv3 counters (FETCH_SIZE and
    # WRITE_SIZE, scaled by a copy kernel of known size), valid only for the
    # kernel source they were taken from
    traffic = measured_traffic(args, dom)

    # every design whose launches were all timed: its step from the per-kernel
    # times, and its algorithmic HBM rate
    designs = {}
    for d, ks in DESIGNS.items():
        if all(k in kern for k in ks):
            ms = sum(kern[k] for k in ks)
            by = sum(alg[k] for k in ks)
            fl = sum(flops[k] for k in ks)
            designs[d] = {"ms_per_step": round(ms, 5), "mpix_per_s": round(mpix / (ms * 1e-3), 1),
                          "hbm_bytes_per_elem": round(by / (N * C * H * W), 2),
                          "algorithmic_gbs": round(by / (ms * 1e-3) / 1e9, 1),
                          "algorithmic_tflops": round(fl / (ms * 1e-3) / 1e12, 2)}

    out = {
        "metric": "Mpix/s fused SSIM fwd+bwd fp32 at 1080p; achieved HBM GB/s as % of peak",
        "value": round(value, 1),
        "unit": "Mpix/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": n_settle},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(value / PAGES_MPIX_S, 2)
                        if args.workload == "1080p-valid" and args.dtype == "float32" else None),
        "dtype": {"float32": "f32", "float16": "f16 I/O, f32 math",
                  "bfloat16": "bf16 I/O, f32 math"}[args.dtype],
        "data": "synthetic",
        "config": {"workload": args.workload, "shape": [N, C, H, W], "padding": w.padding,
                   "design": args.design},
        "roofline": ({
            "bound": "alu",
            "kernel": dom,
            "achieved": round(achieved_tf, 2),
            "peak": FP32_VECTOR_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved_tf / FP32_VECTOR_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flops": flops[dom],
            "hbm": {"achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes": alg[dom]},
        } if alu_bound else {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": alg[dom],
            "alu": {"achieved": round(achieved_tf, 2), "peak": FP32_VECTOR_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved_tf / FP32_VECTOR_PEAK_TFLOPS, 4),
                    "algorithmic_flops": flops[dom]},
        }),
        "counters": committed_counters(args, dom),
        "kernels_ms": {k: round(v, 5) for k, v in kern.items()},
        "designs": designs,
        "autograd": autograd,
        "cold": cold,
        "rates": {
            "melem_per_s": round(N * C * H * W * K / elapsed / 1e6, 1),
            "gbs_at_24_b_per_elem": round(24 * N * C * H * W * K / elapsed / 1e9, 1),
            "copy_gbs_same_bytes": round(cgbs, 1) if cgbs else None,
            "hbm_frac_of_copy": round(achieved / cgbs, 4) if cgbs else None,
        },
        "loss": float(loss.item()),
    }
    # the other configurations the target names, timed in this run: the
    # one-launch step on 1080p with same padding and on the 8 x 4K batch (and
    # the autograd step on the batch)
    if (args.all_kernels and args.dtype == "float32" and args.workload == "1080p-valid"
            and not args.no_workloads):
        out["workloads"] = {}
        for name in ("1080p-same", "4k-batch8"):
            wl = WORKLOADS[name]
            xo, yo = make_workload(name)
            u1 = torch.from_numpy(xo).to(dev)
            u2 = torch.from_numpy(yo).to(dev)
            del xo, yo
            reps = 1000 if u1.numel() < 1e7 else 40
            out["workloads"][name] = one_launch_record(u1, u2, wl.padding, ws, reps)
            if name == "4k-batch8":
                out["autograd"][name] = autograd_record(u1, u2, wl.padding, 20)
            del u1, u2
            torch.cuda.empty_cache()

    if not args.no_cpu:
        # the oracle gets the values the GPU read (half-precision inputs rounded)
        xo = t1.float().cpu().numpy()
        yo = t2.float().cpu().numpy()
        # one fresh step of the timed design, for parity against the oracle
        g1.zero_()
        g2.zero_()
        step()
        torch.cuda.synchronize()
        dl = float(dloss.item())
        out["cpu_baseline"], (ol, ogx, ogy) = cpu_baseline(xo, yo, w.padding, N * H * W, dl)
        gl = float(loss.item())
        par = {"loss_rel_err": abs(gl - ol) / abs(ol),
               "grad1_err_over_max": float(np.abs(g1.float().cpu().numpy() - ogx).max()
                                           / np.abs(ogx).max())}
        if args.design != "one-pass-ref":
            par["grad2_err_over_max"] = float(np.abs(g2.float().cpu().numpy() - ogy).max()
                                              / np.abs(ogy).max())
        out["parity_vs_oracle"] = {k: float(f"{v:.3g}") for k, v in par.items()}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
