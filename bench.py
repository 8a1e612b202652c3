"""Benchmark of the weight-only 4-bit linear layer on one MI355X.

A step is one pass of the layer over the four projections of one
Llama-3.2-1B-shaped decoder layer (2048->2048, 2048->8192 x2, 8192->2048,
group size 32, seeded synthetic inputs):
  * decode (M = 1, the fp32 GEMV): the headline value, in GB/s of
    algorithmic bytes (packed weights + scales + activations + outputs);
  * prefill (M = 512, the binary16 MFMA GEMM): reported beside it in TFLOP/s.

Inputs are resident in HBM before timing starts.  Every projection's packed
weights and scales exist in L rotating copies (L * bytes >= 1 GiB, four times
the 256 MiB Infinity Cache) so each step streams its weights from HBM, as a
token does when each layer has its own weights.  Steps are captured into one
HIP graph (L steps, one per copy) and replayed; timing uses HIP events on the
capture stream, bracketed by synchronisation.

Roofline: each projection's call is timed live with HIP events over
back-to-back launches captured in a graph; the decode roofline counts all
four GEMV launches of the step (the only kernel it runs) against HBM at
8 TB/s, the prefill roofline the calls' binary16 MFMA work against 2516.6
TFLOP/s.  `traffic` (HBM bytes per launch) comes from the committed
rocprofv3 counter summary, and only while the HIP sources still match the
ones it was measured on.

The same run also times the decode step on binary16 scales (q4f16_1
weights, q4_linear_f16_scales), the four projections at a small batch (M = 4,
the kernel the automatic choice runs), the input gradient (M = 1, and at the
prefill size on MFMA) and the
re-quantization of the four projections' weights ("backward" and "requant" objects, GB/s of
algorithmic bytes against HBM).

cpu_baseline: the fp64 oracle (test infrastructure) timed on this host's cores
over a bounded sample of the same step.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2516.6
ROTATE_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--prefill-m", type=int, default=512)
    ap.add_argument("--lowbatch-m", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", choices=["decode", "prefill", "train", "both"], default="both")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also time a plain 256 MiB device-to-device copy (the reference "
                         "kernel for scaling HBM byte counters)")
    return ap.parse_args()


class Suite:
    """Device copies of one set of projections, and graph capture of steps."""

    def __init__(self, projs, torch, b, make_inputs, f16_scales=False):
        self.torch = torch
        self.b = b
        self.projs = projs
        dev = torch.device("cuda")
        sb = 2 if f16_scales else 4
        self.step_bytes = sum(p.alg_bytes(sb) for p in projs)
        self.step_flops = sum(p.flops() for p in projs)
        weight_bytes = sum(p.N * p.Kp + sb * p.G * p.N for p in projs)
        self.copies = max(2, -(-ROTATE_BYTES // weight_bytes))
        self.items = []
        for p in projs:
            x, qw, s, bias = make_inputs(p, 0)
            qd, sd = qw.to(dev), (s.half() if f16_scales else s).to(dev)
            qs = [qd] + [qd.clone() for _ in range(self.copies - 1)]
            ss = [sd] + [sd.clone() for _ in range(self.copies - 1)]
            out = torch.empty((p.M, p.N), dtype=torch.float32, device=dev)
            need = b.workspace_bytes(p.M, p.N, p.K, p.group_size)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need else None
            self.items.append(dict(p=p, x=x.to(dev), qs=qs, ss=ss, out=out, ws=ws,
                                   bias=None if bias is None else bias.to(dev)))
        torch.cuda.synchronize()

    def launch(self, i, c):
        it = self.items[i]
        p = it["p"]
        self.b.linear(it["x"], it["qs"][c], it["ss"][c], it["bias"], K=p.K,
                      group_size=p.group_size, nibble_order=p.order, out=it["out"],
                      workspace=it["ws"])

    def capture(self, body):
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            body()  # warm the code objects outside the capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        torch.cuda.synchronize()
        return g

    def step_graph(self, nsteps):
        """A graph of exactly nsteps steps; step s uses weight copy s % copies,
        so consecutive steps stream different copies from HBM."""
        def body():
            for st in range(nsteps):
                for i in range(len(self.items)):
                    self.launch(i, st % self.copies)
        return self.capture(body)

    def kernel_graph(self, i, reps):
        def body():
            for r in range(reps):
                self.launch(i, r % self.copies)
        return self.capture(body)


class TrainSuite:
    """The input gradient (M = 1) or the re-quantization of every projection
    of a step, each with rotating copies of its large operand (packed weights
    for the gradient, fp32 latents for re-quantization) so that each launch
    reads it from HBM."""

    def __init__(self, projs, torch, b, make_inputs, kind, M=1):
        self.torch = torch
        self.b = b
        self.kind = kind
        self.step_flops = sum(2 * M * p.N * p.K for p in projs)
        dev = torch.device("cuda")
        self.items = []
        per_step = 0
        for p in projs:
            if kind == "backward":
                per_step += p.N * p.Kp + 4 * p.G * p.N
            else:
                per_step += 4 * p.N * p.K
        self.copies = max(2, -(-ROTATE_BYTES // per_step))
        self.step_bytes = 0
        for p in projs:
            _, qw, s, _ = make_inputs(p, 0)
            g = torch.Generator().manual_seed(1)
            sd = s.to(dev)
            it = dict(p=p, s=sd)
            if kind == "backward":
                it["q"] = [qw.to(dev) for _ in range(self.copies)]
                it["dout"] = torch.randn((M, p.N), generator=g).to(dev)
                it["dx"] = torch.empty((M, p.K), device=dev)
                need = b.backward_workspace_bytes(M, p.N, p.K, p.group_size)
                it["ws"] = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
                self.step_bytes += p.N * p.Kp + 4 * p.G * p.N + 4 * M * p.N + 4 * M * p.K
            else:
                w = b.dequant(qw.to(dev), sd, p.K, p.group_size, p.order, torch.float32)
                it["lat"] = [w.clone() for _ in range(self.copies)]
                it["qout"] = torch.empty((p.N, p.Kp), dtype=torch.uint8, device=dev)
                self.step_bytes += 4 * p.N * p.K + 4 * p.G * p.N + p.N * p.Kp
            self.items.append(it)
        torch.cuda.synchronize()

    def launch(self, i, c):
        it = self.items[i]
        p = it["p"]
        if self.kind == "backward":
            self.b.linear_backward(it["dout"], it["q"][c], it["s"], K=p.K,
                                   group_size=p.group_size, nibble_order=p.order,
                                   dx=it["dx"], workspace=it["ws"])
        else:
            self.b.requant(it["lat"][c], it["s"], group_size=p.group_size,
                           nibble_order=p.order, qw=it["qout"])

    capture = Suite.capture
    step_graph = Suite.step_graph
    kernel_graph = Suite.kernel_graph


def train_measure(kind, projs, torch, b, make_inputs, steps, warmup, M=1):
    suite = TrainSuite(projs, torch, b, make_inputs, kind, M)
    m = measure(suite, steps, warmup, torch)
    times = launch_times(suite, torch)
    if M > 1:
        # the prefill-sized input gradient: binary16 operands on MFMA
        tf = suite.step_flops / (m["ms_per_step"] / 1e3) / 1e12
        ach = suite.step_flops / sum(times) / 1e12
        res = dict(
            value=round(tf, 2), unit="TFLOP/s", ms_per_step=round(m["ms_per_step"], 6),
            steps=m["steps"], flops_per_step=suite.step_flops,
            rotating_copies=suite.copies,
            roofline=dict(bound="mfma", achieved=round(ach, 2), peak=MFMA_F16_PEAK_TFLOPS,
                          unit="TFLOP/s", frac=round(ach / MFMA_F16_PEAK_TFLOPS, 4),
                          traffic=None,
                          kernel="dout16 + bwd_mfma (+ split-N reduce), per call",
                          avg_launch_us=round(sum(times) / len(times) * 1e6, 3)),
            per_projection_us=[(p.with_m(M).name, round(t * 1e6, 3))
                               for p, t in zip(projs, times)])
        del suite
        torch.cuda.empty_cache()
        return res
    gbs = suite.step_bytes / (m["ms_per_step"] / 1e3) / 1e9
    ach = suite.step_bytes / sum(times) / 1e9
    res = dict(
        value=round(gbs, 1), unit="GB/s", ms_per_step=round(m["ms_per_step"], 6),
        steps=m["steps"], alg_bytes_per_step=suite.step_bytes, rotating_copies=suite.copies,
        roofline=dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(ach / HBM_PEAK_GBS, 4), traffic=None,
                      kernel="bwd_f32 (+ row-block reduce)" if kind == "backward"
                      else "requant",
                      avg_launch_us=round(sum(times) / len(times) * 1e6, 3)),
        per_projection_us=[(p.name, round(t * 1e6, 3)) for p, t in zip(projs, times)])
    del suite
    torch.cuda.empty_cache()
    return res


def time_graph(torch, g, replays):
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3  # seconds


def measure(suite, steps, warmup, torch):
    """Exactly `warmup` untimed steps, then exactly `steps` timed steps, each
    as one graph replay bracketed by device synchronisation."""
    steps = max(1, steps)
    if warmup > 0:
        gw = suite.step_graph(warmup)
        time_graph(torch, gw, 1)
        del gw
    g = suite.step_graph(steps)
    secs = time_graph(torch, g, 1)
    return dict(steps=steps, warmup=warmup, seconds=secs, ms_per_step=secs / steps * 1e3)


def launch_times(suite, torch, reps=64):
    """Average duration of each projection's call, measured with HIP events
    over `reps` back-to-back launches captured in a graph (rotating weight
    copies, so every launch streams its weights from HBM)."""
    rows = []
    for i, it in enumerate(suite.items):
        g = suite.kernel_graph(i, reps)
        # untimed replays first: the first few milliseconds of a fresh graph
        # on a given set of buffers run measurably slower (up to 15% for the
        # MFMA kernels)
        time_graph(torch, g, 3)
        rows.append(time_graph(torch, g, 4) / (4 * reps))
    return rows


def source_digest():
    """sha256 over the HIP sources with comments and blank space removed: ties
    stored byte counts to the code they were measured on (edits to comments
    alone keep it)."""
    import glob
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "bit_weight_only_int4_amd", "csrc", "*"))):
        with open(f) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(os.path.basename(f).encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def stored_traffic(name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_decode_1b_prefill_1b_m512.md")
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    digest = None
    value = None
    for ln in text.splitlines():
        if ln.startswith("source_sha256:"):
            digest = ln.split(":", 1)[1].strip()
        elif ln.startswith(f"traffic_bytes_per_launch {name}:"):
            value = float(ln.split(":", 1)[1])
    if digest != source_digest():
        return None
    return value


def copy_calibration(torch, mib=1024, reps=8):
    """A plain elementwise copy of known size (dst = -src, fp32): reads and
    writes mib MiB per launch, more than the Infinity Cache holds, so its
    byte counters measure HBM traffic of a known amount."""
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.neg(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return dict(kernel="elementwise neg (fp32)", bytes_read=n * 4, bytes_written=n * 4,
                us=round(secs * 1e6, 2), gbs_read_plus_write=round(2 * n * 4 / secs / 1e9, 1))


def gpu_clocks():
    """Current shader and memory clock levels of cuda:0 (the levels the
    driver's sysfs files mark with '*'; context for the timings), or None.
    Read as plain files: no helper program is started."""
    try:
        import torch
        pr = torch.cuda.get_device_properties(0)
        dev = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (
            pr.pci_domain_id, pr.pci_bus_id, pr.pci_device_id)
        out = {}
        for key, name in (("sclk", "pp_dpm_sclk"), ("mclk", "pp_dpm_mclk")):
            with open(os.path.join(dev, name)) as f:
                cur = [ln.split(":", 1)[1].replace("*", "").strip()
                       for ln in f if ln.rstrip().endswith("*")]
            out[key] = cur[0] if cur else None
        return out
    except Exception:
        return None


def cpu_baseline(projs, budget_s, unit):
    """The oracle, as is, over a bounded sample of the step: a slice of the
    output columns of every projection (whole K, all M rows), repeated until
    about budget_s seconds of CPU work have run."""
    import numpy as np
    from bit_weight_only_int4_amd.workloads import make_inputs
    from oracle import q4_oracle as orc
    data = []
    for p in projs:
        x, qw, s, bias = make_inputs(p, 0)
        data.append((p, x.numpy(), qw.numpy(), s.numpy(),
                     None if bias is None else bias.numpy()))

    def run(f):
        secs = work_b = work_f = 0.0
        for p, x, qw, s, bias in data:
            ncols = max(1, int(round(p.N * f)))
            q_s = np.ascontiguousarray(qw[:ncols])
            s_s = np.ascontiguousarray(s[:ncols] if p.group_size == 0 else s[:, :ncols])
            b_s = None if bias is None else np.ascontiguousarray(bias[:ncols])
            t0 = time.perf_counter()
            orc.linear(x, q_s, s_s, b_s, K=p.K, group_size=p.group_size, order=p.order)
            secs += time.perf_counter() - t0
            share = ncols / p.N
            work_b += p.alg_bytes() * share
            work_f += p.flops() * share
        return secs, work_b, work_f

    # passes over growing column slices until about budget_s seconds of
    # oracle time have run; every pass counts toward the rate
    secs = wb = wf = 0.0
    frac = 1.0 / 256
    passes = 0
    cols = 0.0
    wall0 = time.perf_counter()
    while secs < budget_s and time.perf_counter() - wall0 < 3 * budget_s:
        a, b_, c = run(frac)
        secs += a
        wb += b_
        wf += c
        cols += frac
        passes += 1
        rate = frac / max(a, 1e-9)  # column share per second
        frac = min(1.0, max(frac, rate * (budget_s - secs)))
    value = wb / secs / 1e9 if unit == "GB/s" else wf / secs / 1e12
    return dict(value=round(value, 6), unit=unit, cores=orc.max_threads(), kind="oracle",
                sample=f"fp64 oracle over leading column slices of each of the {len(projs)} "
                       f"projections (whole K, all M rows): {passes} passes covering "
                       f"{cols:.2f} steps' worth of outputs, {secs:.1f} s of CPU time")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); this layer has no "
              "multi-GPU path to time.", file=sys.stderr)
        sys.exit(2)
    import torch
    from bit_weight_only_int4_amd import q4linear as b
    from bit_weight_only_int4_amd.workloads import CONFIGS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    b.lib()  # fail loudly if the HIP library is missing

    result = {}
    clocks_before = gpu_clocks()
    if args.copy_calibration:
        result["copy"] = copy_calibration(torch)
        print(f"[bench] copy: {result['copy']}", file=sys.stderr, flush=True)
    dec_projs = CONFIGS["decode_1b"]
    pre_projs = [p.with_m(args.prefill_m) for p in dec_projs]

    if args.only in ("decode", "both"):
        print(f"[bench] decode: {len(dec_projs)} projections", file=sys.stderr, flush=True)
        dec = Suite(dec_projs, torch, b, make_inputs)
        m = measure(dec, args.steps, args.warmup, torch)
        times = launch_times(dec, torch)
        # the step is four launches of the fp32 GEMV kernel; its roofline
        # counts every one of them
        t_sum = sum(times)
        ach = dec.step_bytes / t_sum / 1e9
        traffic = stored_traffic("gemv_f32")
        result["decode"] = dict(
            m=m, step_bytes=dec.step_bytes, copies=dec.copies,
            per_proj=[(dec_projs[i].name, round(t * 1e6, 3),
                       round(dec_projs[i].alg_bytes() / t / 1e9, 1)) for i, t in enumerate(times)],
            roofline=dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                          frac=round(ach / HBM_PEAK_GBS, 4),
                          traffic=None if traffic is None else round(traffic),
                          traffic_unit="HBM bytes per launch (mean over the step's four launches)",
                          kernel="gemv_f32 (all four projections)",
                          avg_launch_us=round(t_sum / len(times) * 1e6, 3),
                          alg_bytes_per_launch=round(dec.step_bytes / len(times))))
        print(f"[bench] decode done: {m['ms_per_step']:.4f} ms/step", file=sys.stderr,
              flush=True)
        del dec
        torch.cuda.empty_cache()

    if args.only in ("decode", "both"):
        # the same decode step on q4f16_1 weights (binary16 scales)
        print("[bench] decode, binary16 scales", file=sys.stderr, flush=True)
        d16 = Suite(dec_projs, torch, b, make_inputs, f16_scales=True)
        m = measure(d16, max(16, args.steps // 4), max(4, args.warmup // 4), torch)
        times = launch_times(d16, torch)
        ach = d16.step_bytes / sum(times) / 1e9
        result["decode_f16_scales"] = dict(
            value=round(d16.step_bytes / (m["ms_per_step"] / 1e3) / 1e9, 1), unit="GB/s",
            ms_per_step=round(m["ms_per_step"], 6), steps=m["steps"],
            alg_bytes_per_step=d16.step_bytes, rotating_weight_copies=d16.copies,
            config={"workload": "decode_1b projections, scales rounded to binary16 "
                                "(q4_linear_f16_scales)"},
            roofline=dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                          frac=round(ach / HBM_PEAK_GBS, 4), traffic=None,
                          kernel="gemv_f32, binary16 scales (all four projections)",
                          avg_launch_us=round(sum(times) / len(times) * 1e6, 3)),
            per_projection_us=[(dec_projs[i].name, round(t * 1e6, 3))
                               for i, t in enumerate(times)])
        print(f"[bench] binary16 scales done: {m['ms_per_step']:.4f} ms/step", file=sys.stderr,
              flush=True)
        del d16
        torch.cuda.empty_cache()

    if args.only in ("decode", "both") and args.lowbatch_m > 1:
        lb_projs = [p.with_m(args.lowbatch_m) for p in dec_projs]
        print(f"[bench] small batch M={args.lowbatch_m}", file=sys.stderr, flush=True)
        lb = Suite(lb_projs, torch, b, make_inputs)
        m = measure(lb, max(16, args.steps // 4), max(4, args.warmup // 4), torch)
        times = launch_times(lb, torch)
        paths = []
        for it in lb.items:
            p = it["p"]
            _, path = b.linear(it["x"], it["qs"][0], it["ss"][0], None, K=p.K,
                               group_size=p.group_size, nibble_order=p.order,
                               workspace=it["ws"], return_path=True)
            paths.append(path)
        ach = lb.step_bytes / sum(times) / 1e9
        result["lowbatch"] = dict(
            value=round(lb.step_bytes / (m["ms_per_step"] / 1e3) / 1e9, 1), unit="GB/s",
            ms_per_step=round(m["ms_per_step"], 6), steps=m["steps"],
            alg_bytes_per_step=lb.step_bytes, rotating_weight_copies=lb.copies,
            config={"workload": f"decode_1b projections at M={args.lowbatch_m} "
                                "(automatic kernel choice)"},
            roofline=dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                          frac=round(ach / HBM_PEAK_GBS, 4), traffic=None,
                          kernel="per projection: " + ", ".join(paths),
                          avg_launch_us=round(sum(times) / len(times) * 1e6, 3)),
            per_projection_us=[(lb_projs[i].name, round(t * 1e6, 3), paths[i])
                               for i, t in enumerate(times)])
        print(f"[bench] small batch done: {m['ms_per_step']:.4f} ms/step", file=sys.stderr,
              flush=True)
        del lb
        torch.cuda.empty_cache()

    if args.only in ("prefill", "both"):
        print(f"[bench] prefill M={args.prefill_m}", file=sys.stderr, flush=True)
        pre = Suite(pre_projs, torch, b, make_inputs)
        # at least two untimed passes over the rotating copies
        m = measure(pre, max(8, args.steps // 8), max(2 * pre.copies, args.warmup // 8), torch)
        times = launch_times(pre, torch, reps=16)
        # one layer call is the binary16 pre-pass plus the MFMA GEMM (plus the
        # split-K reduce where the plan splits K); timed together per call
        t_sum = sum(times)
        ach = pre.step_flops / t_sum / 1e12
        result["prefill"] = dict(
            m=m, step_flops=pre.step_flops, copies=pre.copies,
            per_proj=[(pre_projs[i].name, round(t * 1e6, 3),
                       round(pre_projs[i].flops() / t / 1e12, 2)) for i, t in enumerate(times)],
            roofline=dict(bound="mfma", achieved=round(ach, 2), peak=MFMA_F16_PEAK_TFLOPS,
                          unit="TFLOP/s", frac=round(ach / MFMA_F16_PEAK_TFLOPS, 4),
                          traffic=None, kernel="gemm_f16 call (pre-pass + GEMM)",
                          avg_launch_us=round(t_sum / len(times) * 1e6, 3)))
        result["clocks_after_prefill"] = gpu_clocks()
        print(f"[bench] prefill done: {m['ms_per_step']:.4f} ms/step", file=sys.stderr,
              flush=True)
        del pre
        torch.cuda.empty_cache()

    if args.only in ("train", "both"):
        for kind in ("backward", "requant"):
            print(f"[bench] {kind}", file=sys.stderr, flush=True)
            result[kind] = train_measure(kind, dec_projs, torch, b, make_inputs,
                                         max(16, args.steps // 4), max(4, args.warmup // 4))
            print(f"[bench] {kind} done: {result[kind]['ms_per_step']:.4f} ms/step",
                  file=sys.stderr, flush=True)
        print(f"[bench] backward at M={args.prefill_m}", file=sys.stderr, flush=True)
        result["backward_prefill"] = train_measure(
            "backward", dec_projs, torch, b, make_inputs, max(8, args.steps // 16),
            max(2, args.warmup // 8), M=args.prefill_m)
        print(f"[bench] backward at M={args.prefill_m} done: "
              f"{result['backward_prefill']['ms_per_step']:.4f} ms/step", file=sys.stderr,
              flush=True)

    cpu = None
    if not args.no_cpu_baseline and "decode" in result:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(dec_projs, args.cpu_seconds, "GB/s")

    line = {"metric": "q4 linear: prefill TFLOP/s (M=512) + decode GEMV HBM GB/s, "
                      "% of MI355X peak"}
    if "decode" in result:
        d = result["decode"]
        gbs = d["step_bytes"] / (d["m"]["ms_per_step"] / 1e3) / 1e9
        line.update({
            "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": d["m"]["steps"], "warmup": d["m"]["warmup"],
            "ms_per_step": round(d["m"]["ms_per_step"], 6), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "decode_1b: M=1, Llama-3.2-1B q/gate/up/down "
                                   "projections (2048x2048, 2048x8192 x2, 8192x2048), "
                                   "group_size 32, fp32 activations N(0,1), "
                                   "scales U[0.005,0.02], seed 0",
                       "rotating_weight_copies": d["copies"],
                       "alg_bytes_per_step": d["step_bytes"]},
            "roofline": d["roofline"],
            "per_projection_us_gbs": d["per_proj"],
        })
    if "prefill" in result:
        pf = result["prefill"]
        tf = pf["step_flops"] / (pf["m"]["ms_per_step"] / 1e3) / 1e12
        line["prefill"] = {
            "value": round(tf, 2), "unit": "TFLOP/s", "dtype": "f16 operands, f32 accumulate",
            "ms_per_step": round(pf["m"]["ms_per_step"], 6), "steps": pf["m"]["steps"],
            "frac_of_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
            "config": {"workload": f"prefill_1b: M={args.prefill_m}, same four projections",
                       "rotating_weight_copies": pf["copies"]},
            "roofline": pf["roofline"],
            "per_projection_us_tflops": pf["per_proj"],
        }
    if "decode_f16_scales" in result:
        line["decode_f16_scales"] = result["decode_f16_scales"]
    if "lowbatch" in result:
        line["lowbatch"] = result["lowbatch"]
    for kind, what in (("backward", "input gradient dx = dout . dequant(W), M=1"),
                       ("backward_prefill", "input gradient at M=%d (automatic choice: "
                        "binary16 operands on MFMA)" % args.prefill_m),
                       ("requant", "re-quantization of fp32 latents into packed codes")):
        if kind in result:
            r = result[kind]
            line[kind] = dict(r, config={"workload": f"decode_1b projections: {what}"})
    line["cpu_baseline"] = cpu
    line["gpu_clocks"] = {"before": clocks_before,
                          "after_prefill": result.get("clocks_after_prefill")}
    if "copy" in result:
        line["copy_calibration"] = result["copy"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
