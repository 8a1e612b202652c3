"""Benchmark of the weight-only 4-bit linear layer on one MI355X.

A step is one pass of the layer over the projections of one workload, each
launched once, on seeded synthetic inputs resident in HBM:

  * decode_1b (the headline value): M = 1, the four Llama-3.2-1B projections
    (2048->2048, 2048->8192 x2, 8192->2048), group size 32, in GB/s of
    algorithmic bytes (packed weights + scales + activations + outputs);
  * every other measured configuration of the workloads, each in its own
    object of the JSON line: prefill_1b at M = 64 / 512 / 2048, the
    Llama-3.1-8B projections (group size 128) at M = 1 and 512, the
    2048 x 128257 per-channel output head at M = 1 / 7 / 333 and the
    2008 x 3000 per-channel projection at M = 65.

Every projection's packed weights and scales exist in L rotating copies
(L * bytes >= 1 GiB, four times the 256 MiB Infinity Cache), so each step
streams its weights from HBM, as a token does when every layer has its own
weights.  Steps are captured into HIP graphs and replayed; timing uses HIP
events on the capture stream, bracketed by synchronisation.

Roofline (per configuration): `achieved` is the configuration's algorithmic
bytes (HBM-bound configurations: M <= 65) or FLOPs (M >= 333, against the
dense binary16 MFMA peak) per step divided by the step time measured over
the timed region, so it is the configuration's own value; `per_projection`
lists each call's own average (HIP events over back-to-back launches) and
the kernel that ran.  `traffic` (HBM bytes per step) comes from the
committed rocprofv3 counter summary, and only while the HIP sources still
hash to the digest it was measured on.

The same run also times the input gradient (M = 1 and 512), the
re-quantization and the decode step on binary16 scales ("train" objects).

cpu_baseline: the fp64 oracle (test infrastructure) timed on this host's
cores over a bounded sample of the decode step; every configuration object
carries the oracle's rate on a bounded sample of its own projections.

`python bench.py --summarize DIR OUT.md --title T --command C` turns the
CSV files of a rocprofv3 run (kernel trace, or FETCH_SIZE / WRITE_SIZE /
SQ counters) into the text summaries kept under profiles/.
"""
import argparse
import glob
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2516.6
ROTATE_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_all_workloads.md")
METRIC = "q4 linear: prefill TFLOP/s (M=512) + decode GEMV HBM GB/s, % of MI355X peak"

# (object name, projections from the workloads): the configurations measured;
# the last is the small-batch regime (M = 4 on the decode projections)
RUNS = [
    ("decode_1b", lambda C: C["decode_1b"]),
    ("prefill_1b_m64", lambda C: [p for p in C["prefill_1b"] if p.M == 64]),
    ("prefill_1b_m512", lambda C: [p for p in C["prefill_1b"] if p.M == 512]),
    ("prefill_1b_m2048", lambda C: [p for p in C["prefill_1b"] if p.M == 2048]),
    ("llama8b_m1", lambda C: [p for p in C["llama8b_gs128"] if p.M == 1]),
    ("llama8b_m512", lambda C: [p for p in C["llama8b_gs128"] if p.M == 512]),
    ("lm_head_m1", lambda C: [p for p in C["per_channel_edges"]
                              if p.name.startswith("lm_head") and p.M == 1]),
    ("lm_head_m7", lambda C: [p for p in C["per_channel_edges"]
                              if p.name.startswith("lm_head") and p.M == 7]),
    ("lm_head_m333", lambda C: [p for p in C["per_channel_edges"]
                                if p.name.startswith("lm_head") and p.M == 333]),
    ("odd_k_m65", lambda C: [p for p in C["per_channel_edges"] if p.name.startswith("odd_k")]),
    ("decode_1b_m4", lambda C: [p.with_m(4) for p in C["decode_1b"]]),
]
TIMED_BUDGET_S = 0.05  # timed steps per non-headline configuration: about 50 ms


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--configs", default="all",
                    help="comma-separated configuration names (default: all)")
    ap.add_argument("--no-train", action="store_true", help="skip the training-side objects")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also time a plain 1 GiB device-to-device copy (the reference "
                         "kernel for scaling HBM byte counters)")
    ap.add_argument("--max-steps", type=int, default=512,
                    help="cap on the timed steps of the configurations after the first")
    ap.add_argument("--reps", type=int, default=0,
                    help="launches per call-timing graph (0: 64, or 16 for large calls)")
    ap.add_argument("--traffic", metavar="ORDER_JSON",
                    help="instead of timing, make one call per projection of each "
                         "configuration, 30 ms apart (for counter runs), and write their "
                         "order to ORDER_JSON")
    ap.add_argument("--summarize", nargs=2, metavar=("DIR", "OUT"),
                    help="summarize the rocprofv3 CSV files in DIR into OUT (markdown)")
    ap.add_argument("--calls-per", type=int, default=1,
                    help="with --traffic: calls per projection, back to back on cycling "
                         "weight copies")
    ap.add_argument("--summarize-calls", nargs=3, metavar=("ORDER_JSON", "DIR", "OUT"),
                    help="per-call median kernel durations from the kernel trace of a "
                         "--traffic run with several calls per projection")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("ORDER_JSON", "DIRS", "OUT"),
                    help="per-projection and per-configuration sums of the counters of "
                         "--traffic runs (DIRS: comma-separated rocprofv3 output folders)")
    ap.add_argument("--bench-json", help="with --summarize-calls: a bench JSON line whose step "
                                          "times the kernel times are set beside")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", default="")
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

    def launch(self, i, c, return_path=False):
        it = self.items[i]
        p = it["p"]
        return self.b.linear(it["x"], it["qs"][c], it["ss"][c], it["bias"], K=p.K,
                             group_size=p.group_size, nibble_order=p.order, out=it["out"],
                             workspace=it["ws"], return_path=return_path)

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
    """The input gradient or the re-quantization of every projection of a
    step, each with rotating copies of its large operand (packed weights for
    the gradient, fp32 latents for re-quantization) so that each launch reads
    it from HBM."""

    def __init__(self, projs, torch, b, make_inputs, kind, M=1):
        self.torch = torch
        self.b = b
        self.kind = kind
        self.step_flops = sum(2 * M * p.N * p.K for p in projs)
        dev = torch.device("cuda")
        self.items = []
        per_step = 0
        for p in projs:
            per_step += (p.N * p.Kp + 4 * p.G * p.N) if kind == "backward" else 4 * p.N * p.K
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
    for i in range(len(suite.items)):
        g = suite.kernel_graph(i, reps)
        # untimed replays first: the first few milliseconds of a fresh graph
        # on a given set of buffers run measurably slower
        time_graph(torch, g, 3)
        rows.append(time_graph(torch, g, 4) / (4 * reps))
        del g
    return rows


def source_digest():
    """The digest the build stamps beside the library: HIP sources and the C
    header, comments and blank space removed."""
    from bit_weight_only_int4_amd import build as hip_build
    return hip_build.source_digest()


def stored_traffic():
    """{configuration: HBM bytes per step} from the committed rocprofv3
    counter summary, or {} if the kernels changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return {}
    digest, values = None, {}
    for ln in text.splitlines():
        if ln.startswith("source_sha256:"):
            digest = ln.split(":", 1)[1].strip()
        elif ln.startswith("traffic_bytes_per_step "):
            name, val = ln[len("traffic_bytes_per_step "):].split(":", 1)
            values[name.strip()] = float(val)
    return values if digest == source_digest() else {}


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


def oracle_rate(projs, budget_s):
    """The oracle, as is, over a bounded sample of the projections: leading
    column slices of every projection (whole K, all M rows), grown until about
    budget_s seconds of CPU work have run.  Returns (GB/s, TFLOP/s, passes,
    steps' worth of outputs, seconds) on the algorithmic denominators."""
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

    secs = wb = wf = cols = 0.0
    frac, passes = 1.0 / 4096, 0
    wall0 = time.perf_counter()
    while secs < budget_s and time.perf_counter() - wall0 < 3 * budget_s:
        a, b_, c = run(frac)
        secs += a
        wb += b_
        wf += c
        cols += frac
        passes += 1
        rate = frac / max(a, 1e-9)
        frac = min(1.0, max(frac, rate * (budget_s - secs)))
    return wb / secs / 1e9, wf / secs / 1e12, passes, cols, secs


def cpu_baseline(projs, budget_s):
    from oracle import q4_oracle as orc
    gbs, _, passes, cols, secs = oracle_rate(projs, budget_s)
    return dict(value=round(gbs, 6), unit="GB/s", cores=orc.max_threads(), kind="oracle",
                sample=f"fp64 oracle over leading column slices of each of the {len(projs)} "
                       f"decode_1b projections (whole K, M = 1): {passes} passes covering "
                       f"{cols:.2f} steps' worth of outputs, {secs:.1f} s of CPU time")


def bound_of(projs):
    """HBM for every projection with M <= 65, dense binary16 MFMA from M = 333
    on (the workloads have no M in between)."""
    return "hbm" if max(p.M for p in projs) <= 65 else "mfma"


def bench_config(name, projs, torch, b, make_inputs, steps, warmup, traffic, cpu_s,
                 max_steps=512, reps=0):
    suite = Suite(projs, torch, b, make_inputs)
    if steps is None:
        # about TIMED_BUDGET_S of timed steps, after two untimed passes over
        # the rotating copies
        probe = measure(suite, 2, 2, torch)
        steps = max(4, min(max_steps, int(TIMED_BUDGET_S / (probe["ms_per_step"] / 1e3))))
        warmup = max(4, 2 * suite.copies if suite.copies * probe["ms_per_step"] < 50 else 8)
        warmup = min(warmup, 2 * max_steps)
    m = measure(suite, steps, warmup, torch)
    times = launch_times(suite, torch, reps=reps or (64 if suite.step_flops < 5e10 else 16))
    paths = [suite.launch(i, 0, return_path=True)[1] for i in range(len(projs))]
    torch.cuda.synchronize()
    step_s = m["ms_per_step"] / 1e3
    gbs = suite.step_bytes / step_s / 1e9
    tfs = suite.step_flops / step_s / 1e12
    bound = bound_of(projs)
    ach, peak, unit = (gbs, HBM_PEAK_GBS, "GB/s") if bound == "hbm" else \
        (tfs, MFMA_F16_PEAK_TFLOPS, "TFLOP/s")
    ai = suite.step_flops / suite.step_bytes
    attainable = min(MFMA_F16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
    tr = traffic.get(name)
    obj = dict(
        value=round(ach, 2), unit=unit, ms_per_step=round(m["ms_per_step"], 6),
        steps=m["steps"], warmup=m["warmup"], rotating_weight_copies=suite.copies,
        alg_bytes_per_step=suite.step_bytes, flops_per_step=suite.step_flops,
        gbs=round(gbs, 1), tflops=round(tfs, 2),
        roofline=dict(bound=bound, achieved=round(ach, 2), peak=peak, unit=unit,
                      frac=round(ach / peak, 4), traffic=None if tr is None else round(tr),
                      traffic_unit="HBM bytes per step (FETCH_SIZE + WRITE_SIZE, scaled)",
                      frac_of_attainable=round(tfs / attainable, 4),
                      attainable_tflops=round(attainable, 1)),
        per_projection=[dict(name=p.name, us=round(t * 1e6, 3),
                             gbs=round(p.alg_bytes() / t / 1e9, 1),
                             tflops=round(p.flops() / t / 1e12, 2), kernel=path)
                        for p, t, path in zip(projs, times, paths)],
        config={"workload": name, "projections": [p.name for p in projs]})
    del suite
    torch.cuda.empty_cache()
    if cpu_s > 0:
        from oracle import q4_oracle as orc
        ogbs, otf, passes, cols, secs = oracle_rate(projs, cpu_s)
        orate = ogbs if unit == "GB/s" else otf
        obj["cpu_oracle"] = dict(value=round(orate, 6), unit=unit, cores=orc.max_threads(),
                                 seconds=round(secs, 2), steps_of_outputs=round(cols, 4),
                                 gpu_over_oracle=round(ach / orate, 1))
    return obj


def train_measure(kind, projs, torch, b, make_inputs, steps, warmup, M=1):
    suite = TrainSuite(projs, torch, b, make_inputs, kind, M)
    m = measure(suite, steps, warmup, torch)
    times = launch_times(suite, torch)
    step_s = m["ms_per_step"] / 1e3
    if M > 1:
        tf = suite.step_flops / step_s / 1e12
        res = dict(value=round(tf, 2), unit="TFLOP/s", ms_per_step=round(m["ms_per_step"], 6),
                   steps=m["steps"], flops_per_step=suite.step_flops,
                   rotating_copies=suite.copies,
                   roofline=dict(bound="mfma", achieved=round(tf, 2), peak=MFMA_F16_PEAK_TFLOPS,
                                 unit="TFLOP/s", frac=round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                                 traffic=None),
                   per_projection_us=[(p.with_m(M).name, round(t * 1e6, 3))
                                      for p, t in zip(projs, times)])
    else:
        gbs = suite.step_bytes / step_s / 1e9
        res = dict(value=round(gbs, 1), unit="GB/s", ms_per_step=round(m["ms_per_step"], 6),
                   steps=m["steps"], alg_bytes_per_step=suite.step_bytes,
                   rotating_copies=suite.copies,
                   roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS,
                                 unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None),
                   per_projection_us=[(p.name, round(t * 1e6, 3)) for p, t in zip(projs, times)])
    del suite
    torch.cuda.empty_cache()
    return res


# ---- rocprofv3 summaries ----------------------------------------------------

def _short(name):
    return name.replace("q4::(anonymous namespace)::", "").replace("q4::", "") \
               .replace("void ", "").split("(")[0]


def summarize(d, out, title, command):
    """Median / mean / min / max duration per (kernel, grid) from a kernel
    trace, or per-dispatch means of every counter from a counter run."""
    import csv
    lines = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "",
             "```", command, "```", ""]
    traces = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    counters = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if traces:
        rows = {}
        for f in traces:
            for r in csv.DictReader(open(f)):
                key = (_short(r["Kernel_Name"]),
                       "%sx%sx%s" % (r["Grid_Size_X"], r["Grid_Size_Y"], r["Grid_Size_Z"]),
                       r["Workgroup_Size_X"])
                us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                rows.setdefault(key, []).append(us)
        lines += ["Durations per kernel and launch shape (grid in work-items x, y, z; "
                  "workgroup size x), in microseconds:", "",
                  "| kernel | grid | wg | calls | median | mean | min | max |",
                  "|---|---|---|---|---|---|---|---|"]
        for key, v in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
            if key[0].startswith("__amd") or len(v) < 4:
                continue
            lines.append(f"| `{key[0]}` | {key[1]} | {key[2]} | {len(v)} | "
                         f"{statistics.median(v):.3f} | {statistics.mean(v):.3f} | "
                         f"{min(v):.3f} | {max(v):.3f} |")
    if counters:
        vals = {}
        for f in counters:
            for r in csv.DictReader(open(f)):
                key = (_short(r["Kernel_Name"]), r["Grid_Size"], r["Counter_Name"])
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
        names = sorted({k[2] for k in vals})
        lines += ["Per-dispatch means of each counter, per kernel and grid size "
                  "(work-items):", "",
                  "| kernel | grid | dispatches | " + " | ".join(names) + " |",
                  "|---|---|---|" + "---|" * len(names)]
        keys = sorted({(k[0], k[1]) for k in vals})
        for k0, k1 in keys:
            cells = []
            n = 0
            for c in names:
                v = vals.get((k0, k1, c))
                n = max(n, len(v) if v else 0)
                cells.append(f"{statistics.mean(v):.6g}" if v else "")
            if k0.startswith("__amd") and "neg" not in k0:
                continue
            lines.append(f"| `{k0}` | {k1} | {n} | " + " | ".join(cells) + " |")
    lines.append("")
    with open(out, "w") as fo:
        fo.write("\n".join(lines))
    print(f"wrote {out}")


LIB_KERNELS = ("gemv_", "gemm_", "x16_kernel", "splitk_reduce_kernel", "bwd_", "dout16_kernel",
               "requant_kernel", "dequant_kernel", "unpack_codes_kernel")


def traffic_run(torch, b, CONFIGS, make_inputs, wanted, order_path, calls_per=1):
    """calls_per calls per projection, back to back, each on a weight copy
    that later copies have pushed out of the caches (copies 1, 2, ...), the
    projections 30 ms apart, so a profiled run's dispatches of the library
    fall into groups that map to the projections in order.  The 30 ms are a
    spin kernel on the GPU, not a host sleep: an idle GPU drops its clocks,
    and the first calls after an idle gap would run slower than the bench's
    back-to-back steps."""
    order = []
    print("[bench] copy calibration", file=sys.stderr, flush=True)
    order.append(dict(config="copy", projection="copy", calibration=copy_calibration(torch)))
    for name, pick in RUNS:
        if wanted is not None and name not in wanted:
            continue
        projs = pick(CONFIGS)
        suite = Suite(projs, torch, b, make_inputs)
        for i, p in enumerate(projs):
            gap(torch)
            for r in range(calls_per):
                _, path = suite.launch(i, 1 + r % (suite.copies - 1), return_path=True)
            torch.cuda.synchronize()
            order.append(dict(config=name, projection=p.name, kernel=path, calls=calls_per,
                              alg_bytes=p.alg_bytes(), flops=p.flops()))
        print(f"[bench] {name}: one call per projection", file=sys.stderr, flush=True)
        del suite
        torch.cuda.empty_cache()
    gap(torch)
    with open(order_path, "w") as f:
        json.dump(order, f)


def gap(torch, seconds=0.03):
    """About `seconds` of GPU time in a spin kernel (torch.cuda._sleep counts
    shader clock cycles, at most 2.4 GHz), then a synchronisation."""
    torch.cuda._sleep(int(seconds * 2.4e9))
    torch.cuda.synchronize()


def _library_groups(events, ncalls, where):
    """The library's dispatches (by kernel name) in start order, split where
    the GPU idled for more than 10 ms: one group per projection."""
    lib = [e for e in sorted(events, key=lambda e: e["t0"])
           if any(t in _short(e["name"]) for t in LIB_KERNELS)]
    groups, last = [], None
    for e in lib:
        if last is None or e["t0"] - last > 10_000_000:
            groups.append([])
        groups[-1].append(e)
        last = e["t1"]
    if len(groups) != ncalls:
        raise SystemExit(f"{where}: {len(groups)} groups of library dispatches for "
                         f"{ncalls} projections")
    return groups


def summarize_calls(order_path, d, out, title, command, bench_path=None):
    """Per projection: the median duration of each of its call's kernels over
    the calls of a --traffic run (the group's dispatches, position by
    position), their sum, and per configuration the kernel time of one step,
    beside the step time of a bench line when one is given."""
    import csv
    order = [o for o in json.load(open(order_path)) if o["config"] != "copy"]
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    ev = [dict(t0=int(r["Start_Timestamp"]), t1=int(r["End_Timestamp"]), name=r["Kernel_Name"])
          for f in files for r in csv.DictReader(open(f))]
    groups = _library_groups(ev, len(order), d)
    bench = {}
    if bench_path:
        line = json.loads(open(bench_path).read().strip().splitlines()[-1])
        bench = dict(line.get("configs", {}))
        if "ms_per_step" in line:
            bench["decode_1b"] = dict(ms_per_step=line["ms_per_step"], roofline=line["roofline"])
    lines = [f"# {title}", "", "Commands (from the repository root, on one MI355X):", "",
             "```", command, "```", "",
             "Per projection: each kernel of its call, the median of its duration over the "
             "calls (microseconds), and their sum:", "",
             "| configuration | projection | calls | kernels (median us) | call (us) |",
             "|---|---|---|---|---|"]
    per_cfg = {}
    for o, g in zip(order, groups):
        k = len(g) // o["calls"]
        if k * o["calls"] != len(g):
            raise SystemExit(f"{o['projection']}: {len(g)} dispatches for {o['calls']} calls")
        meds = [(_short(g[j]["name"]),
                 statistics.median((g[j + c * k]["t1"] - g[j + c * k]["t0"]) / 1e3
                                   for c in range(o["calls"]))) for j in range(k)]
        tot = sum(t for _, t in meds)
        c = per_cfg.setdefault(o["config"], [0.0, 0, 0])
        c[0] += tot
        c[1] += o["alg_bytes"]
        c[2] += o["flops"]
        kern = " + ".join(f"`{n}` {t:.2f}" for n, t in meds)
        lines.append(f"| {o['config']} | {o['projection']} | {o['calls']} | {kern} | {tot:.2f} |")
    lines += ["", "Per configuration (one step = one call of each projection); the roofline "
                  "fraction of the kernel times alone, and of the bench line's step time "
                  "(launch gaps included):", "",
              "| configuration | kernel time per step (us) | bench step time (us) | bound | "
              "fraction of peak, kernel times | fraction of peak, bench step |",
              "|---|---|---|---|---|---|"]
    for cfg, (tot, nbytes, flops) in per_cfg.items():
        bl = bench.get(cfg)
        mfma = (bl["roofline"]["bound"] == "mfma") if bl else flops / max(nbytes, 1) > 300
        frac_k = (flops / (tot * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS) if mfma else \
            (nbytes / (tot * 1e-6) / 1e9 / HBM_PEAK_GBS)
        step = f"{bl['ms_per_step'] * 1e3:.2f}" if bl else ""
        frac_s = f"{bl['roofline']['frac']:.4f}" if bl else ""
        lines.append(f"| {cfg} | {tot:.2f} | {step} | {'mfma' if mfma else 'hbm'} | "
                     f"{frac_k:.4f} | {frac_s} |")
    lines.append("")
    with open(out, "w") as fo:
        fo.write("\n".join(lines))
    print(f"wrote {out}")


def summarize_counters(order_path, dirs, out, title, command):
    """Sums of each counter over the library dispatches of every projection's
    call (groups split at idle gaps of more than 10 ms), per configuration
    per step; HBM bytes from FETCH_SIZE / WRITE_SIZE scaled by what the same
    counters read for the 1 GiB copy; MFMA busy share of the GEMM kernels."""
    import csv
    order = json.load(open(order_path))
    per = {}  # (group index, counter) -> sum;  (group, kernel, counter) -> sum
    kern = {}
    calls_k = {}  # group index -> [(kernel, grid work-items)] of the call
    for d in dirs.split(","):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        disp = {}
        for f in files:
            for r in csv.DictReader(open(f)):
                k = (int(r["Dispatch_Id"]), r["Kernel_Name"])
                disp.setdefault(k, dict(t0=int(r["Start_Timestamp"]), t1=int(r["End_Timestamp"]),
                                        name=r["Kernel_Name"], grid=int(r["Grid_Size"]), c={}))
                disp[k]["c"][r["Counter_Name"]] = float(r["Counter_Value"])
        ev = sorted(disp.values(), key=lambda e: e["t0"])
        cal = [e for e in ev if "neg" in e["name"] or "elementwise" in e["name"]]
        calls = [o for o in order if o["config"] != "copy"]
        groups = _library_groups(ev, len(calls), d)
        for gi, g in enumerate(groups):
            calls_k.setdefault(gi, [(_short(e["name"]), e["grid"]) for e in g])
            for e in g:
                for c, v in e["c"].items():
                    per[(gi, c)] = per.get((gi, c), 0.0) + v
                    kk = (gi, _short(e["name"]), c)
                    kern[kk] = kern.get(kk, 0.0) + v
        if cal:
            e = cal[-1]  # the timed copies: the last of the calibration dispatches
            for c, v in e["c"].items():
                per[("copy", c)] = v
    calls = [o for o in order if o["config"] != "copy"]
    copy = next(o for o in order if o["config"] == "copy")["calibration"]
    scale = {}
    for c, nbytes in (("FETCH_SIZE", copy["bytes_read"]), ("WRITE_SIZE", copy["bytes_written"])):
        v = per.get(("copy", c))
        if v:
            scale[c] = nbytes / (v * 1024)
    lines = [f"# {title}", "", "Commands (from the repository root, on one MI355X):", "",
             "```", command, "```", "",
             f"source_sha256: {source_digest()}", ""]
    if scale:
        lines += ["Scale factors from the 1 GiB elementwise copy (bytes moved / (counter KiB "
                  "x 1024)): " + ", ".join(f"{c} {v:.4f}" for c, v in scale.items()), ""]
    counters = sorted({c for (g, c) in per if g != "copy"})
    lines += ["Per call (sums over the call's library dispatches; counters as read):", "",
              "| configuration | projection | kernel | alg. bytes | " + " | ".join(counters) +
              (" | HBM bytes | HBM / alg." if scale else "") + " |",
              "|---|---|---|---|" + "---|" * len(counters) + ("---|---|" if scale else "")]
    cfg_bytes = {}
    for gi, o in enumerate(calls):
        vals = [per.get((gi, c), 0.0) for c in counters]
        row = f"| {o['config']} | {o['projection']} | {o['kernel']} | {o['alg_bytes']} | " + \
              " | ".join(f"{v:.6g}" for v in vals)
        if scale:
            hbm = sum(per.get((gi, c), 0.0) * 1024 * scale[c] for c in scale)
            cfg_bytes[o["config"]] = cfg_bytes.get(o["config"], 0.0) + hbm
            row += f" | {hbm:.0f} | {hbm / o['alg_bytes']:.3f}"
        lines.append(row + " |")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in counters and "GRBM_GUI_ACTIVE" in counters:
        lines += ["", "MFMA busy share of the GEMM kernels, per call: SQ_VALU_MFMA_BUSY_CYCLES "
                  "(summed over the SIMDs) / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs); the GPU-busy "
                  "cycle count as read is the sum over the 8 XCDs:", "",
                  "| configuration | projection | kernel | MFMA busy |", "|---|---|---|---|"]
        for gi, o in enumerate(calls):
            for (g, kname, c), v in sorted(kern.items()):
                if g != gi or c != "SQ_VALU_MFMA_BUSY_CYCLES" or "gemm" not in kname:
                    continue
                act = kern.get((gi, kname, "GRBM_GUI_ACTIVE"), 0.0)
                if act > 0:
                    lines.append(f"| {o['config']} | {o['projection']} | `{kname}` | "
                                 f"{v / (act / 8 * 1024):.3f} |")
    if cfg_bytes:
        lines += ["", "HBM bytes per step of each configuration (read by bench.py while the "
                  "sources hash to source_sha256):", ""]
        for k, v in cfg_bytes.items():
            lines.append(f"traffic_bytes_per_step {k}: {v:.0f}")
    lines.append("")
    with open(out, "w") as fo:
        fo.write("\n".join(lines))
    with open(out + ".calls.json", "w") as fo:
        json.dump([dict(o, kernels=calls_k.get(gi, [])) for gi, o in enumerate(calls)], fo)
    print(f"wrote {out} and {out}.calls.json")


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize[0], args.summarize[1], args.title, args.command)
        return
    if args.summarize_calls:
        summarize_calls(*args.summarize_calls, args.title, args.command, args.bench_json)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.title, args.command)
        return
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
    b.lib()  # fail loudly if the HIP library is missing or stale

    wanted = None if args.configs == "all" else set(args.configs.split(","))
    if args.traffic:
        traffic_run(torch, b, CONFIGS, make_inputs, wanted, args.traffic, args.calls_per)
        return
    traffic = stored_traffic()
    clocks_before = gpu_clocks()
    result = {}
    copy = copy_calibration(torch) if args.copy_calibration else None
    cpu_s = 0.0 if args.no_cpu_baseline else 1.5
    for name, pick in RUNS:
        if wanted is not None and name not in wanted:
            continue
        projs = pick(CONFIGS)
        head = name == "decode_1b"
        print(f"[bench] {name}: {len(projs)} projection(s)", file=sys.stderr, flush=True)
        result[name] = bench_config(name, projs, torch, b, make_inputs,
                                    args.steps if head else None,
                                    args.warmup if head else None, traffic,
                                    0.0 if head else cpu_s, args.max_steps, args.reps)
        print(f"[bench] {name} done: {result[name]['ms_per_step']:.4f} ms/step, "
              f"{result[name]['value']} {result[name]['unit']}", file=sys.stderr, flush=True)
    clocks_after = gpu_clocks()

    train = {}
    if not args.no_train and (wanted is None or "train" in wanted):
        dec = CONFIGS["decode_1b"]
        for kind, M, what in (("backward", 1, "input gradient dx = dout . dequant(W), M=1"),
                              ("backward", 512, "input gradient at M=512 (automatic choice: "
                                                "binary16 operands on MFMA)"),
                              ("requant", 1, "re-quantization of fp32 latents into packed "
                                             "codes")):
            key = kind if M == 1 else f"{kind}_m{M}"
            print(f"[bench] {key}", file=sys.stderr, flush=True)
            train[key] = train_measure(kind, dec, torch, b, make_inputs,
                                       32 if M == 1 else 8, 4 if M == 1 else 2, M)
            train[key]["config"] = {"workload": f"decode_1b projections: {what}"}
            print(f"[bench] {key} done: {train[key]['ms_per_step']:.4f} ms/step",
                  file=sys.stderr, flush=True)
        print("[bench] decode, binary16 scales", file=sys.stderr, flush=True)
        d16 = Suite(dec, torch, b, make_inputs, f16_scales=True)
        m = measure(d16, 64, 8, torch)
        gbs = d16.step_bytes / (m["ms_per_step"] / 1e3) / 1e9
        train["decode_f16_scales"] = dict(
            value=round(gbs, 1), unit="GB/s", ms_per_step=round(m["ms_per_step"], 6),
            steps=m["steps"], alg_bytes_per_step=d16.step_bytes,
            roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                          frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None),
            config={"workload": "decode_1b projections, scales rounded to binary16 "
                                "(q4_linear_f16_scales)"})
        del d16
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline and "decode_1b" in result:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(CONFIGS["decode_1b"], args.cpu_seconds)

    line = {"metric": METRIC}
    if "decode_1b" in result:
        d = result["decode_1b"]
        line.update({
            "value": d["value"], "unit": "GB/s", "n_gpus": 1, "steps": d["steps"],
            "warmup": d["warmup"], "ms_per_step": d["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "decode_1b: M=1, Llama-3.2-1B q/gate/up/down "
                                   "projections (2048x2048, 2048x8192 x2, 8192x2048), "
                                   "group_size 32, fp32 activations N(0,1), "
                                   "scales U[0.005,0.02], seed 0",
                       "rotating_weight_copies": d["rotating_weight_copies"],
                       "alg_bytes_per_step": d["alg_bytes_per_step"]},
            "roofline": d["roofline"],
            "per_projection": d["per_projection"],
        })
    line["configs"] = {k: v for k, v in result.items() if k != "decode_1b"}
    if "prefill_1b_m512" in result:
        # the metric's prefill figure (the same object as configs.prefill_1b_m512)
        line["prefill"] = result["prefill_1b_m512"]
    if train:
        line["train"] = train
    line["cpu_baseline"] = cpu
    line["gpu_clocks"] = {"before": clocks_before, "after": clocks_after}
    if copy:
        line["copy_calibration"] = copy
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
