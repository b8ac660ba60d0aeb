"""Benchmark of the MoE layer token path (forward + backward) on one MI355X.

A step is one forward and backward pass of the whole layer over one batch:
route -> dispatch -> grouped SwiGLU FFN (+ shared expert) -> combine, then
combine backward -> grouped FFN backward -> dispatch backward -> route
backward. Inputs and weights are seeded synthetic tensors already resident in
HBM when the timed region starts. Before every timed step a 1 GiB scratch
buffer is written and another 1 GiB read, outside the timed events, so that
no step finds its working set in the 256 MB memory-side cache (MALL) or the
L2s. Prints one JSON line.

By default every workload runs: the headline is the largest one that fits one
GPU, the DeepSeek-V3-style FP8 layer (T=8192, d=7168, 256 routed experts +
1 shared, top-8, d_ff=2048, E4M3 with 1x128 / 128x128 fp32 block scales); the
tiny fp32, Mixtral-style, DeepSeek-V3-style bf16 and Qwen3-style skewed
layers follow in the same line under "configs". --config names one workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
CSRC = os.path.join(ROOT, "mixture_experts_layer_gather_amd", "csrc")
# The headline workload: the largest of the five that one GPU holds. The
# others are reported in the same line for context.
HEADLINE = "deepseek_v3_fp8"
CONTEXT_CONFIGS = ("tiny_fp32", "mixtral_bf16", "deepseek_v3_bf16", "qwen3_skew_bf16",
                   "deepseek_v3_mxfp8")
# tokens of the headline workload the CPU oracle runs (a bounded sample)
CPU_SAMPLE_TOKENS = 8
PROFILES = os.path.join(ROOT, "profiles")

# Which library call launches a kernel, from its (demangled) name: the GEMM
# template flags <T, TC, A K-major, B K-major, mode, epilogue, ...> give its
# role. mode 0 = row-grouped, 1 = K split by group; epilogue 0 = store,
# 1 = SwiGLU, 2 = SwiGLU backward.
ROLE_CALL = {"gemm1": "grouped_ffn", "gemm2": "grouped_ffn", "dh": "grouped_ffn_bwd",
             "dx": "grouped_ffn_bwd", "wgrad": "grouped_ffn_bwd"}


def kernel_role(name: str):
    import re
    m = re.search(r"gemm_kernel<[^,]+, [^,]+, (true|false), (true|false), (\d), (\d)", name)
    if not m:
        return None
    ak, bk, mode, epi = m.group(1) == "true", m.group(2) == "true", int(m.group(3)), int(m.group(4))
    if mode == 1:
        return "wgrad"
    if epi == 1:
        return "gemm1"
    if epi == 2:
        return "dh"
    return "gemm2" if bk else "dx"


# the sources the grouped GEMM kernels (whose traffic is stored) are built from
GEMM_SOURCES = ("common.hpp", "gemm.hip", "launch.hpp")


def source_hash() -> str:
    """Hash of the GEMM sources' code, comments and blank space removed (a
    comment edit does not change the kernels the counters measured)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        code = open(os.path.join(CSRC, f)).read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(f.encode())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def step_calls(cfg):
    """The library calls of one step, in launch order."""
    calls = ["route"] + (["aux_loss"] if cfg.aux_coeff else []) + ["dispatch", "grouped_ffn"]
    calls += (["shared_ffn"] if cfg.shared else []) + ["combine", "combine_bwd", "grouped_ffn_bwd"]
    calls += (["shared_ffn_bwd"] if cfg.shared else []) + ["dispatch_bwd", "route_bwd"]
    return calls


def _is_step_start(name):
    import re
    return re.search(r"moe::logits(_small_e)?_kernel<", name) is not None


def _call_ends(call, name, wgrads_seen):
    """Whether the kernel `name` is the last one the library call `call`
    launches (route_bwd, the step's last call, ends at the next step)."""
    if call == "route":
        return "moe::select_kernel<" in name
    if call == "aux_loss":
        return "moe::aux_final_kernel<true>" in name
    if call == "dispatch":
        return "moe::dispatch_gather" in name
    if call in ("grouped_ffn", "shared_ffn"):
        return kernel_role(name) == "gemm2"
    if call in ("combine", "dispatch_bwd"):
        return "moe::combine_kernel<" in name
    if call == "combine_bwd":
        return "moe::combine_bwd_kernel<" in name
    if call in ("grouped_ffn_bwd", "shared_ffn_bwd"):
        return kernel_role(name) == "wgrad" and wgrads_seen == 2
    return False


def attribute_calls(rows, calls, name_key="Kernel_Name"):
    """Library kernels of a rocprofv3 trace or counter CSV, assigned to
    (step, call). Kernels outside the library (torch's fills, the cache
    flush) and those before the first step (weight quantisation at set-up)
    are left out. Returns a list of (step, call, row) in dispatch order."""
    rows = sorted(rows, key=lambda r: int(r["Dispatch_Id"]))
    out = []
    step, ci, wg = -1, 0, 0
    for r in rows:
        n = r[name_key]
        if "moe::" not in n:
            continue
        if _is_step_start(n) and (step < 0 or ci > 0):
            step, ci, wg = step + 1, 0, 0
        if step < 0:
            continue
        if ci >= len(calls):
            raise ValueError(f"kernel {n} past the step's last call")
        if kernel_role(n) == "wgrad":
            wg += 1
        out.append((step, calls[ci], r))
        if _call_ends(calls[ci], n, wg):
            ci, wg = ci + 1, 0
    return out


def summarize_profiles(cfg_name, stats_dir, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir,
                       command):
    """Turn rocprofv3 CSV output into profiles/<cfg>_kernels.md and
    profiles/<cfg>_traffic.json: kernel time per library call and step (every
    kernel a call launches), and HBM bytes per call and per GEMM role, with
    FETCH_SIZE/WRITE_SIZE scaled by what they read for a 1 GiB copy."""
    import csv
    import collections
    import moe_synth as S
    cfg = S.BY_NAME[cfg_name]
    calls = step_calls(cfg)
    stats = list(csv.DictReader(open(os.path.join(stats_dir, "run_kernel_stats.csv"))))
    tot = sum(float(r["TotalDurationNs"]) for r in stats)
    lines = [f"# Kernel time, {cfg_name}, fwd+bwd steps (rocprofv3 --kernel-trace --stats)", "",
             "Command (repository root, one MI355X):", "", "```", command["stats"], "```", "",
             "| avg us | calls | % time | kernel |", "|---:|---:|---:|---|"]
    for r in stats:
        lines.append(f"| {float(r['AverageNs']) / 1e3:.1f} | {r['Calls']} | "
                     f"{100 * float(r['TotalDurationNs']) / tot:.1f} | `{r['Name'][:140]}` |")

    trace = list(csv.DictReader(open(os.path.join(stats_dir, "run_kernel_trace.csv"))))
    att = attribute_calls(trace, calls)
    steps = 1 + max(s for s, _, _ in att)
    dur = lambda r: int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    call_ns = collections.defaultdict(float)
    call_kern = collections.defaultdict(lambda: collections.defaultdict(list))
    for _, c, r in att:
        call_ns[c] += dur(r)
        role = kernel_role(r["Kernel_Name"]) or r["Kernel_Name"].split("(")[0].replace("void ", "")
        call_kern[c][role].append(dur(r))
    lines += ["", "## Library calls per step (every kernel each call launches)", "",
              f"Steps in the trace: {steps} (warm-up included). Kernels are assigned to calls by "
              "their order in the step; a call's time is the sum of its kernels' durations "
              "(gaps between them not counted).", "",
              "| call | ms per step | kernels (avg us x launches per step) |", "|---|---:|---|"]
    for c in calls:
        if c not in call_ns:
            continue
        parts = ", ".join(f"{k} {sum(v) / len(v) / 1e3:.1f} x {len(v) / steps:g}"
                          for k, v in call_kern[c].items())
        lines.append(f"| {c} | {call_ns[c] / steps / 1e6:.3f} | {parts} |")

    def counters(d):
        return list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))

    def copy_kib(d):
        v = [float(r["Counter_Value"]) for r in counters(d) if "copyBuffer" in r["Kernel_Name"]]
        return sum(v) / len(v)

    f_fetch = (1 << 30) / (copy_kib(copy_fetch_dir) * 1024)
    f_write = (1 << 30) / (copy_kib(copy_write_dir) * 1024)

    def per_step(d, factor):
        rows = counters(d)
        a = attribute_calls(rows, calls)
        n = 1 + max(s for s, _, _ in a)
        by_call = collections.defaultdict(float)
        by_role = collections.defaultdict(lambda: collections.defaultdict(list))
        by_kernel = collections.defaultdict(list)
        for _, c, r in a:
            v = float(r["Counter_Value"]) * 1024 * factor
            by_call[c] += v / n
            role = kernel_role(r["Kernel_Name"])
            if role:
                by_role[c][role].append(v)
            else:
                by_kernel[r["Kernel_Name"]].append(v)
        return by_call, by_role, by_kernel

    fc, fr, fk = per_step(fetch_dir, f_fetch)
    wc, wr, wk = per_step(write_dir, f_write)
    roles = {}
    for c in ("grouped_ffn", "grouped_ffn_bwd"):
        for role, v in fr.get(c, {}).items():
            w = wr[c][role]
            roles[role] = [sum(v) / len(v), sum(w) / len(w)]
    out = {"config": cfg_name, "source_hash": source_hash(), "fetch_factor": f_fetch,
           "write_factor": f_write,
           "roles_bytes_per_launch": {k: {"fetch": v[0], "write": v[1]} for k, v in roles.items()},
           "calls_bytes_per_launch": {c: fc[c] + wc.get(c, 0.0) for c in calls if c in fc},
           "calls_ms_per_step": {c: call_ns[c] / steps / 1e6 for c in calls if c in call_ns},
           "commands": command}
    lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
              f"Scaled by a 1 GiB device copy: FETCH_SIZE x {f_fetch:.3f}, WRITE_SIZE x {f_write:.3f}. "
              "Per GEMM role: the routed experts' launches (wgrad: the mean of dW2 and dW1).",
              "", "| GEMM role | fetch GB | write GB |", "|---|---:|---:|"]
    for k, v in roles.items():
        lines.append(f"| {k} | {v[0] / 1e9:.3f} | {v[1] / 1e9:.3f} |")
    lines += ["", "| call | HBM GB per step (fetch + write, every kernel of the call) | GB/s at the "
              "call's kernel time |", "|---|---:|---:|"]
    for c in calls:
        if c in fc:
            b = fc[c] + wc.get(c, 0.0)
            t = call_ns.get(c, 0.0) / steps
            lines.append(f"| {c} | {b / 1e9:.3f} | {b / t:.0f} |" if t else f"| {c} | {b / 1e9:.3f} | |")
    # the other library kernels: measured bytes per launch and the bandwidth
    # they imply at the stats run's mean duration
    avg_ns = {r["Name"]: float(r["AverageNs"]) for r in stats}
    lines += ["", "## Other library kernels: HBM traffic per launch and bandwidth", "",
              "FETCH_SIZE and WRITE_SIZE per launch (scaled as above), divided by the kernel's mean "
              "duration in the stats run; means over every launch inside the steps. 8 TB/s is the "
              "vendor peak; the measured copy peak is in the benchmark line.", "",
              "| kernel | launches | fetch MB | write MB | mean us | GB/s |", "|---|---:|---:|---:|---:|---:|"]
    for n in sorted(fk, key=lambda n: -(sum(fk[n]) / len(fk[n]))):
        if n not in avg_ns:
            continue
        f_ = sum(fk[n]) / len(fk[n])
        w_ = sum(wk.get(n, [0.0])) / max(1, len(wk.get(n, [])))
        us = avg_ns[n] / 1e3
        lines.append(f"| `{n[:110]}` | {len(fk[n])} | {f_ / 1e6:.1f} | {w_ / 1e6:.1f} | "
                     f"{us:.1f} | {(f_ + w_) / (us * 1e3):.0f} |")
    lines += ["", "Commands:", "", "```"] + [command[k] for k in ("fetch", "write", "copy_fetch",
                                                                    "copy_write")] + ["```"]
    os.makedirs(PROFILES, exist_ok=True)
    open(os.path.join(PROFILES, f"{cfg_name}_kernels.md"), "w").write("\n".join(lines) + "\n")
    json.dump(out, open(os.path.join(PROFILES, f"{cfg_name}_traffic.json"), "w"), indent=1)
    print("wrote", os.path.join(PROFILES, f"{cfg_name}_kernels.md"))


def summarize_mfma(cfg_name, pmc_dir):
    """profiles/<cfg>_mfma.md from a `rocprofv3 --pmc MfmaUtil MfmaFlopsBF16`
    run: per GEMM role, the matrix cores' busy share while the kernel runs
    and the MFMA work they did against the algorithmic flops (the excess is
    the zero rows that pad ragged expert tiles)."""
    import csv
    import collections
    import moe_synth as S
    cfg = S.BY_NAME[cfg_name]
    A, d, f = cfg.T * cfg.k, cfg.d, cfg.f
    alg = {"gemm1": 4 * A * d * f, "gemm2": 2 * A * f * d, "dh": 2 * A * d * f, "dx": 4 * A * f * d,
           "wgrad": 3 * A * d * f}  # wgrad: the mean of dW2 (2 A d f) and dW1 (4 A d f)
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(os.path.join(pmc_dir, "run_counter_collection.csv"))):
        role = kernel_role(r["Kernel_Name"])
        if role:
            acc[role][r["Counter_Name"]].append(float(r["Counter_Value"]))
    cmd = (f"rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 --output-format csv -d <dir> -o run -- "
           f"python3 bench.py --steps 2 --warmup 1 --cpu-sample 0 --config {cfg_name}")
    lines = [f"# Matrix-core utilisation, {cfg_name} (rocprofv3 derived counters)", "",
             "Command (repository root, one MI355X):", "", "```", cmd, "```", "",
             "MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs): the share of the "
             "kernel's active cycles in which the matrix cores are busy, at the clock the GPU runs "
             "at under load. MfmaFlopsBF16 = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512: the MFMA work done, "
             "compared with the algorithmic flops of the launch (routed experts and, for a layer "
             "with one, the shared expert averaged in). Means over all launches of the role.", "",
             "| GEMM role | launches | MFMA busy % | MFMA TFLOP per launch | algorithmic TFLOP | ratio |",
             "|---|---:|---:|---:|---:|---:|"]
    for role in ("gemm1", "gemm2", "dh", "dx", "wgrad"):
        v = acc.get(role)
        if not v:
            continue
        u = sum(v["MfmaUtil"]) / len(v["MfmaUtil"])
        fl = sum(v["MfmaFlopsBF16"]) / len(v["MfmaFlopsBF16"])
        lines.append(f"| {role} | {len(v['MfmaUtil'])} | {u:.1f} | {fl / 1e12:.3f} | "
                     f"{alg[role] / 1e12:.3f} | {fl / alg[role]:.3f} |")
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"{cfg_name}_mfma.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print("wrote", out)


def measured_traffic(cfg_name, call):
    """HBM bytes per launch of `call` from the committed counter summary, or
    None when the kernels changed since the counters were taken."""
    f = os.path.join(PROFILES, f"{cfg_name}_traffic.json")
    if not os.path.exists(f):
        return None
    d = json.load(open(f))
    if d.get("source_hash") != source_hash():
        return None
    return d["calls_bytes_per_launch"].get(call)


def stage_work(c):
    """Algorithmic bytes and flops of every call in a step (what the method
    must move or compute; intermediate re-reads are not counted)."""
    T, d, E, k, f, S = c.T, c.d, c.E, c.k, c.f, c.shared
    A = T * k
    R = A + S * T
    bx = 4 if c.act == "f32" else 2
    bo = ba = bx
    bw = {"f32": 4, "bf16": 2, "fp8": 1, "mxfp8": 1}[c.weight]
    bg = 4 if c.weight == "f32" else 2
    # dispatched row: codes + scales (fp32 per 128, or one E8M0 byte per 32)
    bp = {"fp8": d + 4 * d // 128, "mxfp8": d + d // 32}.get(c.weight, d * bx)
    w = {}
    w["route"] = (T * d * bx + 4 * E * d + 4 * T * E + 8 * T * k + T * E, 2 * T * d * E)
    w["dispatch"] = (T * d * bx + A * bp + 16 * A, 0)
    w["grouped_ffn"] = (E * 3 * d * f * bw + A * bp + A * 2 * f * ba + A * d * bo, 6 * d * f * A)
    if S:
        w["shared_ffn"] = (3 * d * f * bw + T * bp + T * 2 * f * ba + T * d * bo, 6 * d * f * T)
    w["combine"] = (A * d * bo + 8 * A + S * T * d * bo + T * d * bo, 2 * A * d)
    w["combine_bwd"] = (T * d * bo + 2 * A * d * bo + 12 * A, 2 * A * d)
    w["grouped_ffn_bwd"] = (E * 3 * d * f * (bw + bg) + A * (2 * d * bo + 2 * f * ba + bp),
                            12 * d * f * A)
    if S:
        w["shared_ffn_bwd"] = (3 * d * f * (bw + bg) + T * (2 * d * bo + 2 * f * ba + bp),
                               12 * d * f * T)
    w["dispatch_bwd"] = (A * d * bo + T * d * bx + 4 * A + S * T * d * bo, A * d)
    w["route_bwd"] = (4 * T * E + 12 * T * k + 3 * T * d * bx + 8 * E * d, 4 * T * d * E)
    if c.aux_coeff:
        w["aux_loss"] = (4 * T * E + 4 * T * k, 0)   # logits and indices, read once
    return w


def make_layer(cfg, device, recompute="none", gemm_tile="auto"):
    import torch
    import moe_synth as S
    from mixture_experts_layer_gather_amd import MoELayer
    layer = MoELayer(**cfg.describe(), recompute=recompute, gemm_tile=gemm_tile, device=device)
    w1, w2 = S.all_expert_weights(cfg, device=device, threads=16)
    bias = S.router_bias(cfg)
    sw1 = S.shared_w1(cfg).to(device) if cfg.shared else None
    sw2 = S.shared_w2(cfg).to(device) if cfg.shared else None
    layer.set_weights(S.w_router(cfg).to(device), w1, w2,
                      bias=None if bias is None else bias.to(device), sw1=sw1, sw2=sw2)
    x = S.x(cfg).to(device)
    dy = S.dy(cfg).to(device)
    torch.cuda.synchronize()
    return layer, x, dy


def timed_step(layer, x, dy, marks):
    """One fwd+bwd step with an event after every library call, on torch's
    current stream (where the library launches)."""
    rec = lambda name: marks.append((name, _event()))
    rec("start")
    layer.forward(x, mark=rec)
    layer.backward(dy, mark=rec)


class CacheFlush:
    """Writes 1 GiB, then reads another 1 GiB, so that the next step finds
    neither its own data nor dirty lines in the L2s or the 256 MB MALL."""

    def __init__(self, device):
        import torch
        self.w = torch.empty(1 << 30, dtype=torch.uint8, device=device)
        self.r = torch.ones(1 << 28, dtype=torch.int32, device=device)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.w.fill_(self.n & 0xFF)
        self.r.sum()


def copy_peak(device, flush):
    """A plain 1 GiB device-to-device copy (torch), after a flush: read +
    written bytes over its event time, best of three."""
    import torch
    a = torch.ones(1 << 30, dtype=torch.uint8, device=device)
    b = torch.empty_like(a)
    best = 0.0
    for _ in range(3):
        flush()
        e0, e1 = _event(), None
        b.copy_(a)
        e1 = _event()
        torch.cuda.synchronize()
        best = max(best, 2 * (1 << 30) / e0.elapsed_time(e1) / 1e6)
    del a, b
    return best


def graph_replay(layer, x, dy, warmup, steps, T, flush):
    """The whole step captured once into a HIP graph (every library call
    only enqueues and reads its shapes from device memory), then replayed,
    each replay after a cache flush."""
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        layer.step(x, dy)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(steps):
        flush()
        a = _event()
        g.replay()
        ts.append((a, _event()))
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ts) / steps
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms / 1e3), 1)}


def _event():
    import torch
    e = torch.cuda.Event(enable_timing=True)
    e.record()
    return e


def cpu_model():
    """The host CPU's model name and logical CPU count (/proc/cpuinfo)."""
    try:
        names = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name")]
        return (names[0] if names else "unknown"), len(names)
    except OSError:  # pragma: no cover
        return "unknown", os.cpu_count()


def cpu_baseline(cfg, sample_tokens):
    """The CPU oracle, as it stands, on the first `sample_tokens` tokens of the
    same workload: routing, dispatch, every expert's SwiGLU FFN forward and
    backward (expert by expert over all experts' weights), combine, and the
    router backward, in fp64."""
    import moe_synth as S
    import oracle
    sub = cfg.replace(T=sample_tokens)
    x = S.x(cfg)[:sample_tokens]
    dy = S.dy(cfg)[:sample_tokens]
    inp = dict(x=x, wr=S.w_router(cfg), bias=S.router_bias(cfg), dy=dy,
               w1=lambda e: S.expert_w1(cfg, e), w2=lambda e: S.expert_w2(cfg, e))
    if cfg.shared:
        inp.update(sw1=S.shared_w1(cfg), sw2=S.shared_w2(cfg))
    t0 = time.perf_counter()
    oracle.layer_stream(sub, inp)
    dt = time.perf_counter() - t0
    threads = os.environ.get("OMP_NUM_THREADS")
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [int(threads or 1)])
    except Exception:  # pragma: no cover
        cores = int(threads or os.cpu_count())
    model, logical = cpu_model()
    return {"value": round(sample_tokens / dt, 3), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", "cpu": model, "host_logical_cpus": logical,
            "sample": f"first {sample_tokens} of {cfg.T} tokens of {cfg.name}: the full layer forward "
                      f"+ backward in fp64 (numpy/OpenBLAS and the C spec with OpenMP), every routed "
                      f"expert's weights quantised and streamed; {dt:.1f} s"}


def run_config(cfg, args, dev, flush, copy_gbps):
    """Warm-up, then `steps` timed steps, each after a cache flush; returns
    the workload's figures (times from events on the library's stream)."""
    import torch
    layer, x, dy = make_layer(cfg, dev, args.recompute, args.gemm_tile)
    for _ in range(args.warmup):
        timed_step(layer, x, dy, [])
    torch.cuda.synchronize()
    steps = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        flush()
        marks = []
        timed_step(layer, x, dy, marks)
        steps.append(marks)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = sorted(m[0][1].elapsed_time(m[-1][1]) for m in steps)
    ms = sum(step_ms) / len(step_ms)
    per = {}
    for marks in steps:
        for (_, a), (name, b) in zip(marks[:-1], marks[1:]):
            per.setdefault(name, []).append(a.elapsed_time(b))
    per_ms = {n: sum(v) / len(v) for n, v in per.items()}
    work = stage_work(cfg)
    dt = "fp8" if cfg.weight in ("fp8", "mxfp8") else cfg.act
    stages = {}
    for n, t in per_ms.items():
        b, fl = work[n]
        stages[n] = {"ms": round(t, 4), "GBps": round(b / t / 1e6, 1),
                     "TFLOPs": round(fl / t / 1e9, 1) if fl else 0.0}
    dom = max(per_ms, key=per_ms.get)
    b, fl = work[dom]
    # the binding roofline of the dominant call: its flops at the matrix
    # cores' peak or its algorithmic bytes at the HBM peak, whichever takes
    # longer (the expert FFN of 256-expert layers streams more weight bytes
    # than it has flops to hide them behind)
    mfma_bound = fl and fl / (MFMA_PEAK_TFLOPS[dt] * 1e12) >= b / (HBM_PEAK_GBPS * 1e9)
    if "ffn" in dom:
        traffic = measured_traffic(cfg.name, dom)
        traffic = None if traffic is None else round(traffic)
        kname = f"moe_{dom.replace('shared_', 'grouped_')} ({dom})"
    else:
        traffic, kname = None, dom
    if mfma_bound:
        ach = fl / per_ms[dom] / 1e9
        roof = {"kernel": kname, "bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_PEAK_TFLOPS[dt],
                "unit": "TFLOP/s", "frac": round(ach / MFMA_PEAK_TFLOPS[dt], 4), "traffic": traffic,
                "algorithmic_flops": fl, "ms": round(per_ms[dom], 4)}
    else:
        ach = b / per_ms[dom] / 1e6
        roof = {"kernel": kname, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "algorithmic_bytes": round(b), "ms": round(per_ms[dom], 4)}
    ffn_f = sum(work[n][1] for n in per_ms if "ffn" in n)
    ffn_t = sum(per_ms[n] for n in per_ms if "ffn" in n)
    hbm = {}
    for n in ("dispatch", "combine", "combine_bwd", "dispatch_bwd"):
        gbps = work[n][0] / per_ms[n] / 1e6
        hbm[n] = {"GBps": round(gbps, 1), "frac_of_8TBps": round(gbps / HBM_PEAK_GBPS, 4),
                  "frac_of_copy": round(gbps / copy_gbps, 4)}
    dc = (work["dispatch"][0] + work["combine"][0]) / (per_ms["dispatch"] + per_ms["combine"]) / 1e6
    out = {
        "workload": f"{cfg.name}: MoE layer fwd+bwd, T={cfg.T} d={cfg.d} E={cfg.E}"
                    f"{'+1 shared' if cfg.shared else ''} top-{cfg.k} {cfg.score}"
                    f"{' renorm' if cfg.renorm else ''}, SwiGLU d_ff={cfg.f}, {cfg.weight}"
                    f"{f', aux loss {cfg.aux_coeff:g}' if cfg.aux_coeff else ''}",
        "tokens_per_s": round(cfg.T / (ms / 1e3), 1),
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(step_ms[len(step_ms) // 2], 4),
        "ms_per_step_min": round(step_ms[0], 4),
        "dtype": dt,
        "dispatch_combine_GBps": round(dc, 1),
        "dispatch_combine_frac_of_8TBps": round(dc / HBM_PEAK_GBPS, 4),
        "dispatch_combine_frac_of_copy": round(dc / copy_gbps, 4),
        "hbm_stages": hbm,
        "grouped_gemm_mfma_pct": round(100 * ffn_f / ffn_t / 1e9 / MFMA_PEAK_TFLOPS[dt], 2),
        "stages": stages,
        "roofline": roof,
        "wall_s": round(wall, 3),
    }
    if args.graph:
        out["graph"] = graph_replay(layer, x, dy, args.warmup, args.steps, cfg.T, flush)
    del layer, x, dy
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def vendor_gemm(name):
    """Context for the grouped GEMM's roofline: the vendor library's dense
    GEMM (torch.matmul, or torch._scaled_mm for the FP8 layers; hipBLASLt) on
    the same per-expert shapes, one call per expert with the mean rows per
    expert, no epilogue work; the first product over all rows against one
    expert's weights (the same flops without streaming 256 weight matrices);
    and a large square GEMM as the library's best case on this GPU."""
    import torch
    import moe_synth as S
    cfg = S.BY_NAME[name]
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    E, d, f = cfg.E, cfg.d, cfg.f
    R = cfg.T * cfg.k // E
    g = torch.Generator(device=dev).manual_seed(0)
    def rnd(*shape):
        return torch.randn(*shape, dtype=bf, device=dev, generator=g)
    x, dy = rnd(E * R, d), rnd(E * R, d)
    h, gu = rnd(E * R, f), rnd(E * R, 2 * f)
    w1, w2 = rnd(E, 2 * f, d), rnd(E, d, f)
    rows = lambda t, e: t[e * R:(e + 1) * R]
    f1, f2 = 2.0 * E * R * d * 2 * f, 2.0 * E * R * f * d
    cases = [("gemm1", "X_e @ W1_e^T", lambda: [rows(x, e) @ w1[e].t() for e in range(E)], f1),
             ("gemm2", "H_e @ W2_e^T", lambda: [rows(h, e) @ w2[e].t() for e in range(E)], f2),
             ("dh", "dY_e @ W2_e", lambda: [rows(dy, e) @ w2[e] for e in range(E)], f2),
             ("dx", "dGU_e @ W1_e", lambda: [rows(gu, e) @ w1[e] for e in range(E)], f1),
             ("wgrad dW1", "X_e^T @ dGU_e", lambda: [rows(x, e).t() @ rows(gu, e) for e in range(E)], f1),
             ("wgrad dW2", "H_e^T @ dY_e", lambda: [rows(h, e).t() @ rows(dy, e) for e in range(E)], f2)]
    sq = rnd(8192, 8192)
    cases.append(("gemm1 dense", "X @ W1_0^T (all rows, one weight)", lambda: x @ w1[0].t(), f1))
    cases.append(("square", "8192 x 8192 x 8192", lambda: sq @ sq, 2.0 * 8192 ** 3))
    peak = 2500
    lib = "torch.matmul (hipBLASLt)"
    dtype_note = "bf16"
    if cfg.weight in ("fp8", "mxfp8"):
        # the same products in E4M3 through torch._scaled_mm with one fp32
        # scale per tensor (no block scales: the library's plain FP8 GEMM),
        # bf16 out; the second operand column-major as the call requires,
        # transposed copies made once before timing
        f8 = torch.float8_e4m3fn
        one = torch.ones((), dtype=torch.float32, device=dev)
        q = lambda t: t.to(f8)
        xq, dyq, hq, guq = q(x), q(dy), q(h), q(gu)
        w1q, w2q = q(w1), q(w2)
        w1t = w1q.transpose(1, 2).contiguous()  # [E, d, 2f]
        w2t = w2q.transpose(1, 2).contiguous()  # [E, f, d]
        xT = [rows(xq, e).t().contiguous() for e in range(E)]
        hT = [rows(hq, e).t().contiguous() for e in range(E)]
        guT = [rows(guq, e).t().contiguous() for e in range(E)]
        dyT = [rows(dyq, e).t().contiguous() for e in range(E)]
        mm = lambda a, b_cm: torch._scaled_mm(a, b_cm, scale_a=one, scale_b=one, out_dtype=bf)
        sq8, sq8t = q(sq), q(sq).t().contiguous()
        w1q0 = w1q[0].t()
        cases = [("gemm1", "X_e @ W1_e^T", lambda: [mm(rows(xq, e), w1q[e].t()) for e in range(E)], f1),
                 ("gemm2", "H_e @ W2_e^T", lambda: [mm(rows(hq, e), w2q[e].t()) for e in range(E)], f2),
                 ("dh", "dY_e @ W2_e", lambda: [mm(rows(dyq, e), w2t[e].t()) for e in range(E)], f2),
                 ("dx", "dGU_e @ W1_e", lambda: [mm(rows(guq, e), w1t[e].t()) for e in range(E)], f1),
                 ("wgrad dW1", "X_e^T @ dGU_e", lambda: [mm(xT[e], guT[e].t()) for e in range(E)], f1),
                 ("wgrad dW2", "H_e^T @ dY_e", lambda: [mm(hT[e], dyT[e].t()) for e in range(E)], f2),
                 ("gemm1 dense", "X @ W1_0^T (all rows, one weight)", lambda: mm(xq, w1q0), f1),
                 ("square", "8192 x 8192 x 8192", lambda: mm(sq8, sq8t.t()), 2.0 * 8192 ** 3)]
        peak = 5000
        lib = "torch._scaled_mm (hipBLASLt)"
        dtype_note = "E4M3 in with one fp32 scale per tensor, bf16 out"
    print(f"# {lib} on the GEMM shapes of {name}\n")
    print(f"{E} experts x {R} rows (mean rows per expert), d={d}, f={f}; {dtype_note}; "
          f"one call per expert; peak {peak} TFLOP/s.\n")
    print("Each case's calls are captured once into a HIP graph and the graph is replayed, so host launch "
          "overhead is not timed (eager replays where capture fails).\n")
    print("| role | product | ms | TFLOP/s | % of peak |\n|---|---|---:|---:|---:|")
    for role, what, fn, flops in cases:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        run = fn
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn()
            run = graph.replay
            run()
        except RuntimeError:
            run = fn
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        print(f"| {role} | {what} | {ms:.3f} | {flops / ms / 1e9:.0f} | {flops / ms / 1e9 / peak * 100:.1f} |",
              flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="all",
                    help="one workload (see moe_synth), or all: the headline workload first, then "
                         "the others in the same line")
    ap.add_argument("--aux-coeff", type=float, default=0.0,
                    help="load-balancing auxiliary loss coefficient (0.01 in the Megatron recipe; "
                         "0: off, as in the workloads' definitions)")
    ap.add_argument("--recompute", choices=["none", "act", "full"], default="none",
                    help="activations the expert FFN keeps for the backward: GU and H (none), "
                         "GU only (act), nothing (full)")
    ap.add_argument("--gemm-tile", choices=["auto", "small", "big"], default="auto",
                    help="force the expert GEMMs' output tile (tuning; default: chosen per GEMM)")
    ap.add_argument("--graph", action="store_true",
                    help="also capture the step into one HIP graph and time its replays")
    ap.add_argument("--cpu-sample", type=int, default=CPU_SAMPLE_TOKENS,
                    help="tokens of the workload timed on the CPU oracle (0: skip)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time torch.matmul (hipBLASLt) on the config's per-expert GEMM shapes")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 output dir; writes profiles/<config>_mfma.md")
    ap.add_argument("--summarize", nargs=5, metavar="DIR",
                    help="rocprofv3 output dirs: stats, FETCH_SIZE, WRITE_SIZE, copy FETCH_SIZE, "
                         "copy WRITE_SIZE; writes profiles/<config>_kernels.md and _traffic.json")
    args = ap.parse_args()
    if args.summarize_mfma:
        summarize_mfma(args.config, args.summarize_mfma)
        return
    if args.summarize:
        c = args.config
        cmd = {"stats": f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
                        f"python3 bench.py --steps 3 --warmup 1 --cpu-sample 0 --config {c}",
               "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- "
                        f"python3 bench.py --steps 2 --warmup 1 --cpu-sample 0 --config {c}",
               "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- "
                        f"python3 bench.py --steps 2 --warmup 1 --cpu-sample 0 --config {c}",
               "copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- "
                             "python3 bench.py --copy-probe",
               "copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- "
                             "python3 bench.py --copy-probe"}
        summarize_profiles(c, *args.summarize, command=cmd)
        return
    if args.vendor_gemm:
        vendor_gemm(args.config)
        return
    if args.copy_probe:
        import torch
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.copy_(a)
        e0.record()
        for _ in range(2):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 2
        print(json.dumps({"copy_probe_bytes": 1 << 30, "launches": 3,
                          "copy_GBps": round(2 * (1 << 30) / ms / 1e6, 1)}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_synth as S
    if args.config == "all":
        order = [HEADLINE] + [n for n in CONTEXT_CONFIGS]
    else:
        order = [args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = CacheFlush(dev)
    copy_gbps = copy_peak(dev, flush)
    results = {}
    for name in order:
        cfg = S.BY_NAME[name]
        if args.aux_coeff:
            cfg = cfg.replace(aux_coeff=args.aux_coeff)
        print(f"[bench] {name}", file=sys.stderr, flush=True)
        results[name] = run_config(cfg, args, dev, flush, copy_gbps)
    head = results[order[0]]
    cfg = S.BY_NAME[order[0]]
    out = {
        "metric": "MoE layer tokens/s; dispatch/combine HBM GB/s; grouped-GEMM MFMA % of peak",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "ms_per_step_median": head["ms_per_step_median"],
        "ms_per_step_min": head["ms_per_step_min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded normal inputs and random-init weights of the layer's shape)",
        "config": {"workload": head["workload"], "tokens": cfg.T, "hidden": cfg.d, "experts": cfg.E,
                   "shared_experts": cfg.shared, "top_k": cfg.k, "ffn_hidden": cfg.f,
                   "parallelism": "none (one GPU)",
                   "timing": "HIP events around each step on the library's stream; 1 GiB written "
                             "and 1 GiB read before every timed step, outside the events"},
        "copy_peak_GBps": round(copy_gbps, 1),
        "dispatch_combine_GBps": head["dispatch_combine_GBps"],
        "dispatch_combine_frac_of_8TBps": head["dispatch_combine_frac_of_8TBps"],
        "dispatch_combine_frac_of_copy": head["dispatch_combine_frac_of_copy"],
        "hbm_stages": head["hbm_stages"],
        "grouped_gemm_mfma_pct": head["grouped_gemm_mfma_pct"],
        "stages": head["stages"],
        "roofline": head["roofline"],
        "wall_s": head["wall_s"],
    }
    if args.recompute != "none":
        out["config"]["recompute"] = args.recompute
    if args.gemm_tile != "auto":
        out["config"]["gemm_tile"] = args.gemm_tile
    if "graph" in head:
        out["graph"] = head["graph"]
    if len(order) > 1:
        out["configs"] = {n: {k: v for k, v in r.items() if k != "stages"} | {"stages": r["stages"]}
                          for n, r in results.items() if n != order[0]}
    if args.cpu_sample > 0:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_sample)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
