"""Benchmark of the FlashAttention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

A step is one FlashAttention forward (attn_fwd_flash through the C ABI) over
the workload's inputs, already resident in HBM.  The default workload is the
Llama-2-7B-shaped causal bf16 forward (batch 4, 32 heads, seq 4096, d 128,
P rounded to bf16).  Timing: the step is enqueued back to back for a fixed
settle time (the power controller drops the shader clock during the first
~30 ms of dense matrix work and then recovers; the settle keeps that
transient out of the figure), then W warm-up steps, then exactly K timed
steps between two HIP events on the launch stream, then a second pass of K
steps with an event after each for the per-launch median, min and max --
all without a host wait in between, so the GPU never idles.  Prints ONE JSON line with:

  value / unit      attention-forward TFLOP/s (MFMA contraction flops over
                    visible (query, key) pairs / mean step time)
  launch_ms         per-launch mean / median / min / max
  shader_clock_mhz  average shader clock over the timed steps (each CU's
                    clock counter sampled before and after)
  roofline          the flash kernel against the bf16 MFMA dense peak
  max_abs_err ...   deviation of the flash output from the FP64 oracle on the
                    oracle's sample, with the count of non-finite elements
  cpu_baseline      the FP64 oracle on the host cores, on a bounded sample
  legs              the other kernels and workloads of the path, each timed
                    alone (the GPT-2-shaped, long-sequence and int8 workloads,
                    the baseline attention, deviation, Wasserstein, rounding
                    bias, delta, backward, fp8 and quantiser legs)
The process exits with status 3 after printing the line when any output
compared with the oracle holds a non-finite element.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "attn fwd TFLOP/s (bf16 causal, % MFMA peak) + max|err| vs FP64 oracle"
PEAK = {"bf16": 2516.6, "int8": 5033.2, "fp8": 5033.2, "f32": 157.3}  # dense MFMA, MI355X
HBM_PEAK_GBS = 8000.0
# the machine's CPU share for one GPU: the oracle's process pool never exceeds it
HOST_CORE_SHARE = 16
SETTLE_S = 0.25
LEG_SETTLE_S = 0.1


# HBM bytes per launch of the flash kernel on c3, from two rocprofv3 --pmc
# passes (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch).  A plain 256 MiB
# device copy reads FETCH_SIZE = 131085 KiB and WRITE_SIZE = 262144 KiB, so
# FETCH_SIZE is scaled by 2 and WRITE_SIZE by 1 (the copy's and the flash
# kernel's reads are all 128-byte requests, TCC_EA0_RDREQ_128B, which the
# FETCH_SIZE formula counts as 64 bytes).  The figure is valid only for the
# kernel sources it was taken on (sha256 of the files below).
TRAFFIC_SOURCES = ("precision_numerics_amd/csrc/flash_fwd.hip",
                   "precision_numerics_amd/csrc/device.hpp",
                   "precision_numerics_amd/csrc/launch.hpp",
                   "precision_numerics_amd/csrc/lds_dma.hpp")
TRAFFIC = {
    "workload": "c3",
    "sources_sha256": "4735a4a0c70ab699fe63c710d0e0c0944a8aebf1d9eab347c979b65a56ba9815",
    "fetch_kib": 305044.0, "fetch_scale": 2.0,
    "write_kib": 131072.0, "write_scale": 1.0,
}


def sources_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch from the counters, or None when they were taken on
    another workload or on different kernel sources."""
    if workload != TRAFFIC["workload"] or sources_digest() != TRAFFIC["sources_sha256"]:
        return None
    return int(1024 * (TRAFFIC["fetch_kib"] * TRAFFIC["fetch_scale"] +
                       TRAFFIC["write_kib"] * TRAFFIC["write_scale"]))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_info():
    """CPU model, the cores this process may use, and numpy's BLAS."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        blas = f"{b.get('name')} {b.get('version')} ({b.get('openblas configuration', '')})"
    except Exception:                                  # noqa: BLE001
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)),
            "numpy": np.__version__, "blas": blas}


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def settle(fn, seconds):
    """Enqueue fn back to back for about `seconds` of GPU time (at most 4000
    calls), without waiting in between: the calls that follow start on a GPU
    that has not idled since."""
    import torch
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(4):
        fn()
    torch.cuda.synchronize()
    per_call = max((time.perf_counter() - t0) / 4, 1e-6)
    calls = int(min(4000, max(0, seconds / per_call)))
    for _ in range(calls):
        fn()
    return calls + 5


def time_steps(fn, steps, warmup, settle_s, pna):
    """Mean ms per call of fn() between two HIP events on torch's current
    stream (the stream every entry point is launched on), then a second pass
    with an event after each call for the per-launch statistics."""
    import torch
    settled = settle(fn, settle_s) if settle_s > 0 else 0
    for _ in range(warmup):
        fn()
    clk0 = torch.zeros((1024, 3), dtype=torch.int64, device="cuda")
    clk1 = torch.zeros_like(clk0)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    pna.attn_clock_sample(clk0)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    pna.attn_clock_sample(clk1)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    mean_ms = start.elapsed_time(end) / steps
    mhz = pna.shader_clock_mhz(clk0.cpu().numpy(), clk1.cpu().numpy())
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
    return {"ms": mean_ms, "median_ms": float(np.median(per)), "min_ms": float(per.min()),
            "max_ms": float(per.max()), "settle_calls": settled,
            "shader_clock_mhz": None if mhz is None else round(mhz, 1)}


def launch_stats(t):
    return {"mean": round(t["ms"], 5), "median": round(t["median_ms"], 5),
            "min": round(t["min_ms"], 5), "max": round(t["max_ms"], 5)}


def mixed_fraction(flops, ms, qk, pv):
    """Fraction of the matrix peak for QK^T on the `qk` engine and P.V on the
    `pv` engine (half of the flops each): ideal time / measured time."""
    ideal_ms = (flops / 2 / (PEAK[qk] * 1e12) + flops / 2 / (PEAK[pv] * 1e12)) * 1e3
    return ideal_ms / ms, flops / (ideal_ms * 1e-3) / 1e12


def to_device(inp):
    import torch

    def bf(x):
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    if inp.cfg.dtype == "bf16":
        return bf(inp.q), bf(inp.k), bf(inp.v)
    if inp.cfg.dtype == "f32":
        return (torch.from_numpy(inp.q).cuda(), torch.from_numpy(inp.k).cuda(),
                torch.from_numpy(inp.v).cuda())
    return torch.from_numpy(inp.q).cuda(), torch.from_numpy(inp.k).cuda(), bf(inp.v)


def deviation_fields(pna, o_sample, ref_t, prefix=""):
    """Error statistics of o_sample against the FP64 reference; the error
    fields are null when any element is non-finite (n_nonfinite says how
    many)."""
    dev = pna.attn_deviation(o_sample, ref_t)
    bad = dev["n_nonfinite"] > 0
    return {prefix + "max_abs_err": None if bad else dev["max_abs"],
            prefix + "mean_abs_err": None if bad else dev["mean_abs"],
            prefix + "mean_signed_err": None if bad else dev["mean_signed"],
            prefix + "n_nonfinite": dev["n_nonfinite"]}


# ---------------------------------------------------------------------------
# the CPU baseline: the FP64 oracle (the only part of the bench that runs it)
# ---------------------------------------------------------------------------

def oracle_unit_fn(cfg, inp):
    """fn(unit) -> the oracle's O of one (batch, head) unit of the workload."""
    import oracle
    b, h, n, d = cfg.shape
    scale = oracle.default_scale(d)
    if cfg.dtype == "int8":
        qc, qs = oracle.quantize_int8(inp.q)
        kc, ks = oracle.quantize_int8(inp.k)
        qc, kc = qc.reshape(b * h, n, d), kc.reshape(b * h, n, d)
        qs, ks = qs.reshape(b * h, n), ks.reshape(b * h, n)
        v = synth.bf16_bits_to_f32(inp.v).reshape(b * h, n, d)

        def unit(u):
            return oracle.attention_int8_head(qc[u], qs[u], kc[u], ks[u], v[u],
                                              causal=cfg.causal, scale=scale)[0]
    else:
        def wide(x):
            return synth.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x
        q, k, v = (wide(x).reshape(b * h, n, d) for x in (inp.q, inp.k, inp.v))

        def unit(u):
            return oracle.attention_head(q[u], k[u], v[u], causal=cfg.causal, scale=scale)[0]
    return unit


def cpu_baseline(cfg, inp, units, workers):
    """The FP64 oracle (as it stands) on the listed (batch, head) units, run in
    a process pool on the host cores.  Returns (oracle O [units, N, d], stats)."""
    import oracle
    b, h, n, d = cfg.shape
    unit = oracle_unit_fn(cfg, inp)
    t0 = time.perf_counter()
    outs, used = oracle.run_heads(unit, units, workers=workers)
    wall = time.perf_counter() - t0
    flops = cfg.scaled(batch=1, heads=len(units)).flops()
    stats = {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
             "sample": f"{len(units)} of {b * h} (batch, head) units of {cfg.name}, all "
                       f"{n} query rows each; FP64 numpy/OpenBLAS, one BLAS thread per worker",
             "seconds": wall, "flops": flops}
    return np.stack(outs), stats


def oracle_refs(cfg, inp, units, workers):
    """Part of the CPU-baseline leg: the oracle's O of the listed units (the
    reference of a workload leg's error figures)."""
    import oracle
    outs, _ = oracle.run_heads(oracle_unit_fn(cfg, inp), list(units), workers=workers)
    return np.stack(outs)


BIAS_BETA = 2.0
BIAS_UNITS = (0, 31)
BIAS_V_SHIFT = -2.0


def bias_inputs(c4_inputs):
    """Inputs of the rounding-bias leg: the rank-4 long-sequence workload with
    V as drawn, V shifted to a negative mean (most columns of V negative, the
    situation the low-precision training page's Figure 5 examines), and that
    with the key rows duplicated in pairs (every token appears twice, so each
    row maximum is repeated).  Returns (cfg, q bits, [(name, k bits, v bits)])."""
    cfg = synth.CONFIGS["c4"]
    b, h, n, d = cfg.shape
    inp = c4_inputs
    v_neg = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(inp.v) + np.float32(BIAS_V_SHIFT))
    k_pair = inp.k.reshape(b, h, n // 2, 2, d)[:, :, :, :1, :].repeat(2, axis=3)
    k_pair = np.ascontiguousarray(k_pair.reshape(b, h, n, d))
    return cfg, inp.q, [("v", inp.k, inp.v), ("v_shifted", inp.k, v_neg),
                        ("v_shifted_keys_paired", k_pair, v_neg)]


def cpu_baseline_bias_refs(c4_inputs, workers):
    """Part of the CPU-baseline leg: the FP64 oracle outputs of the sampled
    heads of every rounding-bias variant."""
    import oracle
    cfg, qbits, variants = bias_inputs(c4_inputs)
    b, h, n, d = cfg.shape
    qf = synth.bf16_bits_to_f32(qbits).reshape(b * h, n, d)
    scale = oracle.default_scale(d)
    refs = {}
    for name, kbits, vbits in variants:
        kf = synth.bf16_bits_to_f32(kbits).reshape(b * h, n, d)
        vf = synth.bf16_bits_to_f32(vbits).reshape(b * h, n, d)

        def unit(u, kf=kf, vf=vf):
            return oracle.attention_head(qf[u], kf[u], vf[u], causal=True, scale=scale)[0]
        outs, _ = oracle.run_heads(unit, list(BIAS_UNITS), workers=workers)
        refs[name] = np.stack(outs)
    return refs


# ---------------------------------------------------------------------------
# legs
# ---------------------------------------------------------------------------

def bias_leg(pna, torch, refs, c4_inputs):
    """Rounding bias of standard versus stabilised FlashAttention: signed and
    absolute error against the FP64 references of the sampled heads, for P
    rounded to bf16 and P kept in fp32, with O stored in bf16 and in fp32 (the
    fp32 O leaves out the rounding of O itself, so what remains is the
    rounding upstream of it: P and the accumulation)."""
    cfg, qbits, variants = bias_inputs(c4_inputs)
    b, h, n, d = cfg.shape

    def dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    q = dev_bf16(qbits)
    out = {"workload": f"c4: {cfg.description}", "beta": BIAS_BETA, "units": list(BIAS_UNITS),
           "v_shift": BIAS_V_SHIFT}
    for name, kbits, vbits in variants:
        kt, vt = dev_bf16(kbits), dev_bf16(vbits)
        ref_t = torch.from_numpy(refs[name]).cuda()
        res = {}
        for o_f32 in (False, True):
            for p_bf16 in (True, False):
                row = {}
                for kind, bb in (("standard", None), ("stabilized", BIAS_BETA)):
                    o = pna.attn_fwd_flash(q, kt, vt, causal=True, p_bf16=p_bf16, beta=bb,
                                           out_f32=o_f32)
                    o_s = torch.stack([o.view(b * h, n, d)[u] for u in BIAS_UNITS]).contiguous()
                    dev = pna.attn_deviation(o_s, ref_t)
                    row[kind] = {key: dev[key] for key in ("mean_signed", "mean_abs", "max_abs",
                                                           "rms", "n_nonfinite")}
                res[("o_fp32_" if o_f32 else "o_bf16_") + ("p_bf16" if p_bf16 else "p_fp32")] = row
        out[name] = res
    return out


def workload_leg(pna, torch, cfg, inp, p_bf16, steps, kernel="flash", ref=None, units=None):
    """Time one workload (flash or baseline kernel) and compare its output on
    the reference units with the oracle."""
    q, k, v = to_device(inp)
    qs = ks = None
    if cfg.dtype == "int8":
        q, qs = pna.attn_quantize_int8(q)
        k, ks = pna.attn_quantize_int8(k)
    out = torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=v.dtype, device="cuda")
    if kernel == "flash":
        def fn():
            pna.attn_fwd_flash(q, k, v, causal=cfg.causal, p_bf16=p_bf16, q_scale=qs,
                               k_scale=ks, out=out)
    else:
        prob = pna.make_problem(q, causal=cfg.causal, p_bf16=p_bf16)
        ws = torch.empty(pna.attn_baseline_workspace_size(prob), dtype=torch.uint8,
                         device="cuda")

        def fn():
            pna.attn_fwd_baseline(q, k, v, causal=cfg.causal, p_bf16=p_bf16, q_scale=qs,
                                  k_scale=ks, workspace=ws, out=out)
    t = time_steps(fn, steps, 3, LEG_SETTLE_S, pna)
    flops = cfg.flops()
    qk = {"bf16": "bf16", "int8": "int8", "f32": "f32"}[cfg.dtype]
    pv = "bf16" if p_bf16 and cfg.dtype != "f32" else "f32"
    frac, peak = mixed_fraction(flops, t["ms"], qk, pv)
    leg = {"workload": f"{cfg.name}: {cfg.description}", "kernel": f"attn_fwd_{kernel}",
           "shape": list(cfg.shape), "causal": cfg.causal, "p_bf16": p_bf16,
           "ms": round(t["ms"], 5), "launch_ms": launch_stats(t),
           "shader_clock_mhz": t["shader_clock_mhz"],
           "tflops": round(flops / (t["ms"] * 1e-3) / 1e12, 2),
           "peak": round(peak, 1), "peak_engines": f"QK^T {qk}, P.V {pv}",
           "frac_of_peak": round(frac, 4)}
    if kernel == "baseline":
        n2 = cfg.batch * cfg.heads * cfg.seq_len * cfg.seq_len
        pbytes = 2 if p_bf16 else 4
        alg = n2 * (4 + 4 + pbytes + pbytes) + 4 * out.numel() * out.element_size()
        leg.update({"alg_bytes": alg, "GB_per_s": round(alg / (t["ms"] * 1e-3) / 1e9, 1),
                    "hbm_frac": round(alg / (t["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        del ws
    if ref is not None:
        b, h, n, d = cfg.shape
        o_s = torch.stack([out.view(b * h, n, d)[u] for u in units]).contiguous()
        leg.update(deviation_fields(pna, o_s, torch.from_numpy(ref).cuda()))
        leg["err_units"] = list(units)
    return leg


def copy_probe():
    """A plain device copy of known size, for scaling the FETCH_SIZE and
    WRITE_SIZE counters (read 256 MiB, write 256 MiB per launch)."""
    import torch
    src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_launch": src.numel() * 4}), flush=True)


LEG_NAMES = ("flash_c2", "baseline_c2", "flash_c4_pbf16", "flash_c4_pfp32", "flash_c5_int8",
             "baseline", "deviation", "wasserstein", "rounding_bias", "bwd_delta",
             "flash_backward", "flash_fp8", "quantize_int8")
C5_ERR_UNITS = (0, 77, 127)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3", choices=sorted(synth.CONFIGS))
    ap.add_argument("--p-fp32", action="store_true", help="keep P in fp32 (P*V on fp32 MFMA)")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of back-to-back steps before the warm-up steps")
    ap.add_argument("--cpu-units", type=int, default=128,
                    help="(batch, head) units in the oracle sample (0: skip the CPU leg)")
    ap.add_argument("--cpu-workers", type=int, default=HOST_CORE_SHARE)
    ap.add_argument("--no-legs", action="store_true", help="time the flash kernel only")
    ap.add_argument("--legs", default="all",
                    help="comma-separated legs to run after the flash kernel (default: all): "
                         + ",".join(LEG_NAMES))
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the kernels shard by (batch, head) with no exchange, so N GPUs would each run "
              "this one-GPU workload on their share", file=sys.stderr)
        sys.exit(2)

    import torch
    import precision_numerics_amd as pna

    if args.copy_probe:
        copy_probe()
        return
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    pna.load()
    legs_on = () if args.no_legs else (LEG_NAMES if args.legs == "all" else
                                       tuple(x for x in args.legs.split(",") if x))

    def want(name):
        return name in legs_on

    cfg = synth.CONFIGS[args.workload]
    p_bf16 = cfg.p_bf16 and not args.p_fp32
    log(f"bench: generating {cfg.name} inputs {cfg.shape}")
    inp = synth.make_inputs(cfg)
    q, k, v = to_device(inp)
    qs = ks = None
    if cfg.dtype == "int8":
        q, qs = pna.attn_quantize_int8(q)
        k, ks = pna.attn_quantize_int8(k)
    out = torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=v.dtype, device="cuda")
    torch.cuda.synchronize()

    def step():
        pna.attn_fwd_flash(q, k, v, causal=cfg.causal, p_bf16=p_bf16, q_scale=qs, k_scale=ks,
                           out=out)

    log(f"bench: timing flash ({args.settle} s settle, {args.warmup} warmup, "
        f"{args.steps} steps)")
    t = time_steps(step, args.steps, args.warmup, args.settle, pna)
    ms = t["ms"]
    flops = cfg.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    qk = {"bf16": "bf16", "int8": "int8", "f32": "f32"}[cfg.dtype]
    pv = "bf16" if p_bf16 and cfg.dtype != "f32" else "f32"
    frac, peak = mixed_fraction(flops, ms, qk, pv)
    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "int8": "int8+bf16"}[cfg.dtype],
        "data": "synthetic (seeded numpy PCG64 draws, see synth)",
        "config": {"workload": f"{cfg.name}: {cfg.description}", "batch": cfg.batch,
                   "heads": cfg.heads, "seq_len": cfg.seq_len, "head_dim": cfg.head_dim,
                   "causal": cfg.causal, "p_bf16": p_bf16, "kernel": "attn_fwd_flash"},
        "pct_peak": round(100 * frac, 2),
        "launch_ms": launch_stats(t),
        "shader_clock_mhz": t["shader_clock_mhz"],
        "settle": {"seconds": args.settle, "calls": t["settle_calls"]},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(frac, 4),
                     "traffic": measured_traffic(args.workload),
                     "peak_dtype": "bf16" if (qk, pv) == ("bf16", "bf16") else f"{qk}+{pv}",
                     "flops_per_launch": flops},
        "host": host_info(),
    }
    nonfinite = 0

    # ---- the oracle on the host cores (the CPU baseline), the flash
    # deviation from it, and the oracle references of the other legs
    refs = {}
    c4_inputs = None
    if want("rounding_bias") or want("flash_c4_pbf16") or want("flash_c4_pfp32"):
        log("bench: generating c4 inputs")
        c4_inputs = synth.make_inputs(synth.CONFIGS["c4"])
    if args.cpu_units > 0:
        b, h = cfg.batch, cfg.heads
        units = list(range(min(args.cpu_units, b * h)))
        workers = max(1, min(args.cpu_workers, len(os.sched_getaffinity(0))))
        log(f"bench: FP64 oracle on {len(units)} units, {workers} workers")
        ref, cpu = cpu_baseline(cfg, inp, units, workers)
        o_s = out.view(b * h, cfg.seq_len, cfg.head_dim)[units[0]:units[-1] + 1].contiguous()
        ref_t = torch.from_numpy(ref).cuda()
        fields = deviation_fields(pna, o_s, ref_t)
        nonfinite += fields["n_nonfinite"]
        result.update(fields)
        result["err_sample"] = f"{len(units)} (batch, head) units"
        result["cpu_baseline"] = {k2: cpu[k2] for k2 in ("value", "unit", "cores", "kind",
                                                          "sample")}
        result["cpu_baseline"]["seconds"] = round(cpu["seconds"], 3)
        result["cpu_baseline"]["host_cores"] = result["host"]["affinity_cores"]
        result["cpu_baseline"]["note"] = (f"process pool capped at {HOST_CORE_SHARE}, the "
                                          "host's CPU share for one GPU")
        result["gpu_over_cpu"] = round(tflops / cpu["value"], 1)
        log("bench: FP64 oracle references for the other legs")
        if want("flash_c2") or want("baseline_c2"):
            c2 = synth.CONFIGS["c2"]
            in2 = synth.make_inputs(c2)
            u2 = list(range(c2.batch * c2.heads))
            refs["c2"] = (in2, u2, oracle_refs(c2, in2, u2, workers))
        if want("flash_c5_int8"):
            c5 = synth.CONFIGS["c5"]
            in5 = synth.make_inputs(c5)
            refs["c5"] = (in5, list(C5_ERR_UNITS), oracle_refs(c5, in5, C5_ERR_UNITS, workers))
        if c4_inputs is not None:
            refs["bias"] = cpu_baseline_bias_refs(c4_inputs, workers)
    else:
        result["cpu_baseline"] = None
        ref_t = None

    # ---- other kernels and workloads of the path, each timed alone
    legs = {}

    def run_leg(name, fn):
        if not want(name):
            return
        log(f"bench: leg {name}")
        try:
            legs[name] = fn()
        except Exception as exc:                         # noqa: BLE001
            legs[name] = {"error": repr(exc)}

    c2 = synth.CONFIGS["c2"]
    r2 = refs.get("c2")
    run_leg("flash_c2", lambda: workload_leg(
        pna, torch, c2, r2[0] if r2 else synth.make_inputs(c2), True, 200,
        ref=r2[2] if r2 else None, units=r2[1] if r2 else None))
    run_leg("baseline_c2", lambda: workload_leg(
        pna, torch, c2, r2[0] if r2 else synth.make_inputs(c2), True, 20, kernel="baseline",
        ref=r2[2] if r2 else None, units=r2[1] if r2 else None))
    c4 = synth.CONFIGS["c4"]
    r4 = refs.get("bias", {}).get("v")
    run_leg("flash_c4_pbf16", lambda: workload_leg(
        pna, torch, c4, c4_inputs, True, 20, ref=r4, units=BIAS_UNITS))
    run_leg("flash_c4_pfp32", lambda: workload_leg(
        pna, torch, c4, c4_inputs, False, 5, ref=r4, units=BIAS_UNITS))
    c5 = synth.CONFIGS["c5"]
    r5 = refs.get("c5")
    run_leg("flash_c5_int8", lambda: workload_leg(
        pna, torch, c5, r5[0] if r5 else synth.make_inputs(c5), True, 100,
        ref=r5[2] if r5 else None, units=r5[1] if r5 else None))

    def baseline_c3():
        leg = workload_leg(pna, torch, cfg, inp, p_bf16, 5, kernel="baseline",
                           ref=ref if ref_t is not None else None,
                           units=units if ref_t is not None else None)
        return leg
    run_leg("baseline", baseline_c3)

    o_s = (out.view(cfg.batch * cfg.heads, cfg.seq_len, cfg.head_dim)[
        units[0]:units[-1] + 1].contiguous() if ref_t is not None else None)

    def deviation_leg():
        scratch = torch.empty(pna.attn_deviation_scratch_size(ref_t.numel()),
                              dtype=torch.uint8, device="cuda")
        tt = time_steps(lambda: pna.attn_deviation(o_s, ref_t, scratch=scratch), 5, 1, 0, pna)
        nb = o_s.numel() * (o_s.element_size() + 8)
        return {"ms": round(tt["ms"], 3), "alg_bytes": nb,
                "GB_per_s": round(nb / (tt["ms"] * 1e-3) / 1e9, 1),
                "note": "includes the host synchronisation per call"}
    if ref_t is not None:
        run_leg("deviation", deviation_leg)

    def wasserstein_leg():
        ws_b = torch.empty(pna.attn_wasserstein_scratch_size(
            ref_t.numel(), pna.ATTN_BF16 if o_s.dtype == torch.bfloat16 else pna.ATTN_F32,
            pna.ATTN_F64), dtype=torch.uint8, device="cuda")
        wf = pna.attn_wasserstein(o_s, ref_t, scratch=ws_b)
        tt = time_steps(lambda: pna.attn_wasserstein(o_s, ref_t, scratch=ws_b), 3, 1, 0, pna)
        leg = {"flash_vs_fp64": {k2: wf[k2] for k2 in ("w1", "w2", "winf", "n_nonfinite")},
               "ms": round(tt["ms"], 3), "n": wf["n"],
               "note": "one call sorts both inputs on the GPU; includes the host "
                       "synchronisation"}
        ob = torch.empty_like(out)
        pna.attn_fwd_baseline(q, k, v, causal=cfg.causal, p_bf16=p_bf16, q_scale=qs,
                              k_scale=ks, out=ob)
        ob_s = ob.view(cfg.batch * cfg.heads, cfg.seq_len, cfg.head_dim)[
            units[0]:units[-1] + 1].contiguous()
        wb = pna.attn_wasserstein(ob_s, ref_t, scratch=ws_b)
        wfb = pna.attn_wasserstein(o_s, ob_s)
        leg["baseline_vs_fp64"] = {k2: wb[k2] for k2 in ("w1", "w2", "winf", "n_nonfinite")}
        leg["flash_vs_baseline"] = {k2: wfb[k2] for k2 in ("w1", "w2", "winf", "n_nonfinite")}
        return leg
    if ref_t is not None and cfg.dtype == "bf16":
        run_leg("wasserstein", wasserstein_leg)
    if "bias" in refs:
        run_leg("rounding_bias", lambda: bias_leg(pna, torch, refs["bias"], c4_inputs))

    def delta_leg():
        g = torch.randn(out.shape, device="cuda").to(out.dtype)
        dl = torch.empty(out.shape[:-1], dtype=torch.float32, device="cuda")
        tt = time_steps(lambda: pna.attn_bwd_delta(out, g, delta=dl), 20, 3, 0, pna)
        nb = 2 * out.numel() * out.element_size() + dl.numel() * 4
        return {"ms": round(tt["ms"], 4), "alg_bytes": nb,
                "GB_per_s": round(nb / (tt["ms"] * 1e-3) / 1e9, 1),
                "hbm_frac": round(nb / (tt["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    run_leg("bwd_delta", delta_leg)

    def backward_leg():
        lse_b = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
        pna.attn_fwd_flash(q, k, v, causal=cfg.causal, out=out, lse=lse_b)
        g_b = torch.randn(out.shape, device="cuda").to(out.dtype)
        dq_b, dk_b, dv_b = (torch.empty_like(x) for x in (q, k, v))
        wsb = torch.empty(pna.attn_bwd_workspace_size(pna.make_problem(q, causal=cfg.causal)),
                          dtype=torch.uint8, device="cuda")
        tt = time_steps(lambda: pna.attn_bwd_flash(
            q, k, v, out, g_b, lse_b, causal=cfg.causal, dq=dq_b, dk=dk_b, dv=dv_b,
            workspace=wsb), 5, 1, LEG_SETTLE_S, pna)
        # the usual accounting: five matrix products against the forward's two
        bflops = 2.5 * flops
        return {"ms": round(tt["ms"], 3), "launch_ms": launch_stats(tt),
                "tflops": round(bflops / (tt["ms"] * 1e-3) / 1e12, 2),
                "frac_of_bf16_peak": round(bflops / (tt["ms"] * 1e-3) / 1e12 / PEAK["bf16"], 4),
                "note": "2.5x the forward's flops; includes the delta kernel"}
    if cfg.dtype == "bf16":
        run_leg("flash_backward", backward_leg)

    def fp8_leg():
        c5c = synth.CONFIGS["c5"]
        in5 = synth.make_inputs(c5c)
        q8, qs8 = pna.attn_quantize_fp8(torch.from_numpy(in5.q).cuda())
        k8, ks8 = pna.attn_quantize_fp8(torch.from_numpy(in5.k).cuda())
        v8 = to_device(in5)[2]
        o8 = torch.empty(q8.shape, dtype=torch.bfloat16, device="cuda")
        tt = time_steps(lambda: pna.attn_fwd_flash(q8, k8, v8, causal=c5c.causal, q_scale=qs8,
                                                   k_scale=ks8, out=o8), 50, 3, LEG_SETTLE_S,
                        pna)
        f5 = c5c.flops()
        fr, pk = mixed_fraction(f5, tt["ms"], "fp8", "bf16")
        return {"workload": f"{c5c.name} shape with E4M3 Q/K", "ms": round(tt["ms"], 4),
                "launch_ms": launch_stats(tt), "tflops": round(f5 / (tt["ms"] * 1e-3) / 1e12, 2),
                "peak": round(pk, 1), "frac_of_fp8_bf16_peak": round(fr, 4)}
    run_leg("flash_fp8", fp8_leg)

    def quant_leg():
        x = torch.randn(cfg.batch * cfg.heads * cfg.seq_len, cfg.head_dim, device="cuda")
        codes = torch.empty(x.shape, dtype=torch.int8, device="cuda")
        scales = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
        tt = time_steps(lambda: pna.attn_quantize_int8(x, codes=codes, scales=scales), 10, 2,
                        0, pna)
        nb = x.numel() * 5 + x.shape[0] * 4
        return {"ms": round(tt["ms"], 4), "alg_bytes": nb,
                "GB_per_s": round(nb / (tt["ms"] * 1e-3) / 1e9, 1)}
    run_leg("quantize_int8", quant_leg)

    for leg in legs.values():
        if isinstance(leg, dict):
            nonfinite += int(leg.get("n_nonfinite", 0) or 0)
    if legs_on:
        result["legs"] = legs
    result["n_nonfinite_total"] = nonfinite
    print(json.dumps(result), flush=True)
    if nonfinite > 0:
        log(f"bench: {nonfinite} non-finite output elements against the oracle")
        sys.exit(3)


if __name__ == "__main__":
    main()
