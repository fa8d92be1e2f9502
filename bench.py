"""Benchmark of the FlashAttention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

A step is one FlashAttention forward (attn_fwd_flash through the C ABI) over
the workload's inputs, already resident in HBM.  The default workload is the
Llama-2-7B-shaped causal bf16 forward (batch 4, 32 heads, seq 4096, d 128,
P rounded to bf16).  Prints ONE JSON line with:

  value / unit      attention-forward TFLOP/s (MFMA contraction flops over
                    visible (query, key) pairs / average step time)
  roofline          the flash kernel against the bf16 MFMA dense peak
  max_abs_err ...   deviation of the flash output from the FP64 oracle on the
                    oracle's sample
  cpu_baseline      the FP64 oracle on the host cores, on a bounded sample
  legs              the other kernels of the path (baseline attention,
                    deviation reduction, int8 quantiser), each timed alone
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


# HBM bytes per launch of the flash kernel on c3, from two rocprofv3 --pmc
# passes (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch).  A plain 256 MiB
# device copy reads FETCH_SIZE = 131085 KiB and WRITE_SIZE = 262144 KiB, so
# FETCH_SIZE is scaled by 2 and WRITE_SIZE by 1.  The figure is valid only for
# the kernel sources it was taken on (sha256 of the files below).
TRAFFIC_SOURCES = ("precision_numerics_amd/csrc/flash_fwd.hip",
                   "precision_numerics_amd/csrc/device.hpp",
                   "precision_numerics_amd/csrc/launch.hpp",
                   "precision_numerics_amd/csrc/lds_dma.hpp")
TRAFFIC = {
    "workload": "c3",
    "sources_sha256": "2af279e559c79fe423a1f6590c67874f50e5e285474e9708ab0e1d8a64ce1f8c",
    "fetch_kib": 301626.7, "fetch_scale": 2.0,
    "write_kib": 138754.2, "write_scale": 1.0,
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


def event_time_ms(fn, steps, warmup):
    """Average ms per call of fn() from HIP events on torch's current stream
    (the stream every entry point is launched on)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


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


def cpu_baseline(cfg, inp, units, workers):
    """The FP64 oracle (as it stands) on the listed (batch, head) units, run in
    a process pool on the host cores.  Returns (oracle O [units, N, d], stats)."""
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
    t0 = time.perf_counter()
    outs, used = oracle.run_heads(unit, units, workers=workers)
    wall = time.perf_counter() - t0
    flops = cfg.scaled(batch=1, heads=len(units)).flops()
    stats = {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
             "sample": f"{len(units)} of {b * h} (batch, head) units of {cfg.name}, all "
                       f"{n} query rows each; FP64 numpy/OpenBLAS, one BLAS thread per worker",
             "seconds": wall, "flops": flops}
    return np.stack(outs), stats


BIAS_BETA = 2.0
BIAS_UNITS = (0, 31)
BIAS_V_SHIFT = -2.0


def bias_inputs():
    """Inputs of the rounding-bias leg: the rank-4 long-sequence workload with
    V as drawn, V shifted to a negative mean (most columns of V negative, the
    situation the low-precision training page's Figure 5 examines), and that
    with the key rows duplicated in pairs (every token appears twice, so each
    row maximum is repeated).  Returns (cfg, q bits, [(name, k bits, v bits)])."""
    cfg = synth.CONFIGS["c4"]
    b, h, n, d = cfg.shape
    inp = synth.make_inputs(cfg)
    v_neg = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(inp.v) + np.float32(BIAS_V_SHIFT))
    k_pair = inp.k.reshape(b, h, n // 2, 2, d)[:, :, :, :1, :].repeat(2, axis=3)
    k_pair = np.ascontiguousarray(k_pair.reshape(b, h, n, d))
    return cfg, inp.q, [("v", inp.k, inp.v), ("v_shifted", inp.k, v_neg),
                        ("v_shifted_keys_paired", k_pair, v_neg)]


def cpu_baseline_bias_refs(workers):
    """Part of the CPU-baseline leg: the FP64 oracle outputs of the sampled
    heads of every rounding-bias variant."""
    import oracle
    cfg, qbits, variants = bias_inputs()
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


def bias_leg(pna, torch, refs):
    """Rounding bias of standard versus stabilised FlashAttention: signed and
    absolute error against the FP64 references of the sampled heads, for P
    rounded to bf16 and P kept in fp32."""
    cfg, qbits, variants = bias_inputs()
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
        for p_bf16 in (True, False):
            row = {}
            for kind, bb in (("standard", None), ("stabilized", BIAS_BETA)):
                o = pna.attn_fwd_flash(q, kt, vt, causal=True, p_bf16=p_bf16, beta=bb)
                o_s = torch.stack([o.view(b * h, n, d)[u] for u in BIAS_UNITS]).contiguous()
                dev = pna.attn_deviation(o_s, ref_t)
                row[kind] = {key: dev[key] for key in ("mean_signed", "mean_abs", "max_abs",
                                                       "rms")}
            res["p_bf16" if p_bf16 else "p_fp32"] = row
        out[name] = res
    return out


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3", choices=sorted(synth.CONFIGS))
    ap.add_argument("--p-fp32", action="store_true", help="keep P in fp32 (P*V on fp32 MFMA)")
    ap.add_argument("--cpu-units", type=int, default=128,
                    help="(batch, head) units in the oracle sample (0: skip the CPU leg)")
    ap.add_argument("--cpu-workers", type=int, default=16)
    ap.add_argument("--no-legs", action="store_true", help="time the flash kernel only")
    ap.add_argument("--legs", default="all",
                    help="comma-separated legs to run after the flash kernel (default: all)")
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

    log(f"bench: timing flash ({args.warmup} warmup, {args.steps} steps)")
    ms = event_time_ms(step, args.steps, args.warmup)
    flops = cfg.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    if cfg.dtype == "int8":
        # int8 QK^T at the int8 peak, P*V at the bf16 (or fp32) peak
        half = flops / 2
        ideal_ms = (half / (PEAK["int8"] * 1e12) +
                    half / (PEAK["bf16" if p_bf16 else "f32"] * 1e12)) * 1e3
        frac = ideal_ms / ms
        peak = flops / (ideal_ms * 1e-3) / 1e12
        bound_dtype = "int8+bf16"
    elif cfg.dtype == "f32" or not p_bf16:
        half = flops / 2
        qk_peak = PEAK["f32"] if cfg.dtype == "f32" else PEAK["bf16"]
        ideal_ms = (half / (qk_peak * 1e12) + half / (PEAK["f32"] * 1e12)) * 1e3
        frac = ideal_ms / ms
        peak = flops / (ideal_ms * 1e-3) / 1e12
        bound_dtype = "mixed"
    else:
        peak = PEAK["bf16"]
        frac = tflops / peak
        bound_dtype = "bf16"
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
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(frac, 4),
                     "traffic": measured_traffic(args.workload),
                     "peak_dtype": bound_dtype,
                     "flops_per_launch": flops},
    }

    # ---- the oracle on the host cores, and the flash deviation from it
    if args.cpu_units > 0:
        b, h = cfg.batch, cfg.heads
        units = list(range(min(args.cpu_units, b * h)))
        workers = min(args.cpu_workers, len(os.sched_getaffinity(0)))
        log(f"bench: FP64 oracle on {len(units)} units, {workers} workers")
        ref, cpu = cpu_baseline(cfg, inp, units, workers)
        o_s = out.view(b * h, cfg.seq_len, cfg.head_dim)[units[0]:units[-1] + 1].contiguous()
        dev = pna.attn_deviation(o_s, torch.from_numpy(ref).cuda())
        result["max_abs_err"] = dev["max_abs"]
        result["mean_abs_err"] = dev["mean_abs"]
        result["mean_signed_err"] = dev["mean_signed"]
        result["err_sample"] = f"{len(units)} (batch, head) units"
        result["cpu_baseline"] = {k2: cpu[k2] for k2 in ("value", "unit", "cores", "kind",
                                                          "sample")}
        result["cpu_baseline"]["seconds"] = round(cpu["seconds"], 3)
        result["gpu_over_cpu"] = round(tflops / cpu["value"], 1)
        ref_t = torch.from_numpy(ref).cuda()
        bias_refs = None
        if not args.no_legs and (args.legs == "all" or "rounding_bias" in args.legs.split(",")):
            log("bench: FP64 oracle references for the rounding-bias leg")
            bias_refs = cpu_baseline_bias_refs(workers)
    else:
        result["cpu_baseline"] = None
        ref_t = None
        bias_refs = None

    # ---- other kernels of the path, each timed alone
    if not args.no_legs:
        legs = {}
        ob_s = None

        def want(name):
            return args.legs == "all" or name in args.legs.split(",")
        try:
            if not want("baseline"):
                raise LookupError
            log("bench: baseline attention leg")
            prob = pna.make_problem(q, causal=cfg.causal, p_bf16=p_bf16)
            ws = torch.empty(pna.attn_baseline_workspace_size(prob), dtype=torch.uint8,
                             device="cuda")
            ob = torch.empty_like(out)

            def base():
                pna.attn_fwd_baseline(q, k, v, causal=cfg.causal, p_bf16=p_bf16, q_scale=qs,
                                      k_scale=ks, workspace=ws, out=ob)
            bms = event_time_ms(base, 3, 1)
            n2 = cfg.batch * cfg.heads * cfg.seq_len * cfg.seq_len
            pbytes = 2 if p_bf16 else 4
            alg = n2 * (4 + 4 + pbytes + pbytes) + 4 * out.numel() * out.element_size()
            legs["baseline"] = {"ms": round(bms, 3), "alg_bytes": alg,
                                "GB_per_s": round(alg / (bms * 1e-3) / 1e9, 1),
                                "hbm_frac": round(alg / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                "tflops": round(flops / (bms * 1e-3) / 1e12, 2)}
            if ref_t is not None:
                ob_s = ob.view(cfg.batch * cfg.heads, cfg.seq_len, cfg.head_dim)[
                    units[0]:units[-1] + 1].contiguous()
                dvb = pna.attn_deviation(ob_s, ref_t)
                legs["baseline"]["max_abs_err"] = dvb["max_abs"]
                legs["baseline"]["mean_abs_err"] = dvb["mean_abs"]
            del ws
        except LookupError:
            pass
        except Exception as exc:                         # noqa: BLE001
            legs["baseline"] = {"error": repr(exc)}
        if ref_t is not None and want("deviation"):
            try:
                log("bench: deviation leg")
                scratch = torch.empty(pna.attn_deviation_scratch_size(ref_t.numel()),
                                      dtype=torch.uint8, device="cuda")
                dms = event_time_ms(lambda: pna.attn_deviation(o_s, ref_t, scratch=scratch), 5, 1)
                nb = o_s.numel() * (o_s.element_size() + 8)
                legs["deviation"] = {"ms": round(dms, 3), "alg_bytes": nb,
                                     "GB_per_s": round(nb / (dms * 1e-3) / 1e9, 1),
                                     "note": "includes the host synchronisation per call"}
            except Exception as exc:                     # noqa: BLE001
                legs["deviation"] = {"error": repr(exc)}
        if ref_t is not None and want("wasserstein"):
            try:
                log("bench: Wasserstein leg")
                ws_b = torch.empty(pna.attn_wasserstein_scratch_size(
                    ref_t.numel(), pna.ATTN_BF16 if o_s.dtype == torch.bfloat16 else pna.ATTN_F32,
                    pna.ATTN_F64), dtype=torch.uint8, device="cuda")
                wf = pna.attn_wasserstein(o_s, ref_t, scratch=ws_b)
                wms = event_time_ms(lambda: pna.attn_wasserstein(o_s, ref_t, scratch=ws_b), 3, 1)
                leg = {"flash_vs_fp64": {k2: wf[k2] for k2 in ("w1", "w2", "winf")},
                       "ms": round(wms, 3), "n": wf["n"],
                       "note": "one call sorts both inputs on the GPU; includes the host "
                               "synchronisation"}
                if ob_s is not None:
                    wb = pna.attn_wasserstein(ob_s, ref_t, scratch=ws_b)
                    wfb = pna.attn_wasserstein(o_s, ob_s)
                    leg["baseline_vs_fp64"] = {k2: wb[k2] for k2 in ("w1", "w2", "winf")}
                    leg["flash_vs_baseline"] = {k2: wfb[k2] for k2 in ("w1", "w2", "winf")}
                legs["wasserstein"] = leg
                del ws_b
            except Exception as exc:                     # noqa: BLE001
                legs["wasserstein"] = {"error": repr(exc)}
        if bias_refs is not None and want("rounding_bias"):
            try:
                log("bench: rounding-bias leg (c4, standard vs stabilised)")
                legs["rounding_bias"] = bias_leg(pna, torch, bias_refs)
            except Exception as exc:                     # noqa: BLE001
                legs["rounding_bias"] = {"error": repr(exc)}
        try:
            if not want("bwd_delta"):
                raise LookupError
            log("bench: delta = rowsum(dO * O) leg")
            g = torch.randn(out.shape, device="cuda").to(out.dtype)
            dl = torch.empty(out.shape[:-1], dtype=torch.float32, device="cuda")
            dms = event_time_ms(lambda: pna.attn_bwd_delta(out, g, delta=dl), 20, 3)
            nb = 2 * out.numel() * out.element_size() + dl.numel() * 4
            legs["bwd_delta"] = {"ms": round(dms, 4), "alg_bytes": nb,
                                 "GB_per_s": round(nb / (dms * 1e-3) / 1e9, 1),
                                 "hbm_frac": round(nb / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        except LookupError:
            pass
        except Exception as exc:                         # noqa: BLE001
            legs["bwd_delta"] = {"error": repr(exc)}
        if cfg.dtype == "bf16" and want("flash_backward"):
            try:
                log("bench: flash backward leg")
                lse_b = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
                pna.attn_fwd_flash(q, k, v, causal=cfg.causal, out=out, lse=lse_b)
                g_b = torch.randn(out.shape, device="cuda").to(out.dtype)
                dq_b, dk_b, dv_b = (torch.empty_like(x) for x in (q, k, v))
                wsb = torch.empty(pna.attn_bwd_workspace_size(pna.make_problem(q, causal=cfg.causal)),
                                  dtype=torch.uint8, device="cuda")
                bwd_ms = event_time_ms(lambda: pna.attn_bwd_flash(
                    q, k, v, out, g_b, lse_b, causal=cfg.causal, dq=dq_b, dk=dk_b, dv=dv_b,
                    workspace=wsb), 5, 1)
                # the usual accounting: five matrix products against the forward's two
                bflops = 2.5 * flops
                legs["flash_backward"] = {"ms": round(bwd_ms, 3),
                                          "tflops": round(bflops / (bwd_ms * 1e-3) / 1e12, 2),
                                          "frac_of_bf16_peak": round(
                                              bflops / (bwd_ms * 1e-3) / 1e12 / PEAK["bf16"], 4),
                                          "note": "2.5x the forward's flops; includes the delta "
                                                  "kernel"}
                del dq_b, dk_b, dv_b, wsb, g_b
            except Exception as exc:                     # noqa: BLE001
                legs["flash_backward"] = {"error": repr(exc)}
        try:
            if not want("flash_fp8"):
                raise LookupError
            log("bench: fp8 (E4M3) Q/K flash leg on the int8 workload's shape")
            c5 = synth.CONFIGS["c5"]
            in5 = synth.make_inputs(c5)
            q8, qs8 = pna.attn_quantize_fp8(torch.from_numpy(in5.q).cuda())
            k8, ks8 = pna.attn_quantize_fp8(torch.from_numpy(in5.k).cuda())
            v8 = to_device(in5)[2]
            o8 = torch.empty(q8.shape, dtype=torch.bfloat16, device="cuda")
            fms = event_time_ms(lambda: pna.attn_fwd_flash(q8, k8, v8, causal=c5.causal,
                                                           q_scale=qs8, k_scale=ks8, out=o8),
                                20, 3)
            f5 = c5.flops()
            # QK^T at the fp8 peak, P*V at the bf16 peak
            ideal = (f5 / 2 / (PEAK["fp8"] * 1e12) + f5 / 2 / (PEAK["bf16"] * 1e12)) * 1e3
            legs["flash_fp8"] = {"workload": f"{c5.name} shape with E4M3 Q/K", "ms": round(fms, 4),
                                 "tflops": round(f5 / (fms * 1e-3) / 1e12, 2),
                                 "frac_of_fp8_bf16_peak": round(ideal / fms, 4)}
            del q8, k8, v8, o8, in5
        except LookupError:
            pass
        except Exception as exc:                         # noqa: BLE001
            legs["flash_fp8"] = {"error": repr(exc)}
        try:
            if not want("quantize_int8"):
                raise LookupError
            log("bench: int8 quantiser leg")
            x = torch.randn(cfg.batch * cfg.heads * cfg.seq_len, cfg.head_dim, device="cuda")
            codes = torch.empty(x.shape, dtype=torch.int8, device="cuda")
            scales = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
            qms = event_time_ms(lambda: pna.attn_quantize_int8(x, codes=codes, scales=scales),
                                10, 2)
            nb = x.numel() * 5 + x.shape[0] * 4
            legs["quantize_int8"] = {"ms": round(qms, 4), "alg_bytes": nb,
                                     "GB_per_s": round(nb / (qms * 1e-3) / 1e9, 1)}
        except LookupError:
            pass
        except Exception as exc:                         # noqa: BLE001
            legs["quantize_int8"] = {"error": repr(exc)}
        result["legs"] = legs

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
