#!/usr/bin/env python3
"""Benchmark of one Beam mixture-of-experts layer on one MI355X.

A step is one ``beam_moe_forward`` call (router -> permutation -> gate/up -> down ->
combine) over one batch of synthetic, seeded tokens already resident in HBM.  The primary
line is the 8192-token prefill layer; the same run also times the 64-token decode layer
(``secondary``).  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload prefill_t8192]
  python bench.py --sweep 16,64,256,1024 [--sweep-md table.md]   # serving shapes, one line per size
  python bench.py --copy-calib 1024      # plain 1 GiB device copy (HBM counter calibration)
  python bench.py --workload W --ingest-pmc FETCH.csv WRITE.csv CALIB_FETCH.csv CALIB_WRITE.csv 1024
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at 1 MI355X (prefill 8192 / decode 64); % MFMA / HBM roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
EXPERTS_SRC = os.path.join(ROOT, "sparse_moe_layer_04_amd", "csrc", "experts.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(text=None) -> str:
    """Hash of the expert-GEMM source with its comments and blank space removed, so that a
    change to the comments alone keeps recorded counter traffic valid."""
    import re
    if text is None:
        with open(EXPERTS_SRC) as f:
            text = f.read()
    code = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    code = re.sub(r"//[^\n]*", " ", code)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def weight_bytes_per_element(cfg):
    """bf16: 2; 8-bit storage: 1 byte per code plus one scale byte per 32 elements; MXFP4:
    half a byte per code plus the scale byte per 32."""
    return {"fp8": 1.0 + 1.0 / 32, "mxfp4": 0.5 + 1.0 / 32}.get(cfg.weights, 2.0)


def gate_up_work(cfg, n_touched):
    """Algorithmic flops and bytes of one gate/up launch.

    flops: 4*H*I per routed pair (gate and up products).
    bytes: each touched expert's gate and up matrices once (2*I*H weights), each token row
    once (H bf16), each h row written once (I bf16)."""
    P = cfg.T * cfg.top_k
    flops = 4.0 * cfg.H * cfg.I * P
    nbytes = n_touched * 2.0 * cfg.I * cfg.H * weight_bytes_per_element(cfg) + cfg.T * cfg.H * 2.0 + P * cfg.I * 2.0
    return flops, nbytes


def down_work(cfg, n_touched):
    """flops 2*H*I per pair; bytes: each touched W_d once, each h row read, each output row written."""
    P = cfg.T * cfg.top_k
    return (2.0 * cfg.H * cfg.I * P,
            n_touched * cfg.H * cfg.I * weight_bytes_per_element(cfg) + P * (cfg.I + cfg.H) * 2.0)


def roofline(flops, nbytes, seconds, traffic=None):
    t_f = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_b = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_f >= t_b:
        ach = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_BF16_TFLOPS, "traffic": traffic}
    ach = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
            "traffic": traffic}


def load_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` ("gate_up" or "down") from the committed counter runs,
    or None when the kernel source changed since they were taken."""
    try:
        with open(TRAFFIC_JSON) as f:
            d = json.load(f)
        ent = d[workload]
        if ent.get("experts_hip_code_sha256_16") != kernel_source_hash():
            return None
        k = ent[kernel]
        return {"fetch_bytes": k["fetch_bytes"], "write_bytes": k["write_bytes"],
                "bytes": k["fetch_bytes"] + k["write_bytes"], "source": os.path.relpath(TRAFFIC_JSON, ROOT)}
    except (OSError, KeyError, ValueError, TypeError):
        return None


# expert GEMM kernels (the decode kernel or the line-streaming kernel) by their GATED template flag
KERNEL_NAMES = {"gate_up": "<true", "down": "<false"}


def _counter_means(path, counter):
    """Mean value of `counter` per dispatch, keyed by kernel name, from a rocprofv3 --pmc csv."""
    import csv
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def ingest_counters(workload, fetch_csv, write_csv, calib_fetch_csv, calib_write_csv, calib_mib):
    """Record HBM traffic per launch of the expert GEMMs into profiles/traffic.json.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the same counters read
    for a plain device copy of calib_mib MiB (the largest kernel in the calibration runs)."""
    n = calib_mib * 2 ** 20
    cf = max(_counter_means(calib_fetch_csv, "FETCH_SIZE").values()) * 1024.0
    cw = max(_counter_means(calib_write_csv, "WRITE_SIZE").values()) * 1024.0
    f_fetch, f_write = n / cf, n / cw
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    ent = {"experts_hip_code_sha256_16": kernel_source_hash(),
           "calibration": {"copy_bytes": n, "fetch_factor": f_fetch, "write_factor": f_write}}
    for key, name in KERNEL_NAMES.items():
        kf = [v for k, v in fetch.items() if "moe_gemm" in k and name in k]
        kw = [v for k, v in write.items() if "moe_gemm" in k and name in k]
        if kf and kw:
            ent[key] = {"fetch_bytes": kf[0] * 1024.0 * f_fetch, "write_bytes": kw[0] * 1024.0 * f_write,
                        "fetch_kib_raw": kf[0], "write_kib_raw": kw[0]}
    try:
        with open(TRAFFIC_JSON) as f:
            d = json.load(f)
    except (OSError, ValueError):
        d = {}
    d[workload] = ent
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({workload: ent}))


def run_workload(cfg, hw, dw, steps, warmup, scales=None):
    """Times `steps` layers of workload `cfg` (weights hw on the host, dw on the device; for
    8-bit weights `scales` = (host scales, device scales))."""
    import numpy as np
    import torch

    import sparse_moe_layer_04_amd as bm
    from synth.configs import make_inputs

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    inp = make_inputs(cfg, weights=hw, w_scales=scales[0] if scales else None)
    shape = bm.make_shape(cfg.T, cfg.H, cfg.E, cfg.I, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho, cfg.dtype)
    op = bm.OP_FORWARD_SUBLAYER if cfg.sublayer else bm.OP_FORWARD
    ws = torch.empty(bm.workspace_size(shape, op), dtype=torch.uint8, device="cuda")
    x, bias = dev(inp.x), dev(inp.bias)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device="cuda")
    sub = None
    if cfg.sublayer:
        g1, g2 = dev(inp.pre_gain), dev(inp.post_gain)
        sub = bm.sublayer(g1, g2, cfg.eps, cfg.residual_k)
    timers = [bm.StageTimer() for _ in range(steps)]

    def step(timer=None):
        bm.forward(shape, x, dw[0], bias, dw[1], dw[2], dw[3], out, ws, sublayer=sub, topk_idx=idx,
                   stage_events=timer.events if timer else None, w_scales=scales[1] if scales else None,
                   w_format=cfg.code_format or "e4m3")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(steps):
        step(timers[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / steps
    stage = np.array([t.elapsed_ms() for t in timers]).mean(axis=0)
    for t in timers:
        t.close()
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=cfg.E)
    n_touched = int((counts > 0).sum())
    return dict(ms_per_step=ms_per_step, wall_s=wall, stage_ms=stage, counts=counts, n_touched=n_touched)


def summarize(cfg, r, steps, warmup):
    ms = r["ms_per_step"]
    P = cfg.T * cfg.top_k
    gu_ms = float(r["stage_ms"][4])
    dn_ms = float(r["stage_ms"][5])
    gu_f, gu_b = gate_up_work(cfg, r["n_touched"])
    dn_f, dn_b = down_work(cfg, r["n_touched"])
    layer_flops = 6.0 * cfg.H * cfg.I * P
    weight_bytes = r["n_touched"] * 3.0 * cfg.H * cfg.I * weight_bytes_per_element(cfg)
    layer_bytes = weight_bytes + cfg.E * cfg.H * 4.0 + 2.0 * cfg.T * cfg.H * 2
    import sparse_moe_layer_04_amd as bm
    return {
        "tokens_per_s": cfg.T / (ms / 1e3),
        "ms_per_step": ms,
        "stages_ms": {n: round(float(v), 4) for n, v in zip(bm.STAGE_NAMES, r["stage_ms"])},
        "layer": {"tflops": layer_flops / (ms / 1e3) / 1e12, "mfma_frac": layer_flops / (ms / 1e3) / 1e12 /
                  PEAK_BF16_TFLOPS, "alg_bytes": layer_bytes, "hbm_gbs": layer_bytes / (ms / 1e3) / 1e9,
                  "hbm_frac": layer_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS},
        "gate_up": roofline(gu_f, gu_b, gu_ms / 1e3, load_traffic(cfg.name, "gate_up")),
        "down": roofline(dn_f, dn_b, dn_ms / 1e3, load_traffic(cfg.name, "down")),
        "experts_touched": r["n_touched"],
        "max_expert_load": int(r["counts"].max()),
        "empty_experts": int((r["counts"] == 0).sum()),
    }


def cpu_baseline(cfg, hw, n_tokens, w_scales=None):
    """The oracle, as it stands, on a seeded sample of the workload's tokens."""
    import oracle
    import synth
    from synth.configs import make_inputs
    inp = make_inputs(cfg, weights=hw, w_scales=w_scales)
    tok = synth.subset(cfg.seed_base + 555, 98, cfg.T, n_tokens)
    t0 = time.perf_counter()
    x = inp.x[tok]
    u = oracle.rmsnorm_pinned(x, inp.pre_gain, cfg.eps) if cfg.sublayer else x
    r = oracle.route(u, inp.w_router, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho, want_margin=False)
    y = oracle.experts(u, inp.w_gate, inp.w_up, inp.w_down, r.idx, r.w, w_scales=inp.w_scales)
    if cfg.sublayer:
        oracle.post_residual(y, x, inp.post_gain, cfg.eps, cfg.residual_k)
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": "%d seeded tokens of %s (router + experts%s), %.1f s" % (
                n_tokens, cfg.name, " + norms" if cfg.sublayer else "", dt)}


def sweep(base, hw, dw, sizes, steps, warmup, md_path="", scales=None):
    """The layer at several token counts with the decode workload's input distributions
    (serving shapes between decode and prefill); one JSON line per size."""
    rows = []
    for T in sizes:
        c = base.replace(name="serve_t%d" % T, T=T)
        r = run_workload(c, hw, dw, steps, warmup, scales=scales)
        s = summarize(c, r, steps, warmup)
        row = {"workload": c.name, "T": T, "tokens_per_s": s["tokens_per_s"], "ms_per_step": s["ms_per_step"],
               "gate_up_ms": s["stages_ms"]["gate_up"], "down_ms": s["stages_ms"]["down"],
               "experts_touched": s["experts_touched"], "rows_per_expert": T * c.top_k / c.E,
               "mfma_frac": s["layer"]["mfma_frac"], "hbm_frac": s["layer"]["hbm_frac"]}
        rows.append(row)
        print(json.dumps(row), flush=True)
    if md_path:
        with open(md_path, "w") as f:
            f.write("| T | rows/expert | experts touched | ms / layer | tokens/s | gate/up ms | down ms | "
                    "MFMA % | HBM % |\n|---|---|---|---|---|---|---|---|---|\n")
            for r in rows:
                f.write("| %d | %.1f | %d | %.3f | %.0f | %.3f | %.3f | %.1f | %.1f |\n" % (
                    r["T"], r["rows_per_expert"], r["experts_touched"], r["ms_per_step"], r["tokens_per_s"],
                    r["gate_up_ms"], r["down_ms"], 100 * r["mfma_frac"], 100 * r["hbm_frac"]))


def copy_calibration(mib):
    import torch
    n = mib * 2 ** 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_t8192",
                    choices=["prefill_t8192", "decode_t64", "skew_t6000", "sublayer_t32768", "decode_t64_fp8",
                             "prefill_t8192_fp8", "decode_t64_mxfp4", "prefill_t8192_mxfp4"])
    ap.add_argument("--secondary", default="decode_t64", help="second workload timed in the same run, or 'none'")
    ap.add_argument("--cpu-tokens", type=int, default=1024, help="oracle sample size for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the decode and prefill layers with 8-bit and 4-bit expert weights")
    ap.add_argument("--sweep", default="", metavar="T1,T2,...",
                    help="time the layer on the decode workload's inputs at each token count (serving shapes) "
                         "and print one JSON line per size instead of the benchmark line")
    ap.add_argument("--sweep-md", default="", metavar="PATH", help="also write the sweep as a markdown table")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MiB")
    ap.add_argument("--ingest-pmc", nargs=5, metavar=("FETCH_CSV", "WRITE_CSV", "CALIB_FETCH_CSV", "CALIB_WRITE_CSV",
                                                      "CALIB_MIB"),
                    help="record counter runs of --workload into profiles/traffic.json (no GPU needed)")
    args = ap.parse_args()
    if args.ingest_pmc:
        a = args.ingest_pmc
        ingest_counters(args.workload, a[0], a[1], a[2], a[3], int(a[4]))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: the layer is built and timed on a single GPU "
              "(no sharding, no collectives); --gpus %d is not supported" % max(args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calib:
        copy_calibration(args.copy_calib)
        return
    import sparse_moe_layer_04_amd  # noqa: F401  (fails loudly without the HIP library)
    from synth.configs import CONFIGS, expert_weights

    cfg = CONFIGS[args.workload]
    t0 = time.time()
    hw = expert_weights(cfg)
    log("weights generated in %.1fs" % (time.time() - t0))

    def dev(a):
        import numpy as np
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    scales = None
    if cfg.weights != "bf16":   # the primary workload reads quantized weights: quantize, keep only those
        from synth.configs import quantized_weights
        hw, hs = quantized_weights(cfg, hw)
        scales = (hs, tuple(dev(a) for a in hs))
    dw = tuple(dev(a) for a in hw)
    torch.cuda.synchronize()
    log("weights uploaded")

    if args.sweep:
        base = CONFIGS["decode_t64" if cfg.weights == "bf16" else "decode_t64_" + cfg.weights]
        sweep(base, hw, dw, [int(t) for t in args.sweep.split(",")], args.steps, args.warmup, args.sweep_md,
              scales=scales)
        return

    prim = run_workload(cfg, hw, dw, args.steps, args.warmup, scales=scales)
    s = summarize(cfg, prim, args.steps, args.warmup)
    log("primary %s: %.3f ms/step" % (cfg.name, s["ms_per_step"]))
    line = {
        "metric": METRIC,
        "value": s["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": s["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "bf16 activations, e4m3 weights", "mxfp4": "bf16 activations, e2m1 (mxfp4) weights"}.get(
            cfg.weights, "bf16"),
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "I": cfg.I, "n_group": cfg.n_group,
                   "topk_group": cfg.topk_group, "top_k": cfg.top_k, "routed_scaling": cfg.rho,
                   "sublayer": cfg.sublayer, "parallelism": "single GPU"},
        "roofline": dict(s["gate_up"], kernel="gate_up (grouped gate/up GEMM + SwiGLU)"),
        "layer": s["layer"],
        "stages_ms": s["stages_ms"],
        "down": s["down"],
        "experts_touched": s["experts_touched"],
        "max_expert_load": s["max_expert_load"],
        "empty_experts": s["empty_experts"],
    }
    if args.secondary and args.secondary != "none" and args.secondary != cfg.name and cfg.weights == "bf16":
        c2 = CONFIGS[args.secondary]
        r2 = run_workload(c2, hw, dw, args.steps, args.warmup)
        s2 = summarize(c2, r2, args.steps, args.warmup)
        log("secondary %s: %.3f ms/step" % (c2.name, s2["ms_per_step"]))
        line["secondary"] = {"workload": c2.name, "tokens_per_s": s2["tokens_per_s"],
                             "ms_per_step": s2["ms_per_step"], "layer": s2["layer"], "stages_ms": s2["stages_ms"],
                             "roofline": dict(s2["gate_up"], kernel="gate_up"), "down": s2["down"],
                             "experts_touched": s2["experts_touched"]}
    del dw
    torch.cuda.empty_cache()
    if not args.no_fp8 and args.workload == "prefill_t8192":
        # the same layers with the expert weights in 8-bit storage (E4M3 codes + E8M0 scales
        # per 32 elements; beam_moe_forward_fp8) and in 4-bit storage (MXFP4: E2M1 codes +
        # E8M0 scales; beam_moe_forward_mxfp4), quantized from the same bf16 weights
        from synth.configs import quantized_weights
        for fmt, key in (("fp8", "fp8_weights"), ("mxfp4", "mxfp4_weights")):
            names = ("decode_t64_" + fmt, "prefill_t8192_" + fmt)
            hq, hs = quantized_weights(CONFIGS[names[0]], hw)
            dq, ds = tuple(dev(a) for a in hq), tuple(dev(a) for a in hs)
            torch.cuda.synchronize()
            line[key] = {}
            for name in names:
                c8 = CONFIGS[name]
                r8 = run_workload(c8, hq, dq, args.steps, args.warmup, scales=(hs, ds))
                s8 = summarize(c8, r8, args.steps, args.warmup)
                log("%s %s: %.3f ms/step" % (fmt, name, s8["ms_per_step"]))
                line[key][name] = {"tokens_per_s": s8["tokens_per_s"], "ms_per_step": s8["ms_per_step"],
                                   "layer": s8["layer"], "stages_ms": s8["stages_ms"],
                                   "gate_up": s8["gate_up"], "down": s8["down"],
                                   "experts_touched": s8["experts_touched"]}
            del dq, ds, hq, hs
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, hw, args.cpu_tokens, w_scales=scales[0] if scales else None)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
