#!/usr/bin/env python3
"""Benchmark of one Beam mixture-of-experts layer on one MI355X.

A step is one ``beam_moe_forward`` call (router -> permutation -> gate/up -> down ->
combine) over one batch of synthetic, seeded tokens already resident in HBM.  The primary
line is the 8192-token prefill layer; the same run times the other four workloads (the
tiny fp32 layer, the 64-token decode layer, the skewed 6000-token layer and the 32768-token
sublayer), the decode and prefill layers with 8-bit and 4-bit expert weights, and the CPU
oracle as a baseline.  Prints ONE JSON line.

Timing: W untimed warm-up steps (every other workload and serving shape also warms for
at least 0.2 s of its own layers, so that it is timed at its own steady clocks), then K
bare forwards, each bracketed by events on the launch stream (``ms_per_step`` is their median; the bracket around all K gives the mean);
the per-stage times come from a separate pass whose forwards record events at every stage
boundary on the same stream.

  python bench.py [--gpus 1] [--steps 20] [--warmup 20] [--workload prefill_t8192]
  python bench.py --sweep 16,64,256,1024 [--sweep-md table.md]   # serving shapes, one line per size
  python bench.py --copy-calib 1024      # plain 1 GiB device copy (HBM counter calibration)
  python bench.py --workload W --ingest-pmc FETCH.csv WRITE.csv CALIB_FETCH.csv CALIB_WRITE.csv 1024
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at 1 MI355X (prefill 8192 / decode 64); % MFMA / HBM roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
GEMM_SOURCES = [os.path.join(ROOT, "sparse_moe_layer_04_amd", "csrc", "experts.hip")]
EXPERTS_SRC = GEMM_SOURCES[0]
# the workloads timed besides the primary one, in this order
OTHER_WORKLOADS = ("tiny_f32", "decode_t64", "skew_t6000", "sublayer_t32768")
# every workload besides the primary one (which warms exactly --warmup layers) and every
# serving shape also warms for at least this long on its own layers before it is timed
SECONDARY_WARM_S = 0.2
# serving shapes timed in the default prefill run (bf16 weights, the decode workload's inputs)
SERVING_SWEEP = (16, 256, 1024, 2048, 4096)
CPU_SUBSET = 256            # seeded token subset of the oracle baseline for the large workloads
CPU_ONE_THREAD_TOKENS = 8   # prefill tokens of the one-thread oracle figure


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(text=None) -> str:
    """Hash of the expert-GEMM sources with their comments and blank space removed, so that a
    change to the comments alone keeps recorded counter traffic valid."""
    import re
    if text is None:
        parts = []
        for p in GEMM_SOURCES:
            with open(p) as f:
                parts.append(f.read())
        text = "\n".join(parts)
    code = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    code = re.sub(r"//[^\n]*", " ", code)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def weight_bytes_per_element(cfg):
    """bf16: 2; fp32: 4; 8-bit storage: 1 byte per code plus one scale byte per 32 elements;
    MXFP4: half a byte per code plus the scale byte per 32."""
    if cfg.dtype == "f32":
        return 4.0
    return {"fp8": 1.0 + 1.0 / 32, "mxfp4": 0.5 + 1.0 / 32}.get(cfg.weights, 2.0)


def act_bytes(cfg):
    return 4.0 if cfg.dtype == "f32" else 2.0


def gate_up_work(cfg, n_touched):
    """Algorithmic flops and bytes of one gate/up launch.

    flops: 4*H*I per routed pair (gate and up products).
    bytes: each touched expert's gate and up matrices once (2*I*H weights), each token row
    once (H activations), each h row written once (I activations)."""
    P = cfg.T * cfg.top_k
    a = act_bytes(cfg)
    flops = 4.0 * cfg.H * cfg.I * P
    nbytes = n_touched * 2.0 * cfg.I * cfg.H * weight_bytes_per_element(cfg) + cfg.T * cfg.H * a + P * cfg.I * a
    return flops, nbytes


def down_work(cfg, n_touched):
    """flops 2*H*I per pair; bytes: each touched W_d once, each h row read, each output row written."""
    P = cfg.T * cfg.top_k
    return (2.0 * cfg.H * cfg.I * P,
            n_touched * cfg.H * cfg.I * weight_bytes_per_element(cfg) + P * (cfg.I + cfg.H) * act_bytes(cfg))


def layer_work(cfg, n_touched):
    """Whole-layer flops (6*H*I per pair; the router's 2*E*H per token excluded) and
    algorithmic bytes (touched experts' weights, W_r, x in, out)."""
    P = cfg.T * cfg.top_k
    flops = 6.0 * cfg.H * cfg.I * P
    nbytes = (n_touched * 3.0 * cfg.H * cfg.I * weight_bytes_per_element(cfg) + cfg.E * cfg.H * 4.0 +
              2.0 * cfg.T * cfg.H * act_bytes(cfg))
    return flops, nbytes


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


# expert GEMM kernels (the decode, line or prefill kernel) by their GATED template flag
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


def trace_summary(csv_path, skip):
    """Markdown table of per-kernel durations from a rocprofv3 --kernel-trace csv, leaving out
    the first `skip` dispatches of every kernel (the untimed warm-up steps of a one-workload
    bench run), so the means cover the same forwards as the bench's timing."""
    import csv
    durs = {}
    for r in csv.DictReader(open(csv_path)):
        durs.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    rows = []
    for name, d in durs.items():
        d = d[skip:] if len(d) > skip else d
        rows.append((name, len(d), sum(d) / len(d), statistics.median(d), min(d), max(d)))
    total = sum(r[1] * r[2] for r in rows)
    rows.sort(key=lambda r: -r[1] * r[2])
    out = ["| kernel | dispatches | mean (us) | median (us) | min (us) | max (us) | share |",
           "|---|---|---|---|---|---|---|"]
    for name, n, mean, med, lo, hi in rows:
        short = name.split("(")[0]
        out.append("| `%s` | %d | %.1f | %.1f | %.1f | %.1f | %.1f%% |" % (short, n, mean, med, lo, hi,
                                                                          100.0 * n * mean / total))
    return "\n".join(out)


def expert_histogram(counts):
    """The per-expert routed-row counts of a step: touched, min, median, max, empty, top-8."""
    import numpy as np
    c = np.asarray(counts)
    return {"touched": int((c > 0).sum()), "min": int(c.min()), "median": float(np.median(c)),
            "max": int(c.max()), "empty": int((c == 0).sum()),
            "top8": [int(v) for v in np.sort(c)[::-1][:8]]}


def _dev(a):
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_workload(cfg, hw, dw, steps, warmup, scales=None, stage_steps=None, min_warm_s=0.0):
    """Times workload `cfg` (weights hw on the host, dw on the device; quantized weights come
    with `scales` = (host scales, device scales)).

    K = `steps` bare forwards, each between two events on the launch stream, give the median
    and mean step times; a separate pass of `stage_steps` forwards records the stage events."""
    import numpy as np
    import torch

    import sparse_moe_layer_04_amd as bm
    from synth.configs import make_inputs

    inp = make_inputs(cfg, weights=hw, w_scales=scales[0] if scales else None)
    shape = bm.make_shape(cfg.T, cfg.H, cfg.E, cfg.I, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho, cfg.dtype)
    op = bm.OP_FORWARD_SUBLAYER if cfg.sublayer else bm.OP_FORWARD
    ws = torch.empty(bm.workspace_size(shape, op), dtype=torch.uint8, device="cuda")
    x, bias = _dev(inp.x), _dev(inp.bias)
    act_dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = torch.empty((cfg.T, cfg.H), dtype=act_dt, device="cuda")
    idx = torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device="cuda")
    sub = None
    if cfg.sublayer:
        g1, g2 = _dev(inp.pre_gain), _dev(inp.post_gain)
        sub = bm.sublayer(g1, g2, cfg.eps, cfg.residual_k)

    def step(timer=None):
        bm.forward(shape, x, dw[0], bias, dw[1], dw[2], dw[3], out, ws, sublayer=sub, topk_idx=idx,
                   stage_events=timer.events if timer else None, w_scales=scales[1] if scales else None,
                   w_format=cfg.code_format or "e4m3")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # then warm for at least min_warm_s of this workload's own layers: after an idle gap (the
    # weights being made and uploaded) the clocks ramp up over the first ~30 ms of load, which
    # a few short decode layers do not cover
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < min_warm_s:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(steps):
        ev[i][0].record()
        step()
        ev[i][1].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per_step = [a.elapsed_time(b) for a, b in ev]
    # stage pass
    n_stage = steps if stage_steps is None else stage_steps
    timers = [bm.StageTimer() for _ in range(n_stage)]
    for t in timers:
        step(t)
    torch.cuda.synchronize()
    stage = np.array([t.elapsed_ms() for t in timers])
    for t in timers:
        t.close()
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=cfg.E)
    return dict(ms_median=statistics.median(per_step), ms_mean=t_start.elapsed_time(t_end) / steps,
                ms_min=min(per_step), wall_s=wall, stage_ms=stage.mean(axis=0), counts=counts,
                n_touched=int((counts > 0).sum()))


def summarize(cfg, r):
    import sparse_moe_layer_04_amd as bm
    ms = r["ms_median"]
    gu_ms = float(r["stage_ms"][4])
    dn_ms = float(r["stage_ms"][5])
    gu_f, gu_b = gate_up_work(cfg, r["n_touched"])
    dn_f, dn_b = down_work(cfg, r["n_touched"])
    lf, lb = layer_work(cfg, r["n_touched"])
    return {
        "workload": cfg.name,
        "T": cfg.T,
        "tokens_per_s": cfg.T / (ms / 1e3),
        "ms_per_step": ms,
        "ms_mean": r["ms_mean"],
        "ms_min": r["ms_min"],
        "stages_ms": {n: round(float(v), 4) for n, v in zip(bm.STAGE_NAMES, r["stage_ms"])},
        "layer": {"tflops": lf / (ms / 1e3) / 1e12, "mfma_frac": lf / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                  "alg_bytes": lb, "hbm_gbs": lb / (ms / 1e3) / 1e9,
                  "hbm_frac": lb / (ms / 1e3) / 1e9 / PEAK_HBM_GBS},
        "gate_up": roofline(gu_f, gu_b, gu_ms / 1e3, load_traffic(cfg.name, "gate_up")),
        "down": roofline(dn_f, dn_b, dn_ms / 1e3, load_traffic(cfg.name, "down")),
        "experts": expert_histogram(r["counts"]),
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_pass(cfg, inp, tok):
    """The oracle on the tokens `tok` of a workload: pre-norm (sublayer), router, experts,
    post-norm and residual (sublayer); returns the seconds it took."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    x = np.ascontiguousarray(inp.x[tok])
    u = oracle.rmsnorm_pinned(x, inp.pre_gain, cfg.eps) if cfg.sublayer else x
    r = oracle.route(u, inp.w_router, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho, want_margin=False)
    y = oracle.experts(u, inp.w_gate, inp.w_up, inp.w_down, r.idx, r.w, w_scales=inp.w_scales)
    if cfg.sublayer:
        oracle.post_residual(y, x, inp.post_gain, cfg.eps, cfg.residual_k)
    return time.perf_counter() - t0


def cpu_baseline(primary, hw, others=(), one_thread=True, w_scales=None):
    """The oracle as it stands, on the host's cores: every token of the tiny and the decode
    workloads, a seeded 256-token subset of the larger ones (router and experts on the
    subset), the router alone over every token of each workload, and a one-thread figure on
    a few prefill tokens.  The primary workload's subset gives `value`."""
    import numpy as np
    import oracle
    import synth
    from synth.configs import CONFIGS, make_inputs
    threads = oracle.threads()
    per = {}
    router_all = {}
    inputs = {}
    names = [primary.name] + [n for n in others if n != primary.name]
    for name in names:
        cfg = CONFIGS[name]
        inp = make_inputs(cfg, weights=None if cfg.dtype == "f32" else hw,
                          w_scales=w_scales if name == primary.name else None)
        inputs[name] = inp
        if cfg.T <= 64:
            tok = np.arange(cfg.T, dtype=np.int64)
            kind = "all %d tokens" % cfg.T
        else:
            tok = synth.subset(cfg.seed_base + 555, 98, cfg.T, CPU_SUBSET)
            kind = "%d seeded tokens of %d" % (CPU_SUBSET, cfg.T)
        dt = _oracle_pass(cfg, inp, tok)
        per[name] = {"tokens": int(tok.size), "seconds": dt, "tokens_per_s": tok.size / dt, "sample": kind}
        log("cpu oracle %s: %s in %.1f s" % (name, kind, dt))
        t0 = time.perf_counter()
        u = oracle.rmsnorm_pinned(inp.x, inp.pre_gain, cfg.eps) if cfg.sublayer else inp.x
        oracle.route(u, inp.w_router, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho, want_margin=False)
        dt = time.perf_counter() - t0
        router_all[name] = {"tokens": cfg.T, "seconds": dt, "tokens_per_s": cfg.T / dt}
    one = None
    if one_thread:
        cfg = primary
        tok = synth.subset(cfg.seed_base + 556, 98, cfg.T, CPU_ONE_THREAD_TOKENS)
        oracle.set_threads(1)
        try:
            dt = _oracle_pass(cfg, inputs[cfg.name], tok)
        finally:
            oracle.set_threads(threads)
        one = {"workload": cfg.name, "tokens": int(tok.size), "seconds": dt, "tokens_per_s": tok.size / dt,
               "threads": 1}
        log("cpu oracle one thread: %d tokens in %.1f s" % (tok.size, dt))
    p = per[primary.name]
    return {"value": p["tokens_per_s"], "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%s of %s (%s), %.1f s" % (
                p["sample"], primary.name,
                "pre-norm, router, experts, post-norm" if primary.sublayer else "router and experts", p["seconds"]),
            "cpu_model": cpu_model(), "per_workload": per, "router_only_all_tokens": router_all,
            "one_thread": one}


def sweep_rows(base, hw, dw, sizes, steps, warmup, scales=None, emit=None):
    """The layer at several token counts with the decode workload's input distributions
    (serving shapes between decode and prefill): one row per size."""
    rows = []
    for T in sizes:
        c = base.replace(name="serve_t%d" % T, T=T)
        r = run_workload(c, hw, dw, steps, warmup, scales=scales, min_warm_s=SECONDARY_WARM_S)
        s = summarize(c, r)
        row = {"workload": c.name, "T": T, "tokens_per_s": s["tokens_per_s"], "ms_per_step": s["ms_per_step"],
               "gate_up_ms": s["stages_ms"]["gate_up"], "down_ms": s["stages_ms"]["down"],
               "experts_touched": s["experts"]["touched"], "rows_per_expert": T * c.top_k / c.E,
               "mfma_frac": s["layer"]["mfma_frac"], "hbm_frac": s["layer"]["hbm_frac"]}
        rows.append(row)
        if emit:
            emit(row)
    return rows


def sweep(base, hw, dw, sizes, steps, warmup, md_path="", scales=None):
    """sweep_rows with one JSON line per size (and optionally a markdown table)."""
    rows = sweep_rows(base, hw, dw, sizes, steps, warmup, scales=scales,
                      emit=lambda row: print(json.dumps(row), flush=True))
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


def dense_gemm_calibration(spec, seconds=3.0):
    """The dense bf16 GEMM rate the board sustains: torch.matmul (hipBLASLt) on contiguous
    M x K and K x N bf16 operands, called back to back for `seconds` after one second of
    warm-up; the median call gives the TFLOP/s.  A reference point for the expert GEMMs,
    not part of the layer."""
    import torch
    m, n, k = (int(v) for v in spec.split(","))
    a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(m, n, device="cuda", dtype=torch.bfloat16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
    times = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for e0, e1 in evs:
            e0.record()
            torch.matmul(a, b, out=c)
            e1.record()
        torch.cuda.synchronize()
        times += [e0.elapsed_time(e1) for e0, e1 in evs]
    ms = statistics.median(times)
    print(json.dumps({"dense_gemm_bf16": [m, n, k], "calls": len(times), "ms_median": ms,
                      "tflops": 2.0 * m * n * k / (ms * 1e-3) / 1e12}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_t8192",
                    choices=["prefill_t8192", "decode_t64", "skew_t6000", "sublayer_t32768", "decode_t64_fp8",
                             "prefill_t8192_fp8", "decode_t64_mxfp4", "prefill_t8192_mxfp4"])
    ap.add_argument("--secondary", default=",".join(OTHER_WORKLOADS),
                    help="comma-separated workloads timed in the same run besides the primary one, or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-serving-sweep", action="store_true",
                    help="skip the serving shapes (decode inputs at %s tokens) of the default prefill run"
                         % ",".join(str(t) for t in SERVING_SWEEP))
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the decode and prefill layers with 8-bit and 4-bit expert weights")
    ap.add_argument("--sweep", default="", metavar="T1,T2,...",
                    help="time the layer on the decode workload's inputs at each token count (serving shapes) "
                         "and print one JSON line per size instead of the benchmark line")
    ap.add_argument("--sweep-md", default="", metavar="PATH", help="also write the sweep as a markdown table")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MiB")
    ap.add_argument("--dense-gemm-calib", default="", metavar="M,N,K",
                    help="time a plain bf16 torch.matmul (hipBLASLt) of this shape back to back: the dense "
                         "GEMM rate the board sustains, a reference for the expert GEMMs")
    ap.add_argument("--trace-summary", nargs=2, metavar=("KERNEL_TRACE_CSV", "SKIP"),
                    help="print the per-kernel duration table of a rocprofv3 kernel trace, leaving out the "
                         "first SKIP dispatches of each kernel (no GPU needed)")
    ap.add_argument("--ingest-pmc", nargs=5, metavar=("FETCH_CSV", "WRITE_CSV", "CALIB_FETCH_CSV", "CALIB_WRITE_CSV",
                                                      "CALIB_MIB"),
                    help="record counter runs of --workload into profiles/traffic.json (no GPU needed)")
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary[0], int(args.trace_summary[1])))
        return
    if args.ingest_pmc:
        a = args.ingest_pmc
        ingest_counters(args.workload, a[0], a[1], a[2], a[3], int(a[4]))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: the layer is built and timed on a single GPU "
              "(no sharding, no collectives); --gpus %d is not supported" % max(args.gpus, world), file=sys.stderr)
        sys.exit(2)

    from synth.configs import CONFIGS as _CONFIGS
    if _CONFIGS[args.workload].weights == "bf16" and args.secondary != "none":
        for n in args.secondary.split(","):   # secondary workloads share the primary's bf16 weights
            if n and (n not in _CONFIGS or _CONFIGS[n].weights != "bf16"):
                print("--secondary takes bf16 workloads only (%s); the 8-bit and 4-bit layers run as "
                      "--workload or in the default prefill run" % n, file=sys.stderr)
                sys.exit(2)

    import torch
    if args.copy_calib:
        copy_calibration(args.copy_calib)
        return
    if args.dense_gemm_calib:
        dense_gemm_calibration(args.dense_gemm_calib)
        return
    import sparse_moe_layer_04_amd  # noqa: F401  (fails loudly without the HIP library)
    from synth.configs import CONFIGS, expert_weights, make_inputs

    cfg = CONFIGS[args.workload]
    t0 = time.time()
    hw = expert_weights(cfg)
    log("weights generated in %.1fs" % (time.time() - t0))

    scales = None
    if cfg.weights != "bf16":   # the primary workload reads quantized weights: quantize, keep only those
        from synth.configs import quantized_weights
        hw, hs = quantized_weights(cfg, hw)
        scales = (hs, tuple(_dev(a) for a in hs))
    dw = tuple(_dev(a) for a in hw)
    torch.cuda.synchronize()
    log("weights uploaded")

    if args.sweep:
        base = CONFIGS["decode_t64" if cfg.weights == "bf16" else "decode_t64_" + cfg.weights]
        sweep(base, hw, dw, [int(t) for t in args.sweep.split(",")], args.steps, args.warmup, args.sweep_md,
              scales=scales)
        return

    bench_wall0 = time.perf_counter()
    prim = run_workload(cfg, hw, dw, args.steps, args.warmup, scales=scales)
    s = summarize(cfg, prim)
    log("primary %s: %.3f ms/step (median), %.3f mean" % (cfg.name, s["ms_per_step"], s["ms_mean"]))
    line = {
        "metric": METRIC,
        "value": s["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": s["ms_per_step"],
        "ms_per_step_mean": s["ms_mean"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "bf16 activations, e4m3 weights", "mxfp4": "bf16 activations, e2m1 (mxfp4) weights"}.get(
            cfg.weights, "bf16"),
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "I": cfg.I, "n_group": cfg.n_group,
                   "topk_group": cfg.topk_group, "top_k": cfg.top_k, "routed_scaling": cfg.rho,
                   "sublayer": cfg.sublayer, "parallelism": "single GPU"},
        "roofline": dict(s["gate_up"], kernel="gate_up (grouped gate/up GEMM + SwiGLU)",
                         kernel_ms=s["stages_ms"]["gate_up"], kernel_ms_source="stage-event pass, mean"),
        "layer": s["layer"],
        "stages_ms": s["stages_ms"],
        "down": s["down"],
        "experts": s["experts"],
        "gemm_code_sha256_16": kernel_source_hash(),
    }
    others = [] if args.secondary == "none" else [n for n in args.secondary.split(",") if n and n != cfg.name]
    if cfg.weights == "bf16" and others:
        line["workloads"] = {}
        for name in others:
            c2 = CONFIGS[name]
            if c2.dtype == "f32":   # the tiny fp32 layer has its own weights
                hw2 = make_inputs(c2)
                hw2 = (hw2.w_router, hw2.w_gate, hw2.w_up, hw2.w_down)
                dw2 = tuple(_dev(a) for a in hw2)
                r2 = run_workload(c2, hw2, dw2, args.steps, args.warmup, min_warm_s=SECONDARY_WARM_S)
                del dw2
            else:
                r2 = run_workload(c2, hw, dw, args.steps, args.warmup, min_warm_s=SECONDARY_WARM_S)
            s2 = summarize(c2, r2)
            log("%s: %.3f ms/step" % (c2.name, s2["ms_per_step"]))
            line["workloads"][c2.name] = s2
    if cfg.name == "prefill_t8192" and not args.no_serving_sweep:
        line["serving_sweep"] = [
            {k: row[k] for k in ("T", "rows_per_expert", "experts_touched", "ms_per_step", "tokens_per_s",
                                 "gate_up_ms", "down_ms", "mfma_frac", "hbm_frac")}
            for row in sweep_rows(CONFIGS["decode_t64"], hw, dw, SERVING_SWEEP, 10, 2,
                                  emit=lambda row: log("serving T=%d: %.3f ms/step" % (row["T"], row["ms_per_step"])))]
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
            dq, ds = tuple(_dev(a) for a in hq), tuple(_dev(a) for a in hs)
            torch.cuda.synchronize()
            line[key] = {}
            for name in names:
                c8 = CONFIGS[name]
                r8 = run_workload(c8, hq, dq, args.steps, args.warmup, scales=(hs, ds), min_warm_s=SECONDARY_WARM_S)
                s8 = summarize(c8, r8)
                log("%s %s: %.3f ms/step" % (fmt, name, s8["ms_per_step"]))
                line[key][name] = s8
            del dq, ds, hq, hs
            torch.cuda.empty_cache()
    line["gpu_wall_s"] = time.perf_counter() - bench_wall0
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, hw, others=others if cfg.weights == "bf16" else (),
                                            w_scales=scales[0] if scales else None)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
