#!/usr/bin/env python3
"""Benchmark of the W8A8 INT8 MoE layer on one MI355X.

One step = one pass of the whole layer (route, quantise x, permute, gate_up
GEMM + SwiGLU, quantise h, down GEMM, combine) over one batch of synthetic
tokens already resident in HBM.  Weights are quantised once before timing
(static per-channel weights) and rotated over several copies so that no step
finds the previous step's weights in the 256 MB last-level cache.

The default workload is the largest MoE layer that fits one GPU, the
235B-shaped layer (T=8192, H=4096, 128 experts, top-8, I=1536, Zipf(1.1)
expert loads); the 30B-shaped prefill and decode layers, the shared-expert and
W4A8 variants and the dense linears are other `--workload` lines.

Prints one JSON line.  `value` is tokens/s of the layer over the timed loop
(wall clock between synchronisations); `step_ms_p10_p50_p90` are per-step
times from HIP events at each layer call's start and end; `roofline` describes
the dominant kernel (the stage with the largest average time in a separate
pass with a HIP event after every stage; in the timed loop that stage is
bracketed by events too, on the layer's stream); `cpu_baseline` is the CPU
oracle timed on a bounded sample of the same tokens, with its threads and on
one thread.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5033.0       # 256 CU x 2.4 GHz x 8192 int8 ops/clk/CU (dense)
HBM_PEAK_GBS = 8000.0
FP32_MATRIX_PEAK_TFLOPS = 157.3
RIDGE = INT8_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
DEFAULT_WORKLOAD = "moe_235b_zipf_T8192"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gate_up_weight_bytes(cfg, E_hit, w4):
    """gate_up_proj weights of the experts hit: int8 codes and one fp32 scale
    per channel, or (W4A8) half a byte per code and an fp32 scale and an int8
    offset per channel and group of 128 inputs."""
    H, I = cfg.H, cfg.I
    if w4:
        return E_hit * 2 * I * (H // 2 + ((H + 127) // 128) * 5)
    return E_hit * 2 * I * (H + 4)


def kernel_model(cfg, E_hit, w4=False):
    """Algorithmic int8 ops and HBM bytes per launch of each stage kernel."""
    T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
    P = T * k
    xb = 2 if cfg.x_dtype == "bf16" else 4
    m = {}
    m["route"] = dict(ops=0, bytes=T * H * xb + E * H * 2 + P * 8)
    m["quant_x"] = dict(ops=0, bytes=T * H * xb + T * H + T * 4)
    m["permute"] = dict(ops=0, bytes=P * 4 * 3 + (E + 1) * 4)
    m["gate_up_gemm"] = dict(ops=2 * P * 2 * I * H,
                             bytes=gate_up_weight_bytes(cfg, E_hit, w4) + T * H + T * 4 + P * 4 + (E + 1) * 4
                             + P * I * 2)
    m["quant_h"] = dict(ops=0, bytes=P * I * 2 + P * I + P * 4)
    # y (the per-pair expert outputs) is 16-bit fixed point with one exponent
    # byte per row and 64 columns
    ybytes = P * H * 2 + P * ((H + 63) // 64)
    m["down_gemm"] = dict(ops=2 * P * H * I, bytes=E_hit * H * I + E_hit * H * 4 + P * I + P * 4 + (E + 1) * 4
                          + ybytes)
    m["combine"] = dict(ops=0, bytes=ybytes + P * 8 + T * H * xb)
    Is = cfg.Is
    if Is:
        # the shared expert's launches sit in the same stages: one group of T
        # rows (no gather), its gate read by the combine with x
        ys = T * H * 2 + T * ((H + 63) // 64)
        m["gate_up_gemm"]["ops"] += 2 * T * 2 * Is * H
        m["gate_up_gemm"]["bytes"] += 2 * Is * (H + 4) + T * Is * 2
        m["quant_h"]["bytes"] += T * Is * 3 + T * 4
        m["down_gemm"]["ops"] += 2 * T * H * Is
        m["down_gemm"]["bytes"] += H * (Is + 4) + T * Is + T * 4 + ys
        m["combine"]["bytes"] += ys + H * 2 + T * H * xb
    return m


def layer_model(cfg, E_hit, w4=False):
    """Whole-layer algorithmic work: int8 ops, and the bytes the method must
    move: quantised weights and scales of the experts hit, the router, x in, out."""
    T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
    xb = 2 if cfg.x_dtype == "bf16" else 4
    ops = 2 * T * k * 3 * H * I
    byts = gate_up_weight_bytes(cfg, E_hit, w4) + E_hit * H * (I + 4) + E * H * 2 + 2 * T * H * xb
    if cfg.Is:   # the shared expert on every token, its int8 weights and bf16 gate
        ops += 2 * T * 3 * H * cfg.Is
        byts += 2 * cfg.Is * (H + 4) + H * (cfg.Is + 4) + H * 2
    return ops, byts


def traffic_for(kernel, workload):
    """HBM bytes per launch measured with rocprofv3 counters, if the record in
    profiles/ was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, "w8a8_int8_quantized_bf16_amd", "csrc", rec["source"]), "rb").read()
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
        return None
    return rec["bytes_per_launch"]


def copy_probe(mib):
    """Plain device-to-device copies of a known size: the reference that
    scales the rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 5}), flush=True)


def counter_kib(csv_path, kernel_prefix, counter):
    """Mean per-dispatch value of a rocprofv3 --pmc counter over the dispatches
    whose kernel name starts with kernel_prefix."""
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if r["Kernel_Name"].startswith(kernel_prefix) and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit("no %s dispatches of %s in %s" % (counter, kernel_prefix, csv_path))
    return sum(vals) / len(vals), len(vals)


def write_traffic(args):
    """profiles/traffic_<stage>_<workload>.json from four rocprofv3 --pmc
    counter files: FETCH_SIZE and WRITE_SIZE of the bench run, and of the copy
    probe (whose true bytes scale the counters)."""
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.traffic
    stage, kernel, source = args.traffic_kernel
    n = args.copy_mib << 20
    cf, _ = counter_kib(cfetch_csv, "__amd_rocclr_copyBuffer", "FETCH_SIZE")
    cw, _ = counter_kib(cwrite_csv, "__amd_rocclr_copyBuffer", "WRITE_SIZE")
    f, nf = counter_kib(fetch_csv, kernel, "FETCH_SIZE")
    w, nw = counter_kib(write_csv, kernel, "WRITE_SIZE")
    sf, sw = n / (cf * 1024.0), n / (cw * 1024.0)
    rec = {"stage": stage, "kernel": kernel, "workload": args.workload, "source": source,
           "source_sha256": hashlib.sha256(open(os.path.join(ROOT, "w8a8_int8_quantized_bf16_amd", "csrc", source),
                                                "rb").read()).hexdigest(),
           "fetch_kib_per_dispatch": f, "write_kib_per_dispatch": w, "dispatches": [nf, nw],
           "copy_probe_bytes": n, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": sf, "write_scale": sw,
           "bytes_per_launch": f * 1024.0 * sf + w * 1024.0 * sw}
    out = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (stage, args.workload))
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec))


SIMDS = 1024                  # 256 CUs x 4 SIMDs
XCDS = 8                      # rocprofv3 sums GRBM_GUI_ACTIVE over the 8 XCDs' graphics blocks
PEAK_CLOCK_HZ = 2.4e9


def _csv_rows(path):
    import csv
    return list(csv.DictReader(open(path)))


def counter_summary(args):
    """Per-kernel summary of one rocprofv3 --pmc run with --kernel-trace:
    matrix-core operations (SQ_INSTS_VALU_MFMA_MOPS_I8, or _F32 for the fp32
    router, x 512), matrix-core busy cycles (SQ_VALU_MFMA_BUSY_CYCLES, summed
    over the SIMDs) against the active cycles of one XCD (GRBM_GUI_ACTIVE,
    summed over the XCDs, / 8) times the SIMDs, the clock those cycles imply
    over the traced duration, and the rate against the dense peak of that
    type (int8 5.0 POP/s, fp32 matrix 157.3 TFLOP/s) at 2.4 GHz and at that
    clock.  Prints markdown."""
    pmc_csv, trace_csv = args.counter_summary
    disp = {}
    for r in _csv_rows(pmc_csv):
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        d = disp.setdefault(key, {"kernel": r["Kernel_Name"], "c": {}})
        d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    dur = {}
    for r in _csv_rows(trace_csv):
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        dur[key] = (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-9
    by_kernel = {}
    for key, d in disp.items():
        if key in dur:
            by_kernel.setdefault(d["kernel"], []).append((d["c"], dur[key]))
    f32 = any("SQ_INSTS_VALU_MFMA_MOPS_F32" in r[0] for rows in by_kernel.values() for r in rows)
    mops, kind, peak = ("SQ_INSTS_VALU_MFMA_MOPS_F32", "fp32", FP32_MATRIX_PEAK_TFLOPS) if f32 else \
        ("SQ_INSTS_VALU_MFMA_MOPS_I8", "int8", INT8_PEAK_TOPS)
    lines = ["| kernel | dispatches | avg us | %s ops (MOPS x 512) | MFMA busy / (XCD active cycles x SIMDs) | "
             "clock = XCD active cycles / duration | %s TOP/s | of peak at 2.4 GHz | of peak at that clock |" % (kind, kind),
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for kern, rows in sorted(by_kernel.items(), key=lambda kv: -sum(t for _, t in kv[1])):
        n = len(rows)
        t = sum(r[1] for r in rows) / n
        c = {name: sum(r[0].get(name, 0.0) for r in rows) / n for name in rows[0][0]}
        ops = c.get(mops, 0.0) * 512
        gui = c.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        util = busy / (gui * SIMDS) if gui else 0.0
        clk = gui / t if t else 0.0
        tops = ops / t / 1e12 if t else 0.0
        at_clk = ops / t / (peak * 1e12 * clk / PEAK_CLOCK_HZ) if ops and clk else 0.0
        name = kern if len(kern) < 90 else kern[:87] + "..."
        # GRBM_GUI_ACTIVE also counts the dispatch's own start and drain, so the
        # implied clock means something only for launches far longer than that
        clk_s = "%.2f GHz" % (clk / 1e9) if t >= 100e-6 else "-"
        at_s = "%.3f" % at_clk if t >= 100e-6 else "-"
        lines.append("| `%s` | %d | %.1f | %.4g | %.3f | %s | %.0f | %.3f | %s |"
                     % (name, n, t * 1e6, ops, util, clk_s, tops, tops / peak, at_s))
    print("\n".join(lines))


def cpu_model():
    """The host CPU's model name and logical core count."""
    name = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                name = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return name, os.cpu_count()


def _time_tokens(layer_tokens, case, wq, tok):
    t0 = time.perf_counter()
    layer_tokens(case["x"], *wq, tok)
    return time.perf_counter() - t0


def cpu_baseline(case, target_s, min_tokens=2048, single_s=6.0):
    """The CPU oracle, as is, on a bounded sample of the workload's tokens (at
    least min_tokens of them, or all): once with the oracle's threads, once on
    a single thread over a smaller sample."""
    import numpy as np

    import oracle
    cfg = case["cfg"]
    t0 = time.time()
    qgu, sgu = oracle.quant_rows(case["gu"].reshape(-1, cfg.H))
    qd, sd = oracle.quant_rows(case["dn"].reshape(-1, cfg.I))
    wq = (case["wg"], qgu.reshape(case["gu"].shape), sgu.reshape(cfg.E, -1), qd.reshape(case["dn"].shape),
          sd.reshape(cfg.E, -1), cfg.k)
    layer_tokens = oracle.moe_layer_tokens
    if cfg.Is:
        sgu_f, sdn_f, wsg = case["shared"]
        qs, ss = oracle.quant_rows(sgu_f)
        qsd, ssd = oracle.quant_rows(sdn_f)
        wq = wq + (dict(wgu=qs, sgu=ss, wd=qsd, sd=ssd, wsg=wsg),)
        layer_tokens = oracle.moe_layer_shared_tokens
    log("oracle weight quantisation (untimed setup): %.1f s" % (time.time() - t0))
    rng = np.random.default_rng(0)
    threads = oracle.num_threads()
    # a short probe sizes the sample so that the timed run takes about target_s
    n = min(64, cfg.T)
    dt = _time_tokens(layer_tokens, case, wq, np.sort(rng.choice(cfg.T, n, replace=False)))
    n = int(min(cfg.T, max(min(min_tokens, cfg.T), n * target_s / max(dt, 1e-6))))
    tok = np.sort(rng.choice(cfg.T, n, replace=False))
    dt = _time_tokens(layer_tokens, case, wq, tok)
    log("oracle, %d threads: %d tokens in %.1f s" % (threads, n, dt))
    # single thread: the same oracle on fewer tokens
    oracle.set_num_threads(1)
    try:
        n1 = max(1, min(n, int(n / dt / threads * single_s)))
        tok1 = np.sort(rng.choice(cfg.T, n1, replace=False))
        dt1 = _time_tokens(layer_tokens, case, wq, tok1)
    finally:
        oracle.set_num_threads(threads)
    log("oracle, 1 thread: %d tokens in %.1f s" % (n1, dt1))
    model, ncpu = cpu_model()
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of the %d tokens of %s (the layer couples no tokens), %.1f s with %d threads; "
                      "weights quantised by the oracle beforehand, untimed" % (n, cfg.T, cfg.name, dt, threads),
            "single_thread": {"value": n1 / dt1, "unit": "tokens/s", "tokens": n1, "seconds": round(dt1, 2)},
            "cpu_model": model, "logical_cpus": ncpu}


def bench_dense(args, cfg):
    """The dense W8A8 linear: one step = quantise x per token + one-group GEMM
    with the dequantising epilogue (bf16 out); W quantised and packed once."""
    import numpy as np
    import torch

    import synth
    import w8a8_int8_quantized_bf16_amd as w8
    M, K, N = cfg.M, cfg.K, cfg.N
    dev = "cuda:0"
    torch.cuda.set_device(0)
    xb, Wf = synth.dense_inputs(cfg)
    x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    qw, sw = w8.quant_act(torch.from_numpy(Wf).to(dev))
    wbytes = N * K
    copies = args.copies or max(1, min(4, (1 << 30) // wbytes + 1))
    packs = [w8.pack_weights(qw.view(1, N, K)) for _ in range(copies)]
    qx = torch.empty((M, K), dtype=torch.int8, device=dev)
    sx = torch.empty((M,), dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    L, st = w8.lib(), w8._stream(x.device)
    P = w8._p
    nws = int(L.w8a8_linear_q_workspace_size(M, N, K))   # split-K partial sums (decode-sized linears)
    lws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)

    # w8a8_linear's kernels, called as its two stages so that events can
    # bracket the GEMM: the per-row quantisation, then w8a8_linear_q (the
    # GEMM, plus the sum of the K slices when K is split)
    def step(i, e0=None, e1=None):
        rc = L.w8a8_quant_act(P(x), w8.BF16, M, K, K, P(qx), P(sx), st)
        if rc:
            raise SystemExit("w8a8_quant_act: %s" % w8.status_string(rc))
        if e0 is not None:
            e0.record()
        rc = L.w8a8_linear_q(P(qx), P(sx), M, K, P(packs[i % copies]), P(sw), N, P(out), w8.BF16, P(lws), nws, st)
        if rc:
            raise SystemExit("w8a8_linear_q: %s" % w8.status_string(rc))
        if e1 is not None:
            e1.record()

    for i in range(args.warmup):
        step(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, *evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gemm_us = sum(a.elapsed_time(b) for a, b in evs) * 1e3 / args.steps
    ops = 2 * M * N * K
    byts = N * K + N * 4 + M * K + M * 4 + M * N * 2   # W codes + scales, x codes + scales, out
    mfma_bound = ops / byts > RIDGE
    if mfma_bound:
        achieved, peak, unit = ops / (gemm_us * 1e-6) / 1e12, INT8_PEAK_TOPS, "TOP/s"
    else:
        achieved, peak, unit = byts / (gemm_us * 1e-6) / 1e9, HBM_PEAK_GBS, "GB/s"
    t_step = elapsed / args.steps
    lbytes = N * K + N * 4 + M * K * 2 + M * N * 2   # W codes + scales, x in (bf16), out (bf16)
    roof_t = max(ops / (INT8_PEAK_TOPS * 1e12), lbytes / (HBM_PEAK_GBS * 1e9))
    result = {
        "metric": "W8A8 linear tokens/s; int8 TOPS as % of MI355X roofline",
        "value": M / t_step, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t_step * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": M, "in_features": K, "out_features": N, "x_dtype": "bf16",
                   "weight_copies_rotated": copies,
                   **({"fused_qkv_widths": list(cfg.split)} if cfg.split else {})},
        "roofline": {"kernel": "dense_gemm", "bound": "mfma" if mfma_bound else "hbm", "achieved": achieved,
                     "peak": peak, "unit": unit, "frac": achieved / peak, "traffic": None, "avg_launch_us": gemm_us,
                     "alg_bytes_per_launch": byts, "int8_ops_per_launch": ops},
        "layer": {"int8_tops": ops / t_step / 1e12, "int8_tops_frac": ops / t_step / 1e12 / INT8_PEAK_TOPS,
                  "roof_time_us": roof_t * 1e6, "roofline_frac": roof_t / t_step,
                  "stage_us": {"quant_x": round(t_step * 1e6 - gemm_us, 2), "gemm": round(gemm_us, 2)}},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_dense(cfg, xb, Wf, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline_dense(cfg, xb, Wf, target_s):
    """The CPU oracle, as is, on a bounded sample of the linear's rows."""
    import numpy as np

    import oracle
    t0 = time.time()
    qw, sw = oracle.quant_rows(Wf)
    log("oracle weight quantisation (untimed setup): %.1f s" % (time.time() - t0))
    rng = np.random.default_rng(0)

    def run(n):
        rows = np.sort(rng.choice(cfg.M, n, replace=False))
        t0 = time.perf_counter()
        qx, sx = oracle.quant_rows(np.ascontiguousarray(xb[rows]))
        oracle.grouped_gemm(qx, sx, None, 1, qw[None], sw[None], np.array([0, n], np.int32), oracle.DEQUANT,
                            oracle.BF16)
        return time.perf_counter() - t0

    n = 16
    dt = run(n)
    n2 = int(min(cfg.M, max(n, n * target_s / max(dt, 1e-6))))
    if n2 > n:
        n, dt = n2, run(n2)
    model, ncpu = cpu_model()
    return {"value": n / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d of the %d rows of %s (rows are independent), %.1f s of CPU time; weights quantised by "
                      "the oracle beforehand, untimed" % (n, cfg.M, cfg.name, dt),
            "cpu_model": model, "logical_cpus": ncpu}


def bench_ep_shares(args, cfg, ngpu):
    """One GPU's share under ngpu-way expert parallelism, at its real shape:
    the routed, quantised pairs of experts [g*E/ngpu, (g+1)*E/ngpu) (taken
    from a full layer run on this GPU, as an all-to-all would deliver them)
    through gate_up GEMM + SwiGLU, h quantisation and the down GEMM, for every
    g.  The layer would run at the pace of the slowest share; the exchanges
    themselves are not part of this (one GPU)."""
    import numpy as np
    import torch

    import synth
    import w8a8_int8_quantized_bf16_amd as w8
    dev = "cuda:0"
    torch.cuda.set_device(0)
    T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
    if E % ngpu:
        raise SystemExit("%d experts do not split over %d GPUs" % (E, ngpu))
    x, wg, gu, dn = synth.moe_inputs(cfg)
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    wgd = torch.from_numpy(wg.view(np.int16)).to(dev).view(torch.bfloat16)
    W = w8.MoEWeights.quantize(wgd, torch.from_numpy(gu).to(dev), torch.from_numpy(dn).to(dev), k)
    del gu, dn
    ws = w8.moe_layer_workspace(W, T, w8.BF16, dev)
    w8.moe_layer(W, xd, ws=ws)
    torch.cuda.synchronize()
    inter = w8.moe_layer_intermediates(W, T, ws, w8.BF16)
    off = inter["offsets"].cpu().numpy().astype(np.int64)
    per = E // ngpu
    gbu = int(w8.lib().w8a8_packed_weights_size(1, 2 * I, H))
    gbd = int(w8.lib().w8a8_packed_weights_size(1, H, I))
    shares = []
    for g in range(ngpu):
        e0, e1 = g * per, (g + 1) * per
        r0, r1 = int(off[e0]), int(off[e1])
        rows = r1 - r0
        loc_off = torch.from_numpy((off[e0:e1 + 1] - r0).astype(np.int32)).to(dev)
        sp = inter["sorted_pair"][r0:r1].clone()   # its own (16-byte aligned) buffer
        Bgu, sgu = W.p_gate_up[e0 * gbu:e1 * gbu], W.s_gate_up[e0:e1]
        Bd, sd = W.p_down[e0 * gbd:e1 * gbd], W.s_down[e0:e1]

        def step():
            h = w8.grouped_gemm(inter["xq"], inter["sx"], sp, k, Bgu, sgu, loc_off, w8.EPI_DEQUANT_SWIGLU, w8.BF16,
                                M_total=rows, b_shape=(per, 2 * I, H))
            hq, sh = w8.quant_act(h)
            w8.grouped_gemm(hq, sh, None, 1, Bd, sd, loc_off, w8.EPI_DEQUANT, w8.BF16, M_total=rows,
                            b_shape=(per, H, I))

        for _ in range(args.warmup):
            step()
        e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e_a.record()
        for _ in range(args.steps):
            step()
        e_b.record()
        torch.cuda.synchronize()
        us = e_a.elapsed_time(e_b) * 1e3 / args.steps
        ops = 2 * rows * 3 * H * I
        wbytes = per * 3 * H * I
        shares.append({"gpu": g, "experts": [e0, e1], "rows": rows, "us": round(us, 2),
                       "int8_tops": ops / us / 1e6, "weight_gbs": wbytes / us / 1e3})
        log("share %d: experts %d..%d, %d rows, %.1f us" % (g, e0, e1 - 1, rows, us))
    slow = max(shares, key=lambda r: r["us"])
    result = {
        "metric": "W8A8 MoE expert compute of one GPU's share under %d-way expert parallelism "
                  "(tokens/s of the layer at the pace of the slowest share; all-to-all not included)" % ngpu,
        "value": T / (slow["us"] * 1e-6), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": slow["us"] / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": cfg.name + "_ep%d_share" % ngpu, "tokens": T, "hidden": H, "experts": E,
                   "experts_per_gpu": per, "top_k": k, "expert_intermediate": I,
                   "placement": "contiguous expert indices"},
        "roofline": None,
        "shares": shares,
    }
    print(json.dumps(result), flush=True)


def vendor_int8(args, cfg):
    """The workload's two expert GEMMs as one dense int8 GEMM each (all T*k
    routed rows against one expert's weights: the same operations, none of the
    grouping), timed in the ROCm BLAS library's int8 GEMM (torch._int_mm,
    int32 out) and in this library's one-group grouped GEMM on the same
    operands (int32 out, and the bf16 dequantised out the layer's GEMMs write).
    The codes are rounded normal draws (std 32, clipped to +-127), seeded.
    Context for the kernels' fractions of peak, not a layer measurement."""
    import torch

    import w8a8_int8_quantized_bf16_amd as w8
    dev = "cuda:0"
    torch.cuda.set_device(0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    M = cfg.T * cfg.k

    def codes(r, c):
        return (torch.randn(r, c, device=dev, generator=gen) * 32).round_().clamp_(-127, 127).to(torch.int8)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(args.steps):
            e_a.record()
            fn()
            e_b.record()
            torch.cuda.synchronize()
            ts.append(e_a.elapsed_time(e_b) * 1e3)
        ts.sort()
        return ts[len(ts) // 2]

    rows = []
    for name, K, N in (("gate_up", cfg.H, 2 * cfg.I), ("down", cfg.I, cfg.H)):
        A, B = codes(M, K), codes(N, K)
        ops = 2.0 * M * N * K
        ref = torch._int_mm(A, B.t())
        t_lib = timed(lambda: torch._int_mm(A, B.t()))
        Bp = w8.pack_weights(B.view(1, N, K))
        off = torch.tensor([0, M], dtype=torch.int32, device=dev)
        sa = torch.ones(M, dtype=torch.float32, device=dev)
        sb = torch.ones(N, dtype=torch.float32, device=dev)
        raw = lambda: w8.grouped_gemm(A, sa, None, 1, Bp, sb, off, w8.EPI_RAW_I32, M_total=M, b_shape=(1, N, K))
        same = bool(torch.equal(raw(), ref))
        t_raw = timed(raw)
        t_bf = timed(lambda: w8.grouped_gemm(A, sa, None, 1, Bp, sb, off, w8.EPI_DEQUANT, w8.BF16, M_total=M,
                                             b_shape=(1, N, K)))
        rows.append({"gemm": name, "M": M, "K": K, "N": N, "torch_int_mm_us": round(t_lib, 1),
                     "own_int32_us": round(t_raw, 1), "own_bf16_us": round(t_bf, 1), "int32_equal": same,
                     "torch_int_mm_tops": round(ops / t_lib / 1e6), "own_int32_tops": round(ops / t_raw / 1e6),
                     "own_bf16_tops": round(ops / t_bf / 1e6)})
        log("%s M=%d K=%d N=%d: torch._int_mm %.1f us, own int32 %.1f us (equal %s), own bf16 %.1f us"
            % (name, M, K, N, t_lib, t_raw, same, t_bf))
        del A, B, Bp, ref
        torch.cuda.empty_cache()
    print(json.dumps({"vendor_int8": cfg.name, "median_of": args.steps, "rows": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay measurement after the timed region")
    ap.add_argument("--w4", action="store_true",
                    help="W4A8 gate_up_proj weights (4-bit codes, groups of 128 with scale and offset)")
    ap.add_argument("--ep-share", type=int, default=0, metavar="G",
                    help="time each GPU's share of the workload's experts under G-way expert parallelism")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run plain device copies of MIB MiB (counter calibration) and exit")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic_<stage>_<workload>.json from rocprofv3 counter files and exit")
    ap.add_argument("--traffic-kernel", nargs=3, metavar=("STAGE", "KERNEL_PREFIX", "SOURCE"),
                    default=["gate_up_gemm", "void w8a8::grouped_gemm_kernel<128, 2, 2, 2, unsigned short, true>",
                             "gemm.hip"])
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--vendor-int8", action="store_true",
                    help="time the workload's GEMMs as dense int8 GEMMs in torch._int_mm and in this library, and exit")
    ap.add_argument("--counter-summary", nargs=2, metavar=("PMC_CSV", "TRACE_CSV"),
                    help="print a per-kernel summary of a rocprofv3 --pmc run (matrix-core counters) and exit")
    args = ap.parse_args()
    if args.counter_summary:
        counter_summary(args)
        return
    if args.traffic:
        write_traffic(args)
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(asked for --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import w8a8_int8_quantized_bf16_amd as w8

    if args.workload in synth.DENSE_CONFIGS:
        return bench_dense(args, synth.DENSE_CONFIGS[args.workload])
    if args.ep_share:
        return bench_ep_shares(args, synth.MOE_CONFIGS[args.workload], args.ep_share)
    if args.vendor_int8:
        return vendor_int8(args, synth.MOE_CONFIGS[args.workload])
    cfg = synth.MOE_CONFIGS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    t0 = time.time()
    x, wg, gu, dn = synth.moe_inputs(cfg)
    log("inputs generated in %.1f s" % (time.time() - t0))
    xd = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).to(dev)
    if x.dtype == np.uint16:
        xd = xd.view(torch.bfloat16)
    wgd = torch.from_numpy(wg.view(np.int16)).to(dev).view(torch.bfloat16)
    shared = synth.shared_expert(cfg) if cfg.Is else None
    shared_d = None
    if shared is not None:
        shared_d = (torch.from_numpy(shared[0]).to(dev), torch.from_numpy(shared[1]).to(dev),
                    torch.from_numpy(shared[2].view(np.int16)).to(dev).view(torch.bfloat16))
    W0 = w8.MoEWeights.quantize(wgd, torch.from_numpy(gu).to(dev), torch.from_numpy(dn).to(dev), cfg.k,
                                w4=args.w4, shared=shared_d)
    del shared_d
    # W4 gate_up: half a byte per weight
    wbytes = cfg.E * cfg.H * cfg.I * (2 if args.w4 else 3) + 3 * cfg.H * cfg.Is

    def clone_weights(W):
        cl = lambda t: None if t is None else t.clone()
        return w8.MoEWeights(*[cl(t) for t in W.tensors], k=cfg.k,
                             w4=None if W.w4 is None else tuple(t.clone() for t in W.w4),
                             shared=None if W.shared is None else tuple(t.clone() for t in W.shared))

    copies = args.copies or max(1, min(4, (1 << 30) // max(wbytes, 1) + 1))
    Ws = [W0] + [clone_weights(W0) for _ in range(copies - 1)]
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    ws = w8.moe_layer_workspace(W0, cfg.T, w8.BF16 if x.dtype == np.uint16 else w8.F32, dev)
    out = torch.empty_like(xd)
    nst = w8.LAYER_STAGES

    def make_events(n):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(n)]
        for row in evs:        # torch creates the HIP event on first record
            for e in row:
                e.record()
        return evs

    for i in range(args.warmup):
        w8.moe_layer(Ws[i % copies], xd, ws=ws, out=out)
    # stage breakdown: a pass of its own with a mark after every stage
    nbr = min(args.steps, 20)
    evs = make_events(nbr)
    torch.cuda.synchronize()
    for i in range(nbr):
        w8.moe_layer(Ws[i % copies], xd, ws=ws, out=out, events=evs[i])
    torch.cuda.synchronize()
    stage_us = [0.0] * nst
    for i in range(nbr):
        for j in range(nst):
            stage_us[j] += evs[i][j].elapsed_time(evs[i][j + 1]) * 1e3 / nbr
    dom = int(np.argmax(stage_us))
    # timed region: the layer with marks only at its start and end and around
    # the dominant stage (HIP events on the layer's stream)
    evs = make_events(args.steps)
    keep = (0, dom, dom + 1, nst)
    sel = [[row[j] if j in keep else None for j in range(nst + 1)] for row in evs]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        w8.moe_layer(Ws[i % copies], xd, ws=ws, out=out, events=sel[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    dom_us = sum(evs[i][dom].elapsed_time(evs[i][dom + 1]) for i in range(args.steps)) * 1e3 / args.steps
    step_ms = np.array([evs[i][0].elapsed_time(evs[i][nst]) for i in range(args.steps)])
    p10, p50, p90 = (float(v) for v in np.percentile(step_ms, [10, 50, 90]))
    # After the timed region: the same steps as replays of a HIP graph of
    # `cap` consecutive layer calls (the layer launches kernels only, so it
    # captures whole).  Reported beside the eager rate, as the share of the
    # step that is launch overhead; marks cannot time stages inside a replay.
    graph_rec = None
    if not args.no_graph:
        cap = next(c for c in (10, 5, 4, 2, 1) if args.steps % c == 0)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(cap):
                w8.moe_layer(Ws[i % copies], xd, ws=ws, out=out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(cap):
                w8.moe_layer(Ws[i % copies], xd, ws=ws, out=out)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for _ in range(args.steps // cap):
            graph.replay()
        torch.cuda.synchronize()
        g_ms = (time.perf_counter() - g0) * 1e3 / args.steps
        graph_rec = {"ms_per_step": g_ms, "value": cfg.T / (g_ms * 1e-3), "layer_calls_per_graph": cap}
        del graph

    inter = w8.moe_layer_intermediates(W0, cfg.T, ws, w8.BF16 if x.dtype == np.uint16 else w8.F32)
    counts = np.diff(inter["offsets"].cpu().numpy())
    E_hit = int(np.sum(counts > 0))
    km = kernel_model(cfg, E_hit, args.w4)
    name = w8.STAGE_NAMES[dom]
    t_dom = dom_us * 1e-6
    ops, byts = km[name]["ops"], km[name]["bytes"]
    mfma_bound = ops > 0 and ops / byts > RIDGE
    if mfma_bound:
        achieved, peak, unit = ops / t_dom / 1e12, INT8_PEAK_TOPS, "TOP/s"
    else:
        achieved, peak, unit = byts / t_dom / 1e9, HBM_PEAK_GBS, "GB/s"
    ms_per_step = elapsed * 1e3 / args.steps
    lops, lbytes = layer_model(cfg, E_hit, args.w4)
    t_step = elapsed / args.steps
    roof_t = max(lops / (INT8_PEAK_TOPS * 1e12), lbytes / (HBM_PEAK_GBS * 1e9))
    result = {
        "metric": "W8A8 MoE layer tokens/s; int8 TOPS and HBM GB/s as % of MI355X roofline",
        "value": cfg.T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "step_ms_p10_p50_p90": [round(p10, 4), round(p50, 4), round(p90, 4)],
        "tokens_per_s_at_median_step": cfg.T / (p50 * 1e-3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": cfg.name + ("_w4a8" if args.w4 else ""), "tokens": cfg.T, "hidden": cfg.H,
                   "experts": cfg.E, "top_k": cfg.k, "gate_up_weights": "w4a8" if args.w4 else "w8a8",
                   "expert_intermediate": cfg.I, "x_dtype": cfg.x_dtype, "experts_hit": E_hit,
                   "weight_copies_rotated": copies},
        "roofline": {"kernel": name, "bound": "mfma" if mfma_bound else "hbm", "achieved": achieved, "peak": peak,
                     "unit": unit, "frac": achieved / peak,
                     "traffic": None if args.w4 or cfg.Is else traffic_for(name, cfg.name),
                     "avg_launch_us": dom_us, "alg_bytes_per_launch": byts, "int8_ops_per_launch": ops},
        "layer": {"int8_tops": lops / t_step / 1e12, "int8_tops_frac": lops / t_step / 1e12 / INT8_PEAK_TOPS,
                  "alg_gbs": lbytes / t_step / 1e9, "alg_gbs_frac": lbytes / t_step / 1e9 / HBM_PEAK_GBS,
                  "roof_time_us": roof_t * 1e6, "roofline_frac": roof_t / t_step,
                  "stage_us": dict(zip(w8.STAGE_NAMES, [round(v, 2) for v in stage_us])),
                  "expert_rows_min_max": [int(counts.min()), int(counts.max())]},
    }
    if graph_rec is not None:
        result["hip_graph_replay"] = graph_rec
    if cfg.Is:
        result["config"]["shared_expert_intermediate"] = cfg.Is
        # the stage's time covers the routed and the shared expert's launches
        result["roofline"]["kernel"] = name + " (routed and shared-expert launches)"
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(dict(cfg=cfg, x=x, wg=wg, gu=gu, dn=dn, shared=shared),
                                              args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
