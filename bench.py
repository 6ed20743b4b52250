#!/usr/bin/env python3
"""Benchmark of the A8W8 decode linears on one MI355X.

One step = one call of a8w8_layer_linears (QKV, O, Gate/Up, split-K Down with all the
quantize / dequant / SiLU / RNE work) on a Qwen3-14B-shaped layer at decode batch 1.
Steps rotate over several independently generated weight sets (1.3 GB at the default
4 sets) so the 256 MB last-level cache cannot serve weights from a previous step.

Prints one JSON line: INT8-weight HBM GB/s (value), microseconds per layer, the
roofline of the dominant kernel (the Gate/Up GEMM) from HIP events recorded around it
on the library's stream, and the CPU oracle's throughput on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--sets S] [--config 2|3]
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/layer and INT8-weight HBM GB/s (% of peak), A8W8 decode linears at batch 1"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
GATEUP_KERNEL = 5     # kernel number of the Gate/Up GEMM inside a8w8_layer_linears
GATEUP_NAME = "decode_kernel<2, 2,"        # its symbol in rocprofv3 counter tables (M <= 16)
GATEUP_NAME_SK = "streamk_kernel<2, 2,"    # ... with more rows (the stream-K kernel)
PACK_NAME = "pack_tiled_kernel"            # plain permuting copy: the counter calibration
PMC_FILE = os.path.join(ROOT, "profiles", "gateup_gemm_pmc.json")
PMC_MD = os.path.join(ROOT, "profiles", "layer_linears_m1_pmc.md")
PMC_FILE_M16 = os.path.join(ROOT, "profiles", "gateup_gemm_m16_pmc.json")
PMC_MD_M16 = os.path.join(ROOT, "profiles", "stack40_m16_pmc.md")


def pmc_target(cfg):
    """(summary json, summary markdown, Gate/Up kernel symbol) of a config's counters."""
    if cfg.M > 4:
        return PMC_FILE_M16, PMC_MD_M16, GATEUP_NAME if cfg.M <= 16 else GATEUP_NAME_SK
    return PMC_FILE, PMC_MD, GATEUP_NAME


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--sets", type=int, default=4, help="weight sets rotated across steps")
    p.add_argument("--config", type=int, default=2,
                   help="0: toy MLP block; 1: Qwen3-14B MLP block M=1; 2: layer M=1; "
                        "3: 40-layer M=16 stack; 4: W8A16 prefill MLP M=256")
    p.add_argument("--stream-ceiling", action="store_true",
                   help="time a plain streaming read of the layer's weight bytes (the "
                        "achievable HBM read rate the decode GEMMs are measured against)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--qk-rope", action="store_true",
                   help="time the QK-norm + RoPE + KV-cache write step (Qwen3-14B heads, M=1 and 16)")
    p.add_argument("--attention", action="store_true",
                   help="time decode attention over the paged cache (Qwen3-14B heads, M=1 and 16)")
    p.add_argument("--context", type=int, default=1024,
                   help="context length for --attention and --decode-layer")
    p.add_argument("--decode-layer", action="store_true",
                   help="time the Qwen3-14B decode layer with real attention (M=1 and 16)")
    p.add_argument("--layer", action="store_true",
                   help="with --config 4: the whole prefill layer (QKV, O and the MLP block)")
    p.add_argument("--graph", type=int, default=1,
                   help="also time the steps replayed from one captured HIP graph (0: skip)")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="summarise two rocprofv3 --pmc runs of this bench (FETCH_SIZE, then "
                        "WRITE_SIZE, csv output) into the profiles/ traffic files; no GPU use")
    p.add_argument("--pmc-commands", nargs=2, default=("?", "?"),
                   help="the two rocprofv3 command lines, recorded in the summary")
    return p.parse_args()


def event_stats(torch, run, n: int) -> dict:
    """Calls run(i) n times back to back on the current stream with a HIP event after
    each call: per-call microseconds as median, 10th and 90th percentile and mean."""
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    evs[0].record(stream)
    for i in range(n):
        run(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    d = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n)])
    return pct_stats(d)


def pct_stats(d) -> dict:
    d = np.asarray(d, dtype=np.float64)
    return {"median": round(float(np.median(d)), 2), "p10": round(float(np.percentile(d, 10)), 2),
            "p90": round(float(np.percentile(d, 90)), 2), "mean": round(float(d.mean()), 2)}


def emit(line: dict) -> None:
    """Prints the bench line; a roofline fraction above 1 means the timing bracketed the
    wrong work, so the run then fails."""
    print(json.dumps(line))
    frac = (line.get("roofline") or {}).get("frac")
    if frac is not None and frac > 1.0:
        print(f"[bench] roofline fraction {frac} > 1: the timed interval cannot hold that "
              f"kernel's bytes; failing", file=sys.stderr)
        sys.exit(3)


def code_text(src: str) -> str:
    """Source text without comments and with whitespace runs collapsed: what the compiler
    sees of it, so that a comment edit does not mark the counters stale."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash(read=None) -> str:
    """Hash of the decode kernels' code (comments and layout excluded)."""
    h = hashlib.sha256()
    for f in ("gemm_decode.hip", "gemm_streamk.hip", "device_common.h", "internal.h"):
        if read is None:
            with open(os.path.join(ROOT, "w8a8_quantized_decode_amd", "csrc", f)) as fh:
                text = fh.read()
        else:
            text = read(f)
        h.update(code_text(text).encode())
    return h.hexdigest()[:16]


def measured_traffic(cfg):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None if the
    summary is missing or was taken on a different kernel source."""
    try:
        with open(pmc_target(cfg)[0]) as f:
            pmc = json.load(f)
    except (OSError, ValueError):
        return None
    if pmc.get("kernel_source_hash") != kernel_source_hash():
        return None
    return pmc.get("hbm_bytes_per_dispatch")


def pmc_summary(fetch_csv: str, write_csv: str, commands, cfg) -> None:
    """Turn two rocprofv3 counter tables of this bench into HBM bytes per dispatch.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled by the factor that
    makes them agree with the known size of the weight-packing copy the bench runs at
    start-up (it reads and writes N*K bytes once), then averaged per kernel."""
    import csv
    from collections import defaultdict

    H, I, n_qkv, M = cfg.H, cfg.I, cfg.n_qkv, cfg.M
    pack_sizes = {n_qkv * H, H * H, I * H}
    pmc_file, pmc_md, gu_name = pmc_target(cfg)

    def load(path, counter):
        per_kernel, pack_alg, pack_cnt = defaultdict(list), 0.0, 0.0
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                kib = float(r["Counter_Value"])
                name = r["Kernel_Name"]
                if PACK_NAME in name:
                    nbytes = int(r["Grid_Size"]) * 16      # one thread per 16-byte chunk
                    if nbytes not in pack_sizes:
                        raise SystemExit(f"pack dispatch of {nbytes} bytes is not a weight")
                    pack_alg += nbytes
                    pack_cnt += kib * 1024
                per_kernel[name].append(kib)
        if pack_cnt == 0:
            raise SystemExit(f"no {PACK_NAME} dispatch in {path}: nothing to calibrate on")
        return per_kernel, pack_alg / pack_cnt

    fetch, f_fetch = load(fetch_csv, "FETCH_SIZE")
    write, f_write = load(write_csv, "WRITE_SIZE")
    rows, gu = [], None
    for name in sorted(set(fetch) & set(write), key=lambda n: -np.mean(fetch[n])):
        fk, wk = float(np.mean(fetch[name])), float(np.mean(write[name]))
        hbm = fk * 1024 * f_fetch + wk * 1024 * f_write
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")[:90]
        rows.append((short, len(fetch[name]), fk, wk, hbm))
        if gu_name in name:
            gu = dict(fetch_kib=fk, write_kib=wk, hbm_bytes_per_dispatch=round(hbm))
    if gu is None:
        raise SystemExit(f"no {gu_name} dispatch in the counter tables")
    gu_alg = 2 * I * H + 2 * I * 4 + M * H + M * 4 + M * I * 4
    summary = dict(kernel=gu_name, workload=cfg.name, kernel_source_hash=kernel_source_hash(),
                   fetch_factor=round(f_fetch, 5), write_factor=round(f_write, 5),
                   algorithmic_bytes_per_dispatch=gu_alg,
                   traffic_over_algorithmic=round(gu["hbm_bytes_per_dispatch"] / gu_alg, 4),
                   commands=list(commands), **gu)
    with open(pmc_file, "w") as f:
        json.dump(summary, f, indent=1)
        f.write("\n")
    lines = [f"# HBM traffic per dispatch, {cfg.name}", "",
             "Two rocprofv3 counter passes over the same bench run:", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", f"Summarised by `python bench.py --pmc-summary <fetch csv> <write csv>`.",
              f"Calibration on the weight-packing copy (reads and writes N*K bytes once): "
              f"FETCH_SIZE x {f_fetch:.4f}, WRITE_SIZE x {f_write:.4f}.", "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (calibrated) |",
              "|---|---|---|---|---|"]
    lines += [f"| `{n}` | {c} | {fk:.1f} | {wk:.1f} | {hbm / 1e6:.2f} MB |" for n, c, fk, wk, hbm in rows]
    lines += ["", f"Gate/Up GEMM: {gu['hbm_bytes_per_dispatch'] / 1e6:.2f} MB per dispatch against "
              f"{gu_alg / 1e6:.2f} MB algorithmic ({summary['traffic_over_algorithmic']:.4f}x).",
              f"Kernel source hash: {summary['kernel_source_hash']}.", ""]
    with open(pmc_md, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(summary))


def cpu_baseline(cfg, seconds: float):
    """The oracle as it stands, timed on whole layers of the same workload."""
    import oracle as O
    from w8a8_quantized_decode_amd import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS default
        cores = os.cpu_count() or 1
    done, t_total = 0, 0.0
    wbytes = 0
    inputs = [synth.layer_inputs(cfg, layer=100 + i, M=cfg.M) for i in range(2)]
    while t_total < seconds:
        d = inputs[done % len(inputs)]
        t0 = time.perf_counter()
        O.layer_linears_decode(d["x"], d["gamma_in"], d["gamma_post"], cfg.eps, d["w_qkv"],
                               d["s_qkv"], d["w_o"], d["s_o"], d["w_gate"], d["s_gate"],
                               d["w_up"], d["s_up"], d["w_down"], d["s_down"], cfg.n_q_heads,
                               cfg.head_dim, cfg.split_k)
        t_total += time.perf_counter() - t0
        wbytes += sum(d[k].nbytes for k in ("w_qkv", "w_o", "w_gate", "w_up", "w_down"))
        done += 1
    return {"value": round(wbytes / t_total / 1e9, 3), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} Qwen3-14B layer-linears decode passes at M={cfg.M} over 2 "
                      f"seeded layers (input generation excluded), {t_total:.1f} s",
            "us_per_layer": round(t_total / done * 1e6, 1)}


def oracle_per_call(run, seconds: float, sample: str):
    """The oracle as it stands, called on the host until about `seconds` have passed (at
    least once) on the benchmarked workload's own inputs: microseconds per call."""
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS default
        cores = os.cpu_count() or 1
    n, t = 0, 0.0
    while n == 0 or t < seconds:
        t0 = time.perf_counter()
        with np.errstate(all="ignore"):  # random bit patterns include BF16 NaN and Inf
            run()
        t += time.perf_counter() - t0
        n += 1
    return {"value": round(t / n * 1e6, 1), "unit": "us per call", "cores": int(cores),
            "kind": "oracle", "sample": f"{n} oracle calls on {sample} (inputs prepared "
                                        f"beforehand), {t:.1f} s"}


def bench_prefill(args, cfg, torch, B) -> None:
    """Secondary line: the W8A16 prefill MLP block (RMSNorm, Gate/Up, SiLU, Down + residual)
    at M = 256; value in TFLOP/s of the three GEMMs, roofline of the Gate/Up GEMM (with
    its leftover-tile reduction) against the BF16 matrix-core peak."""
    from w8a8_quantized_decode_amd import synth
    M, H, I = cfg.M, cfg.H, cfg.I
    d = synth.mlp_inputs(cfg, M=M)

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to("cuda")

    def upw(w, s):
        rm = up(w)
        tiled = torch.empty_like(rm)
        B.a8w8_pack_weight(rm, tiled)
        return (tiled, up(s), B.LAYOUT_TILED)

    gate, upw_, down = upw(d["w_gate"], d["s_gate"]), upw(d["w_up"], d["s_up"]), upw(d["w_down"], d["s_down"])
    x, g, res = up(d["x"]), up(d["gamma_post"]), up(d["res"])
    out = torch.empty_like(res)
    ws = torch.zeros(B.a8w8_workspace_bytes(B.OP_MLP_BLOCK, M, H, I, 0, cfg.split_k,
                                            B.MODE_PREFILL_W8A16), dtype=torch.uint8, device="cuda")

    def step(taps=None):
        B.a8w8_mlp_block(x, g, cfg.eps, gate, upw_, down, res, out, ws, split_k=cfg.split_k,
                         mode=B.MODE_PREFILL_W8A16, taps=taps)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    flops = 2.0 * M * 3 * H * I
    evs = []
    for _ in range(min(args.steps, 50)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    for a, b in evs:
        step({"ev_start": a.cuda_event, "ev_stop": b.cuda_event, "ev_kernel": GATEUP_KERNEL})
    torch.cuda.synchronize()
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    gu_flops = 2.0 * M * 2 * H * I
    achieved = gu_flops / (k_ms * 1e-3) / 1e12
    out_line = {
        "metric": "W8A16 prefill MLP block TFLOP/s (Gate/Up + Down GEMMs), BF16 matrix cores",
        "value": round(flops / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded PCG64, Qwen3-14B shapes, random INT8 weights)",
        "config": {"workload": cfg.name, "M": M, "hidden": H, "intermediate": I},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "prefill_gemm_kernel<EPI_PF_SILU> + reduction",
                     "kernel_us": round(k_ms * 1e3, 2), "algorithmic_flops_per_launch": gu_flops},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle as O
        out_line["cpu_baseline"] = oracle_per_call(
            lambda: O.prefill_mlp(d["x"], d["gamma_post"], cfg.eps, d["w_gate"], d["s_gate"],
                                  d["w_up"], d["s_up"], d["w_down"], d["s_down"], d["res"]),
            args.cpu_seconds, f"the same M={M} prefill MLP block")
    emit((out_line))


def bench_prefill_layer(args, torch, B) -> None:
    """The W8A16 prefill layer at M = 256 (QKV, O, then the MLP block): TFLOP/s of its
    five GEMMs; the roofline is the whole call against the BF16 matrix-core peak."""
    from w8a8_quantized_decode_amd import synth
    cfg = synth.CONFIGS[2]
    M, H, I, n_qkv = synth.CONFIGS[4].M, cfg.H, cfg.I, cfg.n_qkv
    d = synth.layer_inputs(cfg, layer=0, M=M)

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to("cuda")

    def upw(w, s):
        rm = up(w)
        tiled = torch.empty_like(rm)
        B.a8w8_pack_weight(rm, tiled)
        return (tiled, up(s), B.LAYOUT_TILED)

    w = {k: upw(d["w_" + k], d["s_" + k]) for k in ("qkv", "o", "gate", "up", "down")}
    x, gin, gpost = up(d["x"]), up(d["gamma_in"]), up(d["gamma_post"])
    out = torch.empty_like(x)
    ws = torch.zeros(B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, M, H, I, n_qkv, 2,
                                            B.MODE_PREFILL_W8A16), dtype=torch.uint8, device="cuda")

    def step():
        B.a8w8_layer_linears_prefill(x, gin, gpost, cfg.eps, w["qkv"], w["o"], w["gate"], w["up"],
                                     w["down"], out, ws, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    flops = 2.0 * M * (n_qkv * H + H * H + 3 * H * I)
    tf = flops / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        cpu = oracle_per_call(
            lambda: O.layer_linears_prefill(d["x"], d["gamma_in"], d["gamma_post"], cfg.eps,
                                            d["w_qkv"], d["s_qkv"], d["w_o"], d["s_o"],
                                            d["w_gate"], d["s_gate"], d["w_up"], d["s_up"],
                                            d["w_down"], d["s_down"], cfg.n_q_heads,
                                            cfg.head_dim),
            args.cpu_seconds, f"the same M={M} prefill layer")
    emit(({
        "metric": "W8A16 prefill layer TFLOP/s (QKV, O, Gate/Up, Down GEMMs), BF16 matrix cores",
        "value": round(tf, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded PCG64, Qwen3-14B shapes, random INT8 weights)",
        "config": {"workload": "Qwen3-14B W8A16 prefill layer linears, M=256", "M": M,
                   "hidden": H, "intermediate": I, "n_qkv": n_qkv},
        "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "whole call (norm, QKV, slice copy, O, MLP kernels)",
                     "algorithmic_flops_per_launch": flops},
        "cpu_baseline": cpu}))


def bench_qk_rope(args, torch, B) -> None:
    """QK-norm + RoPE + paged BF16 KV-cache write after QKV, Qwen3-14B heads (40 Q and 8 KV
    heads of 128) at the decode batches 1 and 16: microseconds per call from HIP events
    over calls replayed from a captured graph, and the bytes the step must move per call (qkv read, q out,
    K and V written, the gains, the two table rows) over that time against HBM peak."""
    from w8a8_quantized_decode_amd import synth
    nq, nkv, d, bs, bps = 40, 8, 128, 16, 64
    cos, sin = synth.rope_tables(bs * bps, d)
    rows = []
    cpu = None
    for M in (1, 16):
        rng = np.random.default_rng(M)
        qkv_h = rng.integers(0, 1 << 15, size=(M, (nq + 2 * nkv) * d), dtype=np.int16)
        qkv = torch.from_numpy(qkv_h).to("cuda")
        g = torch.full((d,), 0x3F80, dtype=torch.int16, device="cuda")   # BF16 1.0
        pos = torch.from_numpy(rng.integers(0, bs * bps, size=M).astype(np.int32)).to("cuda")
        bt = torch.from_numpy(np.arange(M * bps, dtype=np.int32).reshape(M, bps)).to("cuda")
        kc = torch.zeros((M * bps, bs, nkv, d), dtype=torch.int16, device="cuda")
        vc = torch.zeros_like(kc)
        q = torch.empty((M, nq * d), dtype=torch.int16, device="cuda")
        ct, st = torch.from_numpy(cos).to("cuda"), torch.from_numpy(sin).to("cuda")

        def call():
            B.a8w8_qk_norm_rope_kv(qkv, nq, nkv, d, g, g, 1e-6, ct, st, pos, bt, kc, vc, q)
        for _ in range(args.warmup):
            call()
        # Replayed from a captured graph of 20 calls, so host launch cost does not pace it.
        gr = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(gr):
            for _ in range(20):
                call()
        gr.replay()
        reps = max(1, args.steps // 20)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            gr.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / (reps * 20) * 1e3
        nbytes = M * ((nq + 2 * nkv) * d * 2 + nq * d * 2 + 2 * nkv * d * 2 + 4 + 4 + d * 4) + 2 * d * 2
        if M == 16 and not args.no_cpu_baseline:
            import oracle as O
            g_h = np.full(d, 0x3F80, np.uint16)
            pos_h, bt_h = pos.cpu().numpy(), bt.cpu().numpy()
            kc_h = np.zeros((M * bps, bs, nkv, d), np.uint16)
            cpu = oracle_per_call(
                lambda: O.qk_norm_rope_kv(qkv_h.view(np.uint16), nq, nkv, d, g_h, g_h, 1e-6,
                                          cos, sin, pos_h, bt_h, kc_h, kc_h.copy()),
                min(args.cpu_seconds, 5.0), "the same M=16 inputs")
        rows.append({"M": M, "us_per_call": round(us, 2), "bytes_per_call": nbytes,
                     "gb_s": round(nbytes / (us * 1e-6) / 1e9, 2)})
    r16 = rows[-1]
    emit(({
        "metric": "QK-norm + RoPE + paged BF16 KV-cache write, microseconds per call",
        "value": r16["us_per_call"], "unit": "us", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r16["us_per_call"] / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (Qwen3-14B head counts, random BF16 rows)",
        "config": {"workload": "QK-norm + RoPE + KV write, 40 Q / 8 KV heads of 128, M=16",
                   "per_batch": rows},
        "roofline": {"bound": "hbm", "achieved": r16["gb_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(r16["gb_s"] / HBM_PEAK_GBS, 6), "traffic": None,
                     "kernel": "qk_rope_kernel (latency-bound: a few KB per call)",
                     "algorithmic_bytes_per_launch": r16["bytes_per_call"]},
        "cpu_baseline": cpu}))


def bench_attention(args, torch, B) -> None:
    """Decode attention over the paged BF16 KV cache, Qwen3-14B heads (40 Q, 8 KV of 128),
    every row at the same context length, at the decode batches 1 and 16: microseconds per
    call (graph-replayed) and the cache bytes the step must read (K and V of every
    position of every row) over that time against HBM peak."""
    import math
    nq, nkv, d, bs = 40, 8, 128, 16
    L = args.context
    bps = (L + bs - 1) // bs
    rows = []
    cpu = None
    for M in (1, 16):
        rng = np.random.default_rng(M)
        nblocks = M * bps
        q_h = rng.integers(0x3C00, 0x3F80, size=(M, nq * d), dtype=np.int16)
        kc_h = rng.integers(0x3C00, 0x3F80, size=(nblocks, bs, nkv, d), dtype=np.int16)
        vc_h = rng.integers(0x3C00, 0x3F80, size=(nblocks, bs, nkv, d), dtype=np.int16)
        bt_h = rng.permutation(nblocks).astype(np.int32).reshape(M, bps)
        q, kc, vc = (torch.from_numpy(a).to("cuda") for a in (q_h, kc_h, vc_h))
        bt = torch.from_numpy(bt_h).to("cuda")
        lens = torch.full((M,), L, dtype=torch.int32, device="cuda")
        out = torch.empty_like(q)
        nws = B.a8w8_decode_attention_workspace_bytes(M, nq, nkv, d, bps * bs)
        ws = torch.zeros((nws,), dtype=torch.uint8, device="cuda") if nws else None

        def call():
            B.a8w8_decode_attention(q, nq, nkv, d, kc, vc, bt, lens, 1.0 / math.sqrt(d), out,
                                    workspace=ws)
        for _ in range(3):
            call()
        gr = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(gr):
            for _ in range(10):
                call()
        gr.replay()
        reps = max(1, args.steps // 10)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            gr.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / (reps * 10) * 1e3
        nbytes = M * (L * nkv * d * 2 * 2 + 2 * nq * d * 2)
        if M == 16 and not args.no_cpu_baseline:
            import oracle as O
            cpu = oracle_per_call(
                lambda: O.decode_attention(q_h.view(np.uint16), nq, nkv, d, kc_h.view(np.uint16),
                                           vc_h.view(np.uint16), bt_h, np.full(M, L, np.int32),
                                           1.0 / math.sqrt(d)),
                min(args.cpu_seconds, 10.0), f"the same M=16 inputs at context {L}")
        rows.append({"M": M, "context": L, "workspace_bytes": nws,
                     "us_per_call": round(us, 2), "bytes_per_call": nbytes,
                     "gb_s": round(nbytes / (us * 1e-6) / 1e9, 1)})
    r16 = rows[-1]
    emit(({
        "metric": "decode attention over the paged BF16 KV cache, microseconds per call",
        "value": r16["us_per_call"], "unit": "us", "n_gpus": 1, "steps": args.steps,
        "warmup": 3, "ms_per_step": round(r16["us_per_call"] / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (Qwen3-14B head counts, random BF16 cache)",
        "config": {"workload": f"decode attention, 40 Q / 8 KV heads of 128, context {L}, M=16",
                   "per_batch": rows},
        "roofline": {"bound": "hbm", "achieved": r16["gb_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(r16["gb_s"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "attn_split_kernel + attn_combine_kernel (one call)",
                     "algorithmic_bytes_per_launch": r16["bytes_per_call"]},
        "cpu_baseline": cpu}))


def bench_decode_layer(args, torch, B) -> None:
    """The Qwen3-14B decode layer with real attention (QKV, QK-norm + RoPE + KV write,
    paged attention at context L, O, MLP) at the decode batches 1 and 16: microseconds per
    layer from HIP events over graph-replayed calls, and the bytes the layer must read
    (INT8 weights and scales of the five GEMMs, K and V of every attended position) over
    that time against HBM peak."""
    from w8a8_quantized_decode_amd import synth
    cfg = synth.CONFIGS[2]
    H, I, nq, nkv, hd = cfg.H, cfg.I, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    L = args.context
    rows, cpu = [], None

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to("cuda")

    def upw(w, s):
        rm = up(w)
        tiled = torch.empty_like(rm)
        B.a8w8_pack_weight(rm, tiled)
        return (tiled, up(s), B.LAYOUT_TILED)

    d0 = synth.layer_inputs(cfg, layer=0, M=16)
    w = {k: upw(d0["w_" + k], d0["s_" + k]) for k in ("qkv", "o", "gate", "up", "down")}
    wbytes = sum(d0["w_" + k].nbytes + d0["s_" + k].nbytes for k in ("qkv", "o", "gate", "up", "down"))
    for M in (1, 16):
        d = synth.layer_inputs(cfg, layer=0, M=M)
        a = synth.attention_inputs(cfg, [L] * M, block_size=16)
        x, gin, gpost = up(d["x"]), up(d["gamma_in"]), up(d["gamma_post"])
        kc, vc = up(a["k_cache"]), up(a["v_cache"])
        t = {k: up(a[k]) for k in ("q_gamma", "k_gamma", "cos", "sin", "positions",
                                   "context_lens", "block_table")}
        out = torch.empty_like(x)
        q_rot = torch.empty((M, nq * hd), dtype=torch.int16, device="cuda")
        attn = torch.empty_like(q_rot)
        ws = torch.zeros(B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, M, H, I, cfg.n_qkv,
                                                cfg.split_k), dtype=torch.uint8, device="cuda")
        nws = B.a8w8_decode_attention_workspace_bytes(M, nq, nkv, hd, a["block_table"].shape[1] * 16)
        aws = torch.zeros((max(nws, 256),), dtype=torch.uint8, device="cuda")

        def call():
            B.a8w8_decode_layer(x, gin, gpost, cfg.eps, w["qkv"], w["o"], w["gate"], w["up"],
                                w["down"], out, ws, nq, nkv, hd, q_gamma=t["q_gamma"],
                                k_gamma=t["k_gamma"], qk_eps=cfg.eps, cos_table=t["cos"],
                                sin_table=t["sin"], positions=t["positions"],
                                context_lens=t["context_lens"], block_table=t["block_table"],
                                k_cache=kc, v_cache=vc, scale=a["scale"], q_rot=q_rot,
                                attn=attn, attn_workspace=aws, split_k=cfg.split_k)
        for _ in range(args.warmup):
            call()
        gr = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(gr):
            for _ in range(10):
                call()
        gr.replay()
        reps = max(1, args.steps // 10)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / (reps * 10) * 1e3
        nbytes = wbytes + M * L * nkv * hd * 2 * 2
        rows.append({"M": M, "context": L, "us_per_layer": round(us, 2), "bytes": nbytes,
                     "gb_s": round(nbytes / (us * 1e-6) / 1e9, 1)})
        if M == 1 and not args.no_cpu_baseline:
            import oracle as O
            cpu = oracle_per_call(
                lambda: O.decode_layer(d["x"], d["gamma_in"], d["gamma_post"], cfg.eps,
                                       d["w_qkv"], d["s_qkv"], d["w_o"], d["s_o"], d["w_gate"],
                                       d["s_gate"], d["w_up"], d["s_up"], d["w_down"],
                                       d["s_down"], nq, nkv, hd, cfg.split_k, a["q_gamma"],
                                       a["k_gamma"], cfg.eps, a["cos"], a["sin"],
                                       a["positions"], a["context_lens"], a["block_table"],
                                       a["k_cache"], a["v_cache"], a["scale"]),
                min(args.cpu_seconds, 10.0), f"the same M=1 layer at context {L}")
    r1 = rows[0]
    emit(({
        "metric": "Qwen3-14B A8W8 decode layer with paged attention, microseconds per layer",
        "value": r1["us_per_layer"], "unit": "us", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r1["us_per_layer"] / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic (seeded PCG64, Qwen3-14B shapes, random INT8 weights and BF16 cache)",
        "config": {"workload": f"Qwen3-14B decode layer, real attention at context {L}, M=1",
                   "per_batch": rows},
        "roofline": {"bound": "hbm", "achieved": r1["gb_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(r1["gb_s"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "whole layer (QKV, QK-RoPE, attention split + merge, O, MLP)",
                     "algorithmic_bytes_per_launch": r1["bytes"]},
        "cpu_baseline": cpu}))


def bench_mlp(args, cfg, torch, B) -> None:
    """Configs 0 and 1: the decode MLP block (RMSNorm, quantization, Gate/Up, SiLU * up,
    requantization, split Down + residual) at M = 1.  Value: INT8-weight GB/s; roofline:
    the Gate/Up GEMM from HIP events around its launch.  Weight sets rotate across steps
    so the last-level cache cannot serve them, except for the toy block (0.6 MB of
    weights), which stays cache-resident and is flagged so."""
    from w8a8_quantized_decode_amd import synth
    M, H, I = cfg.M, cfg.H, cfg.I
    toy = cfg.index == 0
    nsets = 1 if toy else max(1, args.sets)

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to("cuda")

    def upw(w, s_):
        rm = up(w)
        tiled = torch.empty_like(rm)
        B.a8w8_pack_weight(rm, tiled)
        return (tiled, up(s_), B.LAYOUT_TILED)

    sets = []
    for si in range(nsets):
        d = synth.mlp_inputs(cfg, layer=si, M=M)
        sets.append(dict(g=up(d["gamma_post"]), gate=upw(d["w_gate"], d["s_gate"]),
                         up=upw(d["w_up"], d["s_up"]), down=upw(d["w_down"], d["s_down"])))
        if si == 0:
            x0, res0, d0 = up(d["x"]), up(d["res"]), d
    out = torch.empty_like(res0)
    ws = torch.zeros(B.a8w8_workspace_bytes(B.OP_MLP_BLOCK, M, H, I, 0, cfg.split_k),
                     dtype=torch.uint8, device="cuda")

    def step(i, taps=None):
        w = sets[i % nsets]
        B.a8w8_mlp_block(x0, w["g"], cfg.eps, w["gate"], w["up"], w["down"], res0, out, ws,
                         split_k=cfg.split_k, taps=taps)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / args.steps * 1e6
    per_step = event_stats(torch, step, min(args.steps, 200))
    wbytes = 3 * I * H
    gbs = wbytes / (us * 1e-6) / 1e9

    n_ev = min(args.steps, 100)
    evs = []
    for _ in range(n_ev):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        step(i, {"ev_start": a.cuda_event, "ev_stop": b.cuda_event, "ev_kernel": GATEUP_KERNEL})
    torch.cuda.synchronize()
    k_us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    gu_bytes = 2 * I * H + 2 * I * 4 + M * H * 2 + H * 2 + M * I * 4
    achieved = gu_bytes / (float(np.mean(k_us)) * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        cpu = oracle_per_call(
            lambda: O.mlp_block_decode(d0["x"], d0["gamma_post"], cfg.eps, d0["w_gate"],
                                       d0["s_gate"], d0["w_up"], d0["s_up"], d0["w_down"],
                                       d0["s_down"], d0["res"], split_k=cfg.split_k),
            args.cpu_seconds, f"the same M={M} MLP block")
    emit({
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic (seeded PCG64, " + ("toy shapes; weights stay cache-resident)"
                                               if toy else "Qwen3-14B shapes, random INT8 weights)"),
        "us_per_block": round(us, 2), "us_per_step_events": per_step,
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "config": {"workload": cfg.name, "M": M, "hidden": H, "intermediate": I,
                   "split_k": cfg.split_k, "weight_sets": nsets, "int8_weight_bytes": wbytes,
                   "cache_resident": toy, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_kernel<EPI_SILU> (Gate/Up)",
                     "kernel_us": round(float(np.mean(k_us)), 2),
                     "kernel_us_stats": pct_stats(k_us),
                     "algorithmic_bytes_per_launch": gu_bytes},
        "cpu_baseline": cpu})


def bench_stream_ceiling(args, torch) -> None:
    """A plain streaming read (measure/stream_read.hip: one 16-wave workgroup per CU, each
    wave reading a contiguous run, 1 KB loads, eight in flight) over the byte counts of
    the layer's weights: the whole layer in one read, and its four GEMMs' weight bytes
    as four reads back to back.  Buffers rotate so the last-level cache cannot serve
    them.  This is the achievable HBM read rate the decode GEMMs are compared against."""
    import ctypes
    from w8a8_quantized_decode_amd import build as BD
    from w8a8_quantized_decode_amd import synth
    if not os.path.exists(BD.MEASURE_LIB):
        raise SystemExit(f"{BD.MEASURE_LIB} is missing: build first")
    L = ctypes.CDLL(BD.MEASURE_LIB)
    L.a8w8m_stream_read.restype = ctypes.c_int
    L.a8w8m_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_void_p]
    cfg = synth.CONFIGS[2]
    H, I, n_qkv = cfg.H, cfg.I, cfg.n_qkv
    parts = [n_qkv * H, H * H, 2 * I * H, H * I]
    total = sum(parts)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nbuf = 4
    bufs = [torch.full((total,), i + 1, dtype=torch.int8, device="cuda") for i in range(nbuf)]
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def read(buf, off, n):
        rc = L.a8w8m_stream_read(buf.data_ptr() + off, n, out.data_ptr(), cus, st)
        if rc:
            raise SystemExit(f"a8w8m_stream_read failed: {rc}")

    def whole(i):
        read(bufs[i % nbuf], 0, total)

    def four(i):
        off = 0
        for n in parts:
            read(bufs[i % nbuf], off, n)
            off += n

    for i in range(args.warmup):
        whole(i)
        four(i)
    torch.cuda.synchronize()
    n = min(args.steps, 200)
    w = event_stats(torch, whole, n)
    f = event_stats(torch, four, n)
    gbs = total / (w["median"] * 1e-6) / 1e9
    emit({
        "metric": "streaming-read ceiling over the layer's INT8 weight bytes", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "ms_per_step": round(w["median"] / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8", "data": "device buffers, rotated (4 x 330 MB)",
        "config": {"workload": "plain streaming read of 330.3 MB (one read) and of the four "
                               "GEMMs' weight bytes (four reads back to back)",
                   "bytes": total, "parts": parts, "cus": cus},
        "one_read_us": w, "four_reads_us": f,
        "four_reads_gb_s": round(total / (f["median"] * 1e-6) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "stream_runs (measure/stream_read.hip)",
                     "algorithmic_bytes_per_launch": total},
        "cpu_baseline": None})


def main():
    args = parse()
    if args.pmc_summary:
        from w8a8_quantized_decode_amd import synth
        pmc_summary(*args.pmc_summary, args.pmc_commands, synth.CONFIGS[args.config])
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1 "
                          "(sharding over several GPUs is not implemented)"}))
        sys.exit(2)
    import torch
    from w8a8_quantized_decode_amd import binding as B
    from w8a8_quantized_decode_amd import synth

    if args.qk_rope:
        bench_qk_rope(args, torch, B)
        return
    if args.attention:
        bench_attention(args, torch, B)
        return
    if args.decode_layer:
        bench_decode_layer(args, torch, B)
        return
    if args.stream_ceiling:
        bench_stream_ceiling(args, torch)
        return
    cfg = synth.CONFIGS[args.config]
    if cfg.kind == "prefill" and args.layer:
        bench_prefill_layer(args, torch, B)
        return
    if cfg.kind == "prefill":
        bench_prefill(args, cfg, torch, B)
        return
    if cfg.kind == "mlp":
        bench_mlp(args, cfg, torch, B)
        return
    if cfg.kind not in ("layer", "stack"):
        raise SystemExit(f"config {cfg.index}: unknown kind {cfg.kind}")
    layers = cfg.layers if cfg.kind == "stack" else 1
    M, H, I, n_qkv = cfg.M, cfg.H, cfg.I, cfg.n_qkv
    nsets = layers if cfg.kind == "stack" else max(1, args.sets)
    print(f"[bench] config {cfg.index}: {cfg.name}; generating {nsets} weight sets",
          file=sys.stderr, flush=True)

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to("cuda")

    def upw(w, s):
        # INT8 weights are converted once to the tiled layout the decode kernels stream.
        rm = up(w)
        tiled = torch.empty_like(rm)
        B.a8w8_pack_weight(rm, tiled)
        del rm
        return (tiled, up(s), B.LAYOUT_TILED)

    sets = []
    for s in range(nsets):
        d = synth.layer_inputs(cfg, layer=s, M=M, with_x=(s == 0))
        sets.append(dict(
            gin=up(d["gamma_in"]), gpost=up(d["gamma_post"]),
            qkv=upw(d["w_qkv"], d["s_qkv"]), o=upw(d["w_o"], d["s_o"]),
            gate=upw(d["w_gate"], d["s_gate"]), up=upw(d["w_up"], d["s_up"]),
            down=upw(d["w_down"], d["s_down"])))
        if s == 0:
            x0 = up(d["x"])
        del d
        if nsets > 4 and (s + 1) % 5 == 0:
            print(f"[bench] {s + 1}/{nsets} weight sets resident", file=sys.stderr, flush=True)
    wbytes_layer = (n_qkv * H + H * H + 2 * I * H + H * I)
    ws = torch.zeros(B.a8w8_workspace_bytes(B.OP_LAYER_LINEARS, M, H, I, n_qkv, cfg.split_k),
                     dtype=torch.uint8, device="cuda")
    xa = torch.empty_like(x0)
    xb = torch.empty_like(x0)

    def layer_call(s, x_in, x_out, taps=None):
        w = sets[s]
        B.a8w8_layer_linears(x_in, w["gin"], w["gpost"], cfg.eps, w["qkv"], w["o"], w["gate"],
                             w["up"], w["down"], x_out, ws, cfg.n_q_heads, cfg.n_kv_heads,
                             cfg.head_dim, split_k=cfg.split_k, taps=taps)

    def step(i, taps_fn=None):
        # One step = one layer (config 2, weight set i mod sets) or the whole 40-layer
        # stack (config 3).  Every step starts from the same input x0.
        if cfg.kind == "stack":
            src, dst = x0, xa
            for l in range(layers):
                layer_call(l, src, dst, taps_fn(l) if taps_fn else None)
                src, dst = dst, (xb if dst is xa else xa)
        else:
            layer_call(i % nsets, x0, xa, taps_fn(0) if taps_fn else None)

    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    layers_per_step = layers
    # The same steps one by one between HIP events: the spread of a step.
    per_step = event_stats(torch, step, min(args.steps, 200 if cfg.kind != "stack" else 20))
    us_per_layer = ms_per_step * 1e3 / layers_per_step
    gbs = wbytes_layer * layers_per_step / (ms_per_step * 1e-3) / 1e9

    # The same steps captured once in a HIP graph (one call per weight set, or the stack)
    # and replayed: the decode GEMMs keep their exchange tags on the device, so replays
    # are valid calls.  Reported beside the plain-launch figure, labelled.
    graph_us = None
    if args.graph:
        n_cap = 1 if cfg.kind == "stack" else nsets
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(n_cap):
                step(i)
        for _ in range(max(1, args.warmup // n_cap)):
            gr.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // n_cap)
        t0 = time.perf_counter()
        for _ in range(reps):
            gr.replay()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - t0) / (reps * n_cap * layers_per_step) * 1e6
        del gr

    # Roofline of the dominant kernel: HIP events recorded by the library right before
    # and after the Gate/Up GEMM launch, on the same stream.
    n_ev = min(args.steps, 100)
    evs = []
    stream = torch.cuda.current_stream()
    for _ in range(n_ev * layers_per_step):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    it = iter(evs)

    def taps_fn(_l):
        a, b = next(it)
        return {"mlp": {"ev_start": a.cuda_event, "ev_stop": b.cuda_event,
                        "ev_kernel": GATEUP_KERNEL}}
    for i in range(n_ev):
        step(i, taps_fn)
    torch.cuda.synchronize()
    k_all = np.array([a.elapsed_time(b) for a, b in evs])
    k_ms = float(np.mean(k_all))
    gu_bytes = 2 * I * H + 2 * I * 4 + M * H + M * 4 + M * I * 4   # weights, scales, q_x, s_x, h
    achieved = gu_bytes / (k_ms * 1e-3) / 1e9
    traffic = measured_traffic(cfg)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "decode_kernel<EPI_SILU> (Gate/Up)" if M <= 16 else
                      "streamk_kernel<EPI_SILU> (Gate/Up)", "kernel_us": round(k_ms * 1e3, 2),
            "kernel_us_stats": pct_stats(k_all * 1e3),
            "algorithmic_bytes_per_launch": gu_bytes}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic (seeded PCG64, Qwen3-14B shapes, random INT8 weights)",
        "us_per_layer": round(us_per_layer, 2),
        "us_per_step_events": per_step,
        "graph_us_per_layer": round(graph_us, 2) if graph_us is not None else None,
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "config": {"workload": cfg.name, "M": M, "hidden": H, "intermediate": I,
                   "n_qkv": n_qkv, "split_k": cfg.split_k, "layers_per_step": layers_per_step,
                   "weight_sets": nsets, "int8_weight_bytes_per_layer": wbytes_layer,
                   "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu,
    }
    emit((out))


if __name__ == "__main__":
    main()
