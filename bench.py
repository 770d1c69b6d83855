#!/usr/bin/env python3
"""Benchmark: ms per DiT denoise step at 1024x1024 (4608 tokens) on one MI355X.

One step = global modulation + embeddings + 5 dual-stream + 20 single-stream
blocks + final layer, through dit_step_forward, on synthetic bf16 weights of
the FLUX.2 [klein] 4B shape and synthetic inputs (512 text rows of width 7680,
64 x 64 latent tokens of width 128), all resident in HBM before timing.

Prints one JSON line (rank 0). Timing: W untimed warm-up steps, then K steps
bracketed by device synchronisation, per-step HIP events on the launch
stream. A second, separate pass records HIP events around every kernel
launch (dit_profile_begin/end) to give per-kernel durations for the
roofline; the headline number comes from the clean pass. The same run also
times the step with one reference image (S = 8704) and the 1920x1088 batch-4
step (S = 8672 per sample) under "workloads", and the latent decoder at
1024x1024 and at 1920x1088 batch 4 under "vae_decode". The CPU baseline times the
oracle in fp32 NumPy on one whole step of the workload's first sample, after
a one-block warm-up.
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per DiT denoise step at 1024² (4608 tok) + attn/GEMM TFLOP/s vs peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
P100A_STEP_MS = 331.0       # per DiT step, 1024^2, Tenstorrent p100a ("flux2-klein-p100a")
COPY_CAL_BYTES = 512 << 20  # device-to-device copy used to calibrate the HBM byte counters
GEMM_SRC = os.path.join(ROOT, "diffusion_transformer_fwd_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_bf16_kernel_step_1024px_hbm_traffic.md")


def gemm_source_hash():
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_gemm_traffic():
    """HBM bytes per GEMM launch from the committed counter summary, or None
    when it is missing or was taken on a different GEMM kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if line.startswith(("bytes_per_launch:",
                                                                         "gemm_source_sha256:")))
    except OSError:
        return None
    if kv.get("gemm_source_sha256", "").strip() != gemm_source_hash():
        return None
    try:
        return float(kv["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def summarize(d):
    """Markdown summary of the rocprofv3 CSV output in directory d: the
    kernel-statistics table, and/or per-kernel counter means with FETCH_SIZE /
    WRITE_SIZE converted to bytes by the calibration kernels (torch
    elementwise kernels that each move COPY_CAL_BYTES, see --copy-calibration)."""
    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        rows = list(csv.DictReader(open(f)))
        out.append("| kernel | calls | avg us | total ms | % |\n|---|---|---|---|---|")
        g_calls, g_ns = 0, 0.0
        for r in rows:
            name = r["Name"].replace("dit::(anonymous namespace)::", "").split("(")[0]
            out.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                       f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['Percentage']):.2f} |")
            if "gemm_bf16_kernel" in name:  # every tile-width instance
                g_calls += int(r["Calls"])
                g_ns += float(r["TotalDurationNs"])
        if g_calls:
            out.append(f"gemm_bf16_kernel, all instances: {g_calls} calls, "
                       f"avg {g_ns / g_calls / 1e3:.1f} us")
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        names = {}
        for r in csv.DictReader(open(f)):
            per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
        by_kernel = collections.defaultdict(list)
        for disp, ctr in per.items():
            by_kernel[names[disp].replace("dit::(anonymous namespace)::", "").split("(")[0]].append(ctr)
        cal = {}
        copies = [x for k, lst in by_kernel.items() if "elementwise_kernel" in k for x in lst]
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            vals = [x[c] for x in copies if c in x]
            if vals:
                cal[c] = COPY_CAL_BYTES / (max(vals) * 1024.0)  # bytes per counted KiB
        out.append(f"counters from {os.path.basename(f)}; calibration kernels moving {COPY_CAL_BYTES} B: "
                   + ", ".join(f"{c} x {1024 * v:.4f}" for c, v in cal.items()))
        out.append("| kernel | dispatches | counter | mean per dispatch |\n|---|---|---|---|")
        for k, lst in sorted(by_kernel.items()):
            for c in sorted({c for x in lst for c in x}):
                vals = [x[c] for x in lst if c in x]
                out.append(f"| {k} | {len(vals)} | {c} | {sum(vals) / len(vals):.6g} |")
        mfma = [(k, lst) for k, lst in sorted(by_kernel.items())
                if any("SQ_INSTS_VALU_MFMA_MOPS_BF16" in x for x in lst)]
        if mfma:
            # MOPS count 512 flops each; MFMA busy cycles are per SIMD (1024 on
            # the chip) and GRBM_GUI_ACTIVE is summed over the 8 XCDs here
            out.append("| kernel | dispatches | counted GFLOP per dispatch | MFMA busy % | "
                       "GUI-active cycles per dispatch |\n|---|---|---|---|---|")
            for k, lst in mfma:
                n = len(lst)
                fl = sum(x.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for x in lst) * 512 / n
                gui = sum(x.get("GRBM_GUI_ACTIVE", 0.0) for x in lst) / n / 8
                busy = sum(x.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for x in lst) / n
                pct = 100.0 * busy / (gui * 1024) if gui else float("nan")
                out.append(f"| {k} | {n} | {fl / 1e9:.2f} | {pct:.1f} | {gui:.0f} |")
        gemm = [x for k, lst in by_kernel.items() if "gemm_bf16_kernel" in k for x in lst]
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            vals = [x[c] for x in gemm if c in x]
            if vals and c in cal:
                out.append(f"gemm_{c.lower()}_bytes_per_launch: {sum(vals) / len(vals) * 1024 * cal[c]:.0f}")
    print("\n".join(out))


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(cfg, mw, wl):
    """Time the oracle as it stands, in fp32 NumPy (its dtype switch), on one
    whole step of one sample of the workload, after a one-block warm-up.
    mw: the synth.ModelWeights the GPU run uploaded (blocks cached in host
    memory, so drawing weights is not timed). Returns (seconds for the step,
    threads, algorithmic FLOPs of the step)."""
    from oracle import dit_oracle as O
    from diffusion_transformer_fwd_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    ins = synth.step_inputs(cfg, wl, batch_row=0)
    txt, lat = ins["txt"][None], ins["latents"][None]
    pos = O.position_ids(wl.n_txt, wl.img_grid, wl.ref_grids)
    S = pos.shape[0]
    # warm-up: one single-stream block on the step's own shapes
    mod = O.modulation(mw.glob, np.array([wl.sigma]), cfg.time_channels, np.float32)
    cos, sin = O.rope_tables(pos, cfg.axes_dim, cfg.theta)
    x = synth.residual(cfg, 0, S)[None]
    O.single_block(x, mw.single(0), mod["single"], cos.astype(np.float32),
                   sin.astype(np.float32), cfg.heads, cfg.eps, cfg.prenorm, np.float32)
    t0 = time.perf_counter()
    v = O.step(cfg, mw, txt, lat, np.array([wl.sigma]), wl.n_img, pos, dtype=np.float32)
    sec = time.perf_counter() - t0
    assert np.all(np.isfinite(v))
    D, F = cfg.hidden, cfg.mlp_hidden
    blk = 2.0 * S * D * (3 * D + 2 * F) + 2.0 * S * (D + F) * D + 4.0 * S * S * D
    flops = (cfg.n_dual + cfg.n_single) * blk + 2.0 * D * (
        wl.n_txt * cfg.txt_channels + (wl.n_img + wl.n_ref) * cfg.in_channels
        + wl.n_img * cfg.in_channels)
    return sec, threads, flops


def cpu_block_baselines(mw):
    """The oracle as it stands, in fp32 NumPy, on the two block workloads:
    the 1024 x 1024 single block (512 text + 64 x 64 image rows, block 0 of
    the step's weights, already in host memory), median of 3 runs after the
    step's timing warmed the same shapes; and the small dual block (hidden
    256, 32 text + 8 x 8 image rows, sigma 0.5) on one BLAS thread, median of
    20 after one warm-up. Returns two dicts of ms and GFLOP/s."""
    from oracle import dit_oracle as O
    from diffusion_transformer_fwd_amd import synth
    from threadpoolctl import threadpool_limits

    def block_flops(S, D, F, dual):
        per_row = 2.0 * D * (4 * D + 3 * F) if dual else 2.0 * D * (3 * D + 2 * F) + 2.0 * (D + F) * D
        return S * per_row + 4.0 * S * S * D

    def setup(cfg, gw, wl):
        pos = O.position_ids(wl.n_txt, wl.img_grid, wl.ref_grids)
        mod = O.modulation(gw, np.array([wl.sigma]), cfg.time_channels, np.float32)
        cos, sin = O.rope_tables(pos, cfg.axes_dim, cfg.theta)
        x = synth.residual(cfg, 0, pos.shape[0])[None]
        return pos.shape[0], mod, cos.astype(np.float32), sin.astype(np.float32), x

    cfg, wl = synth.FLUX2_KLEIN, synth.W_SINGLE_1024
    S, mod, cos, sin, x = setup(cfg, mw.glob, wl)
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        y = O.single_block(x, mw.single(0), mod["single"], cos, sin, cfg.heads, cfg.eps,
                           cfg.prenorm, np.float32)
        ts.append(time.perf_counter() - t0)
    assert np.all(np.isfinite(y))
    sec = float(np.median(ts))
    fl = block_flops(S, cfg.hidden, cfg.mlp_hidden, False)
    single = {"workload": wl.name, "ms": round(sec * 1000.0, 1), "reps": 3,
              "gflops": round(fl / sec / 1e9, 1)}

    c1 = synth.DitConfig(hidden=256, heads=2, head_dim=128, mlp_hidden=768, n_dual=1,
                         n_single=1, in_channels=128, txt_channels=256)
    wl1 = synth.W_DUAL_TINY
    S1, mod1, cos1, sin1, x1 = setup(c1, synth.global_weights(c1, 0), wl1)
    w1 = synth.dual_weights(c1, 0, 0)
    ts = []
    with threadpool_limits(limits=1):
        for i in range(21):
            t0 = time.perf_counter()
            y = O.dual_block(x1, wl1.n_txt, w1, mod1["dual_txt"], mod1["dual_img"], cos1, sin1,
                             c1.heads, c1.eps, c1.prenorm, np.float32)
            if i:
                ts.append(time.perf_counter() - t0)
    assert np.all(np.isfinite(y))
    sec = float(np.median(ts))
    fl = block_flops(S1, c1.hidden, c1.mlp_hidden, True)
    dual = {"workload": wl1.name, "ms": round(sec * 1000.0, 3), "reps": 20, "threads": 1,
            "gflops": round(fl / sec / 1e9, 2)}
    return single, dual


def decode_cpu_baseline(hp=32, wp=32):
    """The decoder oracle as it stands, in fp32 NumPy (its dtype switch), on a
    bounded sample: one decode of an hp x wp token grid (a 512 x 512 image by
    default, 2.6 TFLOP, about 8-25 s on the hosts measured), after a
    64 x 64-image warm-up. Returns (seconds, threads, FLOPs of the sample, FLOPs of a
    1024 x 1024 decode)."""
    from oracle import vae_oracle as V
    from diffusion_transformer_fwd_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    vcfg = synth.VAE_KLEIN
    w = synth.vae_weights(vcfg, 0)
    V.decode(vcfg, w, synth.vae_latents(vcfg, 0, 4, 4)[None], 4, 4, dtype=np.float32)
    z = synth.vae_latents(vcfg, 0, hp, wp)[None]
    t0 = time.perf_counter()
    img = V.decode(vcfg, w, z, hp, wp, dtype=np.float32)
    sec = time.perf_counter() - t0
    assert np.all(np.isfinite(img))
    gh, gw = synth.V_DECODE_1024.grid
    return sec, threads, V.decode_flops(vcfg, 1, hp, wp), V.decode_flops(vcfg, 1, gh, gw)


def matrix_tflops(k):
    """TFLOP/s of the GEMM and attention launches together (plain GEMM,
    plain attention, and attention fused with GEMM tiles), from a per-kernel
    event pass."""
    names = ("gemm", "attention", "attn_gemm")
    fl = sum(k[n]["flops"] for n in names)
    ms = sum(k[n]["total_ms"] for n in names)
    return fl / (ms * 1e-3) / 1e12


def time_workload(dit, synth, torch, cfg, dw, wl, steps=10, warmup=2):
    """Median / p95 ms of one step of workload wl (HIP events on the launch
    stream), its algorithmic TFLOP/s, and the GEMM + attention fraction of
    the bf16 peak from one per-kernel event pass."""
    ins_b = [synth.step_inputs(cfg, wl, batch_row=b) for b in range(wl.batch)]
    txt = dit.to_bf16_device(np.stack([i["txt"] for i in ins_b]))
    lat = dit.to_bf16_device(np.stack([i["latents"] for i in ins_b]))
    pos = dit.position_ids(wl.n_txt, wl.img_grid, wl.ref_grids)
    cos, sin = dit.rope_tables(cfg, pos)
    ws = dit.Workspace()
    out = torch.empty((wl.batch, wl.n_img, cfg.in_channels), dtype=torch.float32, device="cuda")
    sigma = [wl.sigma] * wl.batch

    def one():
        dit.step(cfg, dw, txt, lat, sigma, wl.n_img, cos, sin, ws=ws, out=out)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        one()
        e1.record()
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in evs])
    assert np.all(np.isfinite(out.cpu().numpy())), f"{wl.name}: non-finite output"
    dit.profile_begin()
    one()
    k = dit.profile_end()
    g, a, ag = k["gemm"], k["attention"], k["attn_gemm"]
    flops = sum(s["flops"] for s in k.values())
    ga = matrix_tflops(k)
    med = float(np.median(per))
    res = {"batch": wl.batch, "seq_len": wl.seq, "n_img": wl.n_img, "n_ref": wl.n_ref,
           "ms_median": round(med, 3), "ms_p95": round(float(np.percentile(per, 95)), 3),
           "step_tflop": round(flops / 1e12, 3),
           "step_tflops": round(flops / (med * 1e-3) / 1e12, 1),
           "gemm_tflops": round(g["flops"] / (g["total_ms"] * 1e-3) / 1e12, 1),
           "attention_tflops": round(a["flops"] / (a["total_ms"] * 1e-3) / 1e12, 1)
           if a["total_ms"] > 0 else None,
           "attn_gemm_tflops": round(ag["flops"] / (ag["total_ms"] * 1e-3) / 1e12, 1)
           if ag["total_ms"] > 0 else None,
           "gemm_attn_tflops": round(ga, 1),
           "gemm_attn_frac_of_peak": round(ga / PEAK_BF16_TFLOPS, 4)}
    del ws, out, txt, lat
    torch.cuda.empty_cache()
    return res


def time_decode(dit, synth, torch, vwl, vdw, steps=5, warmup=1):
    """The latent decoder on workload vwl: median / p95 ms of whole decodes
    (HIP events on the launch stream), algorithmic TFLOP/s, and per-kernel
    figures from one event pass (conv TFLOP/s and its fraction of the bf16
    peak; GroupNorm and softmax GB/s)."""
    vcfg = synth.VAE_KLEIN
    hp, wp = vwl.grid
    z = dit.to_f32_device(np.stack([synth.vae_latents(vcfg, b, hp, wp) for b in range(vwl.batch)]))
    ws = dit.Workspace()
    img = torch.empty((vwl.batch, 16 * hp, 16 * wp, 3), dtype=torch.float32, device="cuda")

    def one():
        dit.vae_decode(vcfg, vdw, z, hp, wp, ws=ws, out=img)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        one()
        e1.record()
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in evs])
    assert np.all(np.isfinite(img.cpu().numpy())), f"{vwl.name}: non-finite image"
    dit.profile_begin()
    one()
    k = dit.profile_end()
    flops = sum(s["flops"] for s in k.values())
    med = float(np.median(per))
    res = {"batch": vwl.batch, "image": [16 * hp, 16 * wp], "ms_median": round(med, 3),
           "ms_p95": round(float(np.percentile(per, 95)), 3),
           "tflop": round(flops / 1e12, 3), "tflops": round(flops / (med * 1e-3) / 1e12, 1),
           "frac_of_bf16_peak": round(flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    for name in ("conv_halo", "conv", "group_norm", "softmax", "latent_image"):
        s = k[name]
        if s["launches"] == 0:
            continue
        e = {"launches": s["launches"], "ms": round(s["total_ms"], 3),
             "avg_launch_us": round(1000.0 * s["total_ms"] / s["launches"], 2)}
        if s["flops"] > 0:
            tf = s["flops"] / (s["total_ms"] * 1e-3) / 1e12
            e["tflops"] = round(tf, 1)
            e["frac_of_bf16_peak"] = round(tf / PEAK_BF16_TFLOPS, 4)
            e["alg_bytes"] = s["bytes"]
        else:
            gbs = s["bytes"] / (s["total_ms"] * 1e-3) / 1e9
            e["gbs"] = round(gbs, 1)
            e["frac_of_hbm_peak"] = round(gbs / PEAK_HBM_GBS, 4)
        res[name] = e
    # the decoder's dominant kernel against the bf16 MFMA peak
    h = k["conv_halo"]
    if h["launches"] > 0:
        per_launch = h["flops"] / h["launches"]
        avg_s = h["total_ms"] / h["launches"] * 1e-3
        res["roofline"] = {"bound": "mfma", "kernel": "conv3_halo_kernel",
                           "achieved": round(per_launch / avg_s / 1e12, 1),
                           "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(per_launch / avg_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "per_launch_flop": per_launch, "avg_launch_us": round(avg_s * 1e6, 2),
                           "traffic": None}
    del ws, img, z
    torch.cuda.empty_cache()
    return res


def decode_leg(dit, synth, torch, which):
    """Decoder timings for the named workloads (weights drawn once)."""
    vdw = dit.VaeWeights(synth.VAE_KLEIN, synth.vae_weights(synth.VAE_KLEIN, 0))
    out = {}
    for vwl in which:
        log(f"decode {vwl.name}")
        out[vwl.name] = time_decode(dit, synth, torch, vwl, vdw)
        log(f"  {json.dumps(out[vwl.name])}")
    del vdw
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--profile-steps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="skip the reference-image and batch-4 steps timed after the headline")
    ap.add_argument("--workload", default="step_1024px_s4608",
                    help="step workload to time (the default is the headline one; the others "
                         "are the reference-image, batch-4, three-reference and 512px "
                         "reference steps)")
    ap.add_argument("--denoise-reps", type=int, default=3,
                    help="timed runs of the 4-step sampling loop, eager and graph-replayed")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with three device copies of COPY_CAL_BYTES (counter calibration)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the latent decoder timings (1024x1024 and 1920x1088 batch 4)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the latent decoder and print its JSON record")
    ap.add_argument("--summarize", metavar="DIR",
                    help="print a markdown summary of rocprofv3 CSV output in DIR and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from diffusion_transformer_fwd_amd import dit, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dit.lib()
    torch.cuda.set_device(0)
    if args.decode_only:
        which = (synth.V_DECODE_1024,) if args.no_extra_workloads else (
            synth.V_DECODE_1024, synth.V_DECODE_1920x1088_B4)
        print(json.dumps({"vae_decode": decode_leg(dit, synth, torch, which)}), flush=True)
        return
    cfg = synth.FLUX2_KLEIN
    wl = {w.name: w for w in (synth.W_STEP_1024, synth.W_STEP_1024_REF, synth.W_STEP_1920x1088_B4,
                              synth.W_STEP_848x624_3REF, synth.W_STEP_512_REF)}[args.workload]
    B = wl.batch

    log("drawing weights and inputs")
    t0 = time.time()
    # blocks stay cached in host memory when the CPU baseline will reuse them
    mw = synth.ModelWeights(cfg, 0, cache=not args.no_cpu_baseline)
    dw = dit.ModelWeights(mw)
    ins_b = [synth.step_inputs(cfg, wl, batch_row=b) for b in range(B)]
    ins = ins_b[0]
    txt = dit.to_bf16_device(np.stack([i["txt"] for i in ins_b]))
    lat = dit.to_bf16_device(np.stack([i["latents"] for i in ins_b]))
    pos = dit.position_ids(wl.n_txt, wl.img_grid, wl.ref_grids)
    cos, sin = dit.rope_tables(cfg, pos)
    ws = dit.Workspace()
    out = torch.empty((B, wl.n_img, cfg.in_channels), dtype=torch.float32, device="cuda")
    sigma = [wl.sigma] * B
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f}s")

    def one():
        dit.step(cfg, dw, txt, lat, sigma, wl.n_img, cos, sin, ws=ws, out=out)

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()

    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(K):
        evs[i][0].record()
        one()
        evs[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    per = np.array([a.elapsed_time(b) for a, b in evs])
    ms = float(wall * 1000.0 / K)
    log(f"{K} steps: {ms:.3f} ms/step (wall), events median {np.median(per):.3f} "
        f"p95 {np.percentile(per, 95):.3f}")
    assert np.all(np.isfinite(out.cpu().numpy())), "non-finite output"

    # the 4-step sampling loop on the device (Euler between steps), eager and
    # captured once as a HIP graph and replayed
    den = None
    if args.denoise_reps > 0 and B == 1 and wl.n_ref == 0:
        sched = np.array([[1.0, 0.75, 0.5, 0.25, 0.0]], np.float32)
        z0 = dit.to_f32_device(ins["latents"][None, :wl.n_img])
        z = z0.clone()
        dws = dit.Workspace()
        dws.get(dit.workspace_bytes(cfg, dit.WS_DENOISE, 1, wl.seq))

        def loop():
            dit.denoise(cfg, dw, txt, z, None, sched, cos, sin, ws=dws)

        loop()
        torch.cuda.synchronize()
        t_e = []
        for _ in range(args.denoise_reps):
            z.copy_(z0)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            loop()
            torch.cuda.synchronize()
            t_e.append(time.perf_counter() - t1)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            loop()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            loop()
        t_g = []
        for _ in range(args.denoise_reps):
            z.copy_(z0)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            graph.replay()
            torch.cuda.synchronize()
            t_g.append(time.perf_counter() - t1)
        assert np.all(np.isfinite(z.cpu().numpy())), "non-finite latent"
        del graph
        den = {"steps": 4, "schedule": sched[0].tolist(),
               "eager_ms": round(1000.0 * float(np.median(t_e)), 3),
               "graph_ms": round(1000.0 * float(np.median(t_g)), 3)}
        log(f"4-step loop: eager {den['eager_ms']} ms, graph {den['graph_ms']} ms")

    # per-kernel pass (event pair around every launch)
    P = max(1, args.profile_steps)
    dit.profile_begin()
    for _ in range(P):
        one()
    kstats = dit.profile_end()
    kern = {}
    for name, s in kstats.items():
        if s["launches"] == 0:
            continue
        e = {"launches_per_step": s["launches"] / P, "ms_per_step": s["total_ms"] / P,
             "avg_launch_us": 1000.0 * s["total_ms"] / s["launches"]}
        if s["flops"] > 0 and name in ("gemm", "attention", "attn_gemm"):
            e["tflops"] = s["flops"] / (s["total_ms"] * 1e-3) / 1e12
            e["frac_of_bf16_peak"] = e["tflops"] / PEAK_BF16_TFLOPS
        if s["bytes"] > 0 and name not in ("gemm", "attention", "attn_gemm"):
            e["gbs"] = s["bytes"] / (s["total_ms"] * 1e-3) / 1e9
            e["frac_of_hbm_peak"] = e["gbs"] / PEAK_HBM_GBS
        kern[name] = e
    g = kstats["gemm"]
    step_flops = sum(s["flops"] for s in kstats.values()) / P
    ga_tflops = matrix_tflops(kstats)
    gemm_per_launch = g["flops"] / g["launches"]
    gemm_avg_s = g["total_ms"] / g["launches"] * 1e-3
    achieved = gemm_per_launch / gemm_avg_s / 1e12
    log("kernels: " + json.dumps(kern))

    extra = None
    if not args.no_extra_workloads:
        extra = {}
        for xw in (synth.W_STEP_1024_REF, synth.W_STEP_1920x1088_B4):
            if xw is wl:
                continue
            log(f"workload {xw.name}")
            extra[xw.name] = time_workload(dit, synth, torch, cfg, dw, xw)
            log(f"  {json.dumps(extra[xw.name])}")

    dec = None
    if not args.no_decode:
        which = (synth.V_DECODE_1024,) if args.no_extra_workloads else (
            synth.V_DECODE_1024, synth.V_DECODE_1920x1088_B4)
        dec = decode_leg(dit, synth, torch, which)
        if not args.no_cpu_baseline:
            log("decoder CPU baseline: the oracle in fp32 NumPy on a 512 x 512 decode")
            sec, threads, fl, fl_1024 = decode_cpu_baseline()
            dec[synth.V_DECODE_1024.name]["cpu_baseline"] = {
                "value": round(sec * fl_1024 / fl * 1000.0, 1), "unit": "ms", "cores": threads,
                "kind": "oracle", "gflops": round(fl / sec / 1e9, 1),
                "sample": f"one 512 x 512 decode (32 x 32 tokens, {fl / 1e12:.2f} TFLOP), "
                          f"oracle in fp32 NumPy, timed once after a small warm-up, "
                          f"{sec:.1f} s; scaled by FLOPs to one 1024 x 1024 decode "
                          f"({fl_1024 / 1e12:.2f} TFLOP)"}
            log(f"decoder CPU baseline {sec:.1f} s for the sample")

    cpu = None
    if not args.no_cpu_baseline:
        log("CPU baseline: the oracle in fp32 NumPy, one whole step after a one-block warm-up")
        sec, threads, cflops = cpu_baseline(cfg, mw, wl)
        cpu = {"value": round(sec * 1000.0, 1), "unit": "ms", "cores": threads, "kind": "oracle",
               "gflops": round(cflops / sec / 1e9, 1),
               "sample": f"one whole step (5 dual + 20 single blocks, embeddings, final "
                         f"layer) of batch row 0 of {wl.name} (S={wl.seq}), oracle in fp32 "
                         f"NumPy, timed once after a one-block warm-up"
                         + (f"; the GPU step covers {B} such rows" if B > 1 else "")}
        log(f"CPU baseline {sec:.1f} s/step ({threads} threads, {cpu['gflops']} GFLOP/s)")
        single, dual = cpu_block_baselines(mw)
        cpu["blocks"] = {"single_block_1024px": single, "dual_block_d256_1thread": dual}
        log(f"CPU block baselines: single block {single['ms']} ms, small dual block "
            f"{dual['ms']} ms on one thread")

    if args.copy_calibration:
        # a fill (writes COPY_CAL_BYTES) and elementwise negations (read and
        # write COPY_CAL_BYTES each), so both counters see a known byte count
        src = torch.empty(COPY_CAL_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    traffic = stored_gemm_traffic()
    rec = {
        "metric": METRIC, "value": round(ms, 4), "unit": "ms", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": round(ms / P100A_STEP_MS, 5) if wl is synth.W_STEP_1024 else None,
        "baseline": {"value": P100A_STEP_MS, "unit": "ms",
                     "source": "per DiT step at 1024^2 on a Tenstorrent p100a (context only)"},
        "dtype": "bf16", "data": "synthetic (seeded N(0,1/fan_in) weights, N(0,1) inputs)",
        "config": {"workload": wl.name, "batch": B, "seq_len": wl.seq, "n_txt": wl.n_txt,
                   "n_img": wl.n_img, "blocks": "5 dual + 20 single", "hidden": cfg.hidden,
                   "heads": cfg.heads, "parallelism": "none (1 GPU)"},
        "ms_median": round(float(np.median(per)), 4),
        "ms_p95": round(float(np.percentile(per, 95)), 4),
        "step_tflop": round(step_flops / 1e12, 4),
        "step_tflops": round(step_flops / (ms * 1e-3) / 1e12, 1),
        "gemm_attn_tflops": round(ga_tflops, 1),
        "gemm_attn_frac_of_peak": round(ga_tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": "gemm_bf16_kernel",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "alg_bytes_per_launch": round(g["bytes"] / g["launches"]),
                     "per_launch_flop": gemm_per_launch, "avg_launch_us": gemm_avg_s * 1e6},
        "kernels": kern,
        "workloads": extra,
        "denoise_loop": den,
        "vae_decode": dec,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
