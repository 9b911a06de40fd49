"""Throughput of the packed encoder forward on one MI355X.

Default workload: the Z-Image-style DiT stack as a CFG batch-2 program (30
sandwich layers, d 3840, 30x128 heads, int8 row-scaled weights x f16
activations with f32 accumulation, qk-norm + 2-D RoPE over a 64x64 grid plus
128 caption rows per item, SwiGLU 10240; rows [img0|img1|cap0|cap1] = 8448),
synthetic seeded inputs and random-init weights.  Any other workload is taken
with --workload (the text encoder: gemma_text_f32).  A step is one
encoder_forward over the whole packed batch, inputs already resident in HBM.

Prints one JSON line: value = encoder TFLOP/s, algorithmic (GEMM + attention)
flops / wall time of K steps; the roofline of the dominant kernel class (the
GEMMs) from per-launch HIP events recorded by the library on the stream the
kernels run on; and the f64 oracle timed on the host cores on a bounded sample
of the same workload (the first layers of the f32 batches; layer 0 of the DiT
model over 1600 of its image rows).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"f32": 157.3, "i8f16": 2516.6}  # TFLOP/s, dense MFMA (FP32 / FP16), MI355X datasheet
HBM_PEAK = 8000.0  # GB/s
CPU_LAYERS = 4


def gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm_impl.h", "gemm.hip", "dev.h"):  # dev.h: the epilogues' helpers
        with open(os.path.join(ROOT, "transformer_encoder_forward_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per GEMM launch from the committed rocprofv3 --pmc summary of this
    workload, or None when it is missing or was taken on other GEMM sources."""
    import re
    path = os.path.join(ROOT, "profiles", f"gemm_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    src = re.search(r"gemm_source_sha256:\s*([0-9a-f]+)", txt)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.e+]+)", txt)
    if not src or not val or src.group(1) != gemm_source_hash():
        return None
    return float(val.group(1))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(name, cfg, w):
    """The f64 oracle as it stands, timed on the host cores over a bounded sample of
    the same workload (about 10-30 s): the f32 batches' first CPU_LAYERS layers over
    the whole packed batch; for the int8 DiT, layer 0 of the same model over the
    first 1600 image rows as one 40x40-grid item (each row's GEMM work is the full
    workload's; attention sees 1600 keys instead of the item's own 4224)."""
    import oracle

    from transformer_encoder_forward_amd import workloads as wl

    if cfg["path"] == wl.PATH_F32:
        nl = min(CPU_LAYERS, cfg["layers"])
        sample = wl.make(name, layers=nl)
        sample.cfg["final"] = wl.FINAL_NONE
        what = (f"first {nl} of {cfg['layers']} layers over the same {len(w.items)}-item batch "
                f"({w.rows} rows)")
    else:
        sample = wl.make(name, layers=1, grid=40, ncap=0, cfg_pair=False)
        what = (f"layer 0 of the same model ({cfg['layers']} layers) over its first "
                f"{sample.rows} image rows as one 40x40-grid item, f16 sites on")
    c0 = time.perf_counter()
    oracle.forward(sample)
    cdt = time.perf_counter() - c0
    cfl = wl.gemm_flops(sample) + wl.attn_flops(sample)
    return {"value": round(cfl / cdt / 1e12, 5), "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{what}: {cfl / 1e9:.1f} GFLOP in {cdt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="zimage_dit_cfg_8448")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays")
    ap.add_argument("--layers", type=int, default=None, help="(development) fewer layers")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard by whole items with no exchange step)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from transformer_encoder_forward_amd import binding as B
    from transformer_encoder_forward_amd import model as M
    from transformer_encoder_forward_amd import workloads as wl

    dev = "cuda:0"
    torch.cuda.set_device(0)
    t0 = time.time()
    w = wl.make(args.workload, layers=args.layers, lazy_int8=True)
    cfg = w.cfg
    x = torch.from_numpy(w.x).to(dev)
    out = torch.empty((M.out_rows(w), cfg["d"]), dtype=torch.float32, device=dev)
    ctx = B.context(0)
    stream = torch.cuda.current_stream()
    if w.stages:
        # a staged DiT program: the context refiner runs once (per prompt) on the
        # caption rows; a step is the noise refiner + the main stack
        pre = M.DeviceProgram(w, dev, skip=("noise refiner", "main"))
        prog = M.DeviceProgram(w, dev, skip=("context refiner",))
        ws = torch.empty(max(pre.workspace_bytes(), prog.workspace_bytes()), dtype=torch.uint8,
                         device=dev)
        if pre.parts:
            x0 = x.clone()
            M.stages_forward(pre, x0, x, ws, ctx=ctx, stream=stream)
        timed = [st for lab, st, _ in w.stages if lab != "context refiner"]
    else:
        dm = M.DeviceModel(w, dev)
        db = M.DeviceBatch(w, dev)
        ws = dm.workspace(db, dev)
        timed = [w]
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    print(f"[bench] {args.workload}: rows={w.rows} items={len(w.items)} layers={cfg['layers']} "
          f"setup {setup_s:.1f}s", file=sys.stderr, flush=True)

    def step(st=stream):
        if w.stages:
            M.stages_forward(prog, x, out, ws, ctx=ctx, stream=st)
        else:
            M.encoder_forward(dm, db, x, out, ws, ctx=ctx, stream=st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timed_step = step
    if args.graph:
        # the whole step as one graph, captured on a side stream (the library
        # enqueues kernels and device-to-device copies only) and replayed on
        # the timed stream
        graph, cap = torch.cuda.CUDAGraph(), torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.graph(graph, stream=cap):
            step(cap)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        timed_step = graph.replay
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        timed_step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    assert torch.isfinite(out).all().item(), "non-finite output"

    gflop = sum(wl.gemm_flops(st) for st in timed)
    aflop = sum(wl.attn_flops(st) for st in timed)
    tflops = (gflop + aflop) / (ms * 1e-3) / 1e12
    dtype = "f32" if cfg["path"] == wl.PATH_F32 else "i8f16"
    peak = PEAK[dtype]

    # per-class GPU time from events the library records around each launch
    B.prof_enable(True, ctx)
    B.prof_read(ctx)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = B.prof_read(ctx)
    B.prof_enable(False, ctx)
    g = prof["gemm"]
    gemm_ms_launch = g["ms"] / max(1, g["launches"])
    gemm_tf = g["flops"] / (g["ms"] * 1e-3) / 1e12 if g["ms"] else 0.0
    classes = {k: dict(launches_per_step=v["launches"] / args.steps,
                       ms_per_step=round(v["ms"] / args.steps, 4),
                       tflops=round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 2) if v["flops"] and v["ms"] else None,
                       gbps=round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1) if v["bytes"] and v["ms"] else None)
               for k, v in prof.items()}
    print(f"[bench] {ms:.3f} ms/step, {tflops:.2f} TFLOP/s; classes {classes}", file=sys.stderr,
          flush=True)

    # the chip's MFMA ceiling for this dtype, measured by a register-only kernel
    measured_peak = B.mfma_peak(0 if dtype == "f32" else 1, ctx=ctx)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, cfg, w)
    res = {
        "metric": "encoder TFLOP/s (GEMM+attn) and % of MI355X MFMA peak; tokens/s per layer",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_median": round(per_step[len(per_step) // 2], 4),
        "ms_min": round(per_step[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "launch": "hip graph replay" if args.graph else "eager",
        "pct_of_mfma_peak": round(100.0 * tflops / peak, 2),
        "measured_mfma_peak": round(measured_peak, 1),
        "pct_of_measured_peak": round(100.0 * tflops / measured_peak, 2),
        "tokens_per_s_per_layer": round(sum(st.rows * st.cfg["layers"] for st in timed) / (ms * 1e-3), 1),
        "config": {"workload": args.workload, "rows": w.rows, "items": len(w.items),
                   "layers": cfg["layers"], "d": cfg["d"], "heads": f"{cfg['nq']}x{cfg['hd']}",
                   "kv_heads": cfg["nkv"], "ff": cfg["ff"], "window": cfg["window"],
                   **({"global_every": cfg["global_every"]} if cfg.get("global_every") else {}),
                   **({"v_norm": True} if cfg.get("v_norm") else {}),
                   **({"n_ple": cfg["n_ple"]} if cfg.get("n_ple") else {}),
                   **({"modulated": True} if cfg.get("modulated") else {}),
                   **({"guards": cfg["guards"]} if cfg.get("guards") else {}),
                   **({"step_stages": [f"{lab}: {st.cfg['layers']} layers x {st.rows} rows"
                                       for lab, st, _ in w.stages if lab != "context refiner"]}
                      if w.stages else {}),
                   "gemm_gflop": round(gflop / 1e9, 2), "attn_gflop": round(aflop / 1e9, 2),
                   "parallelism": "single GPU"},
        "roofline": {"kernel": ("GEMM class: gemm_f32d_kernel plain and gated (FP32 MFMA)"
                                if dtype == "f32" else
                                "GEMM class: gemm_q8d_kernel plain and gated (int8 x f16 MFMA)"),
                     "bound": "mfma", "achieved": round(gemm_tf, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(gemm_tf / peak, 4),
                     "traffic": measured_traffic(args.workload),
                     "alg_bytes_per_launch": round(g["bytes"] / max(1, g["launches"])),
                     "launches_per_step": g["launches"] / args.steps,
                     "avg_launch_ms": round(gemm_ms_launch, 5),
                     "gemm_source_sha256": gemm_source_hash()},
        "classes": classes,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
