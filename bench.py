"""Benchmark of the routed-expert MoE FFN on one MI355X.

Default workload: the Qwen3-style decode layer (hidden 2048, expert
intermediate 768, 128 experts, top-8, MXFP8 weights, BF16 activations) at
B = 32 tokens, run by moe_layer's path for that batch (the output-centric
decode kernels).  One step = one layer call over one batch; consecutive steps
cycle through several independent copies of the layer's weights with their
own routing draws (as the layers of a model do), so every step streams its
experts from HBM rather than from a cache warmed by the previous step.

Prints ONE JSON line: value = achieved HBM bandwidth in TB/s counted from the
algorithmic bytes of each step's actual routing (each touched expert's weights
and scales once, plus x, ids, routing weights and y), ms_per_step = time per
layer.  Also: the measured copy-kernel peak and the fraction of it, a batch
sweep, the dominant kernel's roofline entry, and the float64 oracle timed on
the host cores (CPU baseline leg).
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
# MI355X published dense matrix-core peaks (TFLOP/s).  The grouped GEMMs
# take MXFP8 activations as the A operand, so even with E2M1 weights every
# block-scaled MFMA issues at the 8-bit rate.
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "fp4": 10100.0}
DOMINANT = "gate_up_decode_kernel"
KERNEL_SOURCES = ["mixture_experts_decode_amd/csrc/decode.hip",
                  "mixture_experts_decode_amd/csrc/device.h"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="qwen3_decode_mxfp8",
                   help="workload name (see workloads.CONFIGS)")
    p.add_argument("--batch", type=int, default=32)
    p.add_argument("--path", default="auto", choices=["auto", "decode", "grouped"])
    p.add_argument("--block", type=int, default=0)
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-copy-peak", action="store_true")
    p.add_argument("--no-grouped", action="store_true",
                   help="skip the expert-centric (grouped MFMA) report")
    p.add_argument("--crossover", action="store_true",
                   help="also sweep the MXFP4 layer over B with both paths")
    return p.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(cfg_name, batch):
    """HBM traffic per launch of the dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{DOMINANT}_{cfg_name}_b{batch}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU split is a design note only).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import mixture_experts_decode_amd as moe

    moe.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.CONFIGS[args.workload]
    B = args.batch
    stream = torch.cuda.current_stream()

    # ---- weights: one generated layer, copied so steps rotate through
    # independent memory (>= ~2.5 GB in total)
    arrays = W.all_experts(cfg)
    w0 = moe.Weights.from_arrays(cfg, arrays)
    layer_bytes = w0.nbytes()
    n_layers = max(2, min(16, math.ceil(2.5e9 / layer_bytes)))
    layers = [w0]
    for _ in range(n_layers - 1):
        t = [None if a is None else a.clone() for a in w0.tensors]
        layers.append(moe.Weights(cfg.fmt, cfg.hidden, cfg.inter, cfg.num_experts,
                                  cfg.num_shared, *t))
    ebytes = W.expert_bytes(cfg)
    act_bytes = 2 if cfg.act == "bf16" else 4

    def make_inputs(b, variant):
        x = W.activations(cfg, b, variant)
        ids, wts = W.routing(cfg, b, variant=variant)
        xd = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if cfg.act == "bf16"
              else torch.from_numpy(x)).to(dev)
        u = len(W.touched_experts(cfg, ids))
        io = b * cfg.hidden * act_bytes + ids.nbytes + wts.nbytes + b * cfg.hidden * 4
        gate_up_bytes = u * (ebytes - ebytes_down(cfg)) + b * cfg.hidden * act_bytes + ids.nbytes \
            + b * (cfg.top_k + cfg.num_shared) * cfg.inter * (4 if cfg.fmt == "f32" else 2)
        return dict(x=xd, ids=torch.from_numpy(ids).to(dev), wts=torch.from_numpy(wts).to(dev),
                    bytes=u * ebytes + io, gate_up_bytes=gate_up_bytes, U=u)

    def ebytes_down(c):
        shapes = W.weight_shapes(c)
        tot = 0
        for k in ("w2", "w2_scale"):
            if k in shapes:
                s, d = shapes[k]
                tot += int(np.prod(s[1:])) * np.dtype(d).itemsize
        return tot

    # ---- copy peak (read + write bytes), best of 20, 2 GiB each way
    copy_peak = read_peak = None
    if not args.no_copy_peak:
        n = 2 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        moe.util_fill(src, n, 0x3c3c3c3c)
        sink = torch.zeros(4096, dtype=torch.float32, device=dev)
        best_c = best_r = 1e30
        for _ in range(20):
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record(stream)
            moe.util_copy(src, dst, n)
            e1.record(stream)
            moe.util_read(src, n, sink)
            e2.record(stream)
            e2.synchronize()
            best_c = min(best_c, e0.elapsed_time(e1))
            best_r = min(best_r, e1.elapsed_time(e2))
        copy_peak = 2 * n / (best_c * 1e-3) / 1e12
        read_peak = n / (best_r * 1e-3) / 1e12
        del src, dst

    h_dtype = "f32" if cfg.fmt == "f32" else "bf16"   # as moe_layer's decode path

    def run_steps(b, steps, warmup, path):
        ins = [make_inputs(b, v) for v in range(n_layers)]
        need = moe.layer_workspace_bytes(layers[0], b, cfg.top_k, path, args.block)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        y = torch.empty((b, cfg.hidden), dtype=torch.float32, device=dev)
        chosen = moe.choose_path(layers[0], b, cfg.top_k) if path == "auto" else path
        h = torch.empty((b, cfg.top_k + cfg.num_shared, cfg.inter),
                        dtype=torch.float32 if h_dtype == "f32" else torch.bfloat16, device=dev)
        variant = "expert" if b >= 4 else "token"
        dws = torch.empty(max(16, (cfg.top_k + cfg.num_shared) * b * cfg.hidden * 4),
                          dtype=torch.uint8, device=dev)

        def step(i, ev=None):
            L = layers[i % n_layers]
            d = ins[i % n_layers]
            if chosen == "decode":
                if ev is not None:
                    ev[0].record(stream)
                moe.gate_up(L, d["x"], d["ids"], h=h)
                if ev is not None:
                    ev[1].record(stream)
                moe.down(L, h, d["ids"], d["wts"], y=y, variant=variant, workspace=dws)
                if ev is not None:
                    ev[2].record(stream)
            else:
                moe.layer(L, d["x"], d["ids"], d["wts"], path="grouped", block=args.block, y=y,
                          workspace=ws)

        if chosen == "decode":
            # the timed kernel sequence is exactly moe_layer's decode path
            step(0)
            y_ref, _ = moe.layer(layers[0], ins[0]["x"], ins[0]["ids"], ins[0]["wts"], path="decode")
            torch.cuda.synchronize()
            if not torch.equal(y, y_ref):
                raise RuntimeError("timed decode sequence differs from moe_layer(decode)")

        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        # eager pass: per-kernel HIP events on the launch stream
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for i in range(steps):
            step(i, evs[i] if chosen == "decode" else None)
        s1.record(stream)
        torch.cuda.synchronize()
        eager_ms = s0.elapsed_time(s1)
        y_eager = y.clone()
        # timed pass: the same K steps captured once in a HIP graph and
        # replayed, so no host launch cost sits between the kernels (as a
        # decode loop would run them)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        s0.record(stream)
        g.replay()
        s1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        total_ms = s0.elapsed_time(s1)
        del g
        if not torch.equal(y, y_eager):
            raise RuntimeError("graph replay differs from the eager steps")
        tot_bytes = sum(ins[i % n_layers]["bytes"] for i in range(steps))
        res = {"B": b, "path": chosen, "us_per_layer": total_ms * 1e3 / steps,
               "eager_us_per_layer": eager_ms * 1e3 / steps,
               "TBps": tot_bytes / (total_ms * 1e-3) / 1e12,
               "U_mean": float(np.mean([d["U"] for d in ins])), "wall_s": wall}
        if chosen == "decode":
            gu = [evs[i][0].elapsed_time(evs[i][1]) for i in range(steps)]
            dn = [evs[i][1].elapsed_time(evs[i][2]) for i in range(steps)]
            gub = sum(ins[i % n_layers]["gate_up_bytes"] for i in range(steps))
            res["gate_up_us"] = float(np.mean(gu)) * 1e3
            res["down_us"] = float(np.mean(dn)) * 1e3
            res["gate_up_GBps"] = gub / (sum(gu) * 1e-3) / 1e9
            res["gate_up_bytes_per_launch"] = gub / steps
        return res

    main_res = run_steps(B, args.steps, args.warmup, args.path)

    sweep = []
    if not args.no_sweep and cfg is W.QWEN3_DECODE_MXFP8:
        for b in cfg.batches:
            r = run_steps(b, 50, 5, args.path)
            sweep.append({k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()
                          if k in ("B", "path", "us_per_layer", "eager_us_per_layer", "TBps",
                                   "U_mean", "gate_up_us", "down_us")})

    roofline = None
    if main_res["path"] == "decode":
        achieved = main_res["gate_up_GBps"]
        traffic = load_traffic(cfg.name, B)
        roofline = {"kernel": DOMINANT, "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic,
                    "algorithmic_bytes_per_launch": round(main_res["gate_up_bytes_per_launch"]),
                    "avg_launch_us": round(main_res["gate_up_us"], 2)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, B, arrays)
    del layers, arrays, w0
    torch.cuda.empty_cache()

    router = [router_report(moe, W, torch, dev, stream, c, t)
              for c, t in ((W.QWEN3_DECODE_MXFP8, B), (W.DEEPSEEK_V3_FP8_BLK128, 64),
                           (W.PREFILL_ZIPF_MXFP8, 16384))]

    grouped = []
    if not args.no_grouped:
        # DeepSeek-V3-shaped layer at B = 256 (HBM-bound; 32-row blocks,
        # the fastest measured for a dozen tokens per expert) and the Zipf
        # prefill step (MFMA-bound, 128-row blocks)
        for c, t, bs, kind in ((W.DEEPSEEK_V3_FP8_BLK128, 256, 32, None),
                               (W.PREFILL_ZIPF_MXFP8, 16384, 128, "zipf")):
            grouped.append(grouped_report(moe, W, torch, dev, stream, c, t, bs, kind,
                                          steps=min(args.steps, 20)))
            torch.cuda.empty_cache()

    crossover = []
    if args.crossover:
        for c, batches in ((W.MXFP4_SWEEP, None),
                           (W.QWEN3_DECODE_MXFP8, (1, 4, 8, 16, 32, 64, 128, 256)),
                           (W.DEEPSEEK_V3_FP8_BLK128, (1, 8, 16, 32, 64, 128, 224))):
            crossover += crossover_sweep(moe, W, torch, dev, stream, c, batches=batches,
                                         kinds=("uniform", "zipf") if c is W.MXFP4_SWEEP else (None,))
            torch.cuda.empty_cache()

    value = main_res["TBps"]
    out = {
        "metric": "us per MoE layer & achieved HBM TB/s (fraction of peak), 1 GPU",
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["us_per_layer"] / 1e3, 5),
        "us_per_layer": round(main_res["us_per_layer"], 2),
        "eager_us_per_layer": round(main_res["eager_us_per_layer"], 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the multiply-accumulate type of the timed path: BF16 operands (the
        # stored E4M3/E2M1 weights convert to BF16 exactly) with FP32 sums
        "dtype": "f32" if cfg.fmt == "f32" else "bf16",
        "precision": f"{cfg.fmt} weights, {cfg.act} activations, f32 accumulation",
        "data": "synthetic (seeded; random-init weights of the named shape)",
        "config": {"workload": cfg.name, "hidden": cfg.hidden, "inter": cfg.inter,
                   "experts": cfg.num_experts, "top_k": cfg.top_k, "batch": B,
                   "weight_format": cfg.fmt, "path": main_res["path"],
                   "layers_rotated": n_layers, "touched_experts_mean": main_res["U_mean"]},
        "copy_peak_TBps": None if copy_peak is None else round(copy_peak, 3),
        "read_peak_TBps": None if read_peak is None else round(read_peak, 3),
        "frac_of_copy_peak": None if copy_peak is None else round(value / copy_peak, 4),
        "frac_of_hbm_peak": round(value * 1e3 / HBM_PEAK_GBS, 4),
        "kernels_us": {k: round(main_res[k], 2) for k in ("gate_up_us", "down_us") if k in main_res},
        "sweep": sweep,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "router": router,
        "grouped": grouped,
    }
    if crossover:
        out["crossover"] = crossover
    print(json.dumps(out), flush=True)


def _device_inputs(torch, dev, W, cfg, t, kind, variant=0):
    x = W.activations(cfg, t, variant)
    ids, wts = W.routing(cfg, t, kind=kind, variant=variant)
    xd = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if cfg.act == "bf16"
          else torch.from_numpy(x)).to(dev)
    return xd, torch.from_numpy(ids).to(dev), torch.from_numpy(wts).to(dev), ids


def router_report(moe, W, torch, dev, stream, cfg, t, steps=50):
    """Router front-end (gating scores -> top-k ids and weights) timed with
    HIP events; bytes = scores read + ids and weights written."""
    scores, bias = W.gating_scores(cfg, t)
    s = torch.from_numpy(scores).to(dev)
    b = None if bias is None else torch.from_numpy(bias).to(dev)
    ids = torch.empty((t, cfg.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((t, cfg.top_k), dtype=torch.float32, device=dev)
    for _ in range(3):
        moe.topk_route(s, cfg.top_k, bias=b, ids=ids, wts=wts)
    torch.cuda.synchronize()
    # the launch loop calls the library directly with marshalled arguments,
    # so the host keeps ahead of a kernel of a few microseconds
    import ctypes
    args = [ctypes.c_void_p(s.data_ptr()), None if b is None else ctypes.c_void_p(b.data_ptr()),
            t, cfg.num_experts, cfg.top_k, ctypes.c_void_p(ids.data_ptr()),
            ctypes.c_void_p(wts.data_ptr()), ctypes.c_void_p(stream.cuda_stream)]
    fn = moe._lib.moe_topk_route
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn(*args)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = scores.nbytes + (0 if bias is None else bias.nbytes) + t * cfg.top_k * 8
    return {"workload": cfg.name, "tokens": t, "experts": cfg.num_experts, "top_k": cfg.top_k,
            "biased": bias is not None, "us": round(us, 2), "GBps": round(nbytes / us / 1e3, 1)}


def grouped_report(moe, W, torch, dev, stream, cfg, t, bs, kind, steps=20, warmup=3):
    """Expert-centric path on one layer: the five calls moe_layer makes
    (align-sort, gather + MXFP8 quantisation, gate_up GEMM, down GEMM,
    combine), each bracketed by HIP events on the launch stream.  MFMA
    utilisation counts useful FLOPs only (padding rows excluded)."""
    arrays = W.all_experts(cfg)
    Wd = moe.Weights.from_arrays(cfg, arrays)
    del arrays
    x, ids, wts, ids_np = _device_inputs(torch, dev, W, cfg, t, kind)
    k, S = cfg.top_k, cfg.num_shared
    slots = k + S
    y = torch.empty((t, cfg.hidden), dtype=torch.float32, device=dev)
    slot_out = torch.empty((t * slots, cfg.hidden), dtype=torch.bfloat16, device=dev)
    cap = moe.align_sort_capacity(t, k, cfg.num_experts, S, bs)

    def step(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
        rec(0)
        srt = moe.align_sort(ids, cfg.num_experts, S, bs)
        rec(1)
        xq, xs = moe.gather_quant(x, slots, srt["sorted_token_ids"],
                                  srt["num_tokens_post_padded"], cap)
        rec(2)
        hq, hs = moe.grouped_gate_up(Wd, xq, xs, srt["expert_ids"], srt["num_tokens_post_padded"],
                                     cap, bs)
        rec(3)
        moe.grouped_down(Wd, hq, hs, srt["sorted_token_ids"], srt["expert_ids"],
                         srt["num_tokens_post_padded"], cap, bs, wts, t, k, slot_out=slot_out)
        rec(4)
        moe.combine(slot_out, t, slots, y=y)
        rec(5)

    step()
    y_ref, chosen = moe.layer(Wd, x, ids, wts, path="grouped", block=bs)
    torch.cuda.synchronize()
    if not torch.equal(y, y_ref):
        raise RuntimeError("timed grouped sequence differs from moe_layer(grouped)")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    names = ["align_sort", "gather_quant", "gate_up_gemm", "down_gemm", "combine"]
    per = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e3
           for j, n in enumerate(names)}
    total = float(np.mean([e[0].elapsed_time(e[5]) for e in evs])) * 1e3
    entries = t * slots
    fl_gu = 2.0 * entries * cfg.hidden * 2 * cfg.inter
    fl_dn = 2.0 * entries * cfg.inter * cfg.hidden
    peak = MFMA_PEAK_TFLOPS["fp8"]
    u = len(W.touched_experts(cfg, ids_np))
    wbytes = u * W.expert_bytes(cfg)
    act = 2 if cfg.act == "bf16" else 4
    io = t * cfg.hidden * act + ids_np.nbytes * 2 + t * cfg.hidden * 4
    res = {"workload": cfg.name, "tokens": t, "block": bs, "routing": kind or cfg.routing,
           "touched_experts": u, "capacity": cap,
           "us_per_layer": round(total, 2),
           "kernels_us": {n: round(v, 2) for n, v in per.items()},
           "useful_TFLOP": round((fl_gu + fl_dn) / 1e12, 4),
           "gate_up_TFLOPs": round(fl_gu / (per["gate_up_gemm"] * 1e-6) / 1e12, 1),
           "down_TFLOPs": round(fl_dn / (per["down_gemm"] * 1e-6) / 1e12, 1),
           "layer_TFLOPs": round((fl_gu + fl_dn) / (total * 1e-6) / 1e12, 1),
           "mfma_peak_TFLOPs": peak,
           "mfma_frac_gate_up": round(fl_gu / (per["gate_up_gemm"] * 1e-6) / 1e12 / peak, 4),
           "mfma_frac_down": round(fl_dn / (per["down_gemm"] * 1e-6) / 1e12 / peak, 4),
           "mfma_frac_layer": round((fl_gu + fl_dn) / (total * 1e-6) / 1e12 / peak, 4),
           "algorithmic_TBps": round((wbytes + io) / (total * 1e-6) / 1e12, 3)}
    print(f"[bench] grouped {cfg.name} T={t} bs={bs}: {total:.1f} us "
          f"(gate_up {per['gate_up_gemm']:.1f}, down {per['down_gemm']:.1f})",
          file=sys.stderr, flush=True)
    del Wd
    return res


def crossover_sweep(moe, W, torch, dev, stream, cfg, batches=None, kinds=(None,), steps=20,
                    warmup=3, bs=32):
    """Whole-layer time of both paths over a batch list (the configuration's
    own by default) and routing kinds (None: the configuration's own), on one
    layer's weights with several routing draws cycled."""
    arrays = W.all_experts(cfg)
    Wd = moe.Weights.from_arrays(cfg, arrays)
    del arrays
    out = []
    for kind in kinds:
        for t in batches or cfg.batches:
            ins = [_device_inputs(torch, dev, W, cfg, t, kind, v) for v in range(4)]
            row = {"workload": cfg.name, "routing": kind or cfg.routing, "B": t,
                   "entries": t * (cfg.top_k + cfg.num_shared),
                   "auto": moe.choose_path(Wd, t, cfg.top_k),
                   "touched_mean": float(np.mean([len(W.touched_experts(cfg, i[3])) for i in ins]))}
            for path in ("decode", "grouped"):
                if path == "decode" and t * (cfg.top_k + cfg.num_shared) > 2048:
                    continue
                need = moe.layer_workspace_bytes(Wd, t, cfg.top_k, path, bs)
                ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
                y = torch.empty((t, cfg.hidden), dtype=torch.float32, device=dev)
                for i in range(warmup):
                    xd, idd, wd, _ = ins[i % 4]
                    moe.layer(Wd, xd, idd, wd, path=path, block=bs, y=y, workspace=ws)
                torch.cuda.synchronize()
                # the steps replayed from one HIP graph, as in the headline
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(steps):
                        xd, idd, wd, _ = ins[i % 4]
                        moe.layer(Wd, xd, idd, wd, path=path, block=bs, y=y, workspace=ws)
                torch.cuda.synchronize()
                s0 = torch.cuda.Event(enable_timing=True)
                s1 = torch.cuda.Event(enable_timing=True)
                s0.record(stream)
                g.replay()
                s1.record(stream)
                torch.cuda.synchronize()
                del g
                row[path + "_us"] = round(s0.elapsed_time(s1) * 1e3 / steps, 2)
            print(f"[bench] crossover {row}", file=sys.stderr, flush=True)
            out.append(row)
    del Wd
    return out


def cpu_baseline(cfg, B, arrays, budget_s=12.0, max_calls=8):
    """The float64 oracle timed on this host's cores on whole layer calls of
    the same workload (B tokens; successive routing draws) until about
    `budget_s` seconds of CPU work have run (at most `max_calls` calls)."""
    import workloads as W
    from oracle import layer as L

    def get(e):
        return {k: (None if v is None else v[e]) for k, v in arrays.items()}

    kw = dict(fmt=cfg.fmt, num_experts=cfg.num_experts, num_shared=cfg.num_shared, get_expert=get)
    act_bytes = 2 if cfg.act == "bf16" else 4
    spent, nbytes, calls, touched = 0.0, 0, 0, []
    while calls < max_calls and (calls == 0 or spent < budget_s):
        x = W.activations(cfg, B, calls)
        ids, wts = W.routing(cfg, B, variant=calls)
        t0 = time.perf_counter()
        L.moe_layer(L.activations_f64(x, cfg.act), ids, wts, **kw)
        spent += time.perf_counter() - t0
        u = len(W.touched_experts(cfg, ids))
        touched.append(u)
        nbytes += u * W.expert_bytes(cfg) + B * cfg.hidden * act_bytes + ids.nbytes + wts.nbytes \
            + B * cfg.hidden * 4
        calls += 1
    dt = spent / calls
    try:
        import threadpoolctl
        threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    return {"value": round(nbytes / spent / 1e12, 6), "unit": "TB/s", "cores": threads,
            "kind": "oracle", "us_per_layer": round(dt * 1e6, 1), "seconds": round(spent, 2),
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{calls} whole layer calls of {cfg.name} at B={B} (successive routing "
                      f"draws, {min(touched)}-{max(touched)} touched experts), float64"}


if __name__ == "__main__":
    main()
