"""Benchmark of the routed-expert MoE FFN on one MI355X.

Headline workload: the Qwen3-style decode layer (hidden 2048, expert
intermediate 768, 128 experts, top-8, MXFP8 weights, BF16 activations) at
B = 32 tokens, run by moe_layer's path for that batch (the output-centric
decode kernels).  One step = one layer call over one batch; consecutive steps
cycle through several independent copies of the layer's weights with their
own routing draws (as the layers of a model do), so every step streams its
experts from HBM rather than from a cache warmed by the previous step.

Every timed configuration is first checked against the float64 oracle on the
same inputs (per-token cosine, relative L2 and max-abs in the oracle mode of
the path that ran), and the check is printed beside its time.

Prints ONE JSON line: value = achieved HBM bandwidth in TB/s counted from the
algorithmic bytes of each step's actual routing (each touched expert's weights
and scales once, plus x, ids, routing weights and y), ms_per_step = time per
layer.  Also: the measured copy-kernel peak and the fraction of it, the batch
sweep B = 1-256 over the workloads (both paths where both run), the dominant
kernel's roofline entry, the grouped path kernel by kernel with matrix-core
utilisation, the accuracy of the two regimes against exact activations, and
the float64 oracle timed on the host cores (CPU baseline leg).
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

METRIC = "µs per MoE layer & achieved HBM TB/s (fraction of peak), B=1–256, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
# MI355X published dense matrix-core peaks (TFLOP/s).  The grouped GEMMs
# take MXFP8 activations as one operand, so even with E2M1 weights every
# block-scaled MFMA issues at the 8-bit rate.
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "fp4": 10100.0}
DOMINANT = "gate_up_decode_kernel"
KERNEL_SOURCES = ["mixture_experts_decode_amd/csrc/decode.hip",
                  "mixture_experts_decode_amd/csrc/device.h"]
MODE = {"decode": "none", "grouped": "mxfp8"}


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
    p.add_argument("--no-sweep", action="store_true", help="skip the B = 1-256 sweeps")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-copy-peak", action="store_true")
    p.add_argument("--no-grouped", action="store_true",
                   help="skip the expert-centric kernel-by-kernel report")
    p.add_argument("--no-accuracy", action="store_true")
    p.add_argument("--headline-only", action="store_true",
                   help="only the headline workload (for profiler runs)")
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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def spread(values):
    v = np.asarray(values, dtype=np.float64)
    return {"p10": round(float(np.percentile(v, 10)), 2), "p50": round(float(np.median(v)), 2),
            "p90": round(float(np.percentile(v, 90)), 2), "n": int(v.size)}


def sample_rows(t, n):
    if n is None or n >= t:
        return list(range(t))
    return sorted({int(v) for v in np.linspace(0, t - 1, n)})


# ---------------------------------------------------------------------------
# oracle access (test infrastructure: only the parity checks and the CPU
# baseline leg below use it)
# ---------------------------------------------------------------------------

class Oracle:
    """The float64 oracle over one workload's stored weights; each touched
    expert is dequantised once and reused by every check of the run."""

    def __init__(self, cfg, arrays, cache_bytes=8e9):
        from oracle import layer as L
        self.L, self.cfg, self.arrays = L, cfg, arrays
        self.cache = {}
        self.max_entries = max(8, int(cache_bytes // (3 * cfg.hidden * cfg.inter * 8)))

    def _get(self, e):
        if e not in self.cache:
            raw = {k: (None if v is None else v[e]) for k, v in self.arrays.items()}
            wg, wu, wd = self.L.dequant_expert(self.cfg.fmt, raw)
            self.cache[e] = {"w13": np.stack([wg, wu]), "w2": wd}
            if len(self.cache) > self.max_entries:
                self.cache.pop(next(iter(self.cache)))
        return self.cache[e]

    def layer(self, x, ids, w, mode):
        c = self.cfg
        return self.L.moe_layer(self.L.activations_f64(x, c.act), ids, w, act_quant=mode,
                                fmt="f64", num_experts=c.num_experts, num_shared=c.num_shared,
                                get_expert=self._get)


def metrics(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    cos = np.sum(y * ref, 1) / (np.linalg.norm(y, axis=1) * np.linalg.norm(ref, axis=1))
    rel = np.linalg.norm(y - ref, axis=1) / np.linalg.norm(ref, axis=1)
    return {"min_cos": float(np.min(cos)), "max_rel_l2": float(np.max(rel)),
            "rel_l2": float(np.linalg.norm(y - ref) / np.linalg.norm(ref)),
            "max_abs": float(np.max(np.abs(y - ref)))}


def parity(oracle, x, ids, w, rows, y_dev, path):
    """Per-token check of the GPU output rows against the oracle in the mode
    of the path that ran; pass = cosine >= 0.99999 and rel-L2 <= 5e-3."""
    y = y_dev.double().cpu().numpy()[rows]
    ref = oracle.layer(x[rows], ids[rows], w[rows], MODE[path])
    m = metrics(y, ref)
    ok = m["min_cos"] >= 0.99999 and m["max_rel_l2"] <= 5e-3
    return {"tokens": len(rows), "mode": MODE[path], "min_cos": round(m["min_cos"], 8),
            "max_rel_l2": float(f"{m['max_rel_l2']:.3e}"), "max_abs": float(f"{m['max_abs']:.3e}"),
            "pass": bool(ok)}


# ---------------------------------------------------------------------------

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
    ctx = dict(moe=moe, W=W, torch=torch, dev=dev, stream=stream)

    # ---- copy peak (read + write bytes) and read-only peak, best of 20,
    # 4 GiB each way
    copy_peak = read_peak = None
    if not args.no_copy_peak:
        n = 4 << 30
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
        torch.cuda.empty_cache()
        log(f"copy peak {copy_peak:.3f} TB/s, read peak {read_peak:.3f} TB/s (4 GiB)")
    ctx["copy_peak"] = copy_peak

    # ---- headline: weights copied so steps rotate through independent
    # memory (>= ~2.5 GB in total)
    arrays = W.all_experts(cfg)
    oracle = Oracle(cfg, arrays)
    w0 = moe.Weights.from_arrays(cfg, arrays)
    layer_bytes = w0.nbytes()
    n_layers = max(2, min(16, math.ceil(2.5e9 / layer_bytes)))
    layers = [w0]
    for _ in range(n_layers - 1):
        t = [None if a is None else a.clone() for a in w0.tensors]
        layers.append(moe.Weights(cfg.fmt, cfg.hidden, cfg.inter, cfg.num_experts,
                                  cfg.num_shared, *t))
    ebytes = W.expert_bytes(cfg)
    ebytes_dn = down_expert_bytes(W, cfg)
    act_bytes = 2 if cfg.act == "bf16" else 4
    slots = cfg.top_k + cfg.num_shared

    def make_inputs(b, variant):
        x = W.activations(cfg, b, variant)
        ids, wts = W.routing(cfg, b, variant=variant)
        u = len(W.touched_experts(cfg, ids))
        io = b * cfg.hidden * act_bytes + ids.nbytes + wts.nbytes + b * cfg.hidden * 4
        h_el = 4 if cfg.fmt == "f32" else 2
        gate_up_bytes = u * (ebytes - ebytes_dn) + b * cfg.hidden * act_bytes + ids.nbytes \
            + b * slots * cfg.inter * h_el
        # down product: the touched experts' W_down, h, routing, and y
        down_bytes = u * ebytes_dn + b * slots * cfg.inter * h_el + ids.nbytes + wts.nbytes \
            + b * cfg.hidden * 4
        return dict(x=to_dev_x(torch, dev, cfg, x), ids=torch.from_numpy(ids).to(dev),
                    wts=torch.from_numpy(wts).to(dev), bytes=u * ebytes + io,
                    gate_up_bytes=gate_up_bytes, down_bytes=down_bytes, U=u, np=(x, ids, wts))

    h_dtype = "f32" if cfg.fmt == "f32" else "bf16"   # as moe_layer's decode path

    def run_steps(b, steps, warmup, path, n_check=None, replays=5):
        ins = [make_inputs(b, v) for v in range(n_layers)]
        chosen = moe.choose_path(layers[0], b, cfg.top_k) if path == "auto" else path
        need = moe.layer_workspace_bytes(layers[0], b, cfg.top_k, chosen, args.block)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        y = torch.empty((b, cfg.hidden), dtype=torch.float32, device=dev)
        h = torch.empty((b, slots, cfg.inter),
                        dtype=torch.float32 if h_dtype == "f32" else torch.bfloat16, device=dev)
        dws = torch.empty(max(16, slots * b * cfg.hidden * 4), dtype=torch.uint8, device=dev)

        def median_replay_us(graph, launches, n=5):
            """µs per launch: the median over n replays of a graph of
            `launches` launches, each timed alone on the launch stream, after
            0.2 s of untimed replays (the steady state, as for the layer)."""
            t_w = time.perf_counter()
            while time.perf_counter() - t_w < 0.2:
                graph.replay()
                torch.cuda.synchronize()
            t = []
            for _ in range(n):
                s0.record(stream)
                graph.replay()
                s1.record(stream)
                torch.cuda.synchronize()
                t.append(s0.elapsed_time(s1) * 1e3 / launches)
            return float(np.median(t))

        def step(i, ev=None):
            L = layers[i % n_layers]
            d = ins[i % n_layers]
            if chosen == "decode":
                if ev is not None:
                    ev[0].record(stream)
                moe.gate_up(L, d["x"], d["ids"], h=h)
                if ev is not None:
                    ev[1].record(stream)
                moe.down(L, h, d["ids"], d["wts"], y=y, workspace=dws)
                if ev is not None:
                    ev[2].record(stream)
            else:
                moe.layer(L, d["x"], d["ids"], d["wts"], path="grouped", block=args.block, y=y,
                          workspace=ws)

        # verify, then benchmark: the timed kernel sequence is exactly
        # moe_layer's, and its output matches the oracle on every checked token
        step(0)
        y_ref, got = moe.layer(layers[0], ins[0]["x"], ins[0]["ids"], ins[0]["wts"], path=chosen,
                               block=args.block)
        torch.cuda.synchronize()
        if got != chosen or not torch.equal(y, y_ref):
            raise RuntimeError("timed step sequence differs from moe_layer")
        x_np, ids_np, w_np = ins[0]["np"]
        par = parity(oracle, x_np, ids_np, w_np, sample_rows(b, n_check), y_ref, chosen)
        if not par["pass"]:
            raise RuntimeError(f"parity check failed before timing: {par}")

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
        # the graph's first replay, right after the host-side checks left the
        # GPU idle: reported, and checked against the eager steps
        s0.record(stream)
        g.replay()
        s1.record(stream)
        torch.cuda.synchronize()
        first_ms = s0.elapsed_time(s1)
        if not torch.equal(y, y_eager):
            raise RuntimeError("graph replay differs from the eager steps")
        # replays run slower for the first tens of milliseconds of sustained
        # load and then settle; untimed replays for 0.2 s first, so the timed
        # replay sees the steady state a continuously running decode loop sees
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < 0.2:
            g.replay()
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        s0.record(stream)
        g.replay()
        s1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        total_ms = s0.elapsed_time(s1)
        if not torch.equal(y, y_eager):
            raise RuntimeError("graph replay differs from the eager steps")
        # spread: further replays of the same graph, each timed alone
        per = []
        for _ in range(replays):
            s0.record(stream)
            g.replay()
            s1.record(stream)
            torch.cuda.synchronize()
            per.append(s0.elapsed_time(s1) * 1e3 / steps)
        # five replays queued back to back (no host wait between them), as a
        # decode loop would issue them: each replay's launch overlaps the
        # previous one's kernels
        s0.record(stream)
        for _ in range(5):
            g.replay()
        s1.record(stream)
        torch.cuda.synchronize()
        pipelined = s0.elapsed_time(s1) * 1e3 / (5 * steps)
        del g
        tot_bytes = sum(ins[i % n_layers]["bytes"] for i in range(steps))
        res = {"B": b, "path": chosen, "us_per_layer": total_ms * 1e3 / steps,
               "eager_us_per_layer": eager_ms * 1e3 / steps,
               "first_replay_us_per_layer": first_ms * 1e3 / steps,
               "replays_us": spread(per), "pipelined_us_per_layer": pipelined,
               "TBps": tot_bytes / (total_ms * 1e-3) / 1e12,
               "U_mean": float(np.mean([d["U"] for d in ins])), "wall_s": wall, "parity": par}
        if copy_peak:
            res["frac_of_copy_peak"] = res["TBps"] / copy_peak
        if chosen == "decode":
            gu = [evs[i][0].elapsed_time(evs[i][1]) for i in range(steps)]
            dn = [evs[i][1].elapsed_time(evs[i][2]) for i in range(steps)]
            gub = sum(ins[i % n_layers]["gate_up_bytes"] for i in range(steps))
            res["gate_up_us"] = float(np.mean(gu)) * 1e3
            res["down_us"] = float(np.mean(dn)) * 1e3
            res["gate_up_GBps"] = gub / (sum(gu) * 1e-3) / 1e9
            res["gate_up_bytes_per_launch"] = gub / steps
            # the down product alone in each of its launch shapes:
            # token-major buffers nothing; expert-major writes FP32 slot
            # outputs and adds them in a combine kernel
            # the dominant kernel alone, K launches captured in a HIP graph and
            # replayed: no host launch cost sits in the timed interval (the
            # eager per-kernel events above can include the host falling behind)
            gg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gg):
                for i in range(steps):
                    moe.gate_up(layers[i % n_layers], ins[i % n_layers]["x"], ins[i % n_layers]["ids"],
                                h=h)
            torch.cuda.synchronize()
            gg.replay()
            res["gate_up_graph_us"] = median_replay_us(gg, steps)
            del gg
            res["gate_up_graph_GBps"] = gub / (res["gate_up_graph_us"] * steps * 1e-6) / 1e9
            # the down product alone in both launch shapes, timed the same
            # way; GB/s counts the down product's algorithmic bytes (the
            # expert-major shape also writes and re-reads its slot outputs)
            dnb = sum(ins[i % n_layers]["down_bytes"] for i in range(steps)) / steps
            res["down_variants_us"] = {}
            res["down_variants_frac"] = {}
            for var in ("token", "expert"):
                gd = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gd):
                    for i in range(steps):
                        L, d = layers[i % n_layers], ins[i % n_layers]
                        moe.down(L, h, d["ids"], d["wts"], y=y, variant=var, workspace=dws)
                torch.cuda.synchronize()
                gd.replay()
                us = median_replay_us(gd, steps)
                del gd
                res["down_variants_us"][var] = round(us, 2)
                res["down_variants_frac"][var] = round(dnb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
            res["down_bytes_per_launch"] = dnb
        log(f"{cfg.name} B={b} {chosen}: {res['us_per_layer']:.1f} us, {res['TBps']:.3f} TB/s, "
            f"parity {par}")
        return res

    # every token is checked up to B = 64; a spread of tokens beyond
    main_res = run_steps(B, args.steps, args.warmup, args.path, n_check=None if B <= 64 else 4)

    sweep = []
    if not args.no_sweep and not args.headline_only and cfg is W.QWEN3_DECODE_MXFP8:
        for b in cfg.batches:
            r = run_steps(b, 50, 5, args.path, n_check=None)
            sweep.append(rounded(r, ("B", "path", "us_per_layer", "eager_us_per_layer", "replays_us",
                                     "TBps", "frac_of_copy_peak", "U_mean", "gate_up_us",
                                     "down_us", "down_variants_us", "down_variants_frac", "parity")))

    roofline = None
    if main_res["path"] == "decode":
        achieved = main_res["gate_up_graph_GBps"]
        traffic = load_traffic(cfg.name, B)
        roofline = {"kernel": DOMINANT, "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic,
                    "algorithmic_bytes_per_launch": round(main_res["gate_up_bytes_per_launch"]),
                    "avg_launch_us": round(main_res["gate_up_graph_us"], 2),
                    "timing": "HIP events around each of five replays of a graph of the K "
                              "gate_up launches, on their launch stream; the median replay"}

    cpu = None
    if not args.no_cpu_baseline and not args.headline_only:
        cpu = cpu_baseline(cfg, B, oracle)
        cpu["align_sort"] = cpu_align_sort_baseline()
    del layers, w0
    torch.cuda.empty_cache()

    accuracy = []
    if not args.no_accuracy and not args.headline_only:
        accuracy.append(accuracy_report(ctx, cfg, arrays, oracle, 32))
    del arrays, oracle
    if not args.no_accuracy and not args.headline_only:
        # the single-term reading where the matrix cores' accumulation error
        # matters most: an 8-expert prefill-shaped layer at T = 300 (every
        # token), and sampled tokens of the full 16384-token prefill step
        small = W.PREFILL_ZIPF_MXFP8.replace(num_experts=8, tag=31)
        a_small = W.all_experts(small)
        accuracy.append(accuracy_report(ctx, small, a_small, Oracle(small, a_small), 300,
                                        block=128))
        del a_small
        pre = W.PREFILL_ZIPF_MXFP8
        a_pre = W.all_experts(pre)
        accuracy.append(accuracy_report(ctx, pre, a_pre, Oracle(pre, a_pre), 16384, kind="zipf",
                                        rows=sample_rows(16384, 8), block=128))
        del a_pre
        torch.cuda.empty_cache()

    router, grouped, layers_sweep = [], [], []
    if not args.headline_only:
        router = [router_report(ctx, c, t)
                  for c, t in ((W.QWEN3_DECODE_MXFP8, B), (W.DEEPSEEK_V3_FP8_BLK128, 64),
                               (W.PREFILL_ZIPF_MXFP8, 16384))]
    if not args.no_sweep and not args.headline_only:
        # the metric's B = 1-256 over the other workloads: every batch is
        # verified, then timed, on the path moe_layer picks and (where both
        # run) on the other path too
        for c, batches, kinds, n_check in (
                (W.QWEN3_DECODE_MXFP8, (64, 128, 256), (None,), 4),
                (W.DEEPSEEK_V3_FP8_BLK128, (1, 16, 64, 256), (None,), 2),
                (W.MXFP4_SWEEP, (1, 2, 8, 32, 64, 128, 256), ("uniform", "zipf"), 3)):
            layers_sweep += layer_sweep(ctx, c, batches, kinds, n_check,
                                        accuracy if (c is W.MXFP4_SWEEP and not args.no_accuracy)
                                        else None)
            torch.cuda.empty_cache()
    if not args.no_grouped and not args.headline_only:
        # DeepSeek-V3-shaped layer at B = 256 (HBM-bound; 32-row blocks, the
        # fastest measured for a dozen tokens per expert) and the Zipf prefill
        # step (MFMA-bound, 128-row blocks)
        for c, t, bs, kind in ((W.DEEPSEEK_V3_FP8_BLK128, 256, 32, None),
                               (W.PREFILL_ZIPF_MXFP8, 16384, 128, "zipf")):
            grouped.append(grouped_report(ctx, c, t, bs, kind, steps=min(args.steps, 20)))
            torch.cuda.empty_cache()

    value = main_res["TBps"]
    out = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["us_per_layer"] / 1e3, 5),
        "us_per_layer": round(main_res["us_per_layer"], 2),
        "eager_us_per_layer": round(main_res["eager_us_per_layer"], 2),
        "first_replay_us_per_layer": round(main_res["first_replay_us_per_layer"], 2),
        "replays_us": main_res["replays_us"],
        "pipelined_us_per_layer": round(main_res["pipelined_us_per_layer"], 2),
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
        "parity": main_res["parity"],
        "copy_peak_TBps": None if copy_peak is None else round(copy_peak, 3),
        "read_peak_TBps": None if read_peak is None else round(read_peak, 3),
        "frac_of_copy_peak": None if copy_peak is None else round(value / copy_peak, 4),
        "frac_of_hbm_peak": round(value * 1e3 / HBM_PEAK_GBS, 4),
        "kernels_us": {k: round(main_res[k], 2) for k in ("gate_up_us", "down_us") if k in main_res},
        "down_variants_us": main_res.get("down_variants_us"),
        "down_variants_frac_of_hbm_peak": main_res.get("down_variants_frac"),
        "down_bytes_per_launch": round(main_res["down_bytes_per_launch"])
        if "down_bytes_per_launch" in main_res else None,
        "sweep": sweep,
        "layers": layers_sweep,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "accuracy": accuracy,
        "router": router,
        "grouped": grouped,
    }
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------

def rounded(r, keys):
    return {k: (round(r[k], 4) if isinstance(r[k], float) else r[k]) for k in keys if k in r}


def down_expert_bytes(W, c):
    shapes = W.weight_shapes(c)
    tot = 0
    for k in ("w2", "w2_scale"):
        if k in shapes:
            s, d = shapes[k]
            tot += int(np.prod(s[1:])) * np.dtype(d).itemsize
    return tot


def to_dev_x(torch, dev, cfg, x):
    return (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if cfg.act == "bf16"
            else torch.from_numpy(x)).to(dev)


def _device_inputs(ctx, cfg, t, kind, variant=0):
    torch, W, dev = ctx["torch"], ctx["W"], ctx["dev"]
    x = W.activations(cfg, t, variant)
    ids, wts = W.routing(cfg, t, kind=kind, variant=variant)
    return dict(x=to_dev_x(torch, dev, cfg, x), ids=torch.from_numpy(ids).to(dev),
                wts=torch.from_numpy(wts).to(dev), np=(x, ids, wts),
                U=len(W.touched_experts(cfg, ids)))


def layer_sweep(ctx, cfg, batches, kinds, n_check, accuracy=None, steps=10, replays=5, warmup=3):
    """Whole-layer time over a batch list and routing kinds, on the path
    moe_layer(AUTO) picks and on the other path where it runs: each case is
    verified against the oracle first, then its steps (four routing draws
    cycled) are captured in a HIP graph and replayed `replays` times."""
    moe, W, torch, dev, stream = ctx["moe"], ctx["W"], ctx["torch"], ctx["dev"], ctx["stream"]
    arrays = W.all_experts(cfg)
    oracle = Oracle(cfg, arrays)
    Wd = moe.Weights.from_arrays(cfg, arrays)
    del arrays
    ebytes = W.expert_bytes(cfg)
    act = 2 if cfg.act == "bf16" else 4
    out = []
    for kind in kinds:
        for t in batches:
            ins = [_device_inputs(ctx, cfg, t, kind, v) for v in range(4)]
            auto = moe.choose_path(Wd, t, cfg.top_k)
            nbytes = float(np.mean([d["U"] * ebytes + t * cfg.hidden * act + t * cfg.top_k * 8
                                    + t * cfg.hidden * 4 for d in ins]))
            row = {"workload": cfg.name, "routing": kind or cfg.routing, "B": t,
                   "entries": t * (cfg.top_k + cfg.num_shared), "auto": auto,
                   "touched_mean": float(np.mean([d["U"] for d in ins])),
                   "algorithmic_MB": round(nbytes / 1e6, 2)}
            for path in ("decode", "grouped"):
                need = moe.layer_workspace_bytes(Wd, t, cfg.top_k, path, 0)
                y = torch.empty((t, cfg.hidden), dtype=torch.float32, device=dev)
                ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
                try:
                    moe.layer(Wd, ins[0]["x"], ins[0]["ids"], ins[0]["wts"], path=path, y=y,
                              workspace=ws)
                except moe.MoeError as err:
                    if err.status != moe.ERR_UNSUPPORTED:
                        raise
                    continue            # this path does not run at this size
                torch.cuda.synchronize()
                x_np, ids_np, w_np = ins[0]["np"]
                par = parity(oracle, x_np, ids_np, w_np, sample_rows(t, n_check if t > 8 else None),
                             y, path)
                if not par["pass"]:
                    raise RuntimeError(f"parity check failed before timing: {row} {path} {par}")
                for i in range(warmup):
                    d = ins[i % 4]
                    moe.layer(Wd, d["x"], d["ids"], d["wts"], path=path, y=y, workspace=ws)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(steps):
                        d = ins[i % 4]
                        moe.layer(Wd, d["x"], d["ids"], d["wts"], path=path, y=y, workspace=ws)
                torch.cuda.synchronize()
                per = []
                for _ in range(replays):
                    s0 = torch.cuda.Event(enable_timing=True)
                    s1 = torch.cuda.Event(enable_timing=True)
                    s0.record(stream)
                    g.replay()
                    s1.record(stream)
                    torch.cuda.synchronize()
                    per.append(s0.elapsed_time(s1) * 1e3 / steps)
                del g
                us = float(np.median(per))
                entry = {"us": spread(per), "TBps": round(nbytes / (us * 1e-6) / 1e12, 3),
                         "parity": par}
                if ctx["copy_peak"]:
                    entry["frac_of_copy_peak"] = round(nbytes / (us * 1e-6) / 1e12 / ctx["copy_peak"], 4)
                if path == "grouped":
                    fl = 6.0 * cfg.hidden * cfg.inter * t * (cfg.top_k + cfg.num_shared)
                    entry["mfma_frac_useful"] = round(fl / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS["fp8"], 4)
                row[path] = entry
            log(f"layer {row}")
            out.append(row)
            if accuracy is not None and t == 32:
                accuracy.append(accuracy_report(ctx, cfg, None, oracle, t, kind=kind, Wd=Wd))
    del Wd
    return out


def accuracy_report(ctx, cfg, arrays, oracle, t, kind=None, Wd=None, rows=None, block=32):
    """The two regimes on the same inputs against exact activations (oracle
    mode none): the output-centric path keeps activations exact, the
    expert-centric one quantises x and h to MXFP8 and holds slots in BF16
    (the warp-decode post's accuracy section compares the two).  The grouped
    path's h is requantised with two terms; the single-term reading is
    measured too, by running the same kernels with the second term's codes
    set to zero (a zero code contributes nothing whatever its scale)."""
    moe, torch = ctx["moe"], ctx["torch"]
    if Wd is None:
        Wd = moe.Weights.from_arrays(cfg, arrays)
    d = _device_inputs(ctx, cfg, t, kind)
    x_np, ids_np, w_np = d["np"]
    rows = list(range(t)) if rows is None else rows
    entries = t * (cfg.top_k + cfg.num_shared)
    decode_runs = entries <= moe.load().moe_decode_max_entries()
    if decode_runs:
        y_dec, _ = moe.layer(Wd, d["x"], d["ids"], d["wts"], path="decode")
    y_grp, _ = moe.layer(Wd, d["x"], d["ids"], d["wts"], path="grouped", block=block)
    y_one = grouped_single_term(ctx, Wd, cfg, d, t, bs=block)
    torch.cuda.synchronize()
    sel = (x_np[rows], ids_np[rows], w_np[rows])
    exact = oracle.layer(*sel, "none")
    single = oracle.layer(*sel, "mxfp8_single")
    two = oracle.layer(*sel, "mxfp8")
    f = lambda y: y.double().cpu().numpy()[rows]
    fmt = lambda m: {k: float(f"{v:.4e}") for k, v in m.items()}
    m_grp, m_one = metrics(f(y_grp), exact), metrics(f(y_one), exact)
    res = {"workload": cfg.name, "experts": cfg.num_experts, "routing": kind or cfg.routing,
           "B": t, "tokens_compared": len(rows), "block": block,
           "grouped_two_term_vs_exact": fmt(m_grp),
           "grouped_single_term_vs_exact": fmt(m_one),
           "grouped_two_term_vs_its_oracle_mode": fmt(metrics(f(y_grp), two)),
           "grouped_single_term_vs_its_oracle_mode": fmt(metrics(f(y_one), single))}
    if decode_runs:
        m_dec = metrics(f(y_dec), exact)
        res["decode_vs_exact"] = fmt(m_dec)
        res["rel_l2_ratio_grouped_two_term_over_decode"] = round(m_grp["rel_l2"] / m_dec["rel_l2"], 2)
        res["rel_l2_ratio_grouped_single_term_over_decode"] = round(m_one["rel_l2"] / m_dec["rel_l2"], 2)
    log(f"accuracy {res}")
    return res


def grouped_single_term(ctx, Wd, cfg, d, t, bs=32):
    """The grouped path's kernels with h's second term zeroed between the two
    GEMMs: the single-requantisation pipeline."""
    moe, torch = ctx["moe"], ctx["torch"]
    k, S = cfg.top_k, cfg.num_shared
    srt = moe.align_sort(d["ids"], cfg.num_experts, S, bs)
    cap = srt["capacity"]
    xq, xs = moe.quant_rows(d["x"])
    hq, hs = moe.grouped_gate_up(Wd, xq, xs, t, k, srt["sorted_token_ids"], srt["expert_ids"],
                                 srt["num_tokens_post_padded"], cap, bs)
    hq[1].zero_()
    so = moe.grouped_down(Wd, hq, hs, srt["sorted_token_ids"], srt["expert_ids"],
                          srt["num_tokens_post_padded"], cap, bs, d["wts"], t, k)
    return moe.combine(so, t, k + S)


def router_report(ctx, cfg, t, steps=50):
    """Router front-end (gating scores -> top-k ids and weights) timed with
    HIP events; bytes = scores read + ids and weights written."""
    moe, W, torch, dev, stream = ctx["moe"], ctx["W"], ctx["torch"], ctx["dev"], ctx["stream"]
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


def grouped_report(ctx, cfg, t, bs, kind, steps=20, warmup=3, n_check=4):
    """Expert-centric path on one layer: the calls moe_layer makes, each
    bracketed by HIP events on the launch stream, after a check of sampled
    tokens against the oracle.  MFMA utilisation counts useful FLOPs only
    (padding rows excluded)."""
    moe, W, torch, dev, stream = ctx["moe"], ctx["W"], ctx["torch"], ctx["dev"], ctx["stream"]
    arrays = W.all_experts(cfg)
    oracle = Oracle(cfg, arrays)
    Wd = moe.Weights.from_arrays(cfg, arrays)
    del arrays
    d = _device_inputs(ctx, cfg, t, kind)
    x, ids, wts = d["x"], d["ids"], d["wts"]
    x_np, ids_np, w_np = d["np"]
    k, S = cfg.top_k, cfg.num_shared
    slots = k + S
    y = torch.empty((t, cfg.hidden), dtype=torch.float32, device=dev)
    slot_out = torch.empty((t * slots, cfg.hidden), dtype=torch.bfloat16, device=dev)
    cap = moe.align_sort_capacity(t, k, cfg.num_experts, S, bs)
    names = ["align_sort", "quant_rows", "gate_up_gemm", "down_gemm", "combine"]

    def step(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
        rec(0)
        srt = moe.align_sort(ids, cfg.num_experts, S, bs)
        rec(1)
        xq, xs = moe.quant_rows(x)
        rec(2)
        hq, hs = moe.grouped_gate_up(Wd, xq, xs, t, k, srt["sorted_token_ids"], srt["expert_ids"],
                                     srt["num_tokens_post_padded"], cap, bs)
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
    par = parity(oracle, x_np, ids_np, w_np, sample_rows(t, n_check), y_ref, "grouped")
    if not par["pass"]:
        raise RuntimeError(f"parity check failed before timing: {cfg.name} {par}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    per = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e3
           for j, n in enumerate(names)}
    totals = [e[0].elapsed_time(e[-1]) * 1e3 for e in evs]
    total = float(np.mean(totals))
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
           "us_per_layer": round(total, 2), "us_spread": spread(totals),
           "kernels_us": {n: round(v, 2) for n, v in per.items()},
           "useful_TFLOP": round((fl_gu + fl_dn) / 1e12, 4),
           "gate_up_TFLOPs": round(fl_gu / (per["gate_up_gemm"] * 1e-6) / 1e12, 1),
           "down_TFLOPs": round(fl_dn / (per["down_gemm"] * 1e-6) / 1e12, 1),
           "layer_TFLOPs": round((fl_gu + fl_dn) / (total * 1e-6) / 1e12, 1),
           "mfma_peak_TFLOPs": peak,
           "mfma_frac_gate_up": round(fl_gu / (per["gate_up_gemm"] * 1e-6) / 1e12 / peak, 4),
           "mfma_frac_down": round(fl_dn / (per["down_gemm"] * 1e-6) / 1e12 / peak, 4),
           "mfma_frac_layer": round((fl_gu + fl_dn) / (total * 1e-6) / 1e12 / peak, 4),
           "algorithmic_TBps": round((wbytes + io) / (total * 1e-6) / 1e12, 3),
           "parity": par}
    log(f"grouped {cfg.name} T={t} bs={bs}: {total:.1f} us (gate_up {per['gate_up_gemm']:.1f}, "
        f"down {per['down_gemm']:.1f}) parity {par}")
    del Wd
    return res


def cpu_baseline(cfg, B, oracle, budget_s=12.0, max_calls=8):
    """The float64 oracle timed on this host's cores on whole layer calls of
    the same workload (B tokens; successive routing draws) until about
    `budget_s` seconds of CPU work have run (at most `max_calls` calls).
    Each call dequantises the experts it touches (stored format -> float64),
    as the oracle does, without reusing the parity checks' cache."""
    import workloads as W
    from oracle import layer as L

    arrays = oracle.arrays

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


def cpu_align_sort_baseline(budget_s=3.0, max_calls=5):
    """The align-sort oracle (plain Python, one thread) timed on the prefill
    shape the grouped report sorts on the GPU: 16384 tokens x top-8 over 256
    experts, Zipf routing, 128-entry blocks (successive routing draws)."""
    import workloads as W
    from oracle import align_sort as A
    c, t, bs = W.PREFILL_ZIPF_MXFP8, 16384, 128
    spent, calls = 0.0, 0
    while calls < max_calls and (calls == 0 or spent < budget_s):
        ids, _ = W.routing(c, t, kind="zipf", variant=calls)
        t0 = time.perf_counter()
        A.align_sort(ids.reshape(-1), c.num_experts, bs)
        spent += time.perf_counter() - t0
        calls += 1
    n = t * c.top_k
    return {"value": round(n * calls / spent / 1e6, 3), "unit": "M entries/s", "cores": 1,
            "kind": "oracle", "us_per_call": round(spent / calls * 1e6, 1),
            "sample": f"{calls} calls of oracle.align_sort on {t} tokens x top-{c.top_k} over "
                      f"{c.num_experts} experts (Zipf routing), {bs}-entry blocks"}


if __name__ == "__main__":
    main()
