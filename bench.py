"""Benchmark of the MXFP4 routed-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--m 128] [--no-extra] [--no-cpu]
                    [--workload decode|prefill1536|fusedsum4096|mxfp8x4096]

A step is one moe_mxfp4_forward call (route -> FC1 -> FC2 -> combine) over one
batch of the decode workload: hidden 7168, intermediate 2048, 224 resident of
384 experts, top-8, MXFP4 weights (E8M0 scales in [120,130]), bf16 activations
N(0,1), route ids uniform over 0..383 (ids >= 224 contribute an exact zero),
M tokens (default 128).  Inputs are resident in HBM before timing.  Eight
routing/activation sets are rotated so consecutive steps touch different
experts (small-M working sets would otherwise stay in the 256 MB last-level
cache between steps).

--workload picks a single prefill configuration instead (1536 tokens uniform,
4096 tokens Zipf fused-sum, 4096 tokens MXFP8), for profiling one workload at a
time: its tokens/s is the value and its FC1 kernel is priced against the MFMA
peak of its dtype (extras and the CPU baseline are skipped).

Prints ONE JSON line: whole-job tokens/s (`value`, eager launches; the same
steps replayed from captured hipGraphs are reported beside it); the roofline of the
dominant kernel (FC1), timed with HIP events recorded on the launch stream
right before and after that kernel in a second pass over the same steps; the layer's own
HBM fraction; extra entries for the other decode batch sizes and the prefill
workloads (unless --no-extra); the fp64 CPU oracle timed on a bounded sample
(unless --no-cpu).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA
METRIC = "MoE layer tokens/s + % HBM roofline (decode M≤128) / % MFMA peak (prefill)"
STAGES = ("route", "fc1", "fc2", "combine")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def expert_bytes(H, I):
    """Codes + E8M0 scales of one expert: (W13, W2)."""
    return (2 * I * H // 2 + 2 * I * H // 32), (H * I // 2 + H * I // 32)


def build_plan(cid, max_tokens):
    import torch
    import mxfp4_routed_expert_topk_amd as moe
    import workloads as W
    from workloads import device as D
    case = W.config_case(cid, m=max_tokens if cid == 1 else None)
    s = case.shape
    t0 = time.time()
    w = D.upload_experts(case)
    act = moe.MOE_ACT_MXFP8 if case.act == "mxfp8" else moe.MOE_ACT_BF16
    plan = moe.Plan(moe.Config(s.hidden, s.inter, s.experts, s.top_k, max_tokens, act), *w)
    del w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"config {cid}: plan over {s.experts} experts built in {time.time() - t0:.1f}s")
    return plan, case


class Batches:
    """`sets` device-resident input sets of one configuration at T tokens."""

    fused = False   # also time the one-launch forward (--fused)

    def __init__(self, plan, cid, tokens, sets):
        import torch
        import workloads as W
        from workloads import device as D
        self.plan = plan
        base = W.config_case(cid, m=tokens if cid == 1 else None)
        self.base = base
        s = base.shape
        self.T, self.H, self.I, self.E, self.k = s.tokens, s.hidden, s.inter, s.experts, s.top_k
        conf = W.CONFIGS[cid]
        self.inputs, self.touched, self.valid = [], [], []
        for j in range(sets):
            c = base if j == 0 else W.make_case(base.name, s, base.seed + 100000 * j, routing=conf["routing"],
                                                scale_lo=base.scale_lo, scale_hi=base.scale_hi,
                                                invalid_frac=conf.get("invalid_frac", 0.0), act=base.act,
                                                weight_seed=base.wseed)
            self.inputs.append((D.to_dev(c.hidden_bits).view(torch.bfloat16), D.to_dev(c.topk_ids),
                                D.to_dev(c.topk_weights)))
            v = c.topk_ids[(c.topk_ids >= 0) & (c.topk_ids < self.E)]
            self.touched.append(len(np.unique(v)))
            self.valid.append(int(v.size))
        self.acc = torch.full((self.T, self.H), float("nan"), device="cuda") if base.nan_accumulator else None
        self.out = torch.empty((self.T, self.H), dtype=torch.bfloat16, device="cuda")

    def per_step(self, j):
        """Algorithmic layer bytes, FC1 bytes and flops of input set j."""
        w13, w2 = expert_bytes(self.H, self.I)
        t, v = self.touched[j % len(self.touched)], self.valid[j % len(self.valid)]
        layer = t * (w13 + w2) + 2 * self.T * self.H * 2 + self.T * self.k * 8
        if self.acc is not None:
            layer += self.T * self.H * 4
        return layer, t * w13 + self.T * self.H * 2, 6.0 * v * self.H * self.I

    def _loop(self, steps, first, events=None):
        for j in range(steps):
            x, ids, wts = self.inputs[(first + j) % len(self.inputs)]
            if events is not None:
                self.plan.set_stage_events(events[j])
            self.plan.forward(x, ids, wts, out=self.out, acc=self.acc)

    def run(self, steps, warmup):
        """Time `steps` forwards back to back (the headline), then the same
        steps again with stage events recorded between the kernels (per-kernel
        durations on the launch stream)."""
        import torch
        self._loop(warmup, 0)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        self._loop(steps, warmup)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
        for e in evs:
            for ev in e:
                ev.record()              # creates the HIP event before the timed loop
        torch.cuda.synchronize()
        self._loop(steps, warmup, evs)
        torch.cuda.synchronize()
        self.plan.set_stage_events(None)
        stage = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in evs])  # ms
        alg = np.array([self.per_step(warmup + j) for j in range(steps)])
        return {"ms_per_step": ms, "ms_per_step_with_events": float(stage.sum(axis=1).mean()),
                "stage_ms": stage.mean(axis=0), "fc1_ms": stage[:, 1],
                "layer_bytes": alg[:, 0].mean(), "fc1_bytes": alg[:, 1].mean(), "flops": alg[:, 2].mean(),
                "graph_ms_per_step": self.run_graph(steps, warmup),
                "fused_ms_per_step": self.run_fused(steps, warmup) if self.fused else None}

    def run_fused(self, steps, warmup):
        """The same steps through the one-launch forward (bf16, at most 256
        routes), or None where it does not apply."""
        import torch
        if self.base.act != "bf16" or self.T * self.k > 256:
            return None
        for j in range(warmup):
            x, ids, wts = self.inputs[j % len(self.inputs)]
            self.plan.forward_fused(x, ids, wts, out=self.out, acc=self.acc)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for j in range(steps):
            x, ids, wts = self.inputs[(warmup + j) % len(self.inputs)]
            self.plan.forward_fused(x, ids, wts, out=self.out, acc=self.acc)
        end.record()
        torch.cuda.synchronize()
        self.plan.fused_status()   # every wait of the last call completed
        return start.elapsed_time(end) / steps

    def run_graph(self, steps, warmup):
        """The same steps replayed from one captured hipGraph per input set (the
        forward enqueues only kernels, so it captures as is): the per-launch
        host and queue gaps drop out, as in a serving loop."""
        import torch
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for x, ids, wts in self.inputs:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    self.plan.forward(x, ids, wts, out=self.out, acc=self.acc)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(side)
        for j in range(warmup):
            graphs[j % len(graphs)].replay()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for j in range(steps):
            graphs[(warmup + j) % len(graphs)].replay()
        end.record()
        torch.cuda.synchronize()
        del graphs
        return start.elapsed_time(end) / steps

    def summary(self, r):
        ms = r["ms_per_step"]
        gbs = r["layer_bytes"] / (ms * 1e-3) / 1e9
        tflops = r["flops"] / (ms * 1e-3) / 1e12
        peak = FP8_PEAK_TFLOPS if self.base.act == "mxfp8" else BF16_PEAK_TFLOPS
        return {"tokens": self.T, "us_per_step": round(ms * 1e3, 2), "tokens_per_s": round(self.T / (ms * 1e-3), 1),
                "layer_hbm_gbs": round(gbs, 1), "layer_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                "tflops": round(tflops, 2), "mfma_frac": round(tflops / peak, 4),
                "mfma_peak_tflops": peak,
                "stage_us": {k: round(float(v) * 1e3, 2) for k, v in zip(STAGES, r["stage_ms"])},
                "us_per_step_with_stage_events": round(r["ms_per_step_with_events"] * 1e3, 2),
                "graph_us_per_step": round(r["graph_ms_per_step"] * 1e3, 2),
                "graph_tokens_per_s": round(self.T / (r["graph_ms_per_step"] * 1e-3), 1),
                **({"fused_us_per_step": round(r["fused_ms_per_step"] * 1e3, 2),
                    "fused_tokens_per_s": round(self.T / (r["fused_ms_per_step"] * 1e-3), 1)}
                   if r.get("fused_ms_per_step") else {})}


# FC1 kernel source of each workload (the counter records hash it with the shared header)
FC1_SOURCE = {"decode": "gemm.hip", "prefill1536": "gemm_prefill.hip", "fusedsum4096": "gemm_prefill.hip",
              "mxfp8x4096": "gemm_prefill_mx.hip"}
PREFILL = {"prefill1536": 2, "fusedsum4096": 3, "mxfp8x4096": 4}


def source_hash(workload):
    import hashlib
    csrc = os.path.join(ROOT, "mxfp4_routed_expert_topk_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, f), "rb").read() for f in (FC1_SOURCE[workload], "moe_internal.h"))
    return hashlib.sha256(src).hexdigest()


class K3Batches(Batches):
    """Input sets of the K3-shape decode workload at M tokens (see workloads.k3_case)."""

    def __init__(self, plan, m, sets):
        import torch
        import workloads as W
        from workloads import device as D
        self.plan = plan
        base = W.k3_case(m)
        self.base = base
        s = base.shape
        self.T, self.H, self.I, self.E, self.k = s.tokens, s.hidden, s.inter, s.experts, s.top_k
        self.inputs, self.touched, self.valid = [], [], []
        for j in range(sets):
            c = base if j == 0 else W.make_case(base.name, s, base.seed + 100000 * j, routing="uniform",
                                                weight_seed=base.wseed)
            self.inputs.append((D.to_dev(c.hidden_bits).view(torch.bfloat16), D.to_dev(c.topk_ids),
                                D.to_dev(c.topk_weights)))
            v = c.topk_ids[(c.topk_ids >= 0) & (c.topk_ids < self.E)]
            self.touched.append(len(np.unique(v)))
            self.valid.append(int(v.size))
        self.acc = None
        self.out = torch.empty((self.T, self.H), dtype=torch.bfloat16, device="cuda")


def counter_traffic(workload, tag):
    """HBM bytes per FC1 launch from the committed rocprofv3 counter runs, or None
    when the kernel sources changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", f"fc1_{tag}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if source_hash(workload) != rec.get("source_sha256"):
        return None
    return rec["hbm_bytes_per_dispatch"]


def cpu_baseline():
    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    case = W.config_case(1, m=128)
    toks = [0, 1, 2, 3, 4, 5]
    cache = {e: case.expert(e) for e in np.unique(case.topk_ids[toks]) if 0 <= e < case.shape.experts}
    t0 = time.perf_counter()
    oracle.forward(case.hidden_bits, case.topk_ids, case.topk_weights, lambda e: cache[e], case.shape.experts,
                   tokens=toks)
    dt = time.perf_counter() - t0
    return {"value": round(len(toks) / dt, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 numpy oracle over tokens {toks} of the decode M=128 batch ({len(cache)} experts, "
                      f"weight generation excluded): {dt:.1f}s; dequantisation runs on one core, the fp64 "
                      f"matmuls on {threads} BLAS threads"}


def router_timings(reps=200):
    """moe_router_topk alone: microseconds per call at the pages' expert counts and
    batch buckets (logits resident in HBM, back-to-back calls)."""
    import torch
    import mxfp4_routed_expert_topk_amd as moe
    import workloads as W
    from workloads import device as D
    res = {}
    for T, E, k in ((1, 224, 8), (128, 224, 8), (128, 896, 16), (4096, 224, 8), (4096, 896, 16)):
        lg = D.to_dev(W.gen_logits(7, T, E))
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        for _ in range(10):
            moe.router_topk(lg, k, ids, w)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(reps):
            moe.router_topk(lg, k, ids, w)
        end.record()
        torch.cuda.synchronize()
        us = start.elapsed_time(end) / reps * 1e3
        res[f"T{T}_E{E}_k{k}"] = {"us": round(us, 2), "logit_gbs": round(T * E * 4 / (us * 1e-6) / 1e9, 1)}
    return res


def prefill_line(args):
    """The JSON line of one prefill configuration (see --workload)."""
    import workloads as W
    cid = PREFILL[args.workload]
    case = W.config_case(cid)
    pl, _ = build_plan(cid, case.shape.tokens)
    b = Batches(pl, cid, None, 2)
    r = b.run(args.steps, args.warmup)
    summ = b.summary(r)
    mx = case.act == "mxfp8"
    s = case.shape
    valid = float(np.mean(b.valid))
    fc1_us = float(np.mean(r["fc1_ms"])) * 1e3
    fc1_tflops = 2.0 * valid * s.hidden * 2 * s.inter / (fc1_us * 1e-6) / 1e12
    peak = FP8_PEAK_TFLOPS if mx else BF16_PEAK_TFLOPS
    tag = f"{args.workload}"
    line = {
        "metric": METRIC, "value": summ["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8xfp4" if mx else "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: {s.tokens} tokens, hidden {s.hidden}, intermediate {s.inter}, "
                               f"{s.experts} experts, top-{s.top_k}, {W.CONFIGS[cid]['routing']} routing, "
                               f"{'MXFP8' if mx else 'bf16'} activations, MXFP4 weights",
                   "tokens": s.tokens, "hidden": s.hidden, "intermediate": s.inter, "experts_resident": s.experts,
                   "top_k": s.top_k},
        "roofline": {"bound": "mfma", "achieved": round(fc1_tflops, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(fc1_tflops / peak, 4), "traffic": counter_traffic(args.workload, tag),
                     "kernel": ("fc_pre_mx<true,8> (FC1, MXFP8, eight waves)" if mx else "fc_pre<true,128,4> (FC1, bf16)"),
                     "kernel_us": round(fc1_us, 2),
                     "alg_flops_per_launch": 2.0 * valid * s.hidden * 2 * s.inter},
        "layer": summ,
    }
    pl.close()
    return line


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--m", type=int, default=128)
    p.add_argument("--sets", type=int, default=8)
    p.add_argument("--no-extra", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--workload", default="decode", choices=["decode"] + list(PREFILL))
    p.add_argument("--fused", action="store_true",
                   help="also time the one-launch (cooperative) fused forward on decode batches")
    p.add_argument("--copy-probe", action="store_true",
                   help="first copy 512 MiB with torch three times: a kernel of known bytes for counter scaling")
    args = p.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one MI355X; --gpus {args.gpus} is not supported by this single-GPU path",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import mxfp4_routed_expert_topk_amd as moe
    import workloads as W
    moe.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    Batches.fused = args.fused
    if args.workload != "decode":
        print(json.dumps(prefill_line(args)), flush=True)
        return
    plan, _ = build_plan(1, max(max(W.DECODE_M), args.m))
    head_b = Batches(plan, 1, args.m, args.sets)
    r = head_b.run(args.steps, args.warmup)
    head = head_b.summary(r)
    log(f"decode M={args.m}: {head}")
    fc1_us = float(np.mean(r["fc1_ms"])) * 1e3
    fc1_gbs = r["fc1_bytes"] / (fc1_us * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode M={args.m}: hidden 7168, intermediate 2048, 224 resident of 384 experts, "
                               f"top-8, MXFP4 weights, bf16 activations",
                   "tokens": args.m, "hidden": 7168, "intermediate": 2048, "experts_resident": 224,
                   "experts_global": 384, "top_k": 8},
        "roofline": {"bound": "hbm", "achieved": round(fc1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(fc1_gbs / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic("decode", "decode_m128") if args.m == 128 else None,
                     "kernel": "fc_dec<true,false,4,4,2> (FC1, bf16, 16-row tiles)", "kernel_us": round(fc1_us, 2),
                     "alg_bytes_per_launch": int(r["fc1_bytes"])},
        "layer": head,
    }
    if not args.no_extra:
        extra = {}
        for m in W.DECODE_M:
            if m == args.m:
                continue
            b = Batches(plan, 1, m, args.sets)
            extra[f"decode_m{m}"] = b.summary(b.run(max(20, args.steps), args.warmup))
            log(f"decode M={m}: {extra[f'decode_m{m}']}")
            del b
        plan.close()
        del plan, head_b
        torch.cuda.empty_cache()
        for cid in (2, 3, 4):
            pl, case = build_plan(cid, W.config_case(cid).shape.tokens)
            b = Batches(pl, cid, None, 2)
            extra[case.name] = b.summary(b.run(10, 3))
            log(f"config {cid} ({case.name}): {extra[case.name]}")
            pl.close()
            del pl, b
            torch.cuda.empty_cache()
        # the pages' own expert shapes (hidden 3584, intermediate 3072, top-16, 224 of 896 experts)
        case = W.k3_case(max(W.K3_DECODE_M))
        t0 = time.time()
        from workloads import device as D
        w = D.upload_experts(case)
        s = case.shape
        pl = moe.Plan(moe.Config(s.hidden, s.inter, s.experts, s.top_k, max(W.K3_DECODE_M), moe.MOE_ACT_BF16), *w)
        del w
        torch.cuda.synchronize()
        log(f"K3 shapes: plan built in {time.time() - t0:.1f}s")
        for m in W.K3_DECODE_M:
            b = K3Batches(pl, m, args.sets)
            extra[f"k3_decode_m{m}"] = b.summary(b.run(max(20, args.steps), args.warmup))
            log(f"K3 decode M={m}: {extra[f'k3_decode_m{m}']}")
            del b
        pl.close()
        del pl
        torch.cuda.empty_cache()
        extra["router_topk"] = router_timings()
        log(f"router: {extra['router_topk']}")
        line["extra"] = extra
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
