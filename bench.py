"""Benchmark of the MXFP4 routed-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--m 128] [--no-extra] [--no-cpu]
                    [--workload decode|prefill1536|fusedsum4096|mxfp8x4096] [--fused] [--no-power]

A step is one moe_mxfp4_forward call (the whole layer: route -> FC1 -> FC2 ->
weighted sum) over one batch of the decode workload: hidden 7168, intermediate
2048, 224 resident of 384 experts, top-8, MXFP4 weights (E8M0 scales in
[120,130]), bf16 activations N(0,1), route ids uniform over 0..383 (ids >= 224
contribute an exact zero), M tokens (default 128).  Inputs are resident in HBM
before timing.  Eight routing/activation sets are rotated so consecutive steps
touch different experts (small-M working sets would otherwise stay in the
256 MB last-level cache between steps).

--workload picks a single prefill configuration instead (1536 tokens uniform,
4096 tokens Zipf fused-sum, 4096 tokens MXFP8), for profiling one workload at a
time: its tokens/s is the value and its FC1 kernel is priced against the MFMA
peak of its dtype (extras and the CPU baseline are skipped).

Prints ONE JSON line:
 * `value`: whole-job tokens/s of K back-to-back eager steps (one event pair);
 * `layer`: per-step event pairs -- median and p90 with warm caches, and again
   with 1 GiB of other data read between steps (cold: nothing of the last step
   is left in the caches) -- the same steps replayed from captured hipGraphs, per-stage
   times, a SHA-256 prefix of the output (input set 0), the operating point
   (median board power and shader clock over a one-second loop of steps), and
   for batches of up to 16 tokens the stream floor (the layer's bytes read by
   the library's read probe in as many launches as the forward makes);
 * `roofline`: the dominant kernel (FC1) timed by HIP events recorded on its
   launch stream, priced against the published peak and against the ceiling
   measured on the same box (`ceilings`: the library's peak micro-benchmarks);
 * `gpu_state`: clocks, power and performance level before and after timing;
 * `context`: the pages' full-model decode step figures (another machine and
   the whole model: context only);
 * `extra` (unless --no-extra): the other decode batch sizes, the prefill
   workloads, the pages' K3 expert shapes and the router;
 * `cpu_baseline` (unless --no-cpu): the fp64 CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
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
FLUSH_BYTES = 1 << 30
SETTLE_S = 0.05                # minimum untimed warm-up of every workload (clock ramp after host work)
FLOOR_BYTES = 2 << 30          # source of the stream-floor probe: revisited only after 2 GiB of other reads
CONTEXT = {
    "pages_full_model_decode_step_ms": {"fused_megamoe": 43.3, "nccl_fixed_chain": 54.6},
    "hardware": "4x GB300 (SM100), expert parallel over 4 GPUs",
    "workload": "FP8 activations x MXFP4 experts, 93-layer K3 model, one decode stream",
    "source": "pegainfer PR #867 (K3 model line: decode E2E at ep_size 4 with MegaMoE(situ) transport), description",
    "note": "context only: a whole-model step on other hardware, not this layer on one MI355X",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def expert_bytes(H, I):
    """Codes + E8M0 scales of one expert: (W13, W2)."""
    return (2 * I * H // 2 + 2 * I * H // 32), (H * I // 2 + H * I // 32)


def pct(a, q):
    return float(np.percentile(np.asarray(a), q))


# ----------------------------------------------------------------------------- box state and ceilings
def gpu_state():
    """Clock levels, power and performance level of the GPU(s), read from the
    amdgpu sysfs files (the pages saw a clock policy move their numbers).  No
    helper program is started: this process has initialised the GPU by then."""
    out = {}
    try:
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            if not os.path.exists(os.path.join(dev, "pp_dpm_sclk")):
                continue
            rec = {}
            for f in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
                try:
                    cur = [ln.strip() for ln in open(os.path.join(dev, f)) if ln.strip().endswith("*")]
                    rec[f[7:]] = cur[0] if cur else None
                except OSError:
                    pass
            try:
                rec["perf_level"] = open(os.path.join(dev, "power_dpm_force_performance_level")).read().strip()
            except OSError:
                pass
            for pw in glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_*")):
                if pw.endswith(("_average", "_input")):
                    try:
                        rec["power_w"] = round(int(open(pw).read()) / 1e6, 1)
                    except (OSError, ValueError):
                        pass
            out[os.path.basename(os.path.dirname(dev))] = rec
    except Exception as e:          # the state is a record, never a reason to fail the run
        out["error"] = repr(e)[:200]
    return out


def ceilings():
    """Measured peaks on this machine with the library's micro-benchmarks: the two
    MFMA instructions the prefill kernels use, then HBM read (plain and
    non-temporal 128-bit loads over 4 GiB) and copy (2 GiB each way, read +
    write bytes).  Run right before the headline's warm-up: a GPU that idled
    through the seconds of host-side set-up runs its first ~20 ms of work
    3-6 % slower while its clocks come back up, which would otherwise fall
    inside the timed steps."""
    import torch
    import mxfp4_routed_expert_topk_amd as moe
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(16384, dtype=torch.float32, device="cuda")
    res = {}

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts, r = [], None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            r = fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return min(ts), r

    for name, kind, iters in (("mfma_bf16_tflops", moe.MOE_PROBE_MFMA_BF16, 4000),
                              ("mfma_f8f4_tflops", moe.MOE_PROBE_MFMA_F8F4, 8000)):
        t, fl = timed(lambda: moe.probe_mfma(kind, iters, sink, cus * 4))
        res[name] = round(fl / t / 1e12, 1)
    buf = torch.ones(4 << 30, dtype=torch.uint8, device="cuda")
    for name, kind in (("hbm_read_gbs", moe.MOE_PROBE_READ), ("hbm_read_nt_gbs", moe.MOE_PROBE_READ_NT)):
        t, _ = timed(lambda: moe.probe_memory(kind, buf, None, sink, cus * 8))
        res[name] = round(buf.numel() / t / 1e9, 1)
    src, dst = buf[: 2 << 30], buf[2 << 30:]
    t, _ = timed(lambda: moe.probe_memory(moe.MOE_PROBE_COPY, src, dst, sink, cus * 8))
    res["hbm_copy_gbs"] = round(2 * src.numel() / t / 1e9, 1)
    del buf, src, dst
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- workloads
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
    """`sets` device-resident input sets of one workload at T tokens."""

    fused = False   # also time the one-launch forward (--fused)
    power_s = 1.0   # length of the loop that samples power and clock (0: none, --no-power)

    def __init__(self, plan, base, sets, make):
        import torch
        from workloads import device as D
        self.plan = plan
        self.base = base
        s = base.shape
        self.T, self.H, self.I, self.E, self.k = s.tokens, s.hidden, s.inter, s.experts, s.top_k
        self.inputs, self.touched, self.valid = [], [], []
        for j in range(sets):
            c = base if j == 0 else make(j)
            self.inputs.append((D.to_dev(c.hidden_bits).view(torch.bfloat16), D.to_dev(c.topk_ids),
                                D.to_dev(c.topk_weights)))
            v = c.topk_ids[(c.topk_ids >= 0) & (c.topk_ids < self.E)]
            self.touched.append(len(np.unique(v)))
            self.valid.append(int(v.size))
        self.acc = torch.full((self.T, self.H), float("nan"), device="cuda") if base.nan_accumulator else None
        self.out = torch.empty((self.T, self.H), dtype=torch.bfloat16, device="cuda")
        self.flush_buf = None

    @classmethod
    def config(cls, plan, cid, tokens, sets):
        import workloads as W
        base = W.config_case(cid, m=tokens if cid == 1 else None)
        conf = W.CONFIGS[cid]
        return cls(plan, base, sets, lambda j: W.make_case(
            base.name, base.shape, base.seed + 100000 * j, routing=conf["routing"], scale_lo=base.scale_lo,
            scale_hi=base.scale_hi, invalid_frac=conf.get("invalid_frac", 0.0), act=base.act,
            weight_seed=base.wseed))

    @classmethod
    def k3(cls, plan, m, sets):
        import workloads as W
        base = W.k3_case(m)
        return cls(plan, base, sets, lambda j: W.make_case(base.name, base.shape, base.seed + 100000 * j,
                                                           routing="uniform", weight_seed=base.wseed))

    def per_step(self, j):
        """Algorithmic layer bytes, FC1 bytes and flops of input set j."""
        w13, w2 = expert_bytes(self.H, self.I)
        t, v = self.touched[j % len(self.touched)], self.valid[j % len(self.valid)]
        layer = t * (w13 + w2) + 2 * self.T * self.H * 2 + self.T * self.k * 8
        if self.acc is not None:
            layer += self.T * self.H * 4
        return layer, t * w13 + self.T * self.H * 2, 6.0 * v * self.H * self.I

    def step(self, j):
        x, ids, wts = self.inputs[j % len(self.inputs)]
        self.plan.forward(x, ids, wts, out=self.out, acc=self.acc)

    def _flush(self):
        """Read 1 GiB of other data (the library's read probe): the caches then
        hold none of the last step's weights, and nothing dirty is left to
        write back during the next step (a write flush would leave that)."""
        import torch
        import mxfp4_routed_expert_topk_amd as moe
        if self.flush_buf is None:
            self.flush_buf = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
            self.flush_sink = torch.empty(16384, dtype=torch.float32, device="cuda")
            self.flush_grid = torch.cuda.get_device_properties(0).multi_processor_count * 8
            torch.cuda.synchronize()
        moe.probe_memory(moe.MOE_PROBE_READ, self.flush_buf, None, self.flush_sink, self.flush_grid)

    def per_step_times(self, steps, first, flush):
        """One event pair per step; with `flush`, 1 GiB of other data is read
        between steps (outside the timed pairs)."""
        import torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(evs):
            if flush:
                self._flush()
            a.record()
            self.step(first + j)
            b.record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])   # ms

    def run(self, steps, warmup, settle_s=0.0):
        """The headline (back-to-back steps, one event pair), then per-step
        pairs warm and cold, stage events (per-kernel times on the launch
        stream), graph replay, and optionally the one-launch forward.  With
        `settle_s`, the untimed warm-up goes on past `warmup` steps until that
        many seconds have passed (every workload starts after host-side work:
        input generation, or the ceiling probes, with the GPU's clocks not yet
        at the layer's steady state)."""
        import torch
        t0 = time.time()
        j = 0
        while j < warmup or time.time() - t0 < settle_s:
            self.step(j)
            j += 1
            if j >= warmup and settle_s > 0:
                torch.cuda.synchronize()
        warmup = j
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for j in range(steps):
            self.step(warmup + j)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        warm = self.per_step_times(steps, warmup, False)
        cold = self.per_step_times(steps, warmup, True)
        self.flush_buf = None
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
        for e in evs:
            for ev in e:
                ev.record()              # creates the HIP event before the timed loop
        torch.cuda.synchronize()
        for j in range(steps):
            self.plan.set_stage_events(evs[j])
            self.step(warmup + j)
        torch.cuda.synchronize()
        self.plan.set_stage_events(None)
        stage = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in evs])  # ms
        alg = np.array([self.per_step(warmup + j) for j in range(steps)])
        return {"ms_per_step": ms, "warmup_steps_run": warmup, "warm_ms": warm, "cold_ms": cold,
                "ms_per_step_with_events": float(stage.sum(axis=1).mean()),
                "stage_ms": stage.mean(axis=0), "fc1_ms": stage[:, 1],
                "layer_bytes": alg[:, 0].mean(), "fc1_bytes": alg[:, 1].mean(), "flops": alg[:, 2].mean(),
                "graph_ms_per_step": self.run_graph(steps, warmup),
                "fused_ms_per_step": self.run_fused(steps, warmup) if self.fused else None,
                "digest": self.digest(),
                "stream_floor_us": self.stream_floor(),
                "operating_point": self.power_loop(self.power_s) if self.power_s > 0 else None}

    def digest(self):
        """SHA-256 prefix of the outputs of input set 0 (bf16 out, and the fp32
        accumulator where the workload keeps one): equal across runs and boxes
        when the kernels are deterministic."""
        import torch
        self.step(0)
        torch.cuda.synchronize()
        h = hashlib.sha256(self.out.view(torch.uint8).cpu().numpy().tobytes())
        if self.acc is not None:
            h.update(self.acc.view(torch.uint8).cpu().numpy().tobytes())
        return h.hexdigest()[:16]

    def stream_floor(self, reps=40):
        """The layer's algorithmic bytes streamed by the library's read probe
        (non-temporal 128-bit loads) in as many launches as the forward makes
        -- two up to 32 routes (FC1; FC2 with the sum), else four (route, FC1,
        FC2, combine; the route and combine launches read 64 KB and the
        output) -- back to back under one event pair: what a chain of kernels
        that did nothing but move the layer's bytes reaches at this batch size,
        launch gaps and ramp included.  Microseconds per layer; small batches
        only (up to 16 tokens), where launches are a large part of the time."""
        import torch
        import mxfp4_routed_expert_topk_amd as moe
        if self.base.act != "bf16" or self.T > 16:
            return None
        w13, w2 = expert_bytes(self.H, self.I)
        t = float(np.mean(self.touched))
        R = self.T * self.k
        fc1 = t * w13 + self.T * self.H * 2
        fc2 = t * w2 + R * self.I * 2
        sizes = [fc1, fc2] if R <= 32 else [64 << 10, fc1, fc2, (64 << 10) + self.T * self.H * 2]
        sizes = [int(b + 4095) // 4096 * 4096 for b in sizes]
        src = torch.empty(FLOOR_BYTES, dtype=torch.uint8, device="cuda")
        sink = torch.empty(16384, dtype=torch.float32, device="cuda")
        grid = torch.cuda.get_device_properties(0).multi_processor_count * 8
        off = [0]

        def layer():
            for b in sizes:
                if off[0] + b > FLOOR_BYTES:
                    off[0] = 0
                moe.probe_memory(moe.MOE_PROBE_READ_NT, src[off[0]:off[0] + b], None, sink, grid)
                off[0] += b

        for _ in range(10):
            layer()
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            layer()
        e.record()
        torch.cuda.synchronize()
        del src
        return a.elapsed_time(e) / reps * 1e3

    def power_loop(self, seconds):
        """Steps back to back for `seconds` while a thread reads the board power
        and the current shader clock level from sysfs every 20 ms: the operating
        point the timed legs ran at (a layer that reaches the board's power cap
        runs at a lower clock).  Medians over the samples after the first
        quarter of the loop, when the clock has settled."""
        import threading
        import torch
        dev = next((d for d in sorted(glob.glob("/sys/class/drm/card*/device"))
                    if os.path.exists(os.path.join(d, "pp_dpm_sclk"))), None)
        if dev is None:
            return None
        pw = [f for f in glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_*"))
              if f.endswith(("_input", "_average"))]
        cap = glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_cap"))
        samples, stop = [], threading.Event()

        def sample():
            while not stop.is_set():
                try:
                    w = int(open(pw[0]).read()) / 1e6 if pw else None
                    cur = [ln for ln in open(os.path.join(dev, "pp_dpm_sclk")) if ln.strip().endswith("*")]
                    mhz = float(cur[0].split(":")[1].strip().split("Mhz")[0].split("MHz")[0]) if cur else None
                    samples.append((time.time(), w, mhz))
                except (OSError, ValueError, IndexError):
                    pass
                stop.wait(0.02)

        torch.cuda.synchronize()
        th = threading.Thread(target=sample, daemon=True)
        t0 = time.time()
        th.start()
        n = 0
        while time.time() - t0 < seconds:
            for j in range(8):
                self.step(n + j)
            n += 8
            torch.cuda.synchronize()
        t1 = time.time()
        stop.set()
        th.join()
        keep = [x for x in samples if x[0] >= t0 + 0.25 * (t1 - t0)]
        pws = np.array([x[1] for x in keep if x[1] is not None])
        mhz = np.array([x[2] for x in keep if x[2] is not None])
        rec = {"seconds": round(t1 - t0, 2), "steps": n, "us_per_step": round((t1 - t0) / n * 1e6, 1),
               "samples": len(keep),
               "power_w_p50": round(float(np.median(pws)), 1) if pws.size else None,
               "sclk_mhz_p50": round(float(np.median(mhz)), 0) if mhz.size else None}
        try:
            rec["power_cap_w"] = round(int(open(cap[0]).read()) / 1e6, 1) if cap else None
        except (OSError, ValueError):
            rec["power_cap_w"] = None
        return rec

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
        """The same steps replayed from one captured hipGraph that holds a
        forward for every input set in turn (the forward enqueues only kernels,
        so it captures as is), as a serving loop would capture a whole
        model's layers: the per-launch host and queue gaps drop out, and one
        graph launch covers several forwards (at one forward per graph the
        graph launch itself costs more than a small batch's two kernel
        launches).  Replayed until at least `steps` forwards have run;
        microseconds per forward."""
        import torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for x, ids, wts in self.inputs:
                    self.plan.forward(x, ids, wts, out=self.out, acc=self.acc)
        torch.cuda.current_stream().wait_stream(side)
        per = len(self.inputs)
        for _ in range(max(1, -(-warmup // per))):
            g.replay()
        reps = max(1, -(-steps // per))
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(reps):
            g.replay()
        end.record()
        torch.cuda.synchronize()
        del g
        return start.elapsed_time(end) / (reps * per)

    def summary(self, r, ceil=None):
        ms = r["ms_per_step"]
        gbs = r["layer_bytes"] / (ms * 1e-3) / 1e9
        tflops = r["flops"] / (ms * 1e-3) / 1e12
        peak = FP8_PEAK_TFLOPS if self.base.act == "mxfp8" else BF16_PEAK_TFLOPS
        out = {"tokens": self.T, "us_per_step": round(ms * 1e3, 2), "tokens_per_s": round(self.T / (ms * 1e-3), 1),
               "p50_us": round(pct(r["warm_ms"], 50) * 1e3, 2), "p90_us": round(pct(r["warm_ms"], 90) * 1e3, 2),
               "cold_p50_us": round(pct(r["cold_ms"], 50) * 1e3, 2),
               "cold_p90_us": round(pct(r["cold_ms"], 90) * 1e3, 2),
               "layer_hbm_gbs": round(gbs, 1), "layer_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
               "tflops": round(tflops, 2), "mfma_frac": round(tflops / peak, 4), "mfma_peak_tflops": peak,
               "stage_us": {k: round(float(v) * 1e3, 2) for k, v in zip(STAGES, r["stage_ms"])},
               "us_per_step_with_stage_events": round(r["ms_per_step_with_events"] * 1e3, 2),
               "graph_us_per_step": round(r["graph_ms_per_step"] * 1e3, 2),
               "graph_tokens_per_s": round(self.T / (r["graph_ms_per_step"] * 1e-3), 1),
               "output_sha256_16": r["digest"]}
        if ceil:
            out["layer_hbm_frac_of_measured_read"] = round(gbs / ceil["hbm_read_nt_gbs"], 4)
            key = "mfma_f8f4_tflops" if self.base.act == "mxfp8" else "mfma_bf16_tflops"
            out["mfma_frac_of_measured"] = round(tflops / ceil[key], 4)
        if r.get("stream_floor_us"):
            out["stream_floor_us"] = round(r["stream_floor_us"], 2)
            out["frac_of_stream_floor"] = round(r["stream_floor_us"] / (ms * 1e3), 4)
        if r.get("operating_point"):
            out["operating_point"] = r["operating_point"]
        if r.get("fused_ms_per_step"):
            out["fused_us_per_step"] = round(r["fused_ms_per_step"] * 1e3, 2)
            out["fused_tokens_per_s"] = round(self.T / (r["fused_ms_per_step"] * 1e-3), 1)
        return out


# FC1 kernel source of each workload (the counter records hash it with the shared header)
FC1_SOURCE = {"decode": ("gemm.hip", "dec_core.h"), "prefill1536": ("gemm_prefill.hip",),
              "fusedsum4096": ("gemm_prefill.hip",), "mxfp8x4096": ("gemm_prefill_mx.hip",)}
PREFILL = {"prefill1536": 2, "fusedsum4096": 3, "mxfp8x4096": 4}


def source_hash(workload):
    csrc = os.path.join(ROOT, "mxfp4_routed_expert_topk_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, f), "rb").read() for f in FC1_SOURCE[workload] + ("moe_internal.h",))
    return hashlib.sha256(src).hexdigest()


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
    """The fp64 oracle, as it stands, on the whole decode M=128 batch (about
    10 s of host work), its experts evaluated on a thread per host core (BLAS
    single-threaded inside each)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    import oracle
    import workloads as W
    threads = max(1, min(16, os.cpu_count() or 1))
    case = W.config_case(1, m=128)
    toks = list(range(case.shape.tokens))
    cache = {e: case.expert(e) for e in np.unique(case.topk_ids[toks]) if 0 <= e < case.shape.experts}
    with ThreadPoolExecutor(threads) as ex, threadpool_limits(1, "blas"):
        t0 = time.perf_counter()
        oracle.forward(case.hidden_bits, case.topk_ids, case.topk_weights, lambda e: cache[e], case.shape.experts,
                       tokens=toks, pool=ex)
        dt = time.perf_counter() - t0
    return {"value": round(len(toks) / dt, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 numpy oracle over all {len(toks)} tokens of the decode M=128 batch ({len(cache)} experts, "
                      f"weight generation excluded): {dt:.1f}s on {threads} threads (one expert each at a time, "
                      f"BLAS single-threaded); the host reports {os.cpu_count()} CPUs"}


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


def base_line(args, r, summ, config):
    return {"metric": METRIC, "value": summ["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "warmup_steps_run": r["warmup_steps_run"],
            "ms_per_step": round(r["ms_per_step"], 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "data": "synthetic", "config": config, "layer": summ}


def prefill_line(args, measured_ceilings):
    """The JSON line of one prefill configuration (see --workload)."""
    import workloads as W
    cid = PREFILL[args.workload]
    case = W.config_case(cid)
    pl, _ = build_plan(cid, case.shape.tokens)
    b = Batches.config(pl, cid, None, 2)
    ceil = measured_ceilings()
    r = b.run(args.steps, args.warmup, SETTLE_S)
    summ = b.summary(r, ceil)
    mx = case.act == "mxfp8"
    s = case.shape
    valid = float(np.mean(b.valid))
    fc1_us = float(np.mean(r["fc1_ms"])) * 1e3
    fc1_flops = 2.0 * valid * s.hidden * 2 * s.inter
    fc1_tflops = fc1_flops / (fc1_us * 1e-6) / 1e12
    peak = FP8_PEAK_TFLOPS if mx else BF16_PEAK_TFLOPS
    config = {"workload": f"{args.workload}: {s.tokens} tokens, hidden {s.hidden}, intermediate {s.inter}, "
                          f"{s.experts} experts, top-{s.top_k}, {W.CONFIGS[cid]['routing']} routing, "
                          f"{'MXFP8' if mx else 'bf16'} activations, MXFP4 weights",
              "tokens": s.tokens, "hidden": s.hidden, "intermediate": s.inter, "experts_resident": s.experts,
              "top_k": s.top_k}
    line = base_line(args, r, summ, config)
    line["dtype"] = "fp8xfp4" if mx else "bf16"
    line["roofline"] = {
        "bound": "mfma", "achieved": round(fc1_tflops, 1), "peak": peak, "unit": "TFLOP/s",
        "frac": round(fc1_tflops / peak, 4), "traffic": counter_traffic(args.workload, args.workload),
        "kernel": ("fc_pre_mx<true,8> (FC1, MXFP8, eight waves)" if mx else "fc_pre<true,128,4> (FC1, bf16)"),
        "kernel_us": round(fc1_us, 2), "alg_flops_per_launch": fc1_flops}
    if ceil:
        key = "mfma_f8f4_tflops" if mx else "mfma_bf16_tflops"
        line["roofline"]["measured_peak"] = ceil[key]
        line["roofline"]["frac_of_measured"] = round(fc1_tflops / ceil[key], 4)
    pl.close()
    line["_ceil"] = ceil
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
    p.add_argument("--no-ceilings", action="store_true", help="skip the peak micro-benchmarks")
    p.add_argument("--workload", default="decode", choices=["decode"] + list(PREFILL))
    p.add_argument("--fused", action="store_true",
                   help="also time the one-launch (cooperative) fused forward on decode batches")
    p.add_argument("--no-power", action="store_true",
                   help="skip the one-second loop per workload that samples board power and shader clock")
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
    Batches.power_s = 0.0 if args.no_power else 1.0
    state_before = gpu_state()

    def measured_ceilings():
        c = None if args.no_ceilings else ceilings()
        if c:
            log(f"measured ceilings: {c}")
        return c

    if args.workload != "decode":
        line = prefill_line(args, measured_ceilings)
        ceil = line.pop("_ceil")
        line["ceilings"] = ceil
        line["gpu_state"] = {"before": state_before, "after": gpu_state()}
        line["context"] = CONTEXT
        print(json.dumps(line), flush=True)
        return
    plan, _ = build_plan(1, max(max(W.DECODE_M), args.m))
    head_b = Batches.config(plan, 1, args.m, args.sets)
    ceil = measured_ceilings()
    r = head_b.run(args.steps, args.warmup, SETTLE_S)
    head = head_b.summary(r, ceil)
    log(f"decode M={args.m}: {head}")
    fc1_us = float(np.mean(r["fc1_ms"])) * 1e3
    fc1_gbs = r["fc1_bytes"] / (fc1_us * 1e-6) / 1e9
    config = {"workload": f"decode M={args.m}: hidden 7168, intermediate 2048, 224 resident of 384 experts, "
                          f"top-8, MXFP4 weights, bf16 activations",
              "tokens": args.m, "hidden": 7168, "intermediate": 2048, "experts_resident": 224,
              "experts_global": 384, "top_k": 8}
    line = base_line(args, r, head, config)
    line["dtype"] = "bf16"
    line["roofline"] = {
        "bound": "hbm", "achieved": round(fc1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(fc1_gbs / HBM_PEAK_GBS, 4),
        "traffic": counter_traffic("decode", "decode_m128") if args.m == 128 else None,
        "kernel": ("fc_dec<true,false,4,4,2,false,true,2> (FC1, bf16, 16-row tiles, group schedule, two K "
                   "ranges per wave)" if args.m >= 32 else
                   "fc_dec<true,false,4,4,2,false,true,4> (FC1, bf16, 16-row tiles, group schedule)" if args.m > 4
                   else "fc_dec<true,false,2,4,2,true,true,4> (FC1, bf16, one route per tile, group schedule)"),
        "kernel_us": round(fc1_us, 2),
        "alg_bytes_per_launch": int(r["fc1_bytes"])}
    if ceil:
        line["roofline"]["measured_peak"] = ceil["hbm_read_nt_gbs"]
        line["roofline"]["frac_of_measured"] = round(fc1_gbs / ceil["hbm_read_nt_gbs"], 4)
    if not args.no_extra:
        extra = {}
        for m in W.DECODE_M:
            if m == args.m:
                continue
            b = Batches.config(plan, 1, m, args.sets)
            extra[f"decode_m{m}"] = b.summary(b.run(max(20, args.steps), args.warmup, SETTLE_S), ceil)
            log(f"decode M={m}: {extra[f'decode_m{m}']}")
            del b
        plan.close()
        del plan, head_b
        torch.cuda.empty_cache()
        for cid in (2, 3, 4):
            pl, case = build_plan(cid, W.config_case(cid).shape.tokens)
            b = Batches.config(pl, cid, None, 2)
            extra[case.name] = b.summary(b.run(10, 3, SETTLE_S), ceil)
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
            b = Batches.k3(pl, m, args.sets)
            extra[f"k3_decode_m{m}"] = b.summary(b.run(max(20, args.steps), args.warmup, SETTLE_S), ceil)
            log(f"K3 decode M={m}: {extra[f'k3_decode_m{m}']}")
            del b
        pl.close()
        del pl
        torch.cuda.empty_cache()
        extra["router_topk"] = router_timings()
        log(f"router: {extra['router_topk']}")
        line["extra"] = extra
    line["ceilings"] = ceil
    line["gpu_state"] = {"before": state_before, "after": gpu_state()}
    line["context"] = CONTEXT
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
