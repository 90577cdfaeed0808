"""Benchmark of the routed SwiGLU MoE forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|<name>]

One step = the whole hot path over one batch of synthetic inputs already
resident in HBM: the router (moe_route: softmax, top-k, canonical ids) and the
forward (moe_forward: permutation, FC1 + SwiGLU, FC2, fp32 finalize).  W
untimed warm-up steps, then exactly K timed steps between two
torch.cuda.synchronize() calls.  Prints ONE JSON line.

By default every workload is measured in the same run (tiny, decode, logprob,
bf16_16k, mxfp8_16k, bounded_decode, decode_mxfp4, mxfp4_16k); the line's
headline fields are the decode-sized launch (256 tokens, hidden 2048, FFN
1024, 64 experts, top-6, bf16) and `configs` holds every workload's own
record (step time, tokens/s, TFLOP/s, % of MFMA and HBM peak, roofline of its
FC1 stage, CPU oracle baseline).  Kernel-weight buffers are rotated between
steps so that the expert weights cannot be served from the 256 MB Infinity
Cache.  `roofline` reports the dominant kernel's algorithmic bytes
(or flops) per launch over its average duration, measured with HIP events
recorded by the library on the forward's stream during the timed steps.
`cpu_baseline` times the CPU oracle (test infrastructure, never tuned) on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed MoE fwd tokens/s + TFLOP/s (% MFMA peak; % HBM peak at decode)"
HBM_PEAK_GBS = 8000.0
# dense MFMA peaks; MXFP4 weights meet MXFP8 activations, so its MFMA runs at the
# fp8 rate (the 10.1 PF/s fp4 figure is for 4-bit operands on both sides)
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "mxfp4": 5000.0}
MFMA_BOUND = ("bf16_16k", "mxfp8_16k", "mxfp4_16k")
MALL_BYTES = 256 << 20


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="all",
                   help="one workload, or 'all': every configuration in one run, with the "
                        "decode workload as the headline line and the others under 'configs'")
    p.add_argument("--seed", type=int, default=11)
    p.add_argument("--combine", default="fp32", choices=["fp32", "bf16", "rows"],
                   help="how a token's routes are combined (moe_forward_ex): the fp32 chain, "
                        "the fp32 chain rounded to bf16, or every route's row unscaled")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample of the headline workload")
    p.add_argument("--cpu-seconds-other", type=float, default=3.0,
                   help="target CPU time of the oracle sample of every other workload")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy 5 times (to scale HBM counters)")
    return p.parse_args()


def copy_calibration():
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch, the
    reference that converts FETCH_SIZE / WRITE_SIZE counter readings to bytes."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}))


GEMM_SOURCES = ["swiglu_expert_mlp_amd/csrc/gemm_bf16.hip", "swiglu_expert_mlp_amd/csrc/gemm_bf16_small.h",
                "swiglu_expert_mlp_amd/csrc/gemm_bf16_big.h", "swiglu_expert_mlp_amd/csrc/gemm_mxfp8.hip",
                "swiglu_expert_mlp_amd/csrc/gemm_mxfp8_stream.h", "swiglu_expert_mlp_amd/csrc/gemm_mxfp8_lds.h",
                "swiglu_expert_mlp_amd/csrc/gemm_mx4_small.h",
                "swiglu_expert_mlp_amd/csrc/gemm_args.h", "swiglu_expert_mlp_amd/csrc/common.h"]


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    runs (profiles/traffic.json), or None when the GEMM sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    entry = json.load(open(path)).get(workload)
    if not entry:
        return None
    h = hashlib.sha256()
    for s in GEMM_SOURCES:
        with open(os.path.join(ROOT, s), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != entry.get("gemm_source_sha256"):
        return None
    return entry["fetch_bytes_per_launch"] + entry["write_bytes_per_launch"]


def alg_bytes(w, precision: str, touched: int, combine: str = "fp32") -> dict:
    """Algorithmic bytes: each touched expert's weights once, each live token's
    x row once, routed rows written/read once where a stage must (FC1 writes
    the SwiGLU row, FC2 reads it), ids/probs once, the output once (fp32 [T, H],
    bf16 [T, H] or fp32 [T, k, H] by combine)."""
    # weight and activation (SwiGLU row) bytes per element, E8M0 scales included
    ww = {"bf16": 2.0, "mxfp8": 1 + 1.0 / 32, "mxfp4": 0.5 + 1.0 / 32}[precision]
    wa = 2.0 if precision == "bf16" else 1 + 1.0 / 32
    H, F, T, R = w.H, w.F, w.T, w.R
    fc1 = touched * 2 * F * H * ww + T * H * 2 + R * F * wa
    fc2 = touched * H * F * ww + R * F * wa + R * H * 4
    out_b = {"fp32": T * H * 4, "bf16": T * H * 2, "rows": R * H * 4}[combine]
    step = touched * 3 * F * H * ww + T * H * 2 + T * w.k * 8 + out_b
    return dict(fc1=fc1, fc2=fc2, step=step)


class HipEvents:
    """HIP timing events created with a device-scope release
    (hipEventReleaseToDevice), which keeps the record cheap: a default event
    does a system-scope cache write-back at every record."""

    RELEASE_TO_DEVICE = 0x40000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def new(self) -> int:
        ev = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.RELEASE_TO_DEVICE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.made.append(ev.value)
        return ev.value

    def record(self, ev: int, stream: int):
        rc = self.hip.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def ms(self, a: int, b: int) -> float:
        out = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def close(self):
        for ev in self.made:
            self.hip.hipEventDestroy(ev)
        self.made = []


# every configuration the default run measures, the headline first
ALL_WORKLOADS = ("decode", "tiny", "logprob", "bf16_16k", "mxfp8_16k", "bounded_decode",
                 "decode_mxfp4", "mxfp4_16k")
HEADLINE = "decode"
# bf16 workloads whose line also times the single-launch FFN mode (MOE_FUSED_FFN)
FUSED_REPORT = ("decode", "bf16_16k")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_INPUT_CACHE = {}


def inputs_for(w, seed: int):
    """Seeded inputs of workload w (workloads of equal shapes, seed and outlier
    choice share one draw)."""
    key = (w.T, w.T_cap, w.H, w.F, w.E, w.k, w.bias, seed, w.precision != "bf16")
    if key not in _INPUT_CACHE:
        from workloads import make_inputs
        _INPUT_CACHE.clear()
        _INPUT_CACHE[key] = make_inputs(w, seed=seed, outliers=(w.precision != "bf16"))
    return _INPUT_CACHE[key]


def roofline_of(w, ab: dict, fc1_us: float) -> dict:
    """The FC1 + SwiGLU stage against the roofline whose floor is higher for it:
    HBM (its algorithmic bytes) or MFMA (its flops at the precision's peak)."""
    fc1_flops = 4.0 * w.H * w.F * w.R
    t_hbm = ab["fc1"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = fc1_flops / (MFMA_PEAK_TFLOPS[w.precision] * 1e12)
    hbm = dict(bound="hbm", achieved=ab["fc1"] / (fc1_us * 1e-6) / 1e9, peak=HBM_PEAK_GBS,
               unit="GB/s")
    mfma = dict(bound="mfma", achieved=fc1_flops / (fc1_us * 1e-6) / 1e12,
                peak=MFMA_PEAK_TFLOPS[w.precision], unit="TFLOP/s")
    roof, other = (mfma, hbm) if (w.name in MFMA_BOUND or t_mfma > t_hbm) else (hbm, mfma)
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["other_bound"] = {"bound": other["bound"], "frac": other["achieved"] / other["peak"]}
    return roof


def run_workload(name: str, a, cpu_seconds: float, threads1: bool) -> dict:
    import torch
    from workloads import WORKLOADS
    from swiglu_expert_mlp_amd import MoE

    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    inp = inputs_for(w, a.seed)
    bf = lambda arr: torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(
        torch.bfloat16).to(dev)
    x = bf(inp["x_bits"])
    w1 = bf(inp["w1_bits"])
    w2 = bf(inp["w2_bits"])
    logits = torch.from_numpy(inp["logits"]).to(dev)
    live = torch.tensor([w.T], dtype=torch.int32, device=dev)

    # rotate kernel-weight buffers so that their total exceeds twice the MALL
    moe0 = MoE(w.E, w.H, w.F, w.k, w.precision)
    kb = moe0.weight_bytes
    n_rot = max(2, math.ceil(2 * MALL_BYTES / kb) + 1) if kb < 2 * MALL_BYTES else 2
    moes = [moe0] + [MoE(w.E, w.H, w.F, w.k, w.precision) for _ in range(n_rot - 1)]
    for m in moes:
        m.load_weights(w1, w2)
    del w1, w2
    ws = moe0.new_workspace(w.T_cap)
    ids = torch.empty((w.T_cap, w.k), dtype=torch.int32, device=dev)
    probs = torch.empty((w.T_cap, w.k), dtype=torch.float32, device=dev)
    out = {"fp32": lambda: torch.empty((w.T_cap, w.H), dtype=torch.float32, device=dev),
           "bf16": lambda: torch.empty((w.T_cap, w.H), dtype=torch.bfloat16, device=dev),
           "rows": lambda: torch.empty((w.T_cap, w.k, w.H), dtype=torch.float32, device=dev)}[
        a.combine]()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    route_fn = [m.bind_route(logits, live, ids, probs, ws) for m in moes]
    fwd_fn = [m.bind_forward(x, ids, probs, live, out, ws, combine=a.combine) for m in moes]

    def step(i):
        route_fn[i % n_rot]()
        fwd_fn[i % n_rot]()

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    bits = moe0.check(ws)
    if bits:
        raise RuntimeError(f"{name}: device contract violation bits {bits}")
    idx = moe0.get_indices(ws, w.T_cap)
    touched = int(np.count_nonzero(idx["counts"]))
    loads = idx["counts"].astype(np.int64)

    # timed region: K steps with events only around the whole loop (events
    # recorded by the dispatches inside the loop cost about 11 us of gaps per
    # step at decode sizes, so they are kept out of the step time)
    ev = HipEvents()
    t0, t1 = ev.new(), ev.new()
    torch.cuda.synchronize()
    ev.record(t0, sh)
    for i in range(a.steps):
        step(i)
    ev.record(t1, sh)
    torch.cuda.synchronize()
    ms_step = ev.ms(t0, t1) / a.steps

    # the dominant launch (FC1 + SwiGLU): a second timed pass of K steps in
    # which every FC1 launch records its own start and end into two events
    # (hipExtLaunchKernel: the dispatch carries them); its mean duration is the
    # roofline's kernel time
    fc1_ev = [(ev.new(), ev.new()) for _ in range(a.steps)]
    p0, p1 = ev.new(), ev.new()
    torch.cuda.synchronize()
    ev.record(p0, sh)
    for i in range(a.steps):
        m = moes[i % n_rot]
        m.set_stage_events([None, None, fc1_ev[i][0], fc1_ev[i][1], None, None])
        step(i)
    ev.record(p1, sh)
    torch.cuda.synchronize()
    for m in moes:
        m.set_stage_events(None)
    ms_step_instrumented = ev.ms(p0, p1) / a.steps
    fc1_us = float(np.mean([ev.ms(p, q) for p, q in fc1_ev]) * 1e3)

    # the single-launch modes, timed the same way: FC1 + FC2 in one launch
    # (MOE_FUSED_FFN), and FC1 + FC2 + finalize in one launch (MOE_FUSED_FINALIZE)
    fused = None
    if w.precision == "bf16" and name in FUSED_REPORT:
        fused = {}
        for key, kw in (("ffn", {"fused_ffn": True}), ("ffn_finalize", {"fused_finalize": True})):
            fused_fn = [m.bind_forward(x, ids, probs, live, out, ws, combine=a.combine, **kw)
                        for m in moes]
            for i in range(min(a.warmup, 5)):
                route_fn[i % n_rot]()
                fused_fn[i % n_rot]()
            f0, f1 = ev.new(), ev.new()
            torch.cuda.synchronize()
            ev.record(f0, sh)
            for i in range(a.steps):
                route_fn[i % n_rot]()
                fused_fn[i % n_rot]()
            ev.record(f1, sh)
            torch.cuda.synchronize()
            bits = moe0.check(ws)
            if bits:
                raise RuntimeError(f"{name}: single-launch {key}: device contract violation bits {bits}")
            ms_f = ev.ms(f0, f1) / a.steps
            fin = key == "ffn_finalize"
            fused[key] = {"ms_per_step": ms_f, "tokens_per_s": w.T / (ms_f * 1e-3),
                          "speedup_vs_separate_launches": ms_step / ms_f,
                          "kernel": f"moe::gemm_bf16_fused_kernel<false, {str(fin).lower()}> "
                                    "(every tile as a 64-row tile"
                                    + (", the last FC2 tile of a token's 512 columns combines them)"
                                       if fin else ")")}
            del fused_fn

    # stage breakdown (untimed diagnostic pass)
    n_diag = min(10, a.steps)
    diag = [[ev.new() for _ in range(8)] for _ in range(n_diag)]
    for i in range(n_diag):
        m = moes[i % n_rot]
        d = diag[i]
        ev.record(d[6], sh)
        route_fn[i % n_rot]()
        ev.record(d[7], sh)
        m.set_stage_events(d[:6])
        fwd_fn[i % n_rot]()
        m.set_stage_events(None)
    torch.cuda.synchronize()
    names = MoE.STAGES
    stage_us = {n: float(np.mean([ev.ms(d[j], d[j + 1]) for d in diag]) * 1e3)
                for j, n in enumerate(names)}
    stage_us = {"route": float(np.mean([ev.ms(d[6], d[7]) for d in diag]) * 1e3), **stage_us}
    ev.close()

    ab = alg_bytes(w, w.precision, touched, a.combine)
    flops = w.flops()
    tokens_s = w.T / (ms_step * 1e-3)
    tflops = flops / (ms_step * 1e-3) / 1e12
    roof = roofline_of(w, ab, fc1_us)
    # the FC1 + SwiGLU stage: its tiles are 256-row tiles (experts with more than
    # 128 rows) or 64-row tiles (the others); one launch at token capacities up
    # to 1024 (the 64-row kernel takes every tile), else the 256-row launch and
    # then the 64-row launch (MXFP8: one launch for both)
    small = w.T_cap <= 1024
    roof["kernel"] = {"bf16": "moe::gemm_bf16_small_kernel<true, false>" if small else
                              "moe::gemm_bf16_big_kernel<true, false> + moe::gemm_bf16_small_kernel<true, false>",
                      "mxfp8": "moe::gemm_mxfp8_kernel<true, false, false>",
                      "mxfp4": "moe::gemm_mx4_small_kernel<true, false>" if small else
                               "moe::gemm_mxfp8_kernel<true, true, false> + moe::gemm_mx4_small_kernel<true, false>"
                      }[w.precision]
    roof["tiles"] = "256-row" if int(loads.min()) > 128 else (
        "64-row" if int(loads.max()) <= 128 else "256-row + 64-row")
    roof["kernel_us"] = fc1_us
    roof["algorithmic_bytes"] = ab["fc1"]
    roof["algorithmic_flops"] = 4.0 * w.H * w.F * w.R
    roof["traffic"] = measured_traffic(w.name)

    res = {
        "workload": w.name, "tokens": w.T, "token_capacity": w.T_cap, "hidden": w.H,
        "ffn": w.F, "experts": w.E, "topk": w.k, "precision": w.precision,
        "ms_per_step": ms_step, "tokens_per_s": tokens_s, "tflops": tflops,
        "mfma_frac": tflops / MFMA_PEAK_TFLOPS[w.precision],
        "hbm_gbs_step": ab["step"] / (ms_step * 1e-3) / 1e9,
        "hbm_frac_step": ab["step"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "stages_us": stage_us,
        "expert_load": {"touched": touched, "min": int(loads.min()), "mean": float(loads.mean()),
                        "max": int(loads.max())},
        "weight_buffers_rotated": n_rot,
        "ms_per_step_with_fc1_events": ms_step_instrumented,
        "roofline": roof,
    }
    if fused is not None:
        res["single_launch"] = fused
    if w.name == "bounded_decode":
        res["live_tracking"] = live_tracking(w, moes, x, logits, route_fn, fwd_fn, ids, probs, out,
                                             ws, live, sh, n_rot, a.combine)
    del moes, route_fn, fwd_fn, x, logits, ws, out, ids, probs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp, cpu_seconds, a.combine, threads1=threads1)
    return res


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(--gpus {a.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration()
        return

    every = a.workload == "all"
    names = ALL_WORKLOADS if every else (a.workload,)
    headline = HEADLINE if every else a.workload
    results = {}
    t_start = time.time()
    for name in names:
        print(f"[bench] {name} ...", file=sys.stderr, flush=True)
        results[name] = run_workload(name, a, a.cpu_seconds if name == headline else a.cpu_seconds_other,
                                     threads1=name in ("tiny", "decode"))
        r = results[name]
        print(f"[bench] {name}: {r['ms_per_step'] * 1e3:.1f} us/step, "
              f"FC1 {r['roofline']['kernel_us']:.1f} us ({r['roofline']['bound']} "
              f"{100 * r['roofline']['frac']:.1f}%), {time.time() - t_start:.0f} s elapsed",
              file=sys.stderr, flush=True)

    h = results[headline]
    res = {
        "metric": METRIC, "value": h["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": h["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": h["precision"], "data": "synthetic (seeded N(0,1) tokens, N(0,0.02^2) weights)",
        "config": {"workload": h["workload"], "tokens": h["tokens"],
                   "token_capacity": h["token_capacity"], "hidden": h["hidden"], "ffn": h["ffn"],
                   "experts": h["experts"], "topk": h["topk"], "precision": h["precision"],
                   "combine": a.combine, "parallelism": "one GPU, all experts local"},
    }
    for key in ("tflops", "mfma_frac", "hbm_gbs_step", "hbm_frac_step", "stages_us", "expert_load",
                "weight_buffers_rotated", "roofline", "single_launch", "live_tracking", "cpu_baseline"):
        if key in h:
            res[key] = h[key]
    if every:
        res["configs"] = {n: {k: v for k, v in r.items() if k != "stages_us"}
                          for n, r in results.items()}
    print(json.dumps(res))


def live_tracking(w, moes, x, logits, route_fn, fwd_fn, ids, probs, out, ws, live, sh, n_rot,
                  combine: str, steps: int = 20) -> dict:
    """Step time against the live count at the full capacity (live 64 .. 1024),
    and at live = w.T with the buffers sized to the live rows instead.  Rows
    w.T .. 2 w.T - 1 of x and the logits become copies of the first w.T rows,
    so that every swept live count routes real data."""
    import torch
    T = w.T
    x[T:2 * T] = x[:T]
    logits[T:2 * T] = logits[:T]
    ev = HipEvents()

    def time_steps(route, fwd):
        for i in range(3):
            route[i % n_rot]()
            fwd[i % n_rot]()
        a, b = ev.new(), ev.new()
        torch.cuda.synchronize()
        ev.record(a, sh)
        for i in range(steps):
            route[i % n_rot]()
            fwd[i % n_rot]()
        ev.record(b, sh)
        torch.cuda.synchronize()
        return ev.ms(a, b) / steps * 1e3

    by_live = {}
    for n in (64, 128, 256, 512, 1024):
        live.fill_(n)
        by_live[str(n)] = time_steps(route_fn, fwd_fn)
    live.fill_(T)
    # the same live tokens with every buffer sized to them
    xs, ls = x[:T].contiguous(), logits[:T].contiguous()
    ids_s, probs_s, out_s = ids[:T].contiguous(), probs[:T].contiguous(), out[:T].contiguous()
    ws_s = moes[0].new_workspace(T)
    route_s = [m.bind_route(ls, live, ids_s, probs_s, ws_s) for m in moes]
    fwd_s = [m.bind_forward(xs, ids_s, probs_s, live, out_s, ws_s, combine=combine) for m in moes]
    small = time_steps(route_s, fwd_s)
    ev.close()
    return {"token_capacity": w.T_cap, "us_per_step_by_live": by_live,
            f"us_per_step_live_{T}_capacity_{T}": small,
            f"us_per_step_live_{T}_capacity_{w.T_cap}": by_live[str(T)]}


def cpu_baseline(w, inp, target_s: float, combine: str = "fp32", threads1: bool = False) -> dict:
    """The CPU oracle (as it stands) on a bounded sample of the same workload:
    the first S live tokens, S sized from a short calibration run; with
    threads1 also its time on one host thread."""
    import oracle
    cores = oracle.set_threads(0)
    model = oracle.Model(w.E, w.H, w.F, w.k, inp["w1_bits"], inp["w2_bits"], w.precision)
    ids, probs, _ = oracle.route(inp["logits"], w.T, w.k)

    def run(S):
        t = time.time()
        model.forward(inp["x_bits"][:S].copy(), ids[:S].copy(), probs[:S].copy(), S,
                      combine=combine)
        return time.time() - t

    def measure(target):
        S0 = min(w.T, 8)
        t0 = run(S0)
        S = int(min(w.T, max(S0, S0 * target / max(t0, 1e-3))))
        reps = 1
        t = run(S)
        while t * (reps + 1) / reps < target and S == w.T and reps < 8:
            t += run(S)
            reps += 1
        return S, reps, t

    S, reps, t = measure(target_s)
    res = {"value": S * reps / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "cpu_model": cpu_model(),
           "gflops": 6.0 * w.H * w.F * w.k * S * reps / t / 1e9,
           "sample": f"first {S} of {w.T} tokens, {reps} run(s), {t:.1f} s "
                     f"(weights prepared outside the timing)"}
    if threads1:
        oracle.set_threads(1)
        try:
            S1, r1, t1 = measure(min(target_s, 3.0))
        finally:
            oracle.set_threads(cores)
        res["one_thread"] = {"value": S1 * r1 / t1, "unit": "tokens/s", "cores": 1,
                             "sample": f"first {S1} of {w.T} tokens, {r1} run(s), {t1:.1f} s"}
    return res


if __name__ == "__main__":
    main()
