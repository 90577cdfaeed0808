"""Benchmark of the routed SwiGLU MoE forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

One step = the whole hot path over one batch of synthetic inputs already
resident in HBM: the router (moe_route: softmax, top-k, canonical ids) and the
forward (moe_forward: permutation, FC1 + SwiGLU, FC2, fp32 finalize).  W
untimed warm-up steps, then exactly K timed steps between two
torch.cuda.synchronize() calls.  Prints ONE JSON line.

The default workload is the decode-sized launch (256 tokens, hidden 2048, FFN
1024, 64 experts, top-6, bf16).  Kernel-weight buffers are rotated between
steps so that the ~805 MB of expert weights cannot be served from the 256 MB
Infinity Cache.  `roofline` reports the dominant kernel's algorithmic bytes
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
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0}
MALL_BYTES = 256 << 20


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode")
    p.add_argument("--seed", type=int, default=11)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    return p.parse_args()


def alg_bytes(w, precision: str, touched: int) -> dict:
    """Algorithmic bytes: each touched expert's weights once, each live token's
    x row once, routed rows written/read once where a stage must (FC1 writes
    the SwiGLU row, FC2 reads it), ids/probs once, the fp32 output once."""
    wb = 2 if precision == "bf16" else 1
    sb = 0 if precision == "bf16" else 1.0 / 32          # E8M0 bytes per element
    H, F, T, R = w.H, w.F, w.T, w.R
    fc1 = touched * 2 * F * H * (wb + sb) + T * H * 2 + R * F * (wb + sb)
    fc2 = touched * H * F * (wb + sb) + R * F * (wb + sb) + R * H * 4
    step = touched * 3 * F * H * (wb + sb) + T * H * 2 + T * w.k * 8 + T * H * 4
    return dict(fc1=fc1, fc2=fc2, step=step)


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(--gpus {a.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import WORKLOADS, make_inputs
    from swiglu_expert_mlp_amd import MoE

    w = WORKLOADS[a.workload]
    dev = torch.device("cuda:0")
    t_gen = time.time()
    inp = make_inputs(w, seed=a.seed, outliers=(w.precision == "mxfp8"))
    t_gen = time.time() - t_gen
    bf = lambda arr: torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(
        torch.bfloat16).to(dev)
    x = bf(inp["x_bits"])
    w1 = bf(inp["w1_bits"])
    w2 = bf(inp["w2_bits"])
    logits = torch.from_numpy(inp["logits"]).to(dev)
    live = torch.tensor([w.T], dtype=torch.int32, device=dev)

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
    out = torch.empty((w.T_cap, w.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, events=None, rev=None):
        m = moes[i % n_rot]
        if rev is not None:
            rev[0].record(stream)
        m.route(logits, live, ids=ids, probs=probs, ws=ws)
        if rev is not None:
            rev[1].record(stream)
        m.set_stage_events(events)
        m.forward(x, ids, probs, live, out=out, ws=ws)

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    bits = moe0.check(ws)
    if bits:
        raise RuntimeError(f"device contract violation bits {bits}")
    idx = moe0.get_indices(ws, w.T_cap)
    touched = int(np.count_nonzero(idx["counts"]))
    loads = idx["counts"].astype(np.int64)

    mk = lambda: torch.cuda.Event(enable_timing=True)
    stage_ev = [[mk() for _ in range(6)] for _ in range(a.steps)]
    route_ev = [[mk(), mk()] for _ in range(a.steps)]
    t0, t1 = mk(), mk()
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(a.steps):
        step(i, stage_ev[i], route_ev[i])
    t1.record(stream)
    torch.cuda.synchronize()
    for m in moes:
        m.set_stage_events(None)
    ms_step = t0.elapsed_time(t1) / a.steps

    names = MoE.STAGES
    stage_us = {n: float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in stage_ev]) * 1e3)
                for j, n in enumerate(names)}
    route_us = float(np.mean([r[0].elapsed_time(r[1]) for r in route_ev]) * 1e3)

    ab = alg_bytes(w, w.precision, touched)
    flops = w.flops()
    tokens_s = w.T / (ms_step * 1e-3)
    tflops = flops / (ms_step * 1e-3) / 1e12
    if w.precision == "mxfp8" or w.name in ("bf16_16k",):
        fc1_flops = 4.0 * w.H * w.F * w.R
        roof = dict(bound="mfma", achieved=fc1_flops / (stage_us["fc1_swiglu"] * 1e-6) / 1e12,
                    peak=MFMA_PEAK_TFLOPS[w.precision], unit="TFLOP/s")
    else:
        roof = dict(bound="hbm", achieved=ab["fc1"] / (stage_us["fc1_swiglu"] * 1e-6) / 1e9,
                    peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = "gemm_bf16_kernel<FC1>" if w.precision == "bf16" else "gemm_mxfp8_kernel<FC1>"
    roof["traffic"] = None

    res = {
        "metric": METRIC, "value": tokens_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.precision, "data": "synthetic (seeded N(0,1) tokens, N(0,0.02^2) weights)",
        "config": {"workload": w.name, "tokens": w.T, "token_capacity": w.T_cap, "hidden": w.H,
                   "ffn": w.F, "experts": w.E, "topk": w.k, "precision": w.precision,
                   "parallelism": "one GPU, all experts local"},
        "tflops": tflops,
        "mfma_frac": tflops / MFMA_PEAK_TFLOPS[w.precision],
        "hbm_gbs_step": ab["step"] / (ms_step * 1e-3) / 1e9,
        "hbm_frac_step": ab["step"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "stages_us": {"route": route_us, **stage_us},
        "expert_load": {"touched": touched, "min": int(loads.min()), "mean": float(loads.mean()),
                        "max": int(loads.max())},
        "weight_buffers_rotated": n_rot,
        "roofline": roof,
    }

    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp, a.cpu_seconds)
    print(json.dumps(res))


def cpu_baseline(w, inp, target_s: float) -> dict:
    """The CPU oracle (as it stands) on a bounded sample of the same workload:
    the first S live tokens, S sized from a short calibration run."""
    import oracle
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    model = oracle.Model(w.E, w.H, w.F, w.k, inp["w1_bits"], inp["w2_bits"], w.precision)
    ids, probs, _ = oracle.route(inp["logits"], w.T, w.k)

    def run(S):
        t = time.time()
        model.forward(inp["x_bits"][:S].copy(), ids[:S].copy(), probs[:S].copy(), S)
        return time.time() - t

    S0 = min(w.T, 16)
    t0 = run(S0)
    S = int(min(w.T, max(S0, S0 * target_s / max(t0, 1e-3))))
    reps = 1
    t = run(S)
    while t * (reps + 1) / reps < target_s and S == w.T and reps < 8:
        t += run(S)
        reps += 1
    tokens = S * reps
    return {"value": tokens / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {S} of {w.T} tokens, {reps} run(s), {t:.1f} s "
                      f"(weights prepared outside the timing)"}


if __name__ == "__main__":
    main()
