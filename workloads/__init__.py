"""Seeded synthetic inputs for the routed SwiGLU MoE forward.

Shared by the tests, the smoke check and the benchmark; used on both sides
(the HIP path and the CPU oracle).  This module holds no step of the method:
it only draws random tensors, rounds them to bf16 with torch's cast, and
computes the router logits, which are the caller's input (the router GEMM
belongs to the model, not to the expert path).

Workloads (the shapes of the source pages' experiments; every input is
synthetic, there are no trained weights or prompts here):

  tiny            64 tokens, hidden 128, FFN 256, 8 experts, top-2, bf16
  decode          256 tokens, hidden 2048, FFN 1024, 64 experts, top-6, bf16
  logprob         4096 tokens, hidden 2048, FFN 1024, 128 experts, top-8, bf16,
                  router logits with a per-expert bias ~N(0,1) to skew loads
  mxfp8_16k       16384 tokens, hidden 2048, FFN 1024, 128 experts, top-8, MXFP8
  bf16_16k        the same shapes in bf16
  bounded_decode  buffer of 65,536 token rows, 512 live, hidden 2688,
                  FFN 1856, 128 experts, top-6, bf16; rows past the live count
                  are NaN
  decode_mxfp4    the decode shapes with MXFP4 weights (E2M1 + E8M0 per 32)
                  and MXFP8 activations
  mxfp4_16k       the 16K-token shapes with MXFP4 weights and MXFP8 activations

Draw order for one seed (one CPU torch.Generator): x ~ N(0,1) [T_cap, H],
W1 ~ N(0, 0.02^2) [E, 2F, H] (gate rows first), W2 ~ N(0, 0.02^2) [E, H, F],
Wr ~ N(0, 0.1^2) [H, E], then (logprob only) b ~ N(0, 1) [E].  x and the
weights are rounded to bf16 (round to nearest even).  Logits are
fp32(sum_h x_bf16[t, h] * Wr[h, e] + b[e]) computed in fp64.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch

BF16_NAN = 0x7FC0
F32_NAN_BITS = 0x7FC00000


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # live tokens
    T_cap: int        # token rows in the buffers
    H: int
    F: int
    E: int
    k: int
    precision: str    # "bf16" | "mxfp8" | "mxfp4"
    bias: bool = False

    @property
    def R(self) -> int:
        return self.T * self.k

    def flops(self) -> float:
        """FC1 (4HF) + FC2 (2HF) multiply-adds x2 per routed row."""
        return 6.0 * self.H * self.F * self.R

    def with_tokens(self, T: int, T_cap: int | None = None) -> "Workload":
        return replace(self, T=T, T_cap=T if T_cap is None else T_cap)


WORKLOADS = {
    "tiny": Workload("tiny", 64, 64, 128, 256, 8, 2, "bf16"),
    "decode": Workload("decode", 256, 256, 2048, 1024, 64, 6, "bf16"),
    "logprob": Workload("logprob", 4096, 4096, 2048, 1024, 128, 8, "bf16", bias=True),
    "mxfp8_16k": Workload("mxfp8_16k", 16384, 16384, 2048, 1024, 128, 8, "mxfp8"),
    "bf16_16k": Workload("bf16_16k", 16384, 16384, 2048, 1024, 128, 8, "bf16"),
    "bounded_decode": Workload("bounded_decode", 512, 65536, 2688, 1856, 128, 6, "bf16"),
    "decode_mxfp4": Workload("decode_mxfp4", 256, 256, 2048, 1024, 64, 6, "mxfp4"),
    "mxfp4_16k": Workload("mxfp4_16k", 16384, 16384, 2048, 1024, 128, 8, "mxfp4"),
}


def _bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _randn_bf16(gen: torch.Generator, shape, std: float, chunk_rows: int = 1 << 14) -> np.ndarray:
    """N(0, std^2) drawn in fixed row chunks (bounded host memory), rounded to bf16."""
    rows = shape[0]
    rest = tuple(shape[1:])
    out = np.empty(shape, dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        t = torch.randn((r1 - r0,) + rest, generator=gen, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        out[r0:r1] = _bf16_bits(t)
    return out


def make_inputs(w: Workload, seed: int = 11, outliers: bool = False,
                weights: bool = True) -> dict:
    """Seeded inputs for workload ``w``.

    Returns numpy arrays: x_bits uint16 [T_cap, H], w1_bits uint16 [E, 2F, H],
    w2_bits uint16 [E, H, F], logits fp32 [T_cap, E], and ``live``.  Rows at or
    beyond T of x are bf16 NaN and of logits fp32 NaN.  With ``outliers``, 5 %
    of the live tokens (a seeded choice) are scaled by 30 before the bf16 cast.
    """
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn((w.T, w.H), generator=gen, dtype=torch.float32)
    if outliers:
        n_out = max(1, int(round(0.05 * w.T)))
        idx = torch.randperm(w.T, generator=gen)[:n_out]
        x[idx] *= 30.0
    x_bits = np.full((w.T_cap, w.H), BF16_NAN, dtype=np.uint16)
    x_bits[: w.T] = _bf16_bits(x)
    del x
    if weights:
        w1 = _randn_bf16(gen, (w.E * 2 * w.F, w.H), 0.02).reshape(w.E, 2 * w.F, w.H)
        w2 = _randn_bf16(gen, (w.E * w.H, w.F), 0.02).reshape(w.E, w.H, w.F)
    else:
        # skip the weight draws but keep the generator stream aligned
        for shape in ((w.E * 2 * w.F, w.H), (w.E * w.H, w.F)):
            for r0 in range(0, shape[0], 1 << 14):
                torch.randn((min(shape[0], r0 + (1 << 14)) - r0, shape[1]), generator=gen)
        w1 = w2 = None
    wr = torch.randn((w.H, w.E), generator=gen, dtype=torch.float32).mul_(0.1)
    b = torch.randn((w.E,), generator=gen, dtype=torch.float32) if w.bias else None
    xv = (x_bits[: w.T].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    lg = xv @ wr.numpy().astype(np.float64)
    if b is not None:
        lg = lg + b.numpy().astype(np.float64)[None, :]
    logits = np.full((w.T_cap, w.E), np.nan, dtype=np.float32)
    logits[: w.T] = lg.astype(np.float32)
    return dict(x_bits=x_bits, w1_bits=w1, w2_bits=w2, logits=logits, live=w.T,
                wr=wr.numpy(), bias=None if b is None else b.numpy())


def nan_fill_routes(ids: np.ndarray, probs: np.ndarray, live: int):
    """Rows at or beyond ``live`` of ids/probs set to the fp32 NaN bit pattern
    (for ids, 0x7FC00000 is also an out-of-range expert id)."""
    ids = ids.copy()
    probs = probs.copy()
    ids[live:] = np.int32(F32_NAN_BITS)
    probs[live:] = np.uint32(F32_NAN_BITS).view(np.float32)
    return ids, probs
