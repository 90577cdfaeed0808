"""Helpers shared by the GPU tests: run the HIP path through the C ABI and the
oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from workloads import make_inputs

# forward tolerance: relative L2 and max-abs relative to max |ref|
REL_L2 = 5e-3
MAX_ABS = 2e-2


def to_dev_bits(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch bfloat16 on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def live_tensor(n: int) -> torch.Tensor:
    return torch.tensor([n], dtype=torch.int32, device="cuda")


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = got.astype(np.float64) - ref.astype(np.float64)
    nref = np.linalg.norm(ref.astype(np.float64))
    rel = np.linalg.norm(diff) / max(nref, 1e-30)
    mabs = np.abs(diff).max() / max(np.abs(ref).max(), 1e-30)
    assert rel <= REL_L2 and mabs <= MAX_ABS, f"{what}: rel L2 {rel:.3e}, max abs/max {mabs:.3e}"
    return rel, mabs


class Case:
    """Seeded inputs of one workload, with oracle routing, on host and GPU."""

    def __init__(self, w, seed=11, outliers=False, weights=True):
        self.w = w
        self.inp = make_inputs(w, seed=seed, outliers=outliers, weights=weights)
        ids, probs, err = oracle.route(self.inp["logits"], w.T, w.k)
        assert err == 0
        # rows past live: the NaN bit pattern in ids and probs
        ids[w.T:] = np.int32(0x7FC00000)
        probs[w.T:] = np.uint32(0x7FC00000).view(np.float32)
        self.ids, self.probs = ids, probs

    def dev(self):
        x = to_dev_bits(self.inp["x_bits"])
        ids = torch.from_numpy(self.ids).cuda()
        probs = torch.from_numpy(self.probs).cuda()
        return x, ids, probs

    def weights_dev(self):
        return to_dev_bits(self.inp["w1_bits"]), to_dev_bits(self.inp["w2_bits"])

    def oracle_model(self):
        w = self.w
        return oracle.Model(w.E, w.H, w.F, w.k, self.inp["w1_bits"], self.inp["w2_bits"],
                            w.precision)


def sentinel_out(T_cap: int, H: int) -> torch.Tensor:
    """Output buffer pre-filled with a NaN payload that no kernel writes."""
    return torch.full((T_cap, H), 0x7FBADBAD, dtype=torch.int32, device="cuda").view(torch.float32)


SENTINEL_BITS = 0x7FBADBAD
