"""Expert counts, top-k and capacities at the edges of what moe_create accepts.

The benchmark workloads use E <= 128 and top-k <= 8; these cases reach the
other instantiations of the router (64 / 128 / 256 / 512 / 1024 experts per
wave), the prep and finalize templates for top-k 9..16, prep with experts
held by every thread of its finish (E = 1024), and the multi-slab prefix of
prep's finish (more chunks than one LDS slab holds: above 16,384 live tokens
at E = 128).  Routing ids and the permutation bit for bit, probabilities to a
few ulp, the output within the forward tolerance, all against the oracle.
Small H and F keep the oracle fast.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import Workload
from gpu_common import Case, assert_close, live_tensor, sentinel_out, SENTINEL_BITS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import swiglu_expert_mlp_amd  # noqa: F401


WIDE = {
    "e1024_k16": Workload("e1024_k16", 3000, 3000, 64, 64, 1024, 16, "bf16"),
    "e512_k12": Workload("e512_k12", 1000, 1100, 64, 96, 512, 12, "bf16"),
    "e256_k9": Workload("e256_k9", 700, 700, 96, 64, 256, 9, "mxfp8"),
    "e200_k10": Workload("e200_k10", 500, 520, 128, 128, 200, 10, "mxfp4"),
    # 69 chunks of 256 tokens at E = 128: more than the 64 chunk rows one LDS
    # slab of the finish holds
    "multislab": Workload("multislab", 16384 + 1200, 16384 + 1300, 64, 64, 128, 8, "bf16"),
}


@pytest.mark.parametrize("name", list(WIDE))
def test_wide_shapes(name):
    from swiglu_expert_mlp_amd import MoE
    w = WIDE[name]
    print(f"[wide] {name}: T={w.T} T_cap={w.T_cap} E={w.E} k={w.k} H={w.H} F={w.F} "
          f"{w.precision}", flush=True)
    c = Case(w, seed=12, outliers=w.precision != "bf16")
    m = MoE(w.E, w.H, w.F, w.k, w.precision)
    w1, w2 = c.weights_dev()
    m.load_weights(w1, w2)
    ws = m.new_workspace(w.T_cap)
    live = live_tensor(w.T)

    logits = torch.from_numpy(c.inp["logits"]).cuda()
    gi, gp = m.route(logits, live, ws=ws)
    gi, gp = gi.cpu().numpy(), gp.cpu().numpy()
    assert np.array_equal(gi[: w.T], c.ids[: w.T])
    np.testing.assert_allclose(gp[: w.T], c.probs[: w.T], rtol=2e-6, atol=1e-7)

    x, ids, probs = c.dev()
    out = sentinel_out(w.T_cap, w.H)
    m.forward(x, ids, probs, live, out=out, ws=ws)
    torch.cuda.synchronize()
    assert m.check(ws) == 0
    got = out.cpu().numpy()
    assert np.all(got[w.T:].view(np.uint32) == SENTINEL_BITS)
    idx = m.get_indices(ws, w.T_cap)
    ref_idx = oracle.prepare(c.ids, c.probs, w.T, w.E)
    for key in ("counts", "offsets", "perm_src", "dst"):
        assert np.array_equal(idx[key], ref_idx[key]), key
    ref, err, _ = c.oracle_model().forward(c.inp["x_bits"], c.ids, c.probs, w.T)
    assert err == 0
    assert_close(got[: w.T], ref[: w.T], name)
