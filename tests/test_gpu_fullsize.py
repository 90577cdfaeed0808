"""Parity at the full sizes of the benchmark workloads, in the launch
configuration bench.py times: routing ids and the permutation bit for bit over
the whole launch, the output on sampled tokens against the oracle's per-token
evaluation, and (bounded decode) the rows past the live count untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS
from gpu_common import Case, assert_close, live_tensor, sentinel_out, SENTINEL_BITS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import swiglu_expert_mlp_amd  # noqa: F401


def _sample(T, prep, k, n=24, seed=3):
    """24 seeded tokens (first, last, middle and random) plus, for every expert
    with rows, the token of its last grouped row: that row sits in the expert's
    last (ragged) M tile, whichever tile design runs it, so every expert's last
    tile contributes a checked row."""
    rng = np.random.default_rng(seed)
    pick = {0, 1, T - 1, T // 2}
    pick.update(rng.choice(T, size=min(T, n) - len(pick), replace=False).tolist())
    offs, counts, perm = prep["offsets"], prep["counts"], prep["perm_src"]
    for e in np.nonzero(counts)[0]:
        pick.add(int(perm[offs[e + 1] - 1]) // k)
    return np.array(sorted(pick), dtype=np.int64)


@pytest.mark.parametrize("name", ["decode", "logprob", "mxfp8_16k", "bf16_16k", "bounded_decode",
                                  "decode_mxfp4", "mxfp4_16k"])
def test_full_size(name):
    from swiglu_expert_mlp_amd import MoE
    w = WORKLOADS[name]
    print(f"[full-size] {name}: T={w.T} T_cap={w.T_cap} H={w.H} F={w.F} E={w.E} k={w.k} "
          f"{w.precision}", flush=True)
    c = Case(w, seed=11, outliers=w.precision != "bf16")
    m = MoE(w.E, w.H, w.F, w.k, w.precision)
    w1, w2 = c.weights_dev()
    m.load_weights(w1, w2)
    del w1, w2
    ws = m.new_workspace(w.T_cap)
    live = live_tensor(w.T)

    # router: ids bit for bit, probs to a few ulp, rows past live untouched
    logits = torch.from_numpy(c.inp["logits"]).cuda()
    gi = torch.full((w.T_cap, w.k), -5, dtype=torch.int32, device="cuda")
    gp = torch.full((w.T_cap, w.k), -5.0, dtype=torch.float32, device="cuda")
    m.route(logits, live, ids=gi, probs=gp, ws=ws)
    gi, gp = gi.cpu().numpy(), gp.cpu().numpy()
    assert np.array_equal(gi[: w.T], c.ids[: w.T])
    np.testing.assert_allclose(gp[: w.T], c.probs[: w.T], rtol=2e-6, atol=1e-7)
    assert np.all(gi[w.T:] == -5)

    # forward on the oracle's routes
    x, ids, probs = c.dev()
    out = sentinel_out(w.T_cap, w.H)
    m.forward(x, ids, probs, live, out=out, ws=ws)
    torch.cuda.synchronize()
    assert m.check(ws) == 0
    got = out.cpu().numpy()
    assert np.all(got[w.T:].view(np.uint32) == SENTINEL_BITS), "rows past live were written"

    idx = m.get_indices(ws, w.T_cap)
    ref = oracle.prepare(c.ids, c.probs, w.T, w.E)
    for key in ("counts", "offsets", "perm_src", "dst"):
        assert np.array_equal(idx[key], ref[key]), key

    toks = _sample(w.T, ref, w.k)
    print(f"[full-size] {name}: {len(toks)} sampled tokens", flush=True)
    ref_rows = c.oracle_model().forward_tokens(c.inp["x_bits"], c.ids, c.probs, toks)
    assert_close(got[toks], ref_rows, f"{name} sampled tokens")
