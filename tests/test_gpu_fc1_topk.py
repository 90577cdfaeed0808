"""The apply_topk_in_fc1 option on the GPU (cudnn-frontend PR #448, the MoeEp
constructor's apply_topk_in_fc1 flag): each route's probability multiplies its
SwiGLU row inside the FC1 epilogue, before the FC2-input rounding, and the
combine adds the weighted rows.  Against the oracle: the exact hand cases,
small and full-size parity, the bit-for-bit agreement with the default
placement for probabilities that commute with every rounding, and the batch
invariance of every token's bits (launch size, tile design)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, Workload
from gpu_common import Case, assert_close, live_tensor, sentinel_out, to_dev_bits, SENTINEL_BITS

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import swiglu_expert_mlp_amd  # noqa: F401


def _moe(w):
    from swiglu_expert_mlp_amd import MoE
    return MoE(w.E, w.H, w.F, w.k, w.precision)


def _bits(vals):
    v = np.asarray(vals, dtype=np.float32)
    b = v.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0)
    return (b >> 16).astype(np.uint16)


def _cases():
    with open(os.path.join(GOLDEN, "fc1_topk_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("precision", ["bf16", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("c", _cases(), ids=lambda c: c["name"])
def test_hand_cases_exact(c, precision):
    from swiglu_expert_mlp_amd import MoE
    print(f"[fc1-topk] hand case {c['name']} {precision}", flush=True)
    m = MoE(c["E"], c["H"], c["F"], c["k"], precision)
    m.load_weights(to_dev_bits(_bits(c["w1"])), to_dev_bits(_bits(c["w2"])))
    x = to_dev_bits(_bits(c["x"]))
    ids = torch.tensor(c["ids"], dtype=torch.int32, device="cuda")
    probs = torch.tensor(c["probs"], dtype=torch.float32, device="cuda")
    out = sentinel_out(c["T_cap"], c["H"])
    ws = m.new_workspace(c["T_cap"])
    m.forward(x, ids, probs, live_tensor(c["live"]), out=out, ws=ws, topk_in_fc1=True)
    torch.cuda.synchronize()
    assert m.check(ws) == 0
    assert np.array_equal(out.cpu().numpy(), np.array(c["expected"][precision], np.float32))


SMALL = {
    "tiny": WORKLOADS["tiny"],
    "decode_T64": WORKLOADS["decode"].with_tokens(64),
    "odd_bf16": Workload("odd_bf16", 77, 80, 96, 160, 5, 3, "bf16"),
    "odd_bf16_big_cap": Workload("odd_bf16_big_cap", 700, 1100, 96, 160, 5, 3, "bf16"),
    "odd64_bf16_big_cap": Workload("odd64_bf16_big_cap", 700, 1100, 192, 320, 5, 3, "bf16"),
    "mxfp8_T96": WORKLOADS["mxfp8_16k"].with_tokens(96),
    "odd_mxfp8": Workload("odd_mxfp8", 77, 80, 96, 160, 5, 3, "mxfp8"),
    "mx_big": Workload("mx_big", 600, 600, 256, 384, 4, 2, "mxfp8"),
    "mx4_T96": WORKLOADS["mxfp4_16k"].with_tokens(96),
    "odd_mxfp4": Workload("odd_mxfp4", 77, 80, 96, 160, 5, 3, "mxfp4"),
    "mx4_big": Workload("mx4_big", 600, 600, 256, 384, 4, 2, "mxfp4"),
}


@pytest.mark.parametrize("combine", ["fp32", "bf16"])
@pytest.mark.parametrize("name", list(SMALL))
def test_parity_small(name, combine):
    w = SMALL[name]
    print(f"[fc1-topk] parity {name} combine={combine}", flush=True)
    c = Case(w, seed=11, outliers=w.precision != "bf16")
    m = _moe(w)
    m.load_weights(*c.weights_dev())
    x, ids, probs = c.dev()
    ws = m.new_workspace(w.T_cap)
    if combine == "fp32":
        out = sentinel_out(w.T_cap, w.H)
    else:
        out = torch.full((w.T_cap, w.H), -7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    m.forward(x, ids, probs, live_tensor(w.T), out=out, ws=ws, combine=combine, topk_in_fc1=True)
    torch.cuda.synchronize()
    assert m.check(ws) == 0
    ref, err, _ = c.oracle_model().forward(c.inp["x_bits"], c.ids, c.probs, w.T, combine=combine,
                                           topk_in_fc1=True)
    assert err == 0
    if combine == "fp32":
        got = out.cpu().numpy()
        assert np.all(got[w.T:].view(np.uint32) == SENTINEL_BITS)
        assert_close(got[: w.T], ref[: w.T], name)
    else:
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.all(got[w.T:].view(np.int16) == -7)
        assert_close(oracle.bf16_value(got[: w.T]), oracle.bf16_value(ref[: w.T]), name)


@pytest.mark.parametrize("name", ["odd_bf16", "odd_bf16_big_cap", "odd64_bf16_big_cap", "odd_mxfp8",
                                  "odd_mxfp4"])
def test_exact_scalings_match_default_bitwise(name):
    """Probabilities of 1 or powers of two commute with every rounding step, so
    the FC1 placement gives the default placement's bits (on the GPU's own
    arithmetic, both designs of each precision)."""
    w = SMALL[name]
    c = Case(w, seed=12, outliers=w.precision != "bf16")
    m = _moe(w)
    m.load_weights(*c.weights_dev())
    x, ids, _ = c.dev()
    rng = np.random.default_rng(4)
    pw = (2.0 ** -rng.integers(0, 4, (w.T_cap, w.k))).astype(np.float32)
    for probs in (torch.ones((w.T_cap, w.k), device="cuda"), torch.from_numpy(pw).cuda()):
        a = sentinel_out(w.T_cap, w.H)
        b = sentinel_out(w.T_cap, w.H)
        m.forward(x, ids, probs, live_tensor(w.T), out=a, ws=m.new_workspace(w.T_cap))
        m.forward(x, ids, probs, live_tensor(w.T), out=b, ws=m.new_workspace(w.T_cap),
                  topk_in_fc1=True)
        torch.cuda.synchronize()
        assert np.array_equal(a.view(torch.int32).cpu().numpy(), b.view(torch.int32).cpu().numpy())


@pytest.mark.parametrize("name", ["decode_T300", "mxfp8_T300", "mxfp4_T300"])
def test_wide_equals_chunks(name):
    w = {"decode_T300": WORKLOADS["decode"].with_tokens(300),
         "mxfp8_T300": WORKLOADS["mxfp8_16k"].with_tokens(300),
         "mxfp4_T300": WORKLOADS["mxfp4_16k"].with_tokens(300)}[name]
    c = Case(w, seed=13, outliers=w.precision != "bf16")
    m = _moe(w)
    m.load_weights(*c.weights_dev())
    x, ids, probs = c.dev()

    def fwd(xs, i_s, ps, T):
        out = sentinel_out(T, w.H)
        m.forward(xs, i_s, ps, live_tensor(T), out=out, ws=m.new_workspace(T), topk_in_fc1=True)
        return out.view(torch.int32).cpu().numpy()

    wide = fwd(x, ids, probs, w.T)
    for t0 in range(0, w.T, 37):
        t1 = min(w.T, t0 + 37)
        part = fwd(x[t0:t1].clone(), ids[t0:t1].clone(), probs[t0:t1].clone(), t1 - t0)
        assert np.array_equal(part, wide[t0:t1]), t0


def test_tile_designs_agree_bitwise():
    """At a 2048-token capacity the larger experts run on the 256 x 256 kernel;
    the same tokens in launches of 128 run every expert on the 64-row kernel."""
    w = WORKLOADS["logprob"].with_tokens(2048)
    c = Case(w, seed=11)
    m = _moe(w)
    m.load_weights(*c.weights_dev())
    x, ids, probs = c.dev()
    out = sentinel_out(w.T, w.H)
    ws = m.new_workspace(w.T)
    m.forward(x, ids, probs, live_tensor(w.T), out=out, ws=ws, topk_in_fc1=True)
    counts = m.get_indices(ws, w.T)["counts"]
    assert (counts > 128).sum() > 10
    wide = out.view(torch.int32).cpu().numpy()
    for t0 in range(0, w.T, 128):
        part = sentinel_out(128, w.H)
        m.forward(x[t0:t0 + 128].contiguous(), ids[t0:t0 + 128].contiguous(),
                  probs[t0:t0 + 128].contiguous(), live_tensor(128), out=part,
                  ws=m.new_workspace(128), topk_in_fc1=True)
        assert np.array_equal(part.view(torch.int32).cpu().numpy(), wide[t0:t0 + 128]), t0


@pytest.mark.parametrize("name", ["logprob", "mxfp8_16k"])
def test_full_size_sampled(name):
    w = WORKLOADS[name]
    print(f"[fc1-topk] full size {name}", flush=True)
    c = Case(w, seed=11, outliers=w.precision != "bf16")
    m = _moe(w)
    m.load_weights(*c.weights_dev())
    x, ids, probs = c.dev()
    out = sentinel_out(w.T_cap, w.H)
    ws = m.new_workspace(w.T_cap)
    m.forward(x, ids, probs, live_tensor(w.T), out=out, ws=ws, topk_in_fc1=True)
    torch.cuda.synchronize()
    assert m.check(ws) == 0
    got = out.cpu().numpy()
    toks = np.unique(np.r_[np.random.default_rng(2).choice(w.T, 20, replace=False), 0, w.T - 1])
    ref = c.oracle_model().forward_tokens(c.inp["x_bits"], c.ids, c.probs, toks, topk_in_fc1=True)
    assert_close(got[toks], ref, name)


def test_row_mode_rejects_fc1_probabilities():
    w = WORKLOADS["tiny"]
    m = _moe(w)
    g = torch.Generator(device="cuda").manual_seed(1)
    m.load_weights((torch.randn((w.E, 2 * w.F, w.H), generator=g, device="cuda") * 0.02).bfloat16(),
                   (torch.randn((w.E, w.H, w.F), generator=g, device="cuda") * 0.02).bfloat16())
    x = torch.zeros((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((w.T, w.k), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="row mode"):
        m.forward(x, ids, None, live_tensor(w.T), combine="rows", topk_in_fc1=True)
