"""GPU parity of the bf16 combine and the row mode (moe_forward_ex) against the oracle.

Bit-exact: each combine applied by the GPU equals the oracle's applied to the
GPU's own FC2 rows; the GPU's bf16 combine equals torch's bf16 cast of its fp32
combine on the same inputs; row mode without probabilities equals row mode
with them.  End to end: within the forward tolerance of the oracle's forward.
Rows of tokens at or past the live count are never written.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, Workload
from gpu_common import Case, assert_close, live_tensor, sentinel_out, SENTINEL_BITS

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": WORKLOADS["tiny"],
    "decode_T64": WORKLOADS["decode"].with_tokens(64),
    "mxfp8_T96": WORKLOADS["mxfp8_16k"].with_tokens(96),
    "bounded_T40_cap512": WORKLOADS["bounded_decode"].with_tokens(40, 512),
    "odd_bf16_big": Workload("odd_bf16_big", 700, 720, 96, 160, 5, 3, "bf16"),
    "odd_mxfp8": Workload("odd_mxfp8", 77, 80, 96, 160, 5, 3, "mxfp8"),
}
BF16_SENTINEL = 0x7FBB
_cases = {}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import swiglu_expert_mlp_amd  # noqa: F401  (raises if the library is missing)


def get_case(name):
    if name not in _cases:
        w = CASES[name]
        _cases[name] = Case(w, seed=12, outliers=w.precision == "mxfp8")
    return _cases[name]


def new_moe(case):
    from swiglu_expert_mlp_amd import MoE
    w = case.w
    moe = MoE(w.E, w.H, w.F, w.k, w.precision)
    w1, w2 = case.weights_dev()
    moe.load_weights(w1, w2)
    return moe


def run(case, combine, moe=None, no_probs=False):
    w = case.w
    moe = moe or new_moe(case)
    x, ids, probs = case.dev()
    ws = moe.new_workspace(w.T_cap)
    if combine == "fp32":
        out = sentinel_out(w.T_cap, w.H)
    elif combine == "bf16":
        out = torch.full((w.T_cap, w.H), BF16_SENTINEL, dtype=torch.int16, device="cuda")
        out = out.view(torch.bfloat16)
    else:
        out = torch.full((w.T_cap, w.k, w.H), SENTINEL_BITS, dtype=torch.int32, device="cuda")
        out = out.view(torch.float32)
    moe.forward(x, ids, None if no_probs else probs, live_tensor(w.T), out=out, ws=ws,
                combine=combine)
    torch.cuda.synchronize()
    res = out.cpu()
    res = res.view(torch.int16).numpy().view(np.uint16) if combine == "bf16" else res.numpy()
    return moe, ws, res


def check_past_live(out, combine, T):
    if combine == "bf16":
        assert np.all(out[T:] == BF16_SENTINEL), "rows past live were written"
    else:
        assert np.all(out[T:].view(np.uint32) == SENTINEL_BITS), "rows past live were written"


@pytest.mark.parametrize("combine", ["bf16", "rows"])
@pytest.mark.parametrize("name", list(CASES))
def test_combine_bitwise_on_gpu_rows(name, combine):
    """The GPU's combine equals the oracle's applied to the GPU's own FC2 rows."""
    c = get_case(name)
    w = c.w
    moe, ws, out = run(c, combine)
    assert moe.check(ws) == 0
    idx = moe.get_indices(ws, w.T_cap)
    rows = moe.get_rows(ws, w.T_cap, idx["n_rows"], idx["T"])
    if combine == "bf16":
        ref = oracle.finalize_bf16(rows["fc2_rows"], idx["dst"], rows["sorted_probs"], w.H)
        assert np.array_equal(out[: w.T], ref)
    else:
        ref = oracle.finalize_rows(rows["fc2_rows"], idx["dst"], w.H)
        assert np.array_equal(out[: w.T].view(np.uint32), ref.view(np.uint32))
    check_past_live(out, combine, w.T)


@pytest.mark.parametrize("name", list(CASES))
def test_bf16_combine_is_cast_of_fp32_combine(name):
    c = get_case(name)
    moe, _, f32 = run(c, "fp32")
    _, _, b16 = run(c, "bf16", moe=moe)
    T = c.w.T
    ref = torch.from_numpy(f32[:T]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16[:T], ref)


@pytest.mark.parametrize("combine", ["bf16", "rows"])
@pytest.mark.parametrize("name", ["tiny", "decode_T64", "mxfp8_T96", "odd_mxfp8"])
def test_combine_forward_parity(name, combine):
    """End to end against the oracle's forward with the same combine."""
    c = get_case(name)
    w = c.w
    _, _, out = run(c, combine)
    ref, err, _ = c.oracle_model().forward(c.inp["x_bits"], c.ids, c.probs, w.T, combine=combine)
    assert err == 0
    if combine == "bf16":
        assert_close(oracle.bf16_value(out[: w.T]), oracle.bf16_value(ref[: w.T]), name)
    else:
        assert_close(out[: w.T].reshape(-1, w.H), ref[: w.T].reshape(-1, w.H), name)


@pytest.mark.parametrize("name", ["tiny", "odd_bf16_big", "odd_mxfp8"])
def test_rows_without_probabilities(name):
    """Row mode reads no probabilities: a NULL pointer gives the same bits."""
    c = get_case(name)
    moe, _, with_p = run(c, "rows")
    _, _, no_p = run(c, "rows", moe=moe, no_probs=True)
    assert np.array_equal(with_p.view(np.uint32), no_p.view(np.uint32))


def test_probs_required_outside_row_mode():
    c = get_case("tiny")
    with pytest.raises(ValueError):       # MOE_ERR_INVALID_ARG: NULL probabilities
        run(c, "fp32", no_probs=True)
    with pytest.raises(ValueError):
        run(c, "half")
