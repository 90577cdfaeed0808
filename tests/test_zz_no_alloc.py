"""moe_forward_noalloc (the forward with the library's own per-GPU scratch as
workspace) against moe_forward_ex with a caller workspace, through the C ABI:
the same bits, on two calls in a row, the second with a smaller input, for
each precision and combine; and a capacity above the scratch is rejected on
the host with nothing enqueued."""
import numpy as np
import pytest
import torch

from workloads import WORKLOADS, Workload
from gpu_common import Case, live_tensor, sentinel_out

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import swiglu_expert_mlp_amd  # noqa: F401


CASES = {
    "decode_T300": (WORKLOADS["decode"].with_tokens(300), "fp32"),
    "decode_bf16_combine": (WORKLOADS["decode"].with_tokens(200), "bf16"),
    "mxfp8_T200": (WORKLOADS["mxfp8_16k"].with_tokens(200), "fp32"),
    "odd_mxfp4_rows": (Workload("odd_mxfp4", 77, 80, 96, 160, 5, 3, "mxfp4"), "rows"),
}


def _out(m, T_cap, combine):
    if combine == "bf16":
        return torch.full((T_cap, m.H), -7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    if combine == "rows":
        return torch.full((T_cap, m.topk, m.H), float("nan"), device="cuda")
    return sentinel_out(T_cap, m.H)


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_workspace_forward(name):
    from swiglu_expert_mlp_amd import MoE
    w, combine = CASES[name]
    print(f"[noalloc] {name}: T={w.T} cap={w.T_cap} {w.precision} combine={combine}", flush=True)
    c = Case(w, seed=12, outliers=w.precision != "bf16")
    m = MoE(w.E, w.H, w.F, w.k, w.precision)
    w1, w2 = c.weights_dev()
    m.load_weights(w1, w2)
    x, ids, probs = c.dev()
    # two calls in a row, the second on a smaller input (fewer rows and a
    # smaller capacity); the scratch keeps the first call's contents
    for T in (w.T, max(1, w.T // 3)):
        xs, i_s, ps = x[:T].contiguous(), ids[:T].contiguous(), probs[:T].contiguous()
        ref = _out(m, T, combine)
        ws = m.new_workspace(T)
        m.forward(xs, i_s, ps, live_tensor(T), out=ref, ws=ws, combine=combine)
        got = _out(m, T, combine)
        m.forward_noalloc(xs, i_s, ps, live_tensor(T), out=got, combine=combine)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(got), _bits(ref)), f"T={T}"


def test_noalloc_rejects_capacity_above_scratch():
    from swiglu_expert_mlp_amd import MoE
    w = WORKLOADS["decode"]
    m = MoE(w.E, w.H, w.F, w.k, w.precision)
    g = torch.Generator(device="cuda").manual_seed(1)
    m.load_weights((torch.randn((w.E, 2 * w.F, w.H), generator=g, device="cuda") * 0.02).bfloat16(),
                   (torch.randn((w.E, w.H, w.F), generator=g, device="cuda") * 0.02).bfloat16())
    T_cap = 4096
    assert m.workspace_bytes(T_cap) > (64 << 20)
    x = torch.zeros((T_cap, w.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((T_cap, w.k), dtype=torch.int32, device="cuda")
    probs = torch.zeros((T_cap, w.k), dtype=torch.float32, device="cuda")
    out = sentinel_out(T_cap, w.H)
    with pytest.raises(ValueError, match="scratch"):
        m.forward_noalloc(x, ids, probs, live_tensor(T_cap), out=out)
    torch.cuda.synchronize()
    assert np.all(out.view(torch.int32).cpu().numpy() == 0x7FBADBAD)
