"""The single-launch FFN mode (MOE_FUSED_FFN: FC1 and FC2 in one persistent
launch with per-M-tile readiness counters; Megatron-LM PR #7830, "What does
this PR do?", the fused expert MLP kernel).  Against the oracle, and bit for
bit against the two-launch path (the same 64-row tile arithmetic), including
back-to-back calls on one workspace with different inputs (a stale SwiGLU
row would show there), a workspace of garbage bytes (the counters are zeroed
by the forward itself), the other combines, and full-size workloads."""
import numpy as np
import pytest
import torch

from workloads import WORKLOADS, Workload
from gpu_common import Case, assert_close, live_tensor, sentinel_out, SENTINEL_BITS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import swiglu_expert_mlp_amd  # noqa: F401


def _moe(w):
    from swiglu_expert_mlp_amd import MoE
    return MoE(w.E, w.H, w.F, w.k, w.precision)


SMALL = {
    "tiny": WORKLOADS["tiny"],
    "decode_T64": WORKLOADS["decode"].with_tokens(64),
    "odd_bf16": Workload("odd_bf16", 77, 80, 96, 160, 5, 3, "bf16"),
    # experts past 128 rows: their 256-row tiles run as four 64-row tiles
    "mid_bf16_big": Workload("mid_bf16_big", 600, 600, 256, 192, 4, 2, "bf16"),
    # token capacities above 1024 (the mode still takes every tile as 64-row tiles)
    "odd64_bf16_big_cap": Workload("odd64_bf16_big_cap", 700, 1100, 192, 320, 5, 3, "bf16"),
    "mixed129_64_cap": Workload("mixed129_64_cap", 182, 1040, 128, 192, 3, 2, "bf16"),
}


def _fwd(m, x, ids, probs, T, T_cap, H, ws=None, **kw):
    out = sentinel_out(T_cap, H)
    ws = m.new_workspace(T_cap) if ws is None else ws
    m.forward(x, ids, probs, live_tensor(T), out=out, ws=ws, **kw)
    return out, ws


@pytest.mark.parametrize("name", list(SMALL))
def test_parity_and_bitwise_vs_two_launches(name):
    w = SMALL[name]
    print(f"[fused] {name}", flush=True)
    c = Case(w, seed=11)
    m = _moe(w)
    m.load_weights(*c.weights_dev())
    x, ids, probs = c.dev()
    fused, ws = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H, fused_ffn=True)
    two, _ = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H)
    torch.cuda.synchronize()
    assert m.check(ws) == 0
    got = fused.cpu().numpy()
    assert np.all(got[w.T:].view(np.uint32) == SENTINEL_BITS)
    ref, err, _ = c.oracle_model().forward(c.inp["x_bits"], c.ids, c.probs, w.T)
    assert err == 0
    assert_close(got[: w.T], ref[: w.T], name)
    assert np.array_equal(got.view(np.uint32), two.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("combine", ["bf16", "rows"])
def test_other_combines_bitwise(combine):
    w = SMALL["odd_bf16"]
    c = Case(w, seed=12)
    m = _moe(w)
    m.load_weights(*c.weights_dev())
    x, ids, probs = c.dev()
    shape = (w.T_cap, w.k, w.H) if combine == "rows" else (w.T_cap, w.H)
    dt = torch.float32 if combine == "rows" else torch.bfloat16
    outs = []
    for fused in (True, False):
        out = torch.zeros(shape, dtype=dt, device="cuda")
        m.forward(x, ids, probs, live_tensor(w.T), out=out, ws=m.new_workspace(w.T_cap),
                  combine=combine, fused_ffn=fused)
        outs.append(out.view(torch.int16 if dt == torch.bfloat16 else torch.int32).cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def test_topk_in_fc1_bitwise():
    w = SMALL["mid_bf16_big"]
    c = Case(w, seed=13)
    m = _moe(w)
    m.load_weights(*c.weights_dev())
    x, ids, probs = c.dev()
    a, _ = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H, fused_ffn=True, topk_in_fc1=True)
    b, _ = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H, topk_in_fc1=True)
    assert np.array_equal(a.view(torch.int32).cpu().numpy(), b.view(torch.int32).cpu().numpy())


def test_back_to_back_on_one_workspace_and_garbage():
    """Calls with different inputs on one workspace (filled with garbage
    bytes first): every call's rows must be its own."""
    w = WORKLOADS["decode"].with_tokens(200, 256)
    m = _moe(w)
    cases = [Case(w, seed=s) for s in (21, 22, 23)]
    m.load_weights(*cases[0].weights_dev())
    ws = m.new_workspace(w.T_cap)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda"))
    for i, c in enumerate(cases):
        x, ids, probs = c.dev()
        fused, _ = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H, ws=ws, fused_ffn=True)
        two, _ = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H)
        torch.cuda.synchronize()
        assert m.check(ws) == 0, i
        assert torch.equal(fused.view(torch.int32), two.view(torch.int32)), i


@pytest.mark.parametrize("name", ["decode", "bf16_16k"])
def test_full_size_bitwise(name):
    w = WORKLOADS[name]
    print(f"[fused] full size {name}", flush=True)
    m = _moe(w)
    g = torch.Generator(device="cuda").manual_seed(5)
    m.load_weights((torch.randn((w.E, 2 * w.F, w.H), generator=g, device="cuda") * 0.02).bfloat16(),
                   (torch.randn((w.E, w.H, w.F), generator=g, device="cuda") * 0.02).bfloat16())
    x = torch.randn((w.T_cap, w.H), generator=g, device="cuda").bfloat16()
    ids = torch.rand((w.T_cap, w.E), generator=g, device="cuda").argsort(dim=1)[:, : w.k]
    ids = ids.to(torch.int32).contiguous()
    probs = torch.rand((w.T_cap, w.k), generator=g, device="cuda")
    fused, ws = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H, fused_ffn=True)
    two, _ = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H)
    torch.cuda.synchronize()
    assert m.check(ws) == 0
    assert torch.equal(fused.view(torch.int32), two.view(torch.int32))


def test_rejected_for_mx_precisions():
    w = WORKLOADS["mxfp8_16k"].with_tokens(32)
    m = _moe(w)
    c = Case(w, seed=11)
    m.load_weights(*c.weights_dev())
    x, ids, probs = c.dev()
    with pytest.raises(ValueError, match="MOE_FUSED_FFN"):
        m.forward(x, ids, probs, live_tensor(w.T), fused_ffn=True)


# ---------------------------------------------------------------------------
# MOE_FUSED_FINALIZE: the finalize inside the same launch (the last FC2 tile of
# a token's 512-column block combines it).  Bit for bit against the separate
# finalize, in every combine, and against the oracle.

FIN_SHAPES = dict(SMALL)
# hidden sizes that end in a partial 512-column block, and top-16
FIN_SHAPES["h800_k16"] = Workload("h800_k16", 150, 160, 800, 64, 24, 16, "bf16")
FIN_SHAPES["h576_mixed_cap"] = Workload("h576_mixed_cap", 900, 1100, 576, 128, 6, 4, "bf16")


@pytest.mark.parametrize("name", list(FIN_SHAPES))
def test_fused_finalize_parity_and_bitwise(name):
    w = FIN_SHAPES[name]
    print(f"[fused finalize] {name}", flush=True)
    c = Case(w, seed=14)
    m = _moe(w)
    m.load_weights(*c.weights_dev())
    x, ids, probs = c.dev()
    one, ws = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H, fused_finalize=True)
    two, _ = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H)
    torch.cuda.synchronize()
    assert m.check(ws) == 0
    got = one.cpu().numpy()
    assert np.all(got[w.T:].view(np.uint32) == SENTINEL_BITS)
    ref, err, _ = c.oracle_model().forward(c.inp["x_bits"], c.ids, c.probs, w.T)
    assert err == 0
    assert_close(got[: w.T], ref[: w.T], name)
    assert np.array_equal(got.view(np.uint32), two.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("combine", ["bf16", "rows"])
def test_fused_finalize_other_combines_bitwise(combine):
    w = FIN_SHAPES["h800_k16"]
    c = Case(w, seed=15)
    m = _moe(w)
    m.load_weights(*c.weights_dev())
    x, ids, probs = c.dev()
    shape = (w.T_cap, w.k, w.H) if combine == "rows" else (w.T_cap, w.H)
    dt = torch.int32 if combine == "rows" else torch.int16
    outs = []
    for fin in (True, False):
        # a sentinel fill: rows past live must stay as they are
        out = torch.full(shape, 0x7BAD, dtype=dt, device="cuda")
        out = out.view(torch.float32 if combine == "rows" else torch.bfloat16)
        m.forward(x, ids, None if combine == "rows" else probs, live_tensor(w.T), out=out,
                  ws=m.new_workspace(w.T_cap), combine=combine, fused_finalize=fin)
        outs.append(out.view(dt).cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    assert np.all(outs[0][w.T:] == 0x7BAD)


def test_fused_finalize_topk_in_fc1_bitwise():
    w = SMALL["mid_bf16_big"]
    c = Case(w, seed=16)
    m = _moe(w)
    m.load_weights(*c.weights_dev())
    x, ids, probs = c.dev()
    a, _ = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H, fused_finalize=True, topk_in_fc1=True)
    b, _ = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H, topk_in_fc1=True)
    assert np.array_equal(a.view(torch.int32).cpu().numpy(), b.view(torch.int32).cpu().numpy())


@pytest.mark.parametrize("combine", ["fp32", "bf16", "rows"])
def test_fused_finalize_dropped_routes(combine):
    """Tokens with some or all routes dropped (ids out of range or repeated):
    the counts start from the kept routes, and a token with none kept is
    written +0 by the permutation stage, as the separate finalize writes it."""
    w = FIN_SHAPES["odd_bf16"]
    c = Case(w, seed=17)
    m = _moe(w)
    m.load_weights(*c.weights_dev())
    x, ids, probs = c.dev()
    ids = ids.clone()
    ids[3, :] = -5                   # every route out of range
    ids[4, 1] = ids[4, 0]            # a repeat
    ids[9, :] = w.E + 3              # every route out of range
    ids[10, 0] = -1                  # one route out of range
    ids[w.T - 1, :] = ids[w.T - 1, 0]   # every route the same expert: one kept
    shape = (w.T_cap, w.k, w.H) if combine == "rows" else (w.T_cap, w.H)
    dt = torch.int16 if combine == "bf16" else torch.int32
    outs, bits = [], []
    for fin in (True, False):
        out = torch.full(shape, 0x7BAD, dtype=dt, device="cuda")
        out = out.view(torch.bfloat16 if combine == "bf16" else torch.float32)
        ws = m.new_workspace(w.T_cap)
        m.forward(x, ids, None if combine == "rows" else probs, live_tensor(w.T), out=out, ws=ws,
                  combine=combine, fused_finalize=fin)
        torch.cuda.synchronize()
        bits.append(m.check(ws))
        outs.append(out.view(dt).cpu().numpy())
    assert bits[0] == bits[1] and bits[0] != 0
    assert np.array_equal(outs[0], outs[1])
    assert np.all(outs[0][3] == 0) and np.all(outs[0][9] == 0)
    assert np.all(outs[0][w.T:] == 0x7BAD)


def test_fused_finalize_back_to_back_on_garbage():
    """Back-to-back calls with different inputs and live counts on one workspace
    of garbage bytes: the counts are set by each call's permutation stage."""
    w = WORKLOADS["decode"].with_tokens(200, 256)
    m = _moe(w)
    cases = [Case(w, seed=s) for s in (31, 32, 33)]
    m.load_weights(*cases[0].weights_dev())
    ws = m.new_workspace(w.T_cap)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda"))
    for i, (c, live) in enumerate(zip(cases, (200, 37, 200))):
        x, ids, probs = c.dev()
        one, _ = _fwd(m, x, ids, probs, live, w.T_cap, w.H, ws=ws, fused_finalize=True)
        two, _ = _fwd(m, x, ids, probs, live, w.T_cap, w.H)
        torch.cuda.synchronize()
        assert m.check(ws) == 0, i
        assert torch.equal(one.view(torch.int32), two.view(torch.int32)), i


@pytest.mark.parametrize("name", ["decode", "bf16_16k"])
def test_fused_finalize_full_size_bitwise(name):
    w = WORKLOADS[name]
    print(f"[fused finalize] full size {name}", flush=True)
    m = _moe(w)
    g = torch.Generator(device="cuda").manual_seed(6)
    m.load_weights((torch.randn((w.E, 2 * w.F, w.H), generator=g, device="cuda") * 0.02).bfloat16(),
                   (torch.randn((w.E, w.H, w.F), generator=g, device="cuda") * 0.02).bfloat16())
    x = torch.randn((w.T_cap, w.H), generator=g, device="cuda").bfloat16()
    ids = torch.rand((w.T_cap, w.E), generator=g, device="cuda").argsort(dim=1)[:, : w.k]
    ids = ids.to(torch.int32).contiguous()
    probs = torch.rand((w.T_cap, w.k), generator=g, device="cuda")
    one, ws = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H, fused_finalize=True)
    two, _ = _fwd(m, x, ids, probs, w.T, w.T_cap, w.H)
    torch.cuda.synchronize()
    assert m.check(ws) == 0
    assert torch.equal(one.view(torch.int32), two.view(torch.int32))


def test_fused_finalize_rejected_for_mx_precisions():
    w = WORKLOADS["mxfp8_16k"].with_tokens(32)
    m = _moe(w)
    c = Case(w, seed=11)
    m.load_weights(*c.weights_dev())
    x, ids, probs = c.dev()
    with pytest.raises(ValueError, match="MOE_FUSED_FINALIZE"):
        m.forward(x, ids, probs, live_tensor(w.T), fused_finalize=True)
