"""Batch invariance, determinism, live-row bounds, refit and error reporting of
the HIP path (through the C ABI), on the GPU.

Megatron-LM PR #7830, "Tests": a token's output does not depend on how many
tokens shared the launch; repeated launches return identical bits; a refit
without refreshing the kernel weights is stale (negative control); per-layer
buffers are independent.  Megatron-LM PR #8367, "Problem": only the live
rows are touched.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, Workload
from gpu_common import Case, assert_close, live_tensor, sentinel_out, to_dev_bits, SENTINEL_BITS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import swiglu_expert_mlp_amd  # noqa: F401


INV = {
    "decode_T300": WORKLOADS["decode"].with_tokens(300),
    "logprob_T300": WORKLOADS["logprob"].with_tokens(300),
    "mxfp8_T300": WORKLOADS["mxfp8_16k"].with_tokens(300),
    "odd_mxfp8_T300": Workload("odd_mxfp8", 300, 300, 96, 160, 5, 3, "mxfp8"),
    # odd bf16 shapes: 256-row tiles in the wide launch, 64-row tiles with partial
    # 512-column tiles and a half-full last 64-column block in the 8-token chunks
    "odd_bf16_T300": Workload("odd_bf16", 300, 300, 96, 160, 5, 3, "bf16"),
    "mxfp4_T300": WORKLOADS["mxfp4_16k"].with_tokens(300),
    "decode_mxfp4": WORKLOADS["decode_mxfp4"],
}
_cases = {}


def case(name):
    if name not in _cases:
        _cases[name] = Case(INV[name], seed=12, outliers=INV[name].precision != "bf16")
    return _cases[name]


_handles = {}


def handle(name):
    if name not in _handles:
        from swiglu_expert_mlp_amd import MoE
        c = case(name)
        w = c.w
        m = MoE(w.E, w.H, w.F, w.k, w.precision)
        w1, w2 = c.weights_dev()
        m.load_weights(w1, w2)
        _handles[name] = m
    return _handles[name]


def forward(m, x, ids, probs, live, T_cap=None, stream=None):
    T_cap = x.shape[0] if T_cap is None else T_cap
    out = sentinel_out(T_cap, m.H)
    ws = m.new_workspace(T_cap)
    m.forward(x, ids, probs, live_tensor(live), out=out, ws=ws, stream=stream)
    return out, ws


def bits(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("name", list(INV))
def test_wide_equals_chunks_of_8(name):
    c, m = case(name), handle(name)
    x, ids, probs = c.dev()
    T = c.w.T
    wide, _ = forward(m, x, ids, probs, T)
    wide = bits(wide)
    for t0 in range(0, T, 8):
        t1 = min(T, t0 + 8)
        part, _ = forward(m, x[t0:t1].contiguous(), ids[t0:t1].contiguous(),
                          probs[t0:t1].contiguous(), t1 - t0)
        assert np.array_equal(bits(part), wide[t0:t1]), f"tokens {t0}..{t1}"


@pytest.mark.parametrize("name", ["logprob", "mxfp8_16k", "mxfp4_16k"])
def test_64_row_and_256_row_tiles_agree_bitwise(name):
    """Experts with more than 128 rows run on the 256-row tiles, the others on
    the 64-row tiles; a token's bits must not depend on which one ran."""
    from swiglu_expert_mlp_amd import MoE
    w = WORKLOADS[name].with_tokens(2048)
    c = Case(w, seed=11, outliers=w.precision != "bf16")
    m = MoE(w.E, w.H, w.F, w.k, w.precision)
    w1, w2 = c.weights_dev()
    m.load_weights(w1, w2)
    x, ids, probs = c.dev()
    wide, ws = forward(m, x, ids, probs, w.T)
    counts = m.get_indices(ws, w.T)["counts"]
    assert (counts > 128).sum() > 10 and (counts <= 128).sum() > 10, counts
    wide = bits(wide)
    for t0 in range(0, w.T, 128):
        part, _ = forward(m, x[t0:t0 + 128].contiguous(), ids[t0:t0 + 128].contiguous(),
                          probs[t0:t0 + 128].contiguous(), 128)
        assert np.array_equal(bits(part), wide[t0:t0 + 128]), f"tokens {t0}.."


@pytest.mark.parametrize("precision", ["mxfp8", "mxfp4"])
def test_partial_scale_chunk_shapes_agree_bitwise(precision):
    """Hidden 1280 and FFN 1152 are 10 and 9 K steps of 128: the 256-row MX
    tiles load the activation scales in chunks of 8 steps, so both GEMMs end
    on a partial chunk.  Experts with more than 128 rows (256-row tiles) and
    the same tokens in launches of 128 (every expert on the 64-row tiles, which
    take no chunks) must give the same bits."""
    from swiglu_expert_mlp_amd import MoE
    w = Workload("mx_chunks", 2048, 2048, 1280, 1152, 64, 4, precision)
    c = Case(w, seed=17, outliers=True)
    m = MoE(w.E, w.H, w.F, w.k, w.precision)
    w1, w2 = c.weights_dev()
    m.load_weights(w1, w2)
    x, ids, probs = c.dev()
    wide, ws = forward(m, x, ids, probs, w.T)
    counts = m.get_indices(ws, w.T)["counts"]
    assert (counts > 128).sum() > 10, counts
    wide = bits(wide)
    for t0 in range(0, w.T, 128):
        part, _ = forward(m, x[t0:t0 + 128].contiguous(), ids[t0:t0 + 128].contiguous(),
                          probs[t0:t0 + 128].contiguous(), 128)
        assert np.array_equal(bits(part), wide[t0:t0 + 128]), f"tokens {t0}.."


def test_mxfp4_small_capacity_runs_large_experts_as_64_row_tiles_bitwise():
    """MXFP4 at a token capacity <= 1024 runs experts with more than 128 rows as
    four 64-row tiles each (one launch); at a larger capacity they take the
    256-row tiles.  Same tokens, capacity 600 vs 2400: the same bits."""
    from swiglu_expert_mlp_amd import MoE
    w = Workload("mx4_cap", 600, 600, 256, 384, 4, 2, "mxfp4")
    c = Case(w, seed=13, outliers=True)
    m = MoE(w.E, w.H, w.F, w.k, w.precision)
    w1, w2 = c.weights_dev()
    m.load_weights(w1, w2)
    x, ids, probs = c.dev()
    small, ws = forward(m, x, ids, probs, w.T)
    counts = m.get_indices(ws, w.T)["counts"]
    assert (counts > 128).sum() >= 2, counts
    cap = 4 * w.T
    xb = torch.full((cap, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    xb[:w.T] = x
    ib = torch.full((cap, w.k), 0x7FC00000, dtype=torch.int32, device="cuda")
    ib[:w.T] = ids
    pb = torch.full((cap, w.k), float("nan"), dtype=torch.float32, device="cuda")
    pb[:w.T] = probs
    large = bits(forward(m, xb, ib, pb, w.T)[0])
    assert np.array_equal(large[:w.T], bits(small))
    assert np.all(large[w.T:] == SENTINEL_BITS)


def test_mxfp4_fc2_streaming_64_row_tiles_past_2gib_bitwise():
    """The 64-row MXFP4 LDS-staged kernel addresses its activation codes with
    32-bit byte offsets, so FC2's 64-row tiles go to the streaming tiles once
    the SwiGLU buffer (capacity x top-k x FFN bytes) reaches 2 GiB, with K
    (= FFN 1024) still a multiple of 128.  The same 2048 live tokens at
    capacity 2048 (LDS-staged) and 2^20 + 64 (streaming) give the same bits."""
    from swiglu_expert_mlp_amd import MoE
    w = Workload("mx4_w2g", 2048, 2048, 128, 1024, 32, 2, "mxfp4")
    c = Case(w, seed=19, outliers=True)
    m = MoE(w.E, w.H, w.F, w.k, w.precision)
    w1, w2 = c.weights_dev()
    m.load_weights(w1, w2)
    x, ids, probs = c.dev()
    small, ws = forward(m, x, ids, probs, w.T)
    counts = m.get_indices(ws, w.T)["counts"]
    assert ((counts > 0) & (counts <= 128)).sum() >= 2 and (counts > 128).sum() >= 2, counts
    small = bits(small)
    del ws
    cap = (1 << 20) + 64
    assert cap * w.k * w.F >= 1 << 31 and cap * w.H < 1 << 31
    xb = torch.full((cap, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    xb[:w.T] = x
    ib = torch.full((cap, w.k), 0x7FC00000, dtype=torch.int32, device="cuda")
    ib[:w.T] = ids
    pb = torch.full((cap, w.k), float("nan"), dtype=torch.float32, device="cuda")
    pb[:w.T] = probs
    out, ws = forward(m, xb, ib, pb, w.T)
    del ws, xb, ib, pb
    large = bits(out)
    assert np.array_equal(large[:w.T], small)
    assert np.all(large[w.T:] == SENTINEL_BITS)


@pytest.mark.parametrize("name", ["decode_T300", "mxfp8_T300", "mxfp4_T300"])
def test_capacity_and_live_count_invariance(name):
    """Same tokens: capacity T vs 4T, 6000 and 20000 (rows past live are NaN;
    on a 256-CU device the finalize runs a workgroup per token at 6000 and
    loops over tokens at the others), and live counts T, 171, 1, 0 at a fixed
    capacity give the same bits for the live tokens and leave every other
    output row untouched."""
    c, m = case(name), handle(name)
    x, ids, probs = c.dev()
    T = c.w.T
    ref = bits(forward(m, x, ids, probs, T)[0])
    for cap in (4 * T, 6000, 20000):
        xb = torch.full((cap, c.w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        xb[:T] = x
        ib = torch.full((cap, c.w.k), 0x7FC00000, dtype=torch.int32, device="cuda")
        ib[:T] = ids
        pb = torch.full((cap, c.w.k), float("nan"), dtype=torch.float32, device="cuda")
        pb[:T] = probs
        got = bits(forward(m, xb, ib, pb, T)[0])
        assert np.array_equal(got[:T], ref), cap
        assert np.all(got[T:] == SENTINEL_BITS), cap
    for live in (T, 171, 1, 0):
        got = bits(forward(m, x, ids, probs, live)[0])
        assert np.array_equal(got[:live], ref[:live]), live
        assert np.all(got[live:] == SENTINEL_BITS), live


@pytest.mark.parametrize("name", ["decode_T300", "mxfp8_T300", "mxfp4_T300"])
def test_token_order_invariance(name):
    c, m = case(name), handle(name)
    x, ids, probs = c.dev()
    T = c.w.T
    ref = bits(forward(m, x, ids, probs, T)[0])
    perm = torch.from_numpy(np.random.default_rng(5).permutation(T)).cuda()
    got = bits(forward(m, x[perm].contiguous(), ids[perm].contiguous(),
                       probs[perm].contiguous(), T)[0])
    assert np.array_equal(got, ref[perm.cpu().numpy()])
    # a token's routes listed in a different order: the same bits
    rev = bits(forward(m, x, ids.flip(1).contiguous(), probs.flip(1).contiguous(), T)[0])
    assert np.array_equal(rev, ref)


@pytest.mark.parametrize("name", ["decode_T300", "odd_mxfp8_T300", "mxfp4_T300", "decode_mxfp4"])
def test_repeat_and_racing_stream(name):
    """Identical bits across repeated launches, also while a second stream
    (default priority) moves ~1 GB through HBM at the same time (the MXFP4
    64-row kernel waits on per-wave load counts with no barrier on its weight
    ring: other traffic changes the timing such counts have to hold under)."""
    c, m = case(name), handle(name)
    x, ids, probs = c.dev()
    T = c.w.T
    ref = bits(forward(m, x, ids, probs, T)[0])
    for _ in range(3):
        assert np.array_equal(bits(forward(m, x, ids, probs, T)[0]), ref)
    src = torch.empty(256 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    with torch.cuda.stream(side):
        for _ in range(4):
            dst.copy_(src)
    for _ in range(4):
        outs.append(forward(m, x, ids, probs, T)[0])
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(bits(o), ref)


def test_refit_stale_then_fresh():
    """Changing the parameters without reloading leaves the kernel weights (and
    outputs) unchanged; reloading into the same buffer equals a fresh handle."""
    from swiglu_expert_mlp_amd import MoE
    c = case("decode_T300")
    w = c.w
    x, ids, probs = c.dev()
    w1, w2 = c.weights_dev()
    m = MoE(w.E, w.H, w.F, w.k, w.precision)
    kbuf = m.load_weights(w1, w2)
    before = bits(forward(m, x, ids, probs, w.T)[0])
    w1.mul_(-0.5)                      # in-place parameter update, no refresh
    stale = bits(forward(m, x, ids, probs, w.T)[0])
    assert np.array_equal(stale, before), "the kernel weights changed without a refresh"
    m.load_weights(w1, w2, kbuf=kbuf)  # the refit: rewrite the same buffer in place
    refit = bits(forward(m, x, ids, probs, w.T)[0])
    fresh_m = MoE(w.E, w.H, w.F, w.k, w.precision)
    fresh_m.load_weights(w1, w2)
    fresh = bits(forward(fresh_m, x, ids, probs, w.T)[0])
    assert np.array_equal(refit, fresh)
    assert not np.array_equal(refit, before)
    # the reference: oracle with the updated weights
    m_or = oracle.Model(w.E, w.H, w.F, w.k,
                        w1.view(torch.int16).cpu().numpy().view(np.uint16),
                        c.inp["w2_bits"])
    ref, _, _ = m_or.forward(c.inp["x_bits"], c.ids, c.probs, w.T)
    assert_close(refit.view(np.float32)[: w.T], ref[: w.T], "refit")


def test_two_handles_are_independent():
    from swiglu_expert_mlp_amd import MoE
    c = case("decode_T300")
    w = c.w
    x, ids, probs = c.dev()
    w1, w2 = c.weights_dev()
    a = MoE(w.E, w.H, w.F, w.k, w.precision)
    b = MoE(w.E, w.H, w.F, w.k, w.precision)
    a.load_weights(w1, w2)
    b.load_weights((w1 * 2).contiguous(), w2)
    ra = bits(forward(a, x, ids, probs, w.T)[0])
    rb = bits(forward(b, x, ids, probs, w.T)[0])
    assert np.array_equal(ra, bits(forward(handle("decode_T300"), x, ids, probs, w.T)[0]))
    assert not np.array_equal(ra, rb)


@pytest.mark.parametrize("precision", ["bf16", "mxfp8", "mxfp4"])
def test_contract_violations_flagged_and_match_oracle(precision):
    """An out-of-range id drops that route, a repeated id drops the repeat, and
    both set their bit; live above capacity is clamped, below zero writes
    nothing.  The outputs match the oracle's rules for the same cases."""
    from swiglu_expert_mlp_amd import MoE
    w = Workload("viol", 40, 40, 64, 96, 6, 3, precision)
    c = Case(w, seed=13)
    ids = c.ids.copy()
    ids[3, 1] = 6            # out of range
    ids[5, 2] = -1           # out of range
    ids[7, 2] = ids[7, 0]    # duplicate
    m = MoE(w.E, w.H, w.F, w.k, precision)
    w1, w2 = c.weights_dev()
    m.load_weights(w1, w2)
    x = to_dev_bits(c.inp["x_bits"])
    out, ws = forward(m, x, torch.from_numpy(ids).cuda(), torch.from_numpy(c.probs).cuda(), w.T)
    assert m.check(ws) == 3
    assert m.check(ws) == 0, "check clears the bits"
    ref, err, _ = c.oracle_model().forward(c.inp["x_bits"], ids, c.probs, w.T)
    assert err == 3
    assert_close(out.cpu().numpy()[: w.T], ref[: w.T], "violations")
    # live above capacity: clamped, bit 4
    out, ws = forward(m, x, torch.from_numpy(c.ids).cuda(), torch.from_numpy(c.probs).cuda(),
                      w.T + 5)
    assert m.check(ws) == 4
    assert not np.any(bits(out) == SENTINEL_BITS)
    # live below zero: nothing written, bit 8
    out, ws = forward(m, x, torch.from_numpy(c.ids).cuda(), torch.from_numpy(c.probs).cuda(), -3)
    assert m.check(ws) == 8
    assert np.all(bits(out) == SENTINEL_BITS)
    # the router reports its live-count bits too
    logits = torch.from_numpy(c.inp["logits"]).cuda()
    ws = m.new_workspace(w.T_cap)
    m.route(logits, live_tensor(w.T + 1), ws=ws)
    assert m.check(ws) == 4


@pytest.mark.parametrize("name", ["decode_T300", "mxfp8_T300"])
def test_stage_events_leave_outputs_unchanged(name):
    """The stage-timing hook (events 2 and 3 are recorded by the FC1 launch's
    own dispatch) changes no output bit, times a positive FC1 stage and keeps
    the stage boundaries in order."""
    c, m = case(name), handle(name)
    x, ids, probs = c.dev()
    T = c.w.T
    ref = bits(forward(m, x, ids, probs, T)[0])
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    m.set_stage_events(evs)
    try:
        got = bits(forward(m, x, ids, probs, T)[0])
    finally:
        m.set_stage_events(None)
    torch.cuda.synchronize()
    assert np.array_equal(got, ref)
    t = [evs[0].elapsed_time(e) for e in evs]
    assert t[3] - t[2] > 0, t
    assert all(b >= a - 1e-3 for a, b in zip(t, t[1:])), t


@pytest.mark.parametrize("name", ["decode_T300", "mxfp8_T300", "odd_bf16_T300", "decode_mxfp4"])
@pytest.mark.parametrize("fill", [0xFF, 0xA5])
def test_garbage_workspace_gives_identical_results(name, fill):
    """A workspace needs no initialisation: one filled with garbage bytes gives
    the same output bits, indices and (no) error bits as a zeroed one, for the
    router and the forward, in the single-chunk (capacity <= 256 tokens) and
    the multi-chunk prep paths."""
    c, m = case(name), handle(name)
    x, ids, probs = c.dev()
    T = c.w.T
    out0 = sentinel_out(T, m.H)
    ws0 = torch.zeros(m.workspace_bytes(T), dtype=torch.uint8, device="cuda")
    m.forward(x, ids, probs, live_tensor(T), out=out0, ws=ws0)
    ref_idx = m.get_indices(ws0, T)
    out1 = sentinel_out(T, m.H)
    ws1 = torch.full((m.workspace_bytes(T),), fill, dtype=torch.uint8, device="cuda")
    m.forward(x, ids, probs, live_tensor(T), out=out1, ws=ws1)
    assert np.array_equal(bits(out1), bits(out0))
    idx = m.get_indices(ws1, T)
    for key in ("counts", "offsets", "perm_src", "dst"):
        assert np.array_equal(idx[key], ref_idx[key]), key
    assert m.check(ws1) == 0
    # the router on a garbage workspace: no stale error bits, same ids
    logits = torch.from_numpy(c.inp["logits"]).cuda()
    ws2 = torch.full((m.workspace_bytes(T),), fill, dtype=torch.uint8, device="cuda")
    gi, gp = m.route(logits, live_tensor(T), ws=ws2)
    assert m.check(ws2) == 0
    assert np.array_equal(gi.cpu().numpy()[:T], c.ids[:T])
