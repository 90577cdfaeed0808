"""bf16 above a 1024-token capacity: a GEMM stage is a launch of the 256-row
tiles (experts with more than 128 rows) and a launch of the 64-row tiles (the
other experts).  The forward runs the 64-row FC1 -> FC2 chain on the
library's side stream while the 256-row chain runs on the caller's stream,
forked and joined with events; with stage events on (profiling) the stages
stay serial.  The two orders must give the same bits, match the oracle, and
stay correct when two caller streams share one handle (and so one side
stream) at the same time.  Shapes where only one stage has two launches (the
other stage's K not a multiple of 64, or under 128) cover the fork-only and
join-only orders."""
import numpy as np
import pytest
import torch

from workloads import Workload
from gpu_common import Case, assert_close, live_tensor, sentinel_out, SENTINEL_BITS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import swiglu_expert_mlp_amd  # noqa: F401


SHAPES = {
    # both stages have a 256-row and a 64-row launch
    "both_split": Workload("both_split", 1400, 1500, 256, 192, 8, 2, "bf16"),
    # FC1 (K = H = 256) split, FC2 one launch (K = F = 96 is not a multiple of 64)
    "fc1_split": Workload("fc1_split", 1400, 1500, 256, 96, 8, 2, "bf16"),
    # FC1 one launch (K = H = 64, under the 256-row kernel's two stages), FC2
    # (K = F = 192) split
    "fc2_split": Workload("fc2_split", 1400, 1500, 64, 192, 8, 2, "bf16"),
}


def _skewed(c, n_small_tokens=100, seed=7):
    """Routes: the first tokens go to the upper half of the experts (about 50
    rows each: 64-row tiles), the rest to the lower half (hundreds of rows
    each: 256-row tiles)."""
    w = c.w
    rng = np.random.default_rng(seed)
    ids = np.full((w.T_cap, w.k), 0x7FC00000, dtype=np.int32)
    probs = np.full((w.T_cap, w.k), np.uint32(0x7FC00000).view(np.float32), dtype=np.float32)
    half = w.E // 2
    for t in range(w.T):
        pool = np.arange(half, w.E) if t < n_small_tokens else np.arange(half)
        ids[t] = np.sort(rng.choice(pool, size=w.k, replace=False))
        p = rng.random(w.k).astype(np.float32) + np.float32(0.1)
        probs[t] = p / p.sum(dtype=np.float32)
    c.ids, c.probs = ids, probs
    return c


def _run(m, x, ids, probs, T, T_cap, H, ws, stream=None, out=None, live=None):
    out = sentinel_out(T_cap, H) if out is None else out
    m.forward(x, ids, probs, live_tensor(T) if live is None else live, out=out, ws=ws, stream=stream)
    return out


@pytest.mark.parametrize("name", list(SHAPES))
def test_two_streams_match_serial_and_oracle(name):
    from swiglu_expert_mlp_amd import MoE
    w = SHAPES[name]
    print(f"[side stream] {name}", flush=True)
    c = _skewed(Case(w, seed=18))
    m = MoE(w.E, w.H, w.F, w.k, w.precision)
    m.load_weights(*c.weights_dev())
    x = c.dev()[0]
    ids, probs = torch.from_numpy(c.ids).cuda(), torch.from_numpy(c.probs).cuda()
    ws = m.new_workspace(w.T_cap)
    forked = _run(m, x, ids, probs, w.T, w.T_cap, w.H, ws)
    torch.cuda.synchronize()
    assert m.check(ws) == 0
    idx = m.get_indices(ws, w.T_cap)
    counts = idx["counts"]
    assert counts[: w.E // 2].min() > 128 and 0 < counts[w.E // 2:].max() <= 128, counts
    # stage events on: the serial order
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    m.set_stage_events(evs)
    try:
        serial = _run(m, x, ids, probs, w.T, w.T_cap, w.H, m.new_workspace(w.T_cap))
    finally:
        m.set_stage_events(None)
    torch.cuda.synchronize()
    got = forked.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), serial.cpu().numpy().view(np.uint32))
    assert np.all(got[w.T:].view(np.uint32) == SENTINEL_BITS)
    ref, err, _ = c.oracle_model().forward(c.inp["x_bits"], c.ids, c.probs, w.T)
    assert err == 0
    assert_close(got[: w.T], ref[: w.T], name)


def test_two_caller_streams_share_one_handle():
    """Forwards enqueued alternately on two caller streams (one handle, two
    workspaces, different inputs) give each stream's own serial result."""
    from swiglu_expert_mlp_amd import MoE
    w = SHAPES["both_split"]
    c = _skewed(Case(w, seed=19))
    m = MoE(w.E, w.H, w.F, w.k, w.precision)
    m.load_weights(*c.weights_dev())
    x = c.dev()[0]
    x2 = torch.flip(x, dims=[0]).contiguous()
    ids, probs = torch.from_numpy(c.ids).cuda(), torch.from_numpy(c.probs).cuda()
    refs = []
    for xx in (x, x2):
        refs.append(_run(m, xx, ids, probs, w.T, w.T_cap, w.H, m.new_workspace(w.T_cap)))
    torch.cuda.synchronize()
    refs = [r.cpu().numpy().view(np.uint32) for r in refs]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws1, ws2 = m.new_workspace(w.T_cap), m.new_workspace(w.T_cap)
    # every buffer the two streams use is made (on the current stream) before
    # they start
    live = live_tensor(w.T)
    bufs = [sentinel_out(w.T_cap, w.H) for _ in range(6)]
    torch.cuda.synchronize()
    outs = []
    for i in range(3):
        outs.append((0, _run(m, x, ids, probs, w.T, w.T_cap, w.H, ws1, stream=s1, out=bufs[2 * i],
                             live=live)))
        outs.append((1, _run(m, x2, ids, probs, w.T, w.T_cap, w.H, ws2, stream=s2,
                             out=bufs[2 * i + 1], live=live)))
    torch.cuda.synchronize()
    for which, o in outs:
        assert np.array_equal(o.cpu().numpy().view(np.uint32), refs[which]), which
