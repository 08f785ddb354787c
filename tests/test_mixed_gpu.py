"""GPU tests of the mixed decode + prefill step (gdn_mixed_step) and of
prefill split across calls, through the C ABI.

RL-Kernel PR #469, "Not reproducible from this branch: the mixed
decode+prefill measurement": a decode row's state depended on what else its
step held, because mixed steps routed cached rows through another recurrent
kernel; the fix it points to routes them through the decode kernel and aligns
non-final chunked-prefill calls to the 64-token grid.  Checked here:

* parity of a mixed step against the oracle (decode rows: the oracle decode
  step, 1e-5; prefill sequences: the oracle varlen conv, its output rounded to
  bf16 as the step's prefill activations are, then the oracle token-by-token
  prefill, 5e-3; conv rolls bit-exact);
* every decode row bitwise equal (output, recurrent state, conv state) across
  a decode-only step and mixed steps with different prefill compositions;
* a sequence prefilled over two calls split on the 64-token grid equals one
  whole prefill bitwise (mixed step, and the post-conv prefill call alone);
  split off the grid it agrees within the prefill bar only.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_recurrent_gdn_amd as gdn
import oracle
from gpu_helpers import DECODE_TOL, PREFILL_TOL, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu

H, HV, DK = 4, 8, 128
D = 2 * H * DK + HV * DK
SCALE = DK ** -0.5


def _caches(num_slots, seed):
    d = gi.decode_inputs(1, num_slots, H=H, HV=HV, dk=DK, dv=DK, seed=seed, conv_bias=True)
    return d["conv_state"], d["conv_weight"], d["conv_bias"], d["rec_state"]


def _rows(n, seed):
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn(n, D, generator=gen).to(torch.bfloat16)
    g = -torch.rand(n, HV, generator=gen)
    beta = torch.sigmoid(torch.randn(n, HV, generator=gen))
    return x, g, beta


def _mixed(x, g, beta, n_dec, lengths, slots, caches, flags=gdn.DEFAULT_DECODE_FLAGS,
           segment_states=False, streams=None):
    """Run one mixed step on GPU copies of the caches; returns (out, cs, rs).
    segment_states: give the step room for the prefill's segment states;
    streams: a MixedStreams for the overlapped two-stream schedule."""
    cs, w, b, rs = (c.cuda() for c in caches)
    cs, rs = cs.clone(), rs.clone()
    cu = gi.cu_from_lengths(lengths).cuda() if lengths else None
    dims = gdn.make_dims(H, HV, DK, DK, 4)
    out = torch.full((x.shape[0], HV, DK), float("nan"), device="cuda")
    ws = None
    if segment_states:
        T = sum(lengths)
        extra = gdn.gdn_prefill_workspace_size(dims, len(lengths), T)
        assert extra > 0, "these sizes should take the segment-parallel schedule"
        ws = torch.empty(gdn.gdn_mixed_workspace_size(dims, n_dec, T) + extra,
                         dtype=torch.uint8, device="cuda")
    gdn.gdn_mixed_step(x.cuda(), g.cuda(), beta.cuda(), n_dec, cu, slots.cuda(), cs, w, rs, out,
                       dims, SCALE, conv_bias=b, flags=flags, workspace=ws, streams=streams)
    torch.cuda.synchronize()
    return out, cs, rs


def _oracle_mixed(x, g, beta, n_dec, lengths, slots, caches):
    cs, w, b, rs = (f64(c).copy() for c in caches)
    o_dec = oracle.decode_step(f64(x[:n_dec]), f64(g[:n_dec]), f64(beta[:n_dec]),
                               slots[:n_dec].numpy(), cs, w, rs, H, HV, DK, DK, SCALE,
                               conv_bias=b)
    cu = gi.cu_from_lengths(lengths).numpy()
    y = oracle.conv_update(f64(x[n_dec:]), slots[n_dec:].numpy(), cs, w, bias=b, cu_seqlens=cu,
                           flags=oracle.FLAG_SILU)
    y = torch.from_numpy(y).to(torch.bfloat16).double().numpy()     # the step's bf16 activations
    T = y.shape[0]
    q = y[:, :H * DK].reshape(T, H, DK)
    k = y[:, H * DK:2 * H * DK].reshape(T, H, DK)
    v = y[:, 2 * H * DK:].reshape(T, HV, DK)
    o_pre = oracle.prefill(q, k, v, f64(g[n_dec:]), f64(beta[n_dec:]), cu, slots[n_dec:].numpy(),
                           rs, SCALE)
    return o_dec, o_pre, cs, rs


@pytest.mark.parametrize("two_streams", [False, True])
def test_mixed_step_matches_oracle(two_streams):
    n_dec, lengths = 5, [1, 70, 0, 130, 64]
    caches = _caches(16, seed=70)
    x, g, beta = _rows(n_dec + sum(lengths), seed=71)
    slots = torch.tensor([3, 0, 9, 12, 1, 5, 7, 2, -1, 14], dtype=torch.int32)
    slots[8 + 0] = 11          # prefill seq 3 (130 tokens) active
    slots[9] = 0               # prefill seq 4 inactive (64 tokens): zero output
    out, cs, rs = _mixed(x, g, beta, n_dec, lengths, slots, caches,
                         streams=gdn.MixedStreams() if two_streams else None)
    o_dec, o_pre, cs_ref, rs_ref = _oracle_mixed(x, g, beta, n_dec, lengths, slots, caches)
    assert rel_err(f64(out[:n_dec]), o_dec) <= DECODE_TOL
    assert rel_err(f64(out[n_dec:]), o_pre) <= PREFILL_TOL
    for i, s in enumerate(slots.tolist()):
        if s <= 0:
            continue
        tol = DECODE_TOL if i < n_dec else PREFILL_TOL
        assert rel_err(f64(rs[s]), rs_ref[s]) <= tol, (i, s)
        assert np.array_equal(f64(cs[s]), cs_ref[s]), f"conv roll of slot {s}"
    c = [n_dec + t for t in gi.cu_from_lengths(lengths).tolist()]
    assert torch.all(out[c[4]:c[5]] == 0)                 # inactive prefill sequence
    assert torch.all(out[1] == 0)                         # inactive decode row


@pytest.mark.parametrize("n_dec,two_streams", [(0, False), (3, False), (3, True)])
def test_mixed_step_segmented_prefill(n_dec, two_streams):
    """With room for the segment states and no decode rows, the prefill part
    of a mixed step runs segment-parallel (two 1024-token sequences of 16
    chunks over 16 (sequence, value head) runs), meets the prefill bar against
    the oracle and differs from the whole-run schedule only by rounding.
    Beside decode rows it runs whole whatever the workspace and the streams,
    bitwise equal to the minimal-workspace one-stream step; the decode rows
    are bitwise those of the minimal-workspace step either way."""
    lengths = [1024, 1024]
    caches = _caches(12, seed=75)
    x, g, beta = _rows(n_dec + sum(lengths), seed=76)
    # slow decay on the prefill rows, so that a segment's start state still
    # matters at its end (with g ~ U[-1, 0] it fades by ~e^-32 over 64 tokens,
    # and both schedules give the same bits)
    g[n_dec:] *= 0.02
    slots = torch.tensor([2, 0, 7, 5, 9][3 - n_dec:], dtype=torch.int32)
    out, cs, rs = _mixed(x, g, beta, n_dec, lengths, slots, caches, segment_states=True,
                         streams=gdn.MixedStreams() if two_streams else None)
    out_w, cs_w, rs_w = _mixed(x, g, beta, n_dec, lengths, slots, caches)
    o_dec, o_pre, cs_ref, rs_ref = _oracle_mixed(x, g, beta, n_dec, lengths, slots, caches)
    assert torch.equal(out[:n_dec], out_w[:n_dec])
    assert rel_err(f64(out[n_dec:]), o_pre) <= PREFILL_TOL
    if n_dec == 0:
        assert not torch.equal(out[n_dec:], out_w[n_dec:]), "the segment-parallel schedule did not run"
    else:
        assert torch.equal(out[n_dec:], out_w[n_dec:]), "beside decode rows the prefill runs whole"
    for i, s in enumerate(slots.tolist()):
        if s <= 0:
            continue
        tol = DECODE_TOL if i < n_dec else PREFILL_TOL
        assert rel_err(f64(rs[s]), rs_ref[s]) <= tol, (i, s)
        assert np.array_equal(f64(cs[s]), cs_ref[s]), f"conv roll of slot {s}"
        if i < n_dec:
            assert torch.equal(rs[s], rs_w[s]) and torch.equal(cs[s], cs_w[s])


@pytest.mark.parametrize("path", [None, "fused", "split"])
def test_decode_rows_invariant_to_step_composition(path):
    caches = _caches(40, seed=72)
    n_dec = 6
    flags = gdn.DEFAULT_DECODE_FLAGS | {None: 0, "fused": gdn.FLAG_STEP_FUSED,
                                        "split": gdn.FLAG_STEP_SPLIT}[path]
    xd, gd, bd = _rows(n_dec, seed=73)
    dslots = torch.tensor([4, 17, 0, 23, 8, 31], dtype=torch.int32)
    results = []
    for comp, lengths, pslots in (("decode only", [], []),
                                  ("mixed A", [65, 3], [10, 11]),
                                  ("mixed B", [200, 1, 64], [12, 30, 2])):
        xp, gp, bp = _rows(sum(lengths), seed=74 + len(lengths))
        x = torch.cat([xd, xp]); g = torch.cat([gd, gp]); beta = torch.cat([bd, bp])
        slots = torch.tensor(dslots.tolist() + pslots, dtype=torch.int32)
        out, cs, rs = _mixed(x, g, beta, n_dec, lengths, slots, caches, flags=flags)
        results.append((comp, out[:n_dec].clone(), cs, rs))
    ref = results[0]
    for comp, o, cs, rs in results[1:]:
        assert torch.equal(o, ref[1]), comp
        for s in dslots.tolist():
            if s > 0:
                assert torch.equal(rs[s], ref[3][s]), (comp, s)
                assert torch.equal(cs[s], ref[2][s]), (comp, s)


@pytest.mark.parametrize("split,bitwise", [(64, True), (128, True), (100, False)])
def test_split_prefill_vs_whole(split, bitwise):
    L = 200
    caches = _caches(4, seed=75)
    x, g, beta = _rows(L, seed=76)
    slots = torch.tensor([2], dtype=torch.int32)
    out_w, cs_w, rs_w = _mixed(x, g, beta, 0, [L], slots, caches)
    # two calls on one set of caches
    cs, w, b, rs = (c.cuda() for c in caches)
    cs, rs = cs.clone(), rs.clone()
    dims = gdn.make_dims(H, HV, DK, DK, 4)
    out_s = torch.full((L, HV, DK), float("nan"), device="cuda")
    for a, e in ((0, split), (split, L)):
        o = torch.empty(e - a, HV, DK, device="cuda")
        gdn.gdn_mixed_step(x[a:e].cuda(), g[a:e].cuda(), beta[a:e].cuda(), 0,
                           gi.cu_from_lengths([e - a]).cuda(), slots.cuda(), cs, w, rs, o, dims,
                           SCALE, conv_bias=b)
        out_s[a:e] = o
    torch.cuda.synchronize()
    if bitwise:
        assert torch.equal(out_s, out_w)
        assert torch.equal(rs, rs_w)
    else:
        assert rel_err(f64(out_s), f64(out_w)) <= PREFILL_TOL
        assert rel_err(f64(rs[2]), f64(rs_w[2])) <= PREFILL_TOL
    assert torch.equal(cs, cs_w)          # the conv roll never depends on the split


def test_split_post_conv_prefill_on_grid_is_bitwise():
    """gdn_prefill_chunked alone (post-conv q, k, v): 64-aligned splits equal one call."""
    lengths = [300]
    p = to_dev(gi.prefill_inputs(lengths, 4, H=H, HV=HV, dk=DK, dv=DK, seed=77))
    dims = gdn.make_dims(H, HV, DK, DK, 4)
    rs_w = p["rec_state"].clone()
    out_w = torch.empty(300, HV, DK, dtype=torch.bfloat16, device="cuda")
    seq = gdn.FLAG_QK_L2NORM | gdn.FLAG_PREFILL_SEQUENTIAL
    gdn.gdn_prefill_chunked(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu_seqlens"],
                            p["slot_idx"], rs_w, out_w, dims, SCALE, flags=seq)
    rs_s = p["rec_state"].clone()
    out_s = torch.empty_like(out_w)
    for a, e in ((0, 64), (64, 192), (192, 300)):
        o = torch.empty(e - a, HV, DK, dtype=torch.bfloat16, device="cuda")
        gdn.gdn_prefill_chunked(p["q"][a:e].contiguous(), p["k"][a:e].contiguous(),
                                p["v"][a:e].contiguous(), p["g"][a:e].contiguous(),
                                p["beta"][a:e].contiguous(), gi.cu_from_lengths([e - a]).cuda(),
                                p["slot_idx"], rs_s, o, dims, SCALE, flags=seq)
        out_s[a:e] = o
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_w)
    assert torch.equal(rs_s, rs_w)


def test_mixed_validation_covers_both_parts():
    """A slot shared by a decode row and a prefill sequence is a repeat: the
    call fails closed (no output, no cache written)."""
    caches = _caches(8, seed=78)
    x, g, beta = _rows(3 + 10, seed=79)
    slots = torch.tensor([1, 2, 3, 2], dtype=torch.int32)     # decode slot 2 == prefill slot 2
    cs, w, b, rs = (c.cuda() for c in caches)
    cs0, rs0 = cs.clone(), rs.clone()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((13, HV, DK), float("nan"), device="cuda")
    gdn.gdn_mixed_step(x.cuda(), g.cuda(), beta.cuda(), 3, gi.cu_from_lengths([10]).cuda(),
                       slots.cuda(), cs, w, rs, out, gdn.make_dims(H, HV, DK, DK, 4), SCALE,
                       conv_bias=b, flags=gdn.DEFAULT_DECODE_FLAGS | gdn.FLAG_VALIDATE,
                       err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) & gdn.EFLAG_SLOT_REPEAT
    assert torch.isnan(out).all()
    assert torch.equal(cs, cs0) and torch.equal(rs, rs0)


def _graph_vs_eager(n_dec, lengths, streams, capture_first):
    """Capture one mixed step in a HIP graph and compare three replays with
    three consecutive eager steps, bitwise, with eager work between replays.
    capture_first: the capture is this process's first mixed step with these
    arguments (the schedule must not depend on what ran before)."""
    dims = gdn.make_dims(H, HV, DK, DK, 4)
    T = sum(lengths)
    caches = [c.cuda() for c in _caches(16, seed=77)]
    x, g, beta = (t.cuda() for t in _rows(n_dec + T, seed=78))
    g[n_dec:] *= 0.02                 # slow decay: the segment schedule differs from whole runs
    slots = torch.tensor([3, 0, 9, 12, 1, 5, 7][5 - n_dec:], dtype=torch.int32).cuda()
    cu = gi.cu_from_lengths(lengths).cuda()
    extra = gdn.gdn_prefill_workspace_size(dims, len(lengths), T)
    assert extra > 0, "these sizes should take the segment-parallel schedule"
    ws = torch.empty(gdn.gdn_mixed_workspace_size(dims, n_dec, T) + extra, dtype=torch.uint8,
                     device="cuda")

    def step(cs, rs, out):
        gdn.gdn_mixed_step(x, g, beta, n_dec, cu, slots, cs, caches[1], rs, out, dims, SCALE,
                           conv_bias=caches[2], workspace=ws, streams=streams)

    def eager():
        cs_e, rs_e = caches[0].clone(), caches[3].clone()
        ref = []
        for _ in range(3):
            o = torch.empty(n_dec + T, HV, DK, device="cuda")
            step(cs_e, rs_e, o)
            ref.append(o)
        torch.cuda.synchronize()
        return ref, cs_e, rs_e

    if not capture_first:
        ref, cs_e, rs_e = eager()
    cs_g, rs_g = caches[0].clone(), caches[3].clone()
    out = torch.empty(n_dec + T, HV, DK, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(cs_g, rs_g, out)
    torch.cuda.synchronize()
    if capture_first:
        ref, cs_e, rs_e = eager()
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[i]), f"replay {i} output"
        _ = torch.randn(1024, 1024, device="cuda").sum().item()   # eager work between
    assert torch.equal(rs_g, rs_e)
    assert torch.equal(cs_g, cs_e)
    return ref


@pytest.mark.parametrize("two_streams", [False, True])
@pytest.mark.parametrize("capture_first", [False, True])
def test_mixed_step_graph_replay_matches_eager(two_streams, capture_first):
    """A captured HIP graph of a mixed step with decode rows (varlen conv +
    roll, whole prefill runs, the decode rows; on one stream, or forked onto
    a second stream and joined back by events inside the capture) reproduces
    three consecutive eager steps bitwise on every replay, whether the capture
    or the eager steps come first: every call only enqueues work, and the
    schedule depends on the arguments alone."""
    _graph_vs_eager(5, [700, 1300], gdn.MixedStreams() if two_streams else None, capture_first)


def test_mixed_step_graph_replay_segmented():
    """The same for a step without decode rows on the segment-parallel
    schedule (both segment passes and the scan in the graph); the outputs
    differ from the whole-run schedule by rounding, which shows the schedule
    that was captured."""
    ref = _graph_vs_eager(0, [1024, 1024], None, capture_first=True)
    lengths = [1024, 1024]
    x, g, beta = _rows(sum(lengths), seed=78)
    g *= 0.02
    slots = torch.tensor([3, 0, 9, 12, 1, 5, 7][5:], dtype=torch.int32)
    caches = _caches(16, seed=77)
    out_w, _, _ = _mixed(x, g, beta, 0, lengths, slots, caches)
    assert not torch.equal(ref[0], out_w), "the segment-parallel schedule was not captured"
