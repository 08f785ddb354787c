"""GPU state contract, batch invariance and replay of the decode step.

* Slot contract (RL-Kernel PR #469, "State ABI: index validation and the two
  NULL_BLOCK_ID contracts"): rows with slot <= 0 produce zeros and touch no
  cache; slot 0 and every non-addressed slot stay byte-identical; with
  validation on, an out-of-range or repeated active slot sets err_flag and
  the call writes nothing at all (fail closed).
* Batch invariance (RL-Kernel PR #469, "L1, and the bf16 recurrent state";
  RL-Kernel PR #485, "Prior art & reuse decision"): every row computed alone
  equals, bitwise, the same row inside shuffled batches of 2, 7, 64 and 257,
  over three seeds; a deliberately batch-dependent result must fail the same
  check (negative control).
* Replay ("A reduction barrier makes Qwen GDN graph replay bit exact"):
  restoring the caches and rerunning reproduces the hashes of the output, the
  conv cache and the recurrent cache.
"""
import math

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_recurrent_gdn_amd as gdn
from gpu_helpers import fnv64, run_decode_gpu, to_dev

pytestmark = pytest.mark.gpu

SCALE = 128 ** -0.5


def _clone(d):
    return {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


@pytest.mark.parametrize("path", ["fused", "split"])
def test_null_slots_untouched(path):
    d = to_dev(gi.decode_inputs(16, 64, seed=9))
    d["slot_idx"][3] = 0
    d["slot_idx"][7] = -5
    d["slot_idx"][11] = 0
    before_rs, before_cs = d["rec_state"].clone(), d["conv_state"].clone()
    out = run_decode_gpu(d, SCALE, path=path)
    torch.cuda.synchronize()
    for r in (3, 7, 11):
        assert torch.all(out[r] == 0)
    used = [s for s in d["slot_idx"].tolist() if s > 0]
    mask = torch.ones(64, dtype=torch.bool, device="cuda")
    mask[used] = False
    assert torch.equal(before_rs[mask], d["rec_state"][mask])
    assert torch.equal(before_cs[mask], d["conv_state"][mask])
    assert torch.equal(before_rs[0], d["rec_state"][0])


@pytest.mark.parametrize("path", ["fused", "split"])
@pytest.mark.parametrize("bad,bit", [("range", gdn.EFLAG_SLOT_RANGE),
                                     ("repeat", gdn.EFLAG_SLOT_REPEAT)])
def test_validation_fails_closed(bad, bit, path):
    # 33 slots of memory, 32 exposed: slot 32 is out of range for the call but
    # still allocated, so a missed check could not fault
    d = gi.decode_inputs(9, 32, seed=10)
    d["rec_state"] = torch.cat([d["rec_state"], torch.randn(1, *d["rec_state"].shape[1:])])
    d["conv_state"] = torch.cat([d["conv_state"], d["conv_state"][:1]])
    d = to_dev(d)
    full = {k: d[k] for k in ("rec_state", "conv_state")}
    for k in full:
        d[k] = full[k][:32]
    if bad == "range":
        d["slot_idx"][4] = 32
    else:
        d["slot_idx"][6] = d["slot_idx"][2]
    before = {k: v.clone() for k, v in full.items()}
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = run_decode_gpu(d, SCALE, flags=gdn.DEFAULT_DECODE_FLAGS | gdn.FLAG_VALIDATE,
                         err_flag=err, path=path)
    torch.cuda.synchronize()
    assert int(err.item()) & bit
    assert torch.isnan(out).all(), "a rejected call must not write the output"
    for k, v in before.items():
        assert torch.equal(v, full[k]), f"{k} mutated by a rejected call"


def test_validation_clean_call_writes_zero():
    d = to_dev(gi.decode_inputs(9, 32, seed=10))
    d["slot_idx"][0] = 0
    d["slot_idx"][1] = 0           # repeated null slot is fine
    err = torch.full((1,), 123, dtype=torch.int32, device="cuda")
    run_decode_gpu(d, SCALE, flags=gdn.DEFAULT_DECODE_FLAGS | gdn.FLAG_VALIDATE, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0


def _rows_alone(base, rows):
    """Run each row alone (a batch of one) from the original caches; returns
    dict row -> (o, rec slab, conv slab)."""
    res = {}
    d = _clone(base)           # rows use distinct slots: one copy serves them all
    for r in rows:
        for k in ("mixed_qkv", "g", "beta", "slot_idx"):
            d[k] = base[k][r:r + 1].clone()
        o = run_decode_gpu(d, SCALE)
        s = int(base["slot_idx"][r])
        res[r] = (o[0].clone(), d["rec_state"][s].clone(), d["conv_state"][s].clone())
    return res


def _run_batch(base, rows):
    d = _clone(base)
    idx = torch.tensor(rows, device="cuda")
    for k in ("mixed_qkv", "g", "beta", "slot_idx"):
        d[k] = base[k][idx].contiguous()
    o = run_decode_gpu(d, SCALE)
    return o, d


def _invariance_mismatches(alone, rows, o, d, perturb=None):
    bad = 0
    for i, r in enumerate(rows):
        oa, ra, ca = alone[r]
        s = int(d["slot_idx"][i])
        ob = o[i] if perturb is None else perturb(o[i], len(rows))
        bad += int(not torch.equal(oa, ob))
        bad += int(not torch.equal(ra, d["rec_state"][s]))
        bad += int(not torch.equal(ca, d["conv_state"][s]))
    return bad


@pytest.mark.parametrize("seed", [2, 3, 4])
def test_batch_invariance(seed):
    base = to_dev(gi.decode_inputs(257, 300, seed=seed))
    rng = np.random.default_rng(seed)
    alone = _rows_alone(base, list(range(257)))
    for n in (2, 7, 64, 257):
        rows = rng.permutation(257)[:n].tolist()
        o, d = _run_batch(base, rows)
        torch.cuda.synchronize()
        assert _invariance_mismatches(alone, rows, o, d) == 0, (seed, n)


def test_batch_invariance_negative_control():
    """A result that depends on the batch size (a rounding-sized nudge scaled by
    the batch) must be flagged by the same comparison."""
    base = to_dev(gi.decode_inputs(64, 80, seed=3))
    rows = list(range(64))
    alone = _rows_alone(base, rows[:8])
    o, d = _run_batch(base, rows[:8])
    torch.cuda.synchronize()
    assert _invariance_mismatches(alone, rows[:8], o, d) == 0
    nudge = lambda t, n: t * (1 + 2 ** -23 * (n > 1))  # noqa: E731
    assert _invariance_mismatches(alone, rows[:8], o, d, perturb=nudge) > 0


def test_replay_hashes():
    base = to_dev(gi.decode_inputs(16, 40, seed=12))
    hashes = set()
    for _ in range(3):
        d = _clone(base)
        o = run_decode_gpu(d, SCALE)
        torch.cuda.synchronize()
        hashes.add((fnv64(o), fnv64(d["conv_state"]), fnv64(d["rec_state"])))
    assert len(hashes) == 1


def test_replay_under_concurrent_load():
    """Replays stay bitwise identical while another stream keeps the GPU busy
    (a race that depends on scheduling would show up here)."""
    base = to_dev(gi.decode_inputs(64, 80, seed=13))
    ref = None
    side = torch.cuda.Stream()
    big = torch.randn(4096, 4096, device="cuda")
    for i in range(3):
        with torch.cuda.stream(side):
            for _ in range(4):
                big = big @ big.T * 1e-3
        d = _clone(base)
        o = run_decode_gpu(d, SCALE)
        torch.cuda.synchronize()
        h = (fnv64(o), fnv64(d["conv_state"]), fnv64(d["rec_state"]))
        ref = ref or h
        assert h == ref, i


def test_graph_replay_matches_eager():
    """A captured HIP graph of the decode step reproduces the eager results on
    every replay, with eager work and synchronisations between replays (the
    step enqueues kernels only: no allocation, no memset)."""
    base = to_dev(gi.decode_inputs(32, 48, seed=14))
    dims = gdn.make_dims(16, 32, 128, 128, 4)
    ws = torch.empty(gdn.gdn_decode_workspace_size(dims, 32), dtype=torch.uint8, device="cuda")
    # eager reference: three consecutive steps from the base caches
    ref = _clone(base)
    ref_out = []
    for _ in range(3):
        o = torch.empty(32, 32, 128, device="cuda")
        gdn.gdn_decode_step(ref["mixed_qkv"], ref["g"], ref["beta"], ref["slot_idx"],
                            ref["conv_state"], ref["conv_weight"], ref["rec_state"], o, dims,
                            SCALE, workspace=ws)
        ref_out.append(o)
    torch.cuda.synchronize()
    # graph of one step over live buffers, replayed three times
    live = _clone(base)
    out = torch.empty(32, 32, 128, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.gdn_decode_step(live["mixed_qkv"], live["g"], live["beta"], live["slot_idx"],
                            live["conv_state"], live["conv_weight"], live["rec_state"], out,
                            dims, SCALE, workspace=ws)
    torch.cuda.synchronize()
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out[i]), f"replay {i} output"
        _ = torch.randn(1024, 1024, device="cuda").sum().item()   # eager work between
    assert torch.equal(live["rec_state"], ref["rec_state"])
    assert torch.equal(live["conv_state"], ref["conv_state"])
