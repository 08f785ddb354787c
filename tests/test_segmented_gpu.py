"""GPU parity of the segment-parallel prefill (gdn_prefill_segmented, and the
segments gdn_prefill_chunked picks by itself for few long sequences) against
the fp64 token-by-token oracle, through the C ABI.

Bar: output and final state at max|err| / max|ref| <= 5e-3, the prefill bar.
The schedule is a different rounding of the same arithmetic as whole-sequence
runs, so it is compared with the oracle (and with whole-sequence runs at the
same bar), not bitwise -- except where every sequence fits in one segment,
where the first pass is the whole-sequence run and the results are bitwise
equal.  Cases: segment lengths of one to three chunks over ragged lengths
(segment ends on and off the sequence end, one to six segments, so the scan
runs zero to four steps), fp32 and bf16 inputs, inactive and empty
sequences, fused gating, the 64-head-dim and 128-head-dim kernels, the
correlated-key stress sequence of 16384 tokens on both schedules, fail-closed
validation and run-to-run reproducibility.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_recurrent_gdn_amd as gdn
import oracle
from gpu_helpers import PREFILL_TOL, f64, fnv64, rel_err, to_dev
from test_prefill_gpu import check_heads

pytestmark = pytest.mark.gpu

SEQ = gdn.FLAG_QK_L2NORM | gdn.FLAG_PREFILL_SEQUENTIAL


def _dims(p):
    dm = p["dims"]
    return gdn.make_dims(dm["H"], dm["HV"], dm["dk"], dm["dv"], 4)


def run_segmented(g, scale, seg_len, out_dtype=torch.bfloat16, flags=gdn.FLAG_QK_L2NORM,
                  err_flag=None, gate=None, head_len=0):
    dm = g["dims"]
    T = g["q"].shape[0]
    out = torch.full((T, dm["HV"], dm["dv"]), float("nan"), dtype=out_dtype, device="cuda")
    gdn.gdn_prefill_segmented(g["q"], g["k"], g["v"], None if gate else g["g"],
                              None if gate else g["beta"], g["cu_seqlens"], g["slot_idx"],
                              g["rec_state"], out, _dims(g), scale, seg_len, flags=flags,
                              gate=gate, err_flag=err_flag, head_len=head_len)
    return out


def run_whole(g, scale, out_dtype=torch.bfloat16):
    dm = g["dims"]
    T = g["q"].shape[0]
    out = torch.full((T, dm["HV"], dm["dv"]), float("nan"), dtype=out_dtype, device="cuda")
    gdn.gdn_prefill_chunked(g["q"], g["k"], g["v"], g["g"], g["beta"], g["cu_seqlens"],
                            g["slot_idx"], g["rec_state"], out, _dims(g), scale, flags=SEQ)
    return out


LENGTHS = [1, 63, 64, 65, 128, 129, 200, 333, 0, 384]


@pytest.mark.parametrize("seg_len", [64, 128, 192])
@pytest.mark.parametrize("d,in_dtype", [(32, torch.float32), (32, torch.bfloat16),
                                         (64, torch.bfloat16)])
def test_segmented_matches_oracle(seg_len, d, in_dtype):
    p = gi.prefill_inputs(LENGTHS, 16, H=2, HV=4, dk=d, dv=d, seed=21, state_std=0.1,
                          in_dtype=in_dtype, g_mode="softplus")
    g = to_dev(p)
    out = run_segmented(g, d ** -0.5, seg_len, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    eo, es = check_heads(p, g, out, list(range(4)), d ** -0.5)
    print(f"segmented seg={seg_len} d={d} in={in_dtype}: out {eo:.2e} state {es:.2e}")


@pytest.mark.parametrize("seg_len,head_len", [(64, 128), (64, 192), (128, 256), (64, 384)])
def test_head_and_tail_segments_match_oracle(seg_len, head_len):
    """Segment 0 longer than the rest: sequences no longer than the head run
    whole, longer ones get tail segments (zero to five of them here, so the
    scan runs zero to three steps).  A slow decay keeps each segment's start
    state visible at its end, so the composition matters."""
    p = gi.prefill_inputs(LENGTHS, 16, H=2, HV=4, dk=64, dv=64, seed=23, state_std=0.1,
                          g_mode="softplus")
    p["g"] *= 0.02
    g = to_dev(p)
    out = run_segmented(g, 64 ** -0.5, seg_len, out_dtype=torch.float32, head_len=head_len)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    eo, es = check_heads(p, g, out, list(range(4)), 64 ** -0.5)
    print(f"head {head_len} seg {seg_len}: out {eo:.2e} state {es:.2e}")


def test_head_covering_every_sequence_is_the_whole_run_bitwise():
    """With every sequence no longer than the head, each is one segment: the
    first pass is the whole-sequence run, bitwise."""
    p = gi.prefill_inputs(LENGTHS, 16, H=2, HV=4, dk=64, dv=64, seed=24, g_mode="softplus")
    ga, gb = to_dev(p), to_dev(p)
    oa = run_segmented(ga, 0.125, 64, head_len=384)
    ob = run_whole(gb, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    assert torch.equal(ga["rec_state"], gb["rec_state"])


def test_busy_chip_tail_schedule_matches_oracle():
    """The plain call's own schedule on a busy chip (8 sequences x 32 value
    heads, skewed lengths, its workspace given): a head of the balanced
    per-unit chunk count, tails of the longer sequences in parallel.  Against
    the oracle on sampled heads with a slow decay (so the tails' composed start
    states matter), and within the bar of whole-sequence runs."""
    lengths = [1800, 200, 1700, 150, 2300, 100, 1300, 2200]
    p = gi.prefill_inputs(lengths, 10, seed=25)
    p["g"] *= 0.02
    dims = gdn.make_dims(16, 32, 128, 128, 4)
    T = sum(lengths)
    ws_bytes = gdn.gdn_prefill_workspace_size(dims, len(lengths), T)
    if ws_bytes == 0:
        pytest.skip("this device runs the workload whole (fewer than 512 CUs busy is assumed)")
    ga, gb = to_dev(p), to_dev(p)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    oa = torch.full((T, 32, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_prefill_chunked(ga["q"], ga["k"], ga["v"], ga["g"], ga["beta"], ga["cu_seqlens"],
                            ga["slot_idx"], ga["rec_state"], oa, dims, 128 ** -0.5,
                            flags=gdn.FLAG_QK_L2NORM, workspace=ws)
    ob = run_whole(gb, 128 ** -0.5)
    torch.cuda.synchronize()
    assert torch.isfinite(oa).all()
    assert not torch.equal(oa, ob), "the tail schedule did not run"
    assert rel_err(f64(oa), f64(ob)) <= PREFILL_TOL
    eo, es = check_heads(p, ga, oa, [0, 19, 31], 128 ** -0.5)
    print(f"busy-chip tail schedule: out {eo:.2e} state {es:.2e}")


def test_segmented_d128_matches_oracle_and_whole_runs():
    lengths = [700, 130, 1000]
    p = gi.prefill_inputs(lengths, 8, seed=22)
    ga, gb = to_dev(p), to_dev(p)
    for seg in (128, 256):
        ga = to_dev(p)
        out_s = run_segmented(ga, 128 ** -0.5, seg)
        gb = to_dev(p)
        out_w = run_whole(gb, 128 ** -0.5)
        torch.cuda.synchronize()
        assert rel_err(f64(out_s), f64(out_w)) <= PREFILL_TOL
        assert rel_err(f64(ga["rec_state"]), f64(gb["rec_state"])) <= PREFILL_TOL
        eo, es = check_heads(p, ga, out_s, [0, 9, 31], 128 ** -0.5)
        print(f"d=128 seg={seg}: out {eo:.2e} state {es:.2e}")


def test_one_segment_per_sequence_is_the_whole_run_bitwise():
    p = gi.prefill_inputs([300, 64, 17], 8, H=2, HV=4, dk=64, dv=64, seed=23)
    ga, gb = to_dev(p), to_dev(p)
    out_s = run_segmented(ga, 0.125, 320)
    out_w = run_whole(gb, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_w)
    assert torch.equal(ga["rec_state"], gb["rec_state"])


def test_segmented_inactive_and_empty():
    p = gi.prefill_inputs([140, 0, 270, 33], 8, H=2, HV=4, dk=64, dv=64, seed=24)
    p["slot_idx"][2] = 0                    # inactive sequence of 270 tokens
    g = to_dev(p)
    before = g["rec_state"].clone()
    out = run_segmented(g, 0.125, 64)
    torch.cuda.synchronize()
    cu = p["cu_seqlens"].tolist()
    assert torch.all(out[cu[2]:cu[3]] == 0)
    untouched = [s for s in range(8) if s not in (int(p["slot_idx"][0]), int(p["slot_idx"][3]))]
    assert torch.equal(before[untouched], g["rec_state"][untouched])
    check_heads(p, g, out, list(range(4)), 0.125)


def test_segmented_gated_matches_oracle():
    lengths = [260, 77, 400]
    p = gi.prefill_inputs(lengths, 8, H=2, HV=4, dk=64, dv=64, seed=25)
    T = sum(lengths)
    gt = gi.gating_inputs(T, 4, seed=26)
    g_ref, b_ref = oracle.gating(gt["a"].double().numpy(), gt["b"].double().numpy(),
                                 gt["A_log"].double().numpy(), gt["dt_bias"].double().numpy())
    p_ref = dict(p)
    p_ref["g"] = torch.from_numpy(g_ref)
    p_ref["beta"] = torch.from_numpy(b_ref)
    g = to_dev(p)
    gd = {k: v.cuda() for k, v in gt.items()}
    gate = gdn.GateInputs(gd["a"], gd["b"], gd["A_log"], gd["dt_bias"])
    out = run_segmented(g, 0.125, 128, out_dtype=torch.float32, gate=gate)
    torch.cuda.synchronize()
    check_heads(p_ref, g, out, list(range(4)), 0.125)


@pytest.mark.parametrize("schedule", ["auto", "sequential"])
def test_stress_16384_both_schedules(schedule):
    p = gi.stress_prefill_inputs(16384)
    g = to_dev(p)
    dims = _dims(p)
    if schedule == "auto":
        assert gdn.gdn_prefill_workspace_size(dims, 1, 16384) > 0
    out = torch.empty(16384, 32, 128, dtype=torch.bfloat16, device="cuda")
    gdn.gdn_prefill_chunked(g["q"], g["k"], g["v"], g["g"], g["beta"], g["cu_seqlens"],
                            g["slot_idx"], g["rec_state"], out, dims, 128 ** -0.5,
                            flags=gdn.FLAG_QK_L2NORM if schedule == "auto" else SEQ)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(g["rec_state"]).all()
    eo, es = check_heads(p, g, out, [3, 22], 128 ** -0.5)
    print(f"stress 16384 {schedule}: out {eo:.2e} state {es:.2e}")


@pytest.mark.parametrize("bad", ["range", "repeat", "seqlens"])
def test_segmented_validation_fails_closed(bad):
    p = gi.prefill_inputs([140, 150, 260], 8, H=2, HV=4, dk=64, dv=64, seed=27)
    p["rec_state"] = torch.cat([p["rec_state"], torch.randn(1, 4, 64, 64)])
    if bad == "range":
        p["slot_idx"][1] = 8
    elif bad == "repeat":
        p["slot_idx"][2] = p["slot_idx"][0]
    else:
        p["cu_seqlens"][1] = 295            # offsets 0, 295, 290, 550: decreasing
    g = to_dev(p)
    full = g["rec_state"]
    g["rec_state"] = full[:8]
    before = full.clone()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = run_segmented(g, 0.125, 64, flags=gdn.FLAG_QK_L2NORM | gdn.FLAG_VALIDATE, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) != 0
    assert torch.isnan(out.float()).all()
    assert torch.equal(before, full)


def test_segmented_reproducible():
    p = gi.prefill_inputs([900, 500], 8, seed=28)
    hashes = set()
    for _ in range(2):
        g = to_dev(p)
        out = run_segmented(g, 128 ** -0.5, 128)
        torch.cuda.synchronize()
        hashes.add((fnv64(out), fnv64(g["rec_state"])))
    assert len(hashes) == 1
