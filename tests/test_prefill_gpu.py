"""GPU parity of the chunked prefill against the fp64 token-by-token oracle.

Bar: output and final state at max|err| / max|ref| <= 5e-3.  Cases: ragged
lengths around the 16- and 64-token boundaries with random initial states;
the 8-sequence varlen workload (lengths uniform in [512, 8192], H=16, HV=32,
d=128) and the correlated-key stress case (k_t = normalise(base + 0.05 N),
beta = 0.9, g = 0, zero state; vLLM PR #53864, "Test Plan") at 64 and 16384
tokens, both checked against the oracle on sampled value heads (each head's
recurrence is independent) with every output checked finite; inactive and
empty sequences; fail-closed validation; bitwise run-to-run reproducibility.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_recurrent_gdn_amd as gdn
import oracle
from gpu_helpers import PREFILL_TOL, f64, fnv64, rel_err, to_dev

pytestmark = pytest.mark.gpu


def run_prefill_gpu(p, scale, out_dtype=torch.bfloat16, flags=gdn.FLAG_QK_L2NORM,
                    err_flag=None):
    dm = p["dims"]
    dims = gdn.make_dims(dm["H"], dm["HV"], dm["dk"], dm["dv"], 4)
    T = p["q"].shape[0]
    out = torch.full((T, dm["HV"], dm["dv"]), float("nan"), dtype=out_dtype, device="cuda")
    gdn.gdn_prefill_chunked(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu_seqlens"],
                            p["slot_idx"], p["rec_state"], out, dims, scale, flags=flags,
                            err_flag=err_flag)
    return out


def oracle_heads(p_cpu, heads, scale, flags=oracle.FLAG_QK_L2NORM):
    """Oracle on a subset of value heads, each as a one-head problem with its key
    head (hv // (HV / H)); returns o [T, len(heads), dv] and final states
    [n_seqs, len(heads), dv, dk] in the order of slot_idx."""
    dm = p_cpu["dims"]
    grp = dm["HV"] // dm["H"]
    slots = p_cpu["slot_idx"].numpy()
    n = len(slots)
    outs, states = [], []
    for hv in heads:
        h = hv // grp
        rec = np.zeros((n + 1, 1, dm["dv"], dm["dk"]))
        comp = np.where(slots > 0, np.arange(1, n + 1), slots).astype(np.int32)
        for i, s in enumerate(slots):
            if s > 0:
                rec[i + 1, 0] = f64(p_cpu["rec_state"][s, hv])
        o = oracle.prefill(f64(p_cpu["q"][:, h:h + 1]), f64(p_cpu["k"][:, h:h + 1]),
                           f64(p_cpu["v"][:, hv:hv + 1]), f64(p_cpu["g"][:, hv:hv + 1]),
                           f64(p_cpu["beta"][:, hv:hv + 1]), p_cpu["cu_seqlens"].numpy(), comp,
                           rec, scale, flags=flags)
        outs.append(o[:, 0])
        states.append(rec[1:, 0])
    return np.stack(outs, 1), np.stack(states, 1)


def check_heads(p_cpu, p_gpu, out, heads, scale, tol=PREFILL_TOL, flags=oracle.FLAG_QK_L2NORM):
    o_ref, s_ref = oracle_heads(p_cpu, heads, scale, flags=flags)
    o = f64(out[:, heads])
    eo = rel_err(o, o_ref)
    slots = p_cpu["slot_idx"].tolist()
    act = [i for i, s in enumerate(slots) if s > 0]
    sg = np.stack([f64(p_gpu["rec_state"][slots[i]][heads]) for i in act]) if act else None
    es = rel_err(sg, s_ref[act]) if act else 0.0
    assert eo <= tol, f"output rel err {eo:.3e}"
    assert es <= tol, f"state rel err {es:.3e}"
    return eo, es


@pytest.mark.parametrize("d,in_dtype", [(32, torch.bfloat16), (32, torch.float32),
                                         (64, torch.bfloat16), (64, torch.float32),
                                         (128, torch.bfloat16)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_prefill_ragged(d, in_dtype, out_dtype):
    lengths = [1, 15, 16, 17, 63, 64, 65, 130, 200]
    p = gi.prefill_inputs(lengths, 12, H=2, HV=4, dk=d, dv=d, seed=5, state_std=0.1,
                          in_dtype=in_dtype)
    g = to_dev(p)
    out = run_prefill_gpu(g, d ** -0.5, out_dtype=out_dtype)
    torch.cuda.synchronize()
    eo, es = check_heads(p, g, out, list(range(4)), d ** -0.5)
    print(f"ragged d={d} in={in_dtype} out={out_dtype}: out {eo:.2e} state {es:.2e}")
    if out_dtype == torch.float32 and in_dtype == torch.float32:
        # fp32 inputs ride as hi/lo bf16 pairs: far inside the bar
        assert eo <= 1e-3 and es <= 1e-3


def test_prefill_norm_flag_off():
    p = gi.prefill_inputs([70, 64, 5], 6, H=2, HV=4, dk=128, dv=128, seed=6,
                          qk_normalised=True)
    g = to_dev(p)
    out = run_prefill_gpu(g, 128 ** -0.5, out_dtype=torch.float32, flags=0)
    torch.cuda.synchronize()
    check_heads(p, g, out, list(range(4)), 128 ** -0.5, flags=0)


@pytest.fixture(scope="module")
def varlen_workload():
    gen = torch.Generator().manual_seed(3)
    lengths = gi.seqlens_uniform(8, 512, 8192, gen)
    return gi.prefill_inputs(lengths, 16, seed=3)


def test_prefill_varlen_full_size(varlen_workload):
    p = varlen_workload
    g = to_dev(p)
    out = run_prefill_gpu(g, 128 ** -0.5)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    eo, es = check_heads(p, g, out, [0, 13, 31], 128 ** -0.5)
    print(f"varlen T={p['q'].shape[0]}: out {eo:.2e} state {es:.2e}")


@pytest.mark.parametrize("n_seqs", [1, 5, 257])
def test_prefill_many_sequences(n_seqs):
    """vLLM PR #53864, "Test Plan": num_seqs 1, 5 and 257 at the Qwen3-Next-like
    heads (H=16, HV=32, d=128) with short ragged lengths, one sequence inactive
    when there are several; 257 sequences are 8224 workgroups, many rounds of
    the 256 CUs.  Sampled value heads against the oracle, every output and
    state finite, the inactive sequence's rows zero and its slot untouched."""
    gen = torch.Generator().manual_seed(100 + n_seqs)
    lengths = [97] if n_seqs == 1 else gi.seqlens_uniform(n_seqs, 1, 160, gen)
    p = gi.prefill_inputs(lengths, n_seqs + 1, seed=200 + n_seqs)
    dead = None
    if n_seqs > 1:
        dead = n_seqs // 2
        p["slot_idx"][dead] = 0
    g = to_dev(p)
    before = g["rec_state"].clone()
    out = run_prefill_gpu(g, 128 ** -0.5)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.isfinite(g["rec_state"]).all()
    if dead is not None:
        cu = p["cu_seqlens"].tolist()
        assert torch.all(out[cu[dead]:cu[dead + 1]] == 0)
        used = set(p["slot_idx"].tolist())
        free = [s for s in range(n_seqs + 1) if s not in used]
        assert torch.equal(before[free], g["rec_state"][free])
    eo, es = check_heads(p, g, out, [0, 21, 31], 128 ** -0.5)
    print(f"{n_seqs} sequences, T={sum(lengths)}: out {eo:.2e} state {es:.2e}")


@pytest.mark.parametrize("T,heads", [(64, list(range(32))), (16384, [0, 17, 30])])
def test_prefill_correlated_keys(T, heads):
    p = gi.stress_prefill_inputs(T)
    g = to_dev(p)
    out = run_prefill_gpu(g, 128 ** -0.5)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.isfinite(g["rec_state"]).all()
    eo, es = check_heads(p, g, out, heads, 128 ** -0.5)
    print(f"stress T={T}: out {eo:.2e} state {es:.2e}")


def test_prefill_inactive_and_empty():
    p = gi.prefill_inputs([40, 0, 70, 33], 8, H=2, HV=4, dk=64, dv=64, seed=8)
    p["slot_idx"][2] = 0                    # inactive sequence of 70 tokens
    g = to_dev(p)
    before = g["rec_state"].clone()
    out = run_prefill_gpu(g, 0.125)
    torch.cuda.synchronize()
    cu = p["cu_seqlens"].tolist()
    assert torch.all(out[cu[2]:cu[3]] == 0)
    untouched = [s for s in range(8) if s not in (int(p["slot_idx"][0]), int(p["slot_idx"][3]))]
    assert torch.equal(before[untouched], g["rec_state"][untouched])
    check_heads(p, g, out, list(range(4)), 0.125)


@pytest.mark.parametrize("bad", ["range", "repeat", "seqlens"])
def test_prefill_validation_fails_closed(bad):
    # 9 slots of memory, 8 exposed: an index of 8 is out of range for the call
    # but still lands in allocated memory, so a missed check cannot fault
    p = gi.prefill_inputs([40, 50, 60], 8, H=2, HV=4, dk=64, dv=64, seed=9)
    p["rec_state"] = torch.cat([p["rec_state"], torch.randn(1, 4, 64, 64)])
    if bad == "range":
        p["slot_idx"][1] = 8
    elif bad == "repeat":
        p["slot_idx"][2] = p["slot_idx"][0]
    else:
        p["cu_seqlens"][1] = 95             # offsets 0, 95, 90, 150: decreasing
    g = to_dev(p)
    full = g["rec_state"]
    g["rec_state"] = full[:8]
    before = full.clone()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = run_prefill_gpu(g, 0.125, flags=gdn.FLAG_QK_L2NORM | gdn.FLAG_VALIDATE, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) != 0
    assert torch.isnan(out.float()).all()
    assert torch.equal(before, full)


def test_prefill_reproducible(varlen_workload):
    p = varlen_workload
    hashes = set()
    for _ in range(2):
        g = to_dev(p)
        out = run_prefill_gpu(g, 128 ** -0.5)
        torch.cuda.synchronize()
        hashes.add((fnv64(out), fnv64(g["rec_state"])))
    assert len(hashes) == 1


def test_prefill_then_decode_continues_state():
    """Prefill of T tokens followed by a decode token equals the oracle run of
    T + 1 tokens (the caches are the resume mechanism)."""
    d = 128
    p = gi.prefill_inputs([97, 130], 6, H=2, HV=4, dk=d, dv=d, seed=10)
    g = to_dev(p)
    run_prefill_gpu(g, d ** -0.5, out_dtype=torch.float32)
    # one more token per sequence through the recurrent half of the decode step
    gen = torch.Generator().manual_seed(11)
    D = 2 * 2 * d + 4 * d
    qkv = torch.randn(2, D, generator=gen)
    gg = -torch.rand(2, 4, generator=gen)
    bb = torch.sigmoid(torch.randn(2, 4, generator=gen))
    dims = gdn.make_dims(2, 4, d, d, 4)
    o = torch.empty(2, 4, d, device="cuda")
    gdn.gdn_decode_recurrent(qkv.cuda(), gg.cuda(), bb.cuda(), g["slot_idx"], g["rec_state"], o,
                             dims, d ** -0.5)
    torch.cuda.synchronize()
    # oracle: prefill, then one decode-recurrent token via a one-token prefill
    rec = f64(p["rec_state"]).copy()
    oracle.prefill(f64(p["q"]), f64(p["k"]), f64(p["v"]), f64(p["g"]), f64(p["beta"]),
                   p["cu_seqlens"].numpy(), p["slot_idx"].numpy(), rec, d ** -0.5)
    x = qkv.double().numpy()
    o_ref = oracle.prefill(x[:, :2 * d].reshape(2, 2, d), x[:, 2 * d:4 * d].reshape(2, 2, d),
                           x[:, 4 * d:].reshape(2, 4, d), gg.double().numpy(),
                           bb.double().numpy(), [0, 1, 2], p["slot_idx"].numpy(), rec, d ** -0.5)
    assert rel_err(f64(o), o_ref) <= PREFILL_TOL
    act = p["slot_idx"].tolist()
    assert rel_err(f64(g["rec_state"][act]), rec[act]) <= PREFILL_TOL


# ---------------------------------------------------------------------------
# Newton-Schulz A/B variant (vLLM PR #53864, "Numerical root cause and fix"):
# inverting the 16x16 diagonal KK^T blocks by three bf16 Newton-Schulz rounds
# fails on highly correlated keys, four rounds repair it to the bf16-inverse
# level; the default exact fp32 forward substitution stays well inside 5e-3.
def _run_flags(p, extra):
    g = to_dev(p)
    return g, run_prefill_gpu(g, 128 ** -0.5, flags=gdn.FLAG_QK_L2NORM | extra)


def _errs(p, g, out, heads):
    o_ref, s_ref = oracle_heads(p, heads, 128 ** -0.5)
    slots = p["slot_idx"].tolist()
    sg = np.stack([f64(g["rec_state"][s][heads]) for s in slots])
    return rel_err(f64(out[:, heads]), o_ref), rel_err(sg, s_ref)


def test_newton_schulz_three_rounds_fail_on_correlated_keys():
    p = gi.stress_prefill_inputs(64)
    heads = [0, 1, 17, 31]
    g3, o3 = _run_flags(p, gdn.FLAG_PREFILL_NS3)
    g4, o4 = _run_flags(p, gdn.FLAG_PREFILL_NS4)
    gf, of = _run_flags(p, 0)
    torch.cuda.synchronize()
    e3 = _errs(p, g3, o3, heads)
    e4 = _errs(p, g4, o4, heads)
    ef = _errs(p, gf, of, heads)
    print(f"\nNS3 {e3[0]:.2e}/{e3[1]:.2e}  NS4 {e4[0]:.2e}/{e4[1]:.2e}  fwd {ef[0]:.2e}/{ef[1]:.2e}")
    assert not (e3[0] < 1.0), "three bf16 rounds should fail on correlated keys"
    assert e4[0] < 1e-2 and e4[1] < 1e-2, "four rounds should repair it"
    assert ef[0] <= PREFILL_TOL and ef[1] <= PREFILL_TOL
    assert ef[1] < e4[1] / 10, "exact substitution keeps the state far closer than NS4"


def test_newton_schulz_variants_agree_on_random_keys():
    p = gi.prefill_inputs([64, 130, 300], 6, seed=9)
    for fl in (gdn.FLAG_PREFILL_NS3, gdn.FLAG_PREFILL_NS4):
        g, out = _run_flags(p, fl)
        torch.cuda.synchronize()
        eo, es = _errs(p, g, out, [0, 9, 31])
        assert eo <= PREFILL_TOL and es <= PREFILL_TOL, (fl, eo, es)


# ---------------------------------------------------------------------------
# At dk = dv = 128 with bf16 inputs the chunk step runs on the two-role kernel
# (state waves and coefficient waves); GDN_FLAG_PREFILL_SINGLE_ROLE runs it on
# the single-role kernel.  Both take the same arithmetic in the same order, so
# every output and state must match bit for bit, on every schedule.
def _ab_call(p, flags, out_dtype=torch.bfloat16, gate=None, ws=None, seg=None):
    g = to_dev(p)
    dm = p["dims"]
    dims = gdn.make_dims(dm["H"], dm["HV"], dm["dk"], dm["dv"], 4)
    T = p["q"].shape[0]
    out = torch.full((T, dm["HV"], dm["dv"]), float("nan"), dtype=out_dtype, device="cuda")
    if seg is not None:
        seg_len, head_len = seg
        wsb = gdn.gdn_prefill_segmented_workspace_size(dims, len(p["slot_idx"]), T, seg_len)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        gdn.gdn_prefill_segmented(g["q"], g["k"], g["v"], None if gate else g["g"],
                                  None if gate else g["beta"], g["cu_seqlens"], g["slot_idx"],
                                  g["rec_state"], out, dims, 128 ** -0.5, seg_len, flags=flags,
                                  gate=gate, workspace=ws, head_len=head_len)
    elif gate is not None:
        gdn.gdn_prefill_chunked_gated(g["q"], g["k"], g["v"], gate, g["cu_seqlens"],
                                      g["slot_idx"], g["rec_state"], out, dims, 128 ** -0.5,
                                      flags=flags, workspace=ws)
    else:
        gdn.gdn_prefill_chunked(g["q"], g["k"], g["v"], g["g"], g["beta"], g["cu_seqlens"],
                                g["slot_idx"], g["rec_state"], out, dims, 128 ** -0.5,
                                flags=flags, workspace=ws)
    return out, g["rec_state"]


def _ab_equal(p, flags=gdn.FLAG_QK_L2NORM, **kw):
    oa, sa = _ab_call(p, flags, **kw)
    ob, sb = _ab_call(p, flags | gdn.FLAG_PREFILL_SINGLE_ROLE, **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(oa).all() and torch.isfinite(sa).all()
    assert torch.equal(oa, ob), "outputs differ between the two chunk-step kernels"
    assert torch.equal(sa, sb), "states differ between the two chunk-step kernels"
    return oa


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_pipelined_step_equals_single_role_ragged(out_dtype):
    """Whole runs: lengths around the 16- and 64-token boundaries, an empty
    and an inactive sequence, random start states."""
    lengths = [1, 15, 16, 17, 63, 64, 65, 130, 0, 200, 777]
    p = gi.prefill_inputs(lengths, 14, H=2, HV=4, dk=128, dv=128, seed=61, state_std=0.1)
    p["slot_idx"][3] = 0
    out = _ab_equal(p, gdn.FLAG_QK_L2NORM | gdn.FLAG_PREFILL_SEQUENTIAL, out_dtype=out_dtype)
    cu = p["cu_seqlens"].tolist()
    assert torch.all(out[cu[3]:cu[4]] == 0)


def test_pipelined_step_equals_single_role_norm_off_and_gated():
    p = gi.prefill_inputs([70, 64, 5, 300], 6, H=2, HV=4, dk=128, dv=128, seed=62,
                          qk_normalised=True)
    _ab_equal(p, 0)
    T = p["q"].shape[0]
    gt = gi.gating_inputs(T, 4, seed=63)
    gate = gdn.GateInputs(gt["a"].cuda(), gt["b"].cuda(), gt["A_log"].cuda(),
                          gt["dt_bias"].cuda())
    _ab_equal(p, gate=gate)


@pytest.mark.parametrize("seg", [(128, 0), (128, 256), (256, 512)])
def test_pipelined_step_equals_single_role_segmented(seg):
    """Segment runs (pass 1 paired and unpaired, pass 2), ragged tails."""
    p = gi.prefill_inputs([900, 70, 1500, 333], 6, H=2, HV=4, dk=128, dv=128, seed=64,
                          state_std=0.1)
    p["g"] *= 0.05
    _ab_equal(p, seg=seg)


def test_pipelined_step_equals_single_role_auto_schedules():
    """The plain call's own schedules at H=16, HV=32: the busy-chip head/tail
    schedule with its workspace, and the whole-run schedule without one."""
    lengths = [1800, 200, 1700, 150, 2300, 100, 1300, 2200]
    p = gi.prefill_inputs(lengths, 10, seed=65)
    dims = gdn.make_dims(16, 32, 128, 128, 4)
    wsb = gdn.gdn_prefill_workspace_size(dims, len(lengths), sum(lengths))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda") if wsb else None
    _ab_equal(p, ws=ws)
    _ab_equal(p)
