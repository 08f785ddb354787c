"""GPU parity of the fused-gating entry points (gdn_decode_step_gated,
gdn_prefill_chunked_gated) against the oracle, through the C ABI.

RL-Kernel PR #469, "How the golden relates to the kernel", item 1: beta =
sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias) with the softplus
threshold at 20, in fp32.  The oracle computes the gates in fp64
(``oracle.gating``, pinned in the CPU tests) and feeds them to its decode /
token-by-token prefill; the GPU computes them in fp32 inside the kernels.
Bars are the ungated calls': decode 1e-5 (max|err| / max|ref|), prefill 5e-3,
conv roll bit-exact.  Inputs: ``gdn_inputs.gating_inputs`` (about 5% of the
a values pushed past the threshold), a/b in bf16 and fp32.
"""
import math

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_recurrent_gdn_amd as gdn
import oracle
from gpu_helpers import DECODE_TOL, PATH_FLAGS, PREFILL_TOL, f64, oracle_decode_rows, rel_err, to_dev
from test_prefill_gpu import oracle_heads

pytestmark = pytest.mark.gpu


def _gate_dev(gt):
    return gdn.GateInputs(gt["a"].cuda(), gt["b"].cuda(), gt["A_log"].cuda(), gt["dt_bias"].cuda())


def _oracle_gates(gt):
    g, beta = oracle.gating(f64(gt["a"]), f64(gt["b"]), f64(gt["A_log"]), f64(gt["dt_bias"]))
    return torch.from_numpy(g), torch.from_numpy(beta)


@pytest.mark.parametrize("path", ["fused", "split"])
@pytest.mark.parametrize("ab_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(2, 4, 32, 32, 9, 16), (16, 32, 128, 128, 8, 64)],
                         ids=["tiny", "qwen"])
def test_decode_step_gated(shape, ab_dtype, path):
    H, HV, dk, dv, B, ns = shape
    d = gi.decode_inputs(B, ns, H=H, HV=HV, dk=dk, dv=dv, seed=51, conv_bias=True)
    d["slot_idx"][1] = 0
    gt = gi.gating_inputs(B, HV, seed=52, ab_dtype=ab_dtype)
    assert bool(((gt["a"].float() + gt["dt_bias"]) > 20).any()), "threshold branch not exercised"
    ref = dict(d)
    ref["g"], ref["beta"] = _oracle_gates(gt)
    scale = dk ** -0.5
    o_ref, cs_ref, rs_ref, active = oracle_decode_rows(ref, list(range(B)), scale)

    g = to_dev(d)
    dims = gdn.make_dims(H, HV, dk, dv, 4)
    out = torch.full((B, HV, dv), float("nan"), device="cuda")
    gdn.gdn_decode_step_gated(g["mixed_qkv"], _gate_dev(gt), g["slot_idx"], g["conv_state"],
                              g["conv_weight"], g["rec_state"], out, dims, scale,
                              conv_bias=g["conv_bias"],
                              flags=gdn.DEFAULT_DECODE_FLAGS | PATH_FLAGS[path])
    torch.cuda.synchronize()
    assert rel_err(f64(out), o_ref) <= DECODE_TOL
    for i, s in enumerate(d["slot_idx"].tolist()):
        if s <= 0:
            assert torch.all(out[i] == 0)
            continue
        assert rel_err(f64(g["rec_state"][s]), rs_ref[i]) <= DECODE_TOL
        assert np.array_equal(f64(g["conv_state"][s]), cs_ref[i])


def test_decode_gated_matches_precomputed_gates_closely():
    """The gated call and the plain call fed the oracle's gates (rounded to
    fp32) differ only by the fp32 gating rounding."""
    d = gi.decode_inputs(6, 16, H=2, HV=4, dk=64, dv=64, seed=53)
    gt = gi.gating_inputs(6, 4, seed=54, ab_dtype=torch.float32)
    g64, b64 = _oracle_gates(gt)
    a_, b_ = to_dev(d), to_dev(d)
    a_["g"], a_["beta"] = g64.float().cuda(), b64.float().cuda()
    dims = gdn.make_dims(2, 4, 64, 64, 4)
    o1 = torch.empty(6, 4, 64, device="cuda")
    o2 = torch.empty(6, 4, 64, device="cuda")
    gdn.gdn_decode_step(a_["mixed_qkv"], a_["g"], a_["beta"], a_["slot_idx"], a_["conv_state"],
                        a_["conv_weight"], a_["rec_state"], o1, dims, 0.125)
    gdn.gdn_decode_step_gated(b_["mixed_qkv"], _gate_dev(gt), b_["slot_idx"], b_["conv_state"],
                              b_["conv_weight"], b_["rec_state"], o2, dims, 0.125)
    torch.cuda.synchronize()
    assert rel_err(f64(o2), f64(o1)) <= 1e-6
    assert torch.equal(a_["conv_state"], b_["conv_state"])


@pytest.mark.parametrize("d,ab_dtype", [(32, torch.bfloat16), (128, torch.bfloat16),
                                        (64, torch.float32)])
def test_prefill_gated(d, ab_dtype):
    lengths = [1, 63, 64, 65, 130, 0, 200]
    HV, H = 4, 2
    p = gi.prefill_inputs(lengths, 10, H=H, HV=HV, dk=d, dv=d, seed=61)
    p["slot_idx"][5] = 0
    T = int(sum(lengths))
    gt = gi.gating_inputs(T, HV, seed=62, ab_dtype=ab_dtype)
    ref = dict(p)
    ref["g"], ref["beta"] = _oracle_gates(gt)
    scale = d ** -0.5
    o_ref, s_ref = oracle_heads(ref, list(range(HV)), scale)

    g = to_dev(p)
    dims = gdn.make_dims(H, HV, d, d, 4)
    out = torch.full((T, HV, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_prefill_chunked_gated(g["q"], g["k"], g["v"], _gate_dev(gt), g["cu_seqlens"],
                                  g["slot_idx"], g["rec_state"], out, dims, scale)
    torch.cuda.synchronize()
    assert rel_err(f64(out), o_ref) <= PREFILL_TOL
    slots = p["slot_idx"].tolist()
    act = [i for i, s in enumerate(slots) if s > 0]
    sg = np.stack([f64(g["rec_state"][slots[i]]) for i in act])
    assert rel_err(sg, s_ref[act]) <= PREFILL_TOL
    c = p["cu_seqlens"].tolist()
    assert torch.all(out[c[5]:c[6]].float() == 0)        # inactive sequence
