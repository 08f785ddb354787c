"""GPU parity of the decode step (conv -> SiLU -> QK norm -> gated delta rule)
against the fp64 oracle, through the C ABI.

Bars: o and the fp32 state at max|err| / max|ref| <= 1e-5; the conv cache roll
and every untouched slot bit-exact.  Shapes: the tiny fp32 case (H=2, HV=4,
d=32), the Qwen3-Next-like buckets B = 1..16 over a 256-slot cache, and the
large batches B = 256 / 1024 over a 2048-slot cache (sampled rows checked
against the oracle one by one; every row checked for the slot contract).
"""
import math

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_recurrent_gdn_amd as gdn
from gpu_helpers import (DECODE_TOL, f64, oracle_decode_rows, rel_err, run_decode_gpu,
                         to_dev)

pytestmark = pytest.mark.gpu


def _check_rows(d_cpu, d_gpu_after, out_gpu, rows, scale, flags=gdn.DEFAULT_DECODE_FLAGS):
    o_ref, cs_ref, rs_ref, active = oracle_decode_rows(d_cpu, rows, scale, flags=flags)
    o = f64(out_gpu[rows])
    assert rel_err(o, o_ref) <= DECODE_TOL, rel_err(o, o_ref)
    slots = d_cpu["slot_idx"][rows].tolist()
    for i, s in enumerate(slots):
        if s <= 0:
            assert np.all(o[i] == 0.0)
            continue
        rs = f64(d_gpu_after["rec_state"][s])
        assert rel_err(rs, rs_ref[i]) <= DECODE_TOL, (s, rel_err(rs, rs_ref[i]))
        cs = f64(d_gpu_after["conv_state"][s])
        assert np.array_equal(cs, cs_ref[i]), f"conv roll not bit-exact at slot {s}"


def _untouched(before, after, used):
    mask = torch.ones(before.shape[0], dtype=torch.bool)
    mask[[s for s in used if s > 0]] = False
    return torch.equal(before[mask], after.cpu()[mask])


@pytest.mark.parametrize("act_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("bias", [False, True])
def test_decode_tiny(act_dtype, bias):
    d = gi.decode_inputs(6, 8, H=2, HV=4, dk=32, dv=32, act_dtype=act_dtype, seed=0,
                         g_mode="softplus", conv_bias=bias)
    d["slot_idx"][2] = 0           # a padded row
    d["slot_idx"][4] = -1
    g = to_dev(d)
    out = run_decode_gpu(g, 1 / math.sqrt(32))
    torch.cuda.synchronize()
    _check_rows(d, g, out, list(range(6)), 1 / math.sqrt(32))
    assert _untouched(d["rec_state"], g["rec_state"], d["slot_idx"].tolist())
    assert _untouched(d["conv_state"], g["conv_state"], d["slot_idx"].tolist())


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16])
def test_decode_qwen_buckets(B):
    d = gi.decode_inputs(B, 256, seed=1)
    g = to_dev(d)
    out = run_decode_gpu(g, 128 ** -0.5)
    torch.cuda.synchronize()
    _check_rows(d, g, out, list(range(B)), 128 ** -0.5)
    assert _untouched(d["rec_state"], g["rec_state"], d["slot_idx"].tolist())
    assert _untouched(d["conv_state"], g["conv_state"], d["slot_idx"].tolist())


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 96), (256, 128), (32, 128)])
def test_decode_other_head_dims(dk, dv):
    d = gi.decode_inputs(5, 9, H=2, HV=4, dk=dk, dv=dv, seed=7)
    d["slot_idx"][1] = 0
    g = to_dev(d)
    out = run_decode_gpu(g, dk ** -0.5)
    torch.cuda.synchronize()
    _check_rows(d, g, out, list(range(5)), dk ** -0.5)


@pytest.mark.parametrize("flags", [0, gdn.FLAG_SILU, gdn.FLAG_QK_L2NORM])
def test_decode_flag_variants(flags):
    d = gi.decode_inputs(4, 16, seed=5)
    g = to_dev(d)
    out = run_decode_gpu(g, 128 ** -0.5, flags=flags)
    torch.cuda.synchronize()
    _check_rows(d, g, out, list(range(4)), 128 ** -0.5, flags=flags)


def test_decode_bf16_output():
    d = gi.decode_inputs(8, 32, seed=6)
    g = to_dev(d)
    out = run_decode_gpu(g, 128 ** -0.5, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, _, rs_ref, _ = oracle_decode_rows(d, list(range(8)), 128 ** -0.5)
    # the store rounds to bf16 (relative error <= 2^-9 per element)
    assert rel_err(f64(out), o_ref) <= 2 ** -8


@pytest.fixture(scope="module")
def large_cache():
    d = gi.decode_inputs(1024, 2048, seed=2)
    return d


@pytest.mark.parametrize("B", [256, 1024])
def test_decode_large_batch_sampled(large_cache, B):
    d = {k: (v[:B] if k in ("mixed_qkv", "g", "beta", "slot_idx") else v)
         for k, v in large_cache.items()}
    g = to_dev(d)
    out = run_decode_gpu(g, 128 ** -0.5)
    torch.cuda.synchronize()
    rng = np.random.default_rng(B)
    rows = sorted(rng.choice(B, 48, replace=False).tolist())
    _check_rows(d, g, out, rows, 128 ** -0.5)
    assert torch.isfinite(out).all()
    assert _untouched(d["rec_state"], g["rec_state"], d["slot_idx"].tolist())
    del g
    torch.cuda.empty_cache()


def test_decode_empty_batch():
    d = gi.decode_inputs(0, 4, H=2, HV=4, dk=32, dv=32, seed=0)
    g = to_dev(d)
    err = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    out = run_decode_gpu(g, 0.2, flags=gdn.DEFAULT_DECODE_FLAGS | gdn.FLAG_VALIDATE,
                         err_flag=err)
    torch.cuda.synchronize()
    assert out.shape[0] == 0
    assert int(err.item()) == 0
