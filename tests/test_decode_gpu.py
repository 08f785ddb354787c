"""GPU parity of the decode step (conv -> SiLU -> QK norm -> gated delta rule)
against the fp64 oracle, through the C ABI.

Bars: o and the fp32 state at max|err| / max|ref| <= 1e-5; the conv cache roll
and every untouched slot bit-exact.  Shapes: the tiny fp32 case (H=2, HV=4,
d=32), the Qwen3-Next-like buckets B = 1..16 over a 256-slot cache, and the
large batches B = 256 / 1024 over a 2048-slot cache (sampled rows checked
against the oracle one by one; every row checked for the slot contract; at
B = 256 every row is also checked against the oracle).
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


@pytest.mark.parametrize("path", ["fused", "split"])
@pytest.mark.parametrize("act_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("bias", [False, True])
def test_decode_tiny(act_dtype, bias, path):
    d = gi.decode_inputs(6, 8, H=2, HV=4, dk=32, dv=32, act_dtype=act_dtype, seed=0,
                         g_mode="softplus", conv_bias=bias)
    d["slot_idx"][2] = 0           # a padded row
    d["slot_idx"][4] = -1
    g = to_dev(d)
    out = run_decode_gpu(g, 1 / math.sqrt(32), path=path)
    torch.cuda.synchronize()
    _check_rows(d, g, out, list(range(6)), 1 / math.sqrt(32))
    assert _untouched(d["rec_state"], g["rec_state"], d["slot_idx"].tolist())
    assert _untouched(d["conv_state"], g["conv_state"], d["slot_idx"].tolist())


@pytest.mark.parametrize("path", [None, "split"])
@pytest.mark.parametrize("B", [1, 2, 4, 8, 16])
def test_decode_qwen_buckets(B, path):
    d = gi.decode_inputs(B, 256, seed=1)
    g = to_dev(d)
    out = run_decode_gpu(g, 128 ** -0.5, path=path)
    torch.cuda.synchronize()
    _check_rows(d, g, out, list(range(B)), 128 ** -0.5)
    assert _untouched(d["rec_state"], g["rec_state"], d["slot_idx"].tolist())
    assert _untouched(d["conv_state"], g["conv_state"], d["slot_idx"].tolist())


@pytest.mark.parametrize("path", ["fused", "split"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 96), (256, 128), (32, 128)])
def test_decode_other_head_dims(dk, dv, path):
    d = gi.decode_inputs(5, 9, H=2, HV=4, dk=dk, dv=dv, seed=7)
    d["slot_idx"][1] = 0
    g = to_dev(d)
    out = run_decode_gpu(g, dk ** -0.5, path=path)
    torch.cuda.synchronize()
    _check_rows(d, g, out, list(range(5)), dk ** -0.5)


@pytest.mark.parametrize("path", ["fused", "split"])
@pytest.mark.parametrize("flags", [0, gdn.FLAG_SILU, gdn.FLAG_QK_L2NORM])
def test_decode_flag_variants(flags, path):
    d = gi.decode_inputs(4, 16, seed=5)
    g = to_dev(d)
    out = run_decode_gpu(g, 128 ** -0.5, flags=flags, path=path)
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


@pytest.mark.parametrize("path", [None, "fused"])
@pytest.mark.parametrize("B", [256, 1024])
def test_decode_large_batch_sampled(large_cache, B, path):
    d = {k: (v[:B] if k in ("mixed_qkv", "g", "beta", "slot_idx") else v)
         for k, v in large_cache.items()}
    g = to_dev(d)
    out = run_decode_gpu(g, 128 ** -0.5, path=path)
    torch.cuda.synchronize()
    rng = np.random.default_rng(B)
    rows = sorted(rng.choice(B, 48, replace=False).tolist())
    _check_rows(d, g, out, rows, 128 ** -0.5)
    assert torch.isfinite(out).all()
    assert _untouched(d["rec_state"], g["rec_state"], d["slot_idx"].tolist())
    del g
    torch.cuda.empty_cache()


def test_decode_batch256_every_row(large_cache):
    """The batch-256 workload (seed 2, 2048-slot cache): every row's output,
    recurrent state and conv roll against the oracle (checked 64 rows at a
    time), on the library's default path."""
    B = 256
    d = {k: (v[:B] if k in ("mixed_qkv", "g", "beta", "slot_idx") else v)
         for k, v in large_cache.items()}
    g = to_dev(d)
    out = run_decode_gpu(g, 128 ** -0.5)
    torch.cuda.synchronize()
    for r0 in range(0, B, 64):
        _check_rows(d, g, out, list(range(r0, r0 + 64)), 128 ** -0.5)
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


# The fused step and the conv + recurrence pair must agree bitwise on outputs,
# recurrent state and conv cache, for every dtype mix, head shape and flag set.
_PATH_CASES = [
    # (H, HV, dk, dv, x dtype, conv cache dtype, weight dtype, out dtype, bias, flags)
    (2, 4, 32, 32, "f32", "f32", "f32", "f32", True, gdn.DEFAULT_DECODE_FLAGS),
    (16, 32, 128, 128, "bf16", "bf16", "bf16", "f32", False, gdn.DEFAULT_DECODE_FLAGS),
    (16, 32, 128, 128, "bf16", "bf16", "bf16", "bf16", True, gdn.DEFAULT_DECODE_FLAGS),
    (4, 16, 64, 96, "f32", "bf16", "f32", "f32", True, gdn.DEFAULT_DECODE_FLAGS),
    (2, 2, 256, 128, "bf16", "f32", "bf16", "bf16", False, gdn.DEFAULT_DECODE_FLAGS),
    (1, 8, 128, 32, "bf16", "bf16", "f32", "f32", True, gdn.FLAG_SILU),
    (3, 6, 32, 256, "f32", "f32", "bf16", "f32", False, 0),
    (2, 4, 64, 64, "bf16", "bf16", "bf16", "f32", True, gdn.FLAG_QK_L2NORM),
]
_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _batch_for(regime, H):
    """Batch at which the fused step runs double-buffered ("few": at most two
    (row, key head) groups per CU) or single-buffered ("many": more)."""
    if regime == "few":
        return 11
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return max(11, (2 * cus) // H + 5)


@pytest.mark.parametrize("regime", ["few", "many"])
@pytest.mark.parametrize("case", _PATH_CASES, ids=lambda c: "-".join(map(str, c[:8])))
def test_fused_equals_split_bitwise(case, regime):
    H, HV, dk, dv, xd, cd, wd, od, bias, flags = case
    B = _batch_for(regime, H)
    d = gi.decode_inputs(B, B + 13, H=H, HV=HV, dk=dk, dv=dv, seed=40 + dk + dv, conv_bias=bias)
    d["mixed_qkv"] = d["mixed_qkv"].to(_DT[xd])
    d["conv_state"] = d["conv_state"].to(_DT[cd])
    d["conv_weight"] = d["conv_weight"].to(_DT[wd])
    if bias:
        d["conv_bias"] = d["conv_bias"].to(_DT[wd])
    d["slot_idx"][3] = 0
    d["slot_idx"][8] = -2
    a, b = to_dev(d), to_dev(d)
    oa = run_decode_gpu(a, dk ** -0.5, flags=flags, out_dtype=_DT[od], path="fused")
    ob = run_decode_gpu(b, dk ** -0.5, flags=flags, out_dtype=_DT[od], path="split")
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    assert torch.equal(a["rec_state"], b["rec_state"])
    assert torch.equal(a["conv_state"], b["conv_state"])
    assert not torch.isnan(oa).any()
