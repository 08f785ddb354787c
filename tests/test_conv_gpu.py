"""GPU parity of gdn_conv_update (decode and varlen forms) against the oracle.

RL-Kernel PR #469, "Summary" and "The conv half: coverage and the two
mismatch mechanisms": the rolled conv state must equal the last W-1 raw
inputs exactly (compared bitwise there); outputs are a bias-first fp32
accumulation over the window, optionally followed by SiLU.  Bars: outputs
max|err| / max|ref| <= 1e-5 (fp32 output) or within bf16 rounding (bf16
output); rolled state bit-exact (in the cache dtype); untouched slots and
inactive rows byte-identical.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_recurrent_gdn_amd as gdn
import oracle
from gpu_helpers import f64, rel_err

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _case(T_rows, dim, ns, x_dt, cs_dt, w_dt, bias, seed):
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn(T_rows, dim, generator=gen).to(DT[x_dt])
    cs = torch.randn(ns, dim, 3, generator=gen).to(DT[cs_dt])
    w = (torch.rand(dim, 4, generator=gen) - 0.5).to(DT[w_dt])
    b = (torch.rand(dim, generator=gen) - 0.5).to(DT[w_dt]) if bias else None
    return x, cs, w, b


def _expected_cache(cs_before, cs_oracle, dtype):
    """The oracle keeps fp64 taps; the cache stores them rounded to its dtype."""
    return torch.from_numpy(cs_oracle).to(dtype)


@pytest.mark.parametrize("x_dt,cs_dt,w_dt", [("bf16", "bf16", "bf16"), ("f32", "f32", "f32"),
                                             ("f32", "bf16", "f32"), ("bf16", "f32", "bf16")])
@pytest.mark.parametrize("bias,silu", [(False, True), (True, True), (True, False)])
def test_conv_decode_form(x_dt, cs_dt, w_dt, bias, silu):
    B, dim, ns = 9, 520, 12
    x, cs, w, b = _case(B, dim, ns, x_dt, cs_dt, w_dt, bias, seed=31)
    slots = torch.tensor([3, 0, 7, 11, -1, 1, 5, 9, 2], dtype=torch.int32)
    flags = gdn.FLAG_SILU if silu else 0
    cs_g = cs.cuda()
    out = torch.full((B, dim), float("nan"), device="cuda")
    gdn.gdn_conv_update(x.cuda(), slots.cuda(), cs_g, w.cuda(), out,
                        bias=None if b is None else b.cuda(), flags=flags)
    torch.cuda.synchronize()
    cs_o = f64(cs).copy()
    ref = oracle.conv_update(f64(x), slots.numpy(), cs_o, f64(w),
                             bias=None if b is None else f64(b),
                             flags=oracle.FLAG_SILU if silu else 0)
    assert rel_err(f64(out), ref) <= 1e-5
    assert torch.equal(cs_g.cpu(), _expected_cache(cs, cs_o, cs.dtype))
    for r, s in enumerate(slots.tolist()):
        if s <= 0:
            assert torch.all(out[r] == 0)


@pytest.mark.parametrize("x_dt,cs_dt,w_dt", [("bf16", "bf16", "bf16"), ("f32", "f32", "f32"),
                                             ("f32", "bf16", "f32")])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
@pytest.mark.parametrize("dim", [264, 262])   # token-parallel kernel; general kernel (dim % 4 != 0)
def test_conv_varlen_form(x_dt, cs_dt, w_dt, out_dt, dim):
    lengths = [1, 2, 3, 0, 17, 64, 5, 200]
    cu = gi.cu_from_lengths(lengths)
    T, ns = int(cu[-1]), 12
    x, cs, w, b = _case(T, dim, ns, x_dt, cs_dt, w_dt, True, seed=32)
    slots = torch.tensor([4, 8, 0, 2, 11, 1, 6, 9], dtype=torch.int32)
    cs_g = cs.cuda()
    out = torch.full((T, dim), float("nan"), dtype=DT[out_dt], device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.gdn_conv_update(x.cuda(), slots.cuda(), cs_g, w.cuda(), out, bias=b.cuda(),
                        cu_seqlens=cu.cuda(), flags=gdn.FLAG_SILU | gdn.FLAG_VALIDATE,
                        err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    cs_o = f64(cs).copy()
    ref = oracle.conv_update(f64(x), slots.numpy(), cs_o, f64(w), bias=f64(b),
                             cu_seqlens=cu.numpy(), flags=oracle.FLAG_SILU)
    tol = 1e-5 if out_dt == "f32" else 2 ** -8
    assert rel_err(f64(out), ref) <= tol
    assert torch.equal(cs_g.cpu(), _expected_cache(cs, cs_o, cs.dtype))
    c = cu.tolist()
    assert torch.all(out[c[2]:c[3]].float() == 0)          # inactive sequence


def test_conv_varlen_equals_token_by_token():
    """One varlen call over L tokens == L decode-form calls (bitwise)."""
    lengths = [7, 1, 30]
    cu = gi.cu_from_lengths(lengths)
    T, dim, ns = int(cu[-1]), 256, 6
    x, cs, w, b = _case(T, dim, ns, "bf16", "bf16", "bf16", False, seed=33)
    slots = torch.tensor([2, 5, 3], dtype=torch.int32)
    cs_a = cs.cuda()
    out_a = torch.empty(T, dim, device="cuda")
    gdn.gdn_conv_update(x.cuda(), slots.cuda(), cs_a, w.cuda(), out_a, cu_seqlens=cu.cuda())
    cs_b = cs.cuda()
    out_b = torch.empty(T, dim, device="cuda")
    c = cu.tolist()
    for t in range(max(lengths)):
        rows = [n for n in range(3) if t < lengths[n]]
        idx = torch.tensor([c[n] + t for n in rows])
        o = torch.empty(len(rows), dim, device="cuda")
        gdn.gdn_conv_update(x[idx].contiguous().cuda(), slots[rows].cuda(), cs_b, w.cuda(), o)
        out_b[idx.cuda()] = o
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    assert torch.equal(cs_a, cs_b)


@pytest.mark.parametrize("x_dt,cs_dt", [("bf16", "bf16"), ("f32", "bf16")])
def test_conv_varlen_many_short_sequences(x_dt, cs_dt):
    """Sequences of 0..20 tokens starting anywhere inside the 16-token tiles of
    the token-parallel kernel (several sequence starts per tile), some inactive."""
    gen = torch.Generator().manual_seed(35)
    n = 120
    lengths = torch.randint(0, 21, (n,), generator=gen).tolist()
    cu = gi.cu_from_lengths(lengths)
    T, dim, ns = int(cu[-1]), 256, n + 7
    x, cs, w, b = _case(T, dim, ns, x_dt, cs_dt, "bf16", True, seed=36)
    slots = (torch.randperm(ns - 1, generator=gen)[:n] + 1).to(torch.int32)
    slots[::9] = 0                                         # inactive sequences
    cs_g = cs.cuda()
    out = torch.full((T, dim), float("nan"), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.gdn_conv_update(x.cuda(), slots.cuda(), cs_g, w.cuda(), out, bias=b.cuda(),
                        cu_seqlens=cu.cuda(), flags=gdn.FLAG_SILU | gdn.FLAG_VALIDATE,
                        err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    cs_o = f64(cs).copy()
    ref = oracle.conv_update(f64(x), slots.numpy(), cs_o, f64(w), bias=f64(b),
                             cu_seqlens=cu.numpy(), flags=oracle.FLAG_SILU)
    assert rel_err(f64(out), ref) <= 1e-5
    assert torch.equal(cs_g.cpu(), _expected_cache(cs, cs_o, cs.dtype))


def test_conv_varlen_paths_agree_bitwise():
    """The token-parallel kernel (16-byte aligned tensors) and the general one
    (taken for a misaligned output view) give identical outputs and caches."""
    lengths = [3, 1, 0, 70, 2, 33]
    cu = gi.cu_from_lengths(lengths)
    T, dim, ns = int(cu[-1]), 256, 9
    x, cs, w, b = _case(T, dim, ns, "bf16", "bf16", "bf16", True, seed=37)
    slots = torch.tensor([3, 1, 5, 8, 0, 2], dtype=torch.int32)
    cs_a, cs_b = cs.cuda(), cs.cuda()
    out_a = torch.empty(T, dim, device="cuda")
    gdn.gdn_conv_update(x.cuda(), slots.cuda(), cs_a, w.cuda(), out_a, bias=b.cuda(),
                        cu_seqlens=cu.cuda(), flags=gdn.FLAG_SILU)
    buf = torch.empty(T * dim + 1, device="cuda")
    out_b = buf[1:].view(T, dim)                           # 4-byte aligned only
    gdn.gdn_conv_update(x.cuda(), slots.cuda(), cs_b, w.cuda(), out_b, bias=b.cuda(),
                        cu_seqlens=cu.cuda(), flags=gdn.FLAG_SILU)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    assert torch.equal(cs_a, cs_b)
