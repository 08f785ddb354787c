"""GPU parity of gdn_gated_rmsnorm against the oracle's plain definition.

The gated RMSNorm after the GDN core (RL-Kernel PR #469, "Latest Status":
SiLU or sigmoid gate, optional zero-centred weight).  Bars: fp32 output
max|err| / max|ref| <= 1e-5; bf16 output within bf16 rounding (2^-8).  Also:
in place (out is x), zero rows, and bitwise batch invariance (a row alone
equals the row inside a batch).
"""
import numpy as np
import pytest
import torch

import gated_deltanet_recurrent_gdn_amd as gdn
import oracle
from gpu_helpers import f64, rel_err

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _inputs(rows, dim, x_dt, w_dt, seed):
    gen = torch.Generator().manual_seed(seed)
    x = (torch.randn(rows, dim, generator=gen) * torch.rand(rows, 1, generator=gen) * 4).to(DT[x_dt])
    z = (2 * torch.randn(rows, dim, generator=gen)).to(DT[x_dt])
    w = (1 + 0.3 * torch.randn(dim, generator=gen)).to(DT[w_dt])
    return x, z, w


@pytest.mark.parametrize("x_dt,w_dt,out_dt", [("bf16", "f32", "bf16"), ("f32", "f32", "f32"),
                                              ("bf16", "bf16", "f32"), ("f32", "bf16", "bf16")])
@pytest.mark.parametrize("gate,flags", [("silu", 0), ("sigmoid", gdn.NORM_GATE_SIGMOID),
                                        ("none", 0), ("silu", gdn.NORM_ZERO_CENTRED)])
@pytest.mark.parametrize("dim", [128, 4, 36, 1024])
def test_gated_rmsnorm_parity(x_dt, w_dt, out_dt, gate, flags, dim):
    rows = 37
    x, z, w = _inputs(rows, dim, x_dt, w_dt, seed=dim + flags)
    x[5] = 0
    if flags & gdn.NORM_ZERO_CENTRED:
        w = (w.float() - 1).to(w.dtype)
    zz = None if gate == "none" else z
    out = torch.full((rows, dim), float("nan"), dtype=DT[out_dt], device="cuda")
    gdn.gdn_gated_rmsnorm(x.cuda(), w.cuda(), out, z=None if zz is None else zz.cuda(), eps=1e-6,
                          flags=flags)
    torch.cuda.synchronize()
    oflags = (oracle.NORM_GATE_SIGMOID if flags & gdn.NORM_GATE_SIGMOID else 0) | \
             (oracle.NORM_ZERO_CENTRED if flags & gdn.NORM_ZERO_CENTRED else 0)
    ref = oracle.gated_rmsnorm(f64(x), f64(w), z=None if zz is None else f64(zz), eps=1e-6,
                               flags=oflags)
    tol = 1e-5 if out_dt == "f32" else 2 ** -8
    assert rel_err(f64(out), ref) <= tol
    assert torch.all(out[5] == 0)


def test_gated_rmsnorm_in_place_and_batch_invariant():
    rows, dim = 64, 128
    x, z, w = _inputs(rows, dim, "bf16", "f32", seed=3)
    xg, zg, wg = x.cuda(), z.cuda(), w.cuda()
    full = torch.empty(rows, dim, dtype=torch.bfloat16, device="cuda")
    gdn.gdn_gated_rmsnorm(xg, wg, full, z=zg)
    for r in (0, 17, 63):
        one = torch.empty(1, dim, dtype=torch.bfloat16, device="cuda")
        gdn.gdn_gated_rmsnorm(xg[r:r + 1].contiguous(), wg, one, z=zg[r:r + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(one[0], full[r])
    inplace = xg.clone()
    gdn.gdn_gated_rmsnorm(inplace, wg, inplace, z=zg)
    torch.cuda.synchronize()
    assert torch.equal(inplace, full)


def test_gated_rmsnorm_on_prefill_output():
    """The epilogue on a real prefill output: o [T, HV, dv] normalised per head."""
    import gdn_inputs as gi
    p = gi.prefill_inputs([100, 37], 4, H=2, HV=4, dk=128, dv=128, seed=5)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    dims = gdn.make_dims(2, 4, 128, 128, 4)
    o = torch.empty(137, 4, 128, dtype=torch.bfloat16, device="cuda")
    gdn.gdn_prefill_chunked(g["q"], g["k"], g["v"], g["g"], g["beta"], g["cu_seqlens"],
                            g["slot_idx"], g["rec_state"], o, dims, 128 ** -0.5)
    gen = torch.Generator().manual_seed(6)
    zt = torch.randn(137, 4, 128, generator=gen).to(torch.bfloat16)
    w = torch.ones(128)
    y = torch.empty_like(o)
    gdn.gdn_gated_rmsnorm(o, w.cuda(), y, z=zt.cuda())
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(f64(o), f64(w), z=f64(zt), eps=1e-6)
    assert rel_err(f64(y), ref) <= 2 ** -8
