"""The tiny end-to-end configuration on the GPU: 2 sequences, 2 key heads, 4
value heads, d = 32, conv width 4, fp32 everywhere; a 64-token prefill per
sequence (one chunk) and then 8 decode steps, against the fp64 oracle.

* Each decode step is compared with the oracle run from the GPU's own caches
  before that step (isolating one step's error; bar 1e-5 on o and state, conv
  roll bit-exact).
* The whole chain is compared with one oracle run from the initial inputs
  (bar 5e-3, the prefill bar, since the prefill's error carries forward).
* A full pipeline variant runs the varlen conv update over the prompt's mixed
  q|k|v, splits it, prefills, then decodes; the oracle does the same steps.

Reading (the pages leave it open): the prefill consumes the given q, k, v (no
conv), the conv state starts at zero, and the decode steps feed fresh N(0, 1)
mixed q|k|v through the conv path.
"""
import math

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_recurrent_gdn_amd as gdn
import oracle
from gpu_helpers import DECODE_TOL, PREFILL_TOL, f64, rel_err

pytestmark = pytest.mark.gpu


def _dims(c):
    dm = c["dims"]
    return gdn.make_dims(dm["H"], dm["HV"], dm["dk"], dm["dv"], dm["W"])


def test_tiny_prefill_then_decode():
    c = gi.tiny_config(seed=0)
    dm, scale = c["dims"], c["scale"]
    H, HV, d = dm["H"], dm["HV"], dm["dk"]
    dims = _dims(c)
    pre = c["prefill"]
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in pre.items()}
    conv = c["conv_state"].cuda()
    weight = c["conv_weight"].cuda()
    T = pre["q"].shape[0]
    out = torch.empty(T, HV, d, device="cuda")
    gdn.gdn_prefill_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                            dev["cu_seqlens"], dev["slot_idx"], dev["rec_state"], out, dims, scale,
                            flags=gdn.FLAG_QK_L2NORM | gdn.FLAG_VALIDATE,
                            err_flag=torch.zeros(1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    # oracle chain from the initial inputs
    rec_o = f64(pre["rec_state"]).copy()
    conv_o = f64(c["conv_state"]).copy()
    o_ref = oracle.prefill(f64(pre["q"]), f64(pre["k"]), f64(pre["v"]), f64(pre["g"]),
                           f64(pre["beta"]), pre["cu_seqlens"].numpy(), pre["slot_idx"].numpy(),
                           rec_o, scale)
    assert rel_err(f64(out), o_ref) <= PREFILL_TOL
    slots = pre["slot_idx"].numpy()
    assert rel_err(f64(dev["rec_state"][slots]), rec_o[slots]) <= PREFILL_TOL

    for step, dec in enumerate(c["decode"]):
        x = dec["mixed_qkv"]
        # one-step oracle from the GPU's caches before this step
        rec_1 = f64(dev["rec_state"]).copy()
        conv_1 = f64(conv).copy()
        o_step = oracle.decode_step(f64(x), f64(dec["g"]), f64(dec["beta"]), slots, conv_1,
                                    f64(c["conv_weight"]), rec_1, H, HV, d, d, scale)
        o_chain = oracle.decode_step(f64(x), f64(dec["g"]), f64(dec["beta"]), slots, conv_o,
                                     f64(c["conv_weight"]), rec_o, H, HV, d, d, scale)
        o = torch.empty(2, HV, d, device="cuda")
        gdn.gdn_decode_step(x.cuda(), dec["g"].cuda(), dec["beta"].cuda(), dev["slot_idx"], conv,
                            weight, dev["rec_state"], o, dims, scale)
        torch.cuda.synchronize()
        assert rel_err(f64(o), o_step) <= DECODE_TOL, step
        assert rel_err(f64(dev["rec_state"][slots]), rec_1[slots]) <= DECODE_TOL, step
        assert np.array_equal(f64(conv), conv_1), step
        assert rel_err(f64(o), o_chain) <= PREFILL_TOL, step
        assert rel_err(f64(dev["rec_state"][slots]), rec_o[slots]) <= PREFILL_TOL, step


def test_full_pipeline_conv_prefill_decode():
    """varlen conv over the prompt's mixed q|k|v -> split -> prefill -> decode."""
    H, HV, d, W = 2, 4, 32, 4
    D = 2 * H * d + HV * d
    scale = d ** -0.5
    gen = torch.Generator().manual_seed(21)
    lengths = [37, 64, 90]
    cu = gi.cu_from_lengths(lengths)
    T = int(cu[-1])
    x = torch.randn(T, D, generator=gen)
    g = -torch.nn.functional.softplus(torch.randn(T, HV, generator=gen))
    b = torch.sigmoid(torch.randn(T, HV, generator=gen))
    weight = torch.rand(D, W, generator=gen) - 0.5
    slots = torch.tensor([3, 1, 5], dtype=torch.int32)
    ns = 6
    conv = torch.zeros(ns, D, W - 1)
    rec = torch.zeros(ns, HV, d, d)
    dims = gdn.make_dims(H, HV, d, d, W)
    # GPU
    conv_g, rec_g = conv.cuda(), rec.cuda()
    y = torch.empty(T, D, device="cuda")
    gdn.gdn_conv_update(x.cuda(), slots.cuda(), conv_g, weight.cuda(), y,
                        cu_seqlens=cu.cuda(), flags=gdn.FLAG_SILU)
    q = y[:, :H * d].reshape(T, H, d).contiguous()
    k = y[:, H * d:2 * H * d].reshape(T, H, d).contiguous()
    v = y[:, 2 * H * d:].reshape(T, HV, d).contiguous()
    out = torch.empty(T, HV, d, device="cuda")
    gdn.gdn_prefill_chunked(q, k, v, g.cuda(), b.cuda(), cu.cuda(), slots.cuda(), rec_g, out,
                            dims, scale)
    xd = torch.randn(3, D, generator=gen)
    gd = -torch.rand(3, HV, generator=gen)
    bd = torch.sigmoid(torch.randn(3, HV, generator=gen))
    od = torch.empty(3, HV, d, device="cuda")
    gdn.gdn_decode_step(xd.cuda(), gd.cuda(), bd.cuda(), slots.cuda(), conv_g, weight.cuda(),
                        rec_g, od, dims, scale)
    torch.cuda.synchronize()
    # oracle, same steps
    conv_o, rec_o = f64(conv).copy(), f64(rec).copy()
    y_o = oracle.conv_update(f64(x), slots.numpy(), conv_o, f64(weight), cu_seqlens=cu.numpy(),
                             flags=oracle.FLAG_SILU)
    assert rel_err(f64(y), y_o) <= 1e-6
    o_o = oracle.prefill(y_o[:, :H * d].reshape(T, H, d), y_o[:, H * d:2 * H * d].reshape(T, H, d),
                         y_o[:, 2 * H * d:].reshape(T, HV, d), f64(g), f64(b), cu.numpy(),
                         slots.numpy(), rec_o, scale)
    assert rel_err(f64(out), o_o) <= PREFILL_TOL
    od_o = oracle.decode_step(f64(xd), f64(gd), f64(bd), slots.numpy(), conv_o, f64(weight),
                              rec_o, H, HV, d, d, scale)
    assert rel_err(f64(od), od_o) <= PREFILL_TOL
    assert np.array_equal(f64(conv_g), conv_o), "conv roll across varlen + decode"
    s = slots.numpy()
    assert rel_err(f64(rec_g[s]), rec_o[s]) <= PREFILL_TOL
