"""gdn_decode_step_noalloc: the decode step for callers that cannot allocate
(HIP graph capture, tight serving loops, harnesses without hipMalloc).

Through the C ABI, the entry point must give bitwise the outputs and cache
updates of gdn_decode_step with a caller workspace, on the conv + recurrence
path (the one that puts the fp32 activations in the library's scratch array)
and on the library's default path, over two calls in a row with the second
smaller than the first (the scratch keeps the first call's contents).  On the
CPU: the size limit of the scratch is a synchronous GDN_ERR_WORKSPACE.
"""
import ctypes

import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_recurrent_gdn_amd as gdn
from gated_deltanet_recurrent_gdn_amd import _abi

H, HV, DK = 16, 32, 128
D = 2 * H * DK + HV * DK
SCALE = DK ** -0.5
SCRATCH_BYTES = 16 << 20


def test_noalloc_rejects_batches_past_the_scratch():
    """More than 512 rows at D = 8192 do not fit the 16 MiB scratch on the conv +
    recurrence path: rejected before anything is looked up or enqueued."""
    lib = gdn.load_library()
    fake = ctypes.c_void_p(0x10000)
    dims = gdn.make_dims(H, HV, DK, DK, 4)
    batch = SCRATCH_BYTES // (D * 4) + 1
    st = lib.gdn_decode_step_noalloc(fake, 1, fake, fake, fake, batch, fake, 1, fake, None, 1,
                                     fake, 4096, fake, 0, ctypes.byref(dims), SCALE,
                                     gdn.DEFAULT_DECODE_FLAGS | gdn.FLAG_STEP_SPLIT, None, None)
    assert st == 5, _abi._STATUS.get(st, st)          # GDN_ERR_WORKSPACE
    assert lib.gdn_decode_step_noalloc(fake, 1, fake, fake, None, 4, fake, 1, fake, None, 1,
                                       fake, 64, fake, 0, ctypes.byref(dims), SCALE, 3, None,
                                       None) == 1      # GDN_ERR_NULL (slot_idx)


def _pair(batch, seed, flags):
    """One decode batch run twice from the same caches: through gdn_decode_step
    (caller workspace) and through gdn_decode_step_noalloc.  Returns both
    (out, conv cache, recurrent cache) triples."""
    d = gi.decode_inputs(batch, batch + 8, seed=seed)
    d["slot_idx"][1] = 0                                   # one padded row
    runs = []
    for noalloc in (False, True):
        g = {k: (v.cuda().clone() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
        dims = gdn.make_dims(H, HV, DK, DK, 4)
        out = torch.full((batch, HV, DK), float("nan"), device="cuda")
        fn = gdn.gdn_decode_step_noalloc if noalloc else gdn.gdn_decode_step
        fn(g["mixed_qkv"], g["g"], g["beta"], g["slot_idx"], g["conv_state"], g["conv_weight"],
           g["rec_state"], out, dims, SCALE, flags=flags)
        torch.cuda.synchronize()
        runs.append((out, g["conv_state"], g["rec_state"]))
    return runs


@pytest.mark.gpu
@pytest.mark.parametrize("path", ["split", None])
def test_noalloc_equals_decode_step(path):
    flags = gdn.DEFAULT_DECODE_FLAGS | {None: 0, "split": gdn.FLAG_STEP_SPLIT}[path]
    for batch, seed in ((96, 11), (20, 12)):               # the second call smaller
        (o_ws, cs_ws, rs_ws), (o_na, cs_na, rs_na) = _pair(batch, seed, flags)
        assert not torch.isnan(o_na).any(), (path, batch)
        assert torch.equal(o_na, o_ws), (path, batch)
        assert torch.equal(rs_na, rs_ws), (path, batch)
        assert torch.equal(cs_na, cs_ws), (path, batch)


@pytest.mark.gpu
def test_noalloc_past_the_scratch_takes_the_fused_kernel():
    """520 rows need 16.25 MiB of activations on the conv + recurrence pair,
    past the scratch: the default noalloc call then takes the fused kernel,
    while gdn_decode_step takes the pair for that batch -- the same bits."""
    dims = gdn.make_dims(H, HV, DK, DK, 4)
    assert gdn.gdn_decode_step_fused(dims, 520) == 0       # the plain call: the pair
    (o_ws, cs_ws, rs_ws), (o_na, cs_na, rs_na) = _pair(520, 13, gdn.DEFAULT_DECODE_FLAGS)
    assert not torch.isnan(o_na).any()
    assert torch.equal(o_na, o_ws)
    assert torch.equal(rs_na, rs_ws)
    assert torch.equal(cs_na, cs_ws)
