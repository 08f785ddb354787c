"""Shared helpers of the GPU tests: run the HIP path through the C ABI, run the
oracle on the same inputs, and compare.

The error metric is max|gpu - ref| / max|ref| against the fp64 oracle (the
metric of RL-Kernel PR #485, "Prior art & reuse decision", reused with the
bars stated for this method: 1e-5 for the decode output and state, 5e-3 for
the prefill output and final state; slot handling and conv rolls bit-exact).
"""
import hashlib

import numpy as np
import torch

import gated_deltanet_recurrent_gdn_amd as gdn
import oracle

DECODE_TOL = 1e-5
PREFILL_TOL = 5e-3


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(gpu - ref).max() if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def fnv64(t: torch.Tensor) -> str:
    """A content hash of a tensor's bytes (the replay check of the GDN graph
    post compares FNV64 hashes; any stable byte hash serves)."""
    b = t.detach().contiguous().cpu().view(torch.uint8).numpy().tobytes()
    return hashlib.blake2b(b, digest_size=8).hexdigest()


def to_dev(inp, device="cuda"):
    out = {}
    for k, v in inp.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out


PATH_FLAGS = {None: 0, "fused": gdn.FLAG_STEP_FUSED, "split": gdn.FLAG_STEP_SPLIT}


def run_decode_gpu(d, scale, flags=gdn.DEFAULT_DECODE_FLAGS, out_dtype=torch.float32,
                   err_flag=None, path=None):
    """d: dict of GPU tensors (decode_inputs layout); caches updated in place.
    path: None (the library's choice), "fused" or "split" (forced kernel path)."""
    flags |= PATH_FLAGS[path]
    dims = gdn.make_dims(d["dims"]["H"], d["dims"]["HV"], d["dims"]["dk"], d["dims"]["dv"],
                         d["dims"]["W"])
    B = d["mixed_qkv"].shape[0]
    out = torch.full((B, dims.num_v_heads, dims.head_v_dim), float("nan"),
                     dtype=out_dtype, device=d["mixed_qkv"].device)
    gdn.gdn_decode_step(d["mixed_qkv"], d["g"], d["beta"], d["slot_idx"], d["conv_state"],
                        d["conv_weight"], d["rec_state"], out, dims, scale,
                        conv_bias=d.get("conv_bias"), flags=flags, err_flag=err_flag)
    return out


def oracle_decode_rows(d_cpu, rows, scale, flags=oracle.FLAG_SILU | oracle.FLAG_QK_L2NORM):
    """Oracle decode for a subset of rows, on compact fp64 caches.

    Rows are independent, so each selected active row gets its own slot in a
    small cache (slot r+1 for the r-th selected row); inactive rows keep their
    index.  Returns (o [len(rows), HV, dv], conv rows, rec rows) in fp64."""
    dm = d_cpu["dims"]
    slots = d_cpu["slot_idx"][rows].numpy().astype(np.int32)
    active = slots > 0
    comp = np.where(active, np.arange(1, len(rows) + 1), slots).astype(np.int32)
    cs = np.zeros((len(rows) + 1,) + tuple(d_cpu["conv_state"].shape[1:]))
    rs = np.zeros((len(rows) + 1,) + tuple(d_cpu["rec_state"].shape[1:]))
    for i, (r, s) in enumerate(zip(rows, slots)):
        if s > 0:
            cs[i + 1] = f64(d_cpu["conv_state"][s])
            rs[i + 1] = f64(d_cpu["rec_state"][s])
    bias = None if d_cpu.get("conv_bias") is None else f64(d_cpu["conv_bias"])
    o = oracle.decode_step(f64(d_cpu["mixed_qkv"][rows]), f64(d_cpu["g"][rows]),
                           f64(d_cpu["beta"][rows]), comp, cs, f64(d_cpu["conv_weight"]), rs,
                           dm["H"], dm["HV"], dm["dk"], dm["dv"], scale, conv_bias=bias,
                           flags=flags)
    return o, cs[1:], rs[1:], active
