"""Seeded synthetic inputs for the GDN decode step and chunked prefill.

This module is shared by the tests, the benchmark and the smoke check.  It
draws random numbers and lays them out; it holds none of the method's
arithmetic, and it imports neither the oracle nor the HIP binding.

Shapes and distributions follow the workloads described for the method:
  * decode at the Qwen3-Next-like shape (16 key heads, 32 value heads,
    d_k = d_v = 128, conv width 4 over 8192 channels, bf16 conv cache, fp32
    recurrent state, shuffled slot indices; RL-Kernel PR #469, "Summary" and
    the provider-agreement test dims);
  * chunked varlen prefill with cu_seqlens and 64-token chunks;
  * the correlated-key stress prefill (beta = 0.9, g = 0, zero fp32 state;
    vLLM PR #53864, "Numerical root cause and fix").
Where the pages leave a distribution open, the choice is stated inline.

Everything is generated with ``torch.Generator`` seeded per call on the CPU
(or on ``gen_device`` when given, for the multi-GiB caches of the benchmark);
the caller moves tensors to the GPU.
"""
import math

import torch

SLOT_NULL = 0  # slot 0 is reserved and never addressed


def _gen(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def draw_slots(n_active, num_slots, gen, device="cpu"):
    """n_active distinct slots from 1..num_slots-1, in shuffled order."""
    if n_active > num_slots - 1:
        raise ValueError("not enough slots")
    perm = torch.randperm(num_slots - 1, generator=gen, device=device)[:n_active] + 1
    return perm.to(torch.int32)


def conv_dim(H, HV, dk, dv):
    return 2 * H * dk + HV * dv


def decode_inputs(batch, num_slots, H=16, HV=32, dk=128, dv=128, W=4,
                  act_dtype=torch.bfloat16, seed=1, state_std=0.1,
                  g_mode="uniform", qkv_normalised=False, conv_cache_std=1.0,
                  conv_bias=False, gen_device="cpu"):
    """One decode step's inputs plus fresh caches.

    * mixed_qkv [B, D] act_dtype ~ N(0, 1)        (q | k | v channel order)
    * g [B, HV] fp32: U[-1, 0] ("uniform"), or -softplus(N(0,1)) ("softplus")
    * beta [B, HV] fp32 = sigmoid(N(0, 1))
    * slot_idx [B] int32: distinct, shuffled, drawn from 1..num_slots-1
    * conv_state [num_slots, D, W-1] act_dtype ~ N(0, conv_cache_std^2)
    * conv_weight [D, W] act_dtype ~ U(-1/2, 1/2) (depthwise-conv default bound
      1/sqrt(W) at W = 4); conv_bias [D] ~ U(-1/2, 1/2) when requested
    * rec_state [num_slots, HV, dv, dk] fp32 ~ N(0, state_std^2)
      ("N(0, 0.1)" is read as standard deviation 0.1)
    """
    gen = _gen(seed, gen_device)
    D = conv_dim(H, HV, dk, dv)
    dev = gen_device
    x = torch.randn(batch, D, generator=gen, device=dev)
    if g_mode == "uniform":
        g = -torch.rand(batch, HV, generator=gen, device=dev)
    elif g_mode == "softplus":
        g = -torch.nn.functional.softplus(torch.randn(batch, HV, generator=gen, device=dev))
    else:
        raise ValueError(g_mode)
    beta = torch.sigmoid(torch.randn(batch, HV, generator=gen, device=dev))
    slots = draw_slots(batch, num_slots, gen, device=dev)
    conv_state = (torch.randn(num_slots, D, W - 1, generator=gen, device=dev)
                  * conv_cache_std).to(act_dtype)
    weight = (torch.rand(D, W, generator=gen, device=dev) - 0.5).to(act_dtype)
    bias = ((torch.rand(D, generator=gen, device=dev) - 0.5).to(act_dtype)
            if conv_bias else None)
    if state_std == 0:
        rec = torch.zeros(num_slots, HV, dv, dk, device=dev)
    else:
        rec = torch.randn(num_slots, HV, dv, dk, generator=gen, device=dev).mul_(state_std)
    return dict(mixed_qkv=x.to(act_dtype), g=g.float(), beta=beta.float(),
                slot_idx=slots, conv_state=conv_state, conv_weight=weight,
                conv_bias=bias, rec_state=rec,
                dims=dict(H=H, HV=HV, dk=dk, dv=dv, W=W))


def gating_inputs(rows, HV, seed=0, ab_dtype=torch.bfloat16, threshold_frac=0.05):
    """Raw projections for fused gating.

    * a [rows, HV] ab_dtype ~ 3 N(0, 1); a fraction ``threshold_frac`` of the
      entries is shifted by +25 so that a + dt_bias exceeds the softplus
      threshold (20)
    * b [rows, HV] ab_dtype ~ 2 N(0, 1)
    * A_log [HV] fp32 ~ U(0, log 16)
    * dt_bias [HV] fp32 ~ U(-7, -2)
    """
    gen = torch.Generator().manual_seed(seed + 3000)
    a = 3.0 * torch.randn(rows, HV, generator=gen)
    big = torch.rand(rows, HV, generator=gen) < threshold_frac
    a = a + 25.0 * big
    b = 2.0 * torch.randn(rows, HV, generator=gen)
    A_log = torch.rand(HV, generator=gen) * 2.772588722239781
    dt_bias = -2.0 - 5.0 * torch.rand(HV, generator=gen)
    return dict(a=a.to(ab_dtype), b=b.to(ab_dtype), A_log=A_log.float(), dt_bias=dt_bias.float())


def seqlens_uniform(n_seqs, lo, hi, gen):
    """n_seqs integer lengths uniform in [lo, hi]."""
    return torch.randint(lo, hi + 1, (n_seqs,), generator=gen).tolist()


def cu_from_lengths(lengths):
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32)


def prefill_inputs(lengths, num_slots, H=16, HV=32, dk=128, dv=128,
                   in_dtype=torch.bfloat16, seed=3, state_std=0.1,
                   g_mode="uniform", qk_normalised=False, gen_device="cpu"):
    """Varlen prefill inputs: q, k [T, H, dk], v [T, HV, dv], g, beta [T, HV].

    q, k, v ~ N(0, 1) (q and k L2-normalised first when ``qk_normalised``);
    g ~ U[-1, 0] ("uniform") or -softplus(N(0,1)) ("softplus");
    beta = sigmoid(N(0, 1)); initial states ~ N(0, state_std^2) in the slots
    the sequences use (zero when state_std == 0); slots distinct and shuffled.
    """
    gen = _gen(seed, gen_device)
    dev = gen_device
    T = int(sum(lengths))
    q = torch.randn(T, H, dk, generator=gen, device=dev)
    k = torch.randn(T, H, dk, generator=gen, device=dev)
    if qk_normalised:
        q = q / q.norm(dim=-1, keepdim=True)
        k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn(T, HV, dv, generator=gen, device=dev)
    if g_mode == "uniform":
        g = -torch.rand(T, HV, generator=gen, device=dev)
    elif g_mode == "softplus":
        g = -torch.nn.functional.softplus(torch.randn(T, HV, generator=gen, device=dev))
    else:
        raise ValueError(g_mode)
    beta = torch.sigmoid(torch.randn(T, HV, generator=gen, device=dev))
    slots = draw_slots(len(lengths), num_slots, gen, device=dev)
    rec = torch.zeros(num_slots, HV, dv, dk, device=dev)
    if state_std:
        for s in slots.tolist():
            rec[s].normal_(0.0, state_std, generator=gen)
    return dict(q=q.to(in_dtype), k=k.to(in_dtype), v=v.to(in_dtype), g=g.float(),
                beta=beta.float(), cu_seqlens=cu_from_lengths(lengths).to(dev),
                slot_idx=slots, rec_state=rec, dims=dict(H=H, HV=HV, dk=dk, dv=dv))


def stress_prefill_inputs(T, H=16, HV=32, d=128, noise=0.05, beta=0.9, seed=4,
                          in_dtype=torch.bfloat16, num_slots=2):
    """Correlated-key stress case (vLLM PR #53864, "Numerical root cause and fix").

    One sequence of T tokens; k_t = normalise(base_h + noise * N(0,1)) with one
    base_h ~ N(0, 1) per key head; q, v ~ N(0, 1); beta = 0.9; g = 0; zero fp32
    initial state.
    """
    gen = _gen(seed)
    base = torch.randn(1, H, d, generator=gen)
    k = base + noise * torch.randn(T, H, d, generator=gen)
    k = k / k.norm(dim=-1, keepdim=True)
    q = torch.randn(T, H, d, generator=gen)
    v = torch.randn(T, HV, d, generator=gen)
    g = torch.zeros(T, HV)
    b = torch.full((T, HV), float(beta))
    rec = torch.zeros(num_slots, HV, d, d)
    return dict(q=q.to(in_dtype), k=k.to(in_dtype), v=v.to(in_dtype), g=g, beta=b,
                cu_seqlens=torch.tensor([0, T], dtype=torch.int32),
                slot_idx=torch.tensor([1], dtype=torch.int32), rec_state=rec,
                dims=dict(H=H, HV=HV, dk=d, dv=d))


def tiny_config(seed=0):
    """The tiny end-to-end case: 2 sequences, H=2, HV=4, d=32, W=4, fp32
    everywhere; prefill of 64 tokens each then 8 decode steps; q, k L2-normalised,
    v ~ N(0,1), beta = sigmoid(N(0,1)), g = -softplus(N(0,1)), zero states,
    8-slot cache; decode mixed_qkv ~ N(0, 1), conv weight ~ U(-1/2, 1/2)."""
    H, HV, d, W, n_seqs, T_each, steps, num_slots = 2, 4, 32, 4, 2, 64, 8, 8
    gen = _gen(seed + 1000)            # decode draws: a stream apart from the prefill's
    pre = prefill_inputs([T_each] * n_seqs, num_slots, H=H, HV=HV, dk=d, dv=d,
                         in_dtype=torch.float32, seed=seed, state_std=0.0,
                         g_mode="softplus", qk_normalised=True)
    D = conv_dim(H, HV, d, d)
    dec = []
    for _ in range(steps):
        dec.append(dict(
            mixed_qkv=torch.randn(n_seqs, D, generator=gen),
            g=-torch.nn.functional.softplus(torch.randn(n_seqs, HV, generator=gen)),
            beta=torch.sigmoid(torch.randn(n_seqs, HV, generator=gen))))
    weight = torch.rand(D, W, generator=gen) - 0.5
    conv_state = torch.zeros(num_slots, D, W - 1)
    return dict(prefill=pre, decode=dec, conv_weight=weight, conv_state=conv_state,
                dims=dict(H=H, HV=HV, dk=d, dv=d, W=W), scale=1.0 / math.sqrt(d))
