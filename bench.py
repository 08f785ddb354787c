#!/usr/bin/env python3
"""Benchmark of the GDN hot path on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
  * decode step at batch 256 drawn from a 2048-slot cache (16 key heads,
    32 value heads, d = 128, conv width 4 over 8192 channels, bf16 conv cache,
    fp32 state): gdn_decode_step, the headline workload;
  * decode step at batch 16 from a 256-slot cache (the small bucket);
  * chunked prefill of 8 sequences with lengths uniform in [512, 8192]
    (about 32k tokens), bf16 q/k/v, fp32 states (when the prefill is built).
Inputs are resident in HBM before the timed region.  Successive steps rotate
over disjoint slot sets so the 256 MB Infinity Cache (MALL) cannot serve a
state written in a recent step.

Prints ONE JSON line.  `value` is the decode step's algorithmic HBM bytes per
second at batch 256 (GB/s); the batch-16 decode rate and the prefill tokens/s
ride along in "extra".  "roofline" reports the headline step's dominant kernel
timed alone: at batch 256 the step is the conv kernel followed by the
recurrence kernel (the library's choice for that batch; the fused one-kernel
step serves one or two (row, key head) groups per CU), and the recurrence kernel
carries ~92% of its time.  Timing: blocks of back-to-back eager launches, one
HIP event pair on their stream per block, the block time divided by its
launches; the whole step and the fused kernel are timed the same way alongside.  "cpu_baseline" is the
fp64 oracle on a bounded sample of the same workload, run over independent
rows on the host's threads (at most 16); the one-thread figure is in "extra".
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA

H, HV, DK, DV, W = 16, 32, 128, 128, 4
D = 2 * H * DK + HV * DV


def decode_bytes_per_seq(x_bytes=2, cs_bytes=2, out_bytes=4):
    """Algorithmic HBM bytes of one decode row: state read + write, conv state
    read + write, the new token, g and beta, the slot index and the output."""
    state = 2 * HV * DV * DK * 4
    conv = 2 * D * (W - 1) * cs_bytes
    return state + conv + D * x_bytes + 2 * HV * 4 + 4 + HV * DV * out_bytes


def rec_bytes_per_seq(y_bytes=4, out_bytes=4):
    """Algorithmic bytes of the recurrence kernel alone (post-conv activations in)."""
    return 2 * HV * DV * DK * 4 + D * y_bytes + 2 * HV * 4 + 4 + HV * DV * out_bytes


def conv_weight_bytes(w_bytes=2):
    return D * W * w_bytes


def prefill_flops(lengths, chunk=64):
    """MFMA-shaped FLOPs of the chunked prefill: per chunk of length L,
    HV (6 L^2 d + 6 L d^2) + H (4 L^2 d)."""
    f = 0
    for n in lengths:
        for c0 in range(0, n, chunk):
            L = min(chunk, n - c0)
            f += HV * (6 * L * L * DK + 6 * L * DK * DV) + H * 4 * L * L * DK
    return f


def prefill_bytes(total_tokens, n_seqs, in_bytes=2, out_bytes=2):
    per_tok = (2 * H * DK + HV * DV) * in_bytes + 2 * HV * 4 + HV * DV * out_bytes
    return total_tokens * per_tok + n_seqs * 2 * HV * DV * DK * 4


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_kernel_b256_traffic.txt")
REC_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_rec_kernel_b256_traffic.txt")
DECODE_SRC = os.path.join(ROOT, "gated_deltanet_recurrent_gdn_amd", "csrc", "decode.hip")


PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_call_varlen_traffic.txt")
PREFILL_SRC = os.path.join(ROOT, "gated_deltanet_recurrent_gdn_amd", "csrc", "prefill.hip")
CONV_COUNTER_FILE = os.path.join(ROOT, "profiles", "conv_varlen_tok_kernel_valu.txt")
CONV_SRC = os.path.join(ROOT, "gated_deltanet_recurrent_gdn_amd", "csrc", "conv.hip")
# vector ALU issue peak: 256 CUs x 4 SIMDs, one wave64 instruction per SIMD every
# 4 cycles (16 lanes wide), 2.4 GHz
VALU_PEAK_WAVE_INSTS = 256 * 2.4e9


def sources_sha256(src_path):
    """sha256 over a kernel's source file followed by every header it can
    include (the package's csrc/*.hpp, then include/*.h, each set in name
    order): a change to any of them invalidates counters taken before it."""
    import glob
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "gated_deltanet_recurrent_gdn_amd", "csrc")
    for f in [src_path] + sorted(glob.glob(os.path.join(pkg, "*.hpp"))) + \
            sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()


def counter_summary(path, src_path, key):
    """The key = value lines of a committed counter summary, or None when the
    kernel's sources have changed since those counters were taken."""
    try:
        kv = {}
        for line in open(path):
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        return kv if kv.get(key) == sources_sha256(src_path) else None
    except OSError:
        return None


def measured_traffic(path=TRAFFIC_FILE, src_path=DECODE_SRC, key="decode_sources_sha256"):
    """HBM bytes per launch from a committed counter summary (FETCH_SIZE +
    WRITE_SIZE, copy-calibrated) -- by default the fused step kernel at batch
    256 -- or None when the kernel's source has changed since those counters
    were taken."""
    kv = counter_summary(path, src_path, key)
    try:
        return int(kv["fetch_bytes_per_launch"]) + int(kv["write_bytes_per_launch"])
    except (TypeError, KeyError, ValueError):
        return None


def conv_roofline(ms, alg_bytes):
    """The varlen conv call (token kernel + roll kernel) against HBM: algorithmic
    bytes over the call's live mean time; traffic and the token kernel's vector
    ALU issue rate come from the committed counter summary (SQ_INSTS_VALU over
    the same live time, against 256 CUs x one wave64 instruction per cycle) and
    are None once the conv sources have changed since those counters."""
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    kv = counter_summary(CONV_COUNTER_FILE, CONV_SRC, "conv_sources_sha256")
    out = {"bound": "hbm", "kernel": "conv_varlen_tok_kernel + conv_roll_kernel",
           "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": alg_bytes,
           "traffic": None, "valu_issue_frac": None}
    if kv is not None:
        out["traffic"] = int(kv["fetch_bytes_per_launch"]) + int(kv["write_bytes_per_launch"])
        out["valu_issue_frac"] = round(float(kv["valu_wave_insts_per_launch"]) / (ms * 1e-3) /
                                       VALU_PEAK_WAVE_INSTS, 4)
    return out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle sample")
    ap.add_argument("--validate", action="store_true",
                    help="time with device-side index validation on")
    ap.add_argument("--eager", action="store_true",
                    help="time decode steps as eager launches instead of graph replay "
                         "(for counter collection)")

    return ap.parse_args()


class DecodeSetup:
    """A decode workload with K disjoint slot sets rotated step to step."""

    def __init__(self, batch, num_slots, seed, dev):
        import torch
        import gdn_inputs as gi
        import gated_deltanet_recurrent_gdn_amd as gdn
        self.torch, self.gdn = torch, gdn
        self.batch = batch
        d = gi.decode_inputs(batch, num_slots, seed=seed, gen_device=dev)
        self.d = d
        gen = torch.Generator(device="cpu")
        gen.manual_seed(seed + 100)
        perm = (torch.randperm(num_slots - 1, generator=gen) + 1).to(torch.int32)
        nsets = max(1, (num_slots - 1) // batch)
        self.slot_sets = [perm[i * batch:(i + 1) * batch].to(dev) for i in range(nsets)]
        self.dims = gdn.make_dims(H, HV, DK, DV, W)
        self.out = torch.empty(batch, HV, DV, device=dev)
        self.ws = torch.empty(gdn.gdn_decode_workspace_size(self.dims, batch),
                              dtype=torch.uint8, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.y = torch.empty(batch, D, device=dev)          # post-conv activations
        self.scale = DK ** -0.5
        self.i = 0
        self.gate = None
        self.extra_flags = 0                                 # e.g. force a step path

    def use_gating(self, seed):
        """Switch the step to the fused-gating call (raw a, b projections in bf16)."""
        import gdn_inputs as gi
        gt = gi.gating_inputs(self.batch, HV, seed=seed)
        gt = {k: v.to(self.out.device) for k, v in gt.items()}
        self.gate = self.gdn.GateInputs(gt["a"], gt["b"], gt["A_log"], gt["dt_bias"])

    def step(self, validate=False):
        gdn = self.gdn
        d = self.d
        slots = self.slot_sets[self.i % len(self.slot_sets)]
        self.i += 1
        flags = (gdn.DEFAULT_DECODE_FLAGS | (gdn.FLAG_VALIDATE if validate else 0) |
                 self.extra_flags)
        if self.gate is not None:
            gdn.gdn_decode_step_gated(d["mixed_qkv"], self.gate, slots, d["conv_state"],
                                      d["conv_weight"], d["rec_state"], self.out, self.dims,
                                      self.scale, flags=flags, workspace=self.ws,
                                      err_flag=self.err if validate else None)
            return
        gdn.gdn_decode_step(d["mixed_qkv"], d["g"], d["beta"], slots, d["conv_state"],
                            d["conv_weight"], d["rec_state"], self.out, self.dims, self.scale,
                            flags=flags, workspace=self.ws,
                            err_flag=self.err if validate else None)

    def capture(self, validate=False):
        """One HIP graph holding one step per disjoint slot set, in order
        (replayed as a unit)."""
        torch = self.torch
        self.i = 0
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):          # warm the capture path once
            self.step(validate)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        self.i = 0
        with torch.cuda.graph(graph):
            for _ in range(len(self.slot_sets)):
                self.step(validate)
        torch.cuda.synchronize()
        return graph, len(self.slot_sets)

    def prepare_rec(self):
        gdn = self.gdn
        d = self.d
        gdn.gdn_conv_update(d["mixed_qkv"], self.slot_sets[0], d["conv_state"].clone(),
                            d["conv_weight"], self.y, flags=gdn.FLAG_SILU)

    def rec_step(self):
        gdn = self.gdn
        d = self.d
        slots = self.slot_sets[self.i % len(self.slot_sets)]
        self.i += 1
        gdn.gdn_decode_recurrent(self.y, d["g"], d["beta"], slots, d["rec_state"], self.out,
                                 self.dims, self.scale)


class MixedSetup:
    """A mixed step on the batch-256 decode workload's caches: its first slot
    set's 256 decode rows plus two 1024-token prefill sequences on slots that
    no decode slot set uses."""

    def __init__(self, big, seed, dev):
        import torch
        import gdn_inputs as gi
        self.torch, self.gdn, self.big = torch, big.gdn, big
        self.lengths = [1024, 1024]
        T = sum(self.lengths)
        gen = torch.Generator().manual_seed(seed)
        xp = torch.randn(T, D, generator=gen).to(torch.bfloat16)
        gp = -torch.rand(T, HV, generator=gen)
        bp = torch.sigmoid(torch.randn(T, HV, generator=gen))
        d = big.d
        self.x = torch.cat([d["mixed_qkv"], xp.to(dev)])
        self.g = torch.cat([d["g"], gp.to(dev)])
        self.beta = torch.cat([d["beta"], bp.to(dev)])
        used = set(torch.cat(big.slot_sets).tolist())
        spare = [s for s in range(1, d["rec_state"].shape[0]) if s not in used][:2]
        self.slots = torch.cat([big.slot_sets[0],
                                torch.tensor(spare, dtype=torch.int32, device=dev)])
        self.cu = gi.cu_from_lengths(self.lengths).to(dev)
        self.out = torch.empty(256 + T, HV, DV, device=dev)
        dims = big.dims
        # beside decode rows the prefill part runs whole sequences: the
        # minimal workspace is all the step uses
        self.ws = torch.empty(big.gdn.gdn_mixed_workspace_size(dims, 256, T),
                              dtype=torch.uint8, device=dev)
        self.T = T

        self.streams = big.gdn.MixedStreams()

    def step(self, overlap=True):
        """One mixed step; overlap: the prefill part on the caller-owned second
        stream (forked and joined by events), else both parts in order."""
        b = self.big
        d = b.d
        self.gdn.gdn_mixed_step(self.x, self.g, self.beta, 256, self.cu, self.slots,
                                d["conv_state"], d["conv_weight"], d["rec_state"], self.out,
                                b.dims, b.scale, workspace=self.ws,
                                streams=self.streams if overlap else None)

    def step_serial(self):
        self.step(overlap=False)


class PrefillSetup:
    """The varlen prefill workload: 8 sequences, lengths uniform in [512, 8192]
    (drawn with the workload's seed).  `copies` input sets of those lengths
    (the first with the workload's seed, the others with their own), each with
    its own states, slots and output, are rotated call to call so that no call
    finds the previous call's inputs in the 256 MB Infinity Cache."""

    def __init__(self, seed, dev, copies=3):
        import torch
        import gdn_inputs as gi
        import gated_deltanet_recurrent_gdn_amd as gdn
        self.torch, self.gdn = torch, gdn
        gen = torch.Generator().manual_seed(seed)
        self.lengths = gi.seqlens_uniform(8, 512, 8192, gen)
        self.sets = []
        for c in range(copies):
            p = gi.prefill_inputs(self.lengths, 16, seed=seed + 1000 * c)
            self.sets.append({k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
                              for k, v in p.items()})
        self.p = self.sets[0]
        self.T = int(sum(self.lengths))
        self.dims = gdn.make_dims(H, HV, DK, DV, W)
        self.outs = [torch.empty(self.T, HV, DV, dtype=torch.bfloat16, device=dev)
                     for _ in range(copies)]
        self.out = self.outs[0]
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.gate = None
        self.i = 0
        # the workspace with which the call takes the schedule it picks for
        # these sizes (on a busy chip: heads plus tail segments)
        self.ws = torch.empty(max(1, gdn.gdn_prefill_workspace_size(self.dims, 8, self.T)),
                              dtype=torch.uint8, device=dev)
        self.whole = False

    def rotate(self):
        """Move to the next input set (and its output buffer)."""
        self.i = (self.i + 1) % len(self.sets)
        self.p, self.out = self.sets[self.i], self.outs[self.i]

    def use_gating(self, seed):
        import gdn_inputs as gi
        gt = gi.gating_inputs(self.T, HV, seed=seed)
        gt = {k: v.to(self.out.device) for k, v in gt.items()}
        self.gate = self.gdn.GateInputs(gt["a"], gt["b"], gt["A_log"], gt["dt_bias"])

    def step(self, validate=False):
        gdn = self.gdn
        self.rotate()
        p = self.p
        flags = gdn.FLAG_QK_L2NORM | (gdn.FLAG_VALIDATE if validate else 0)
        if self.whole:
            flags |= gdn.FLAG_PREFILL_SEQUENTIAL
        if self.gate is not None:
            gdn.gdn_prefill_chunked_gated(p["q"], p["k"], p["v"], self.gate, p["cu_seqlens"],
                                          p["slot_idx"], p["rec_state"], self.out, self.dims,
                                          DK ** -0.5, flags=flags, workspace=self.ws,
                                          err_flag=self.err if validate else None)
            return
        gdn.gdn_prefill_chunked(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu_seqlens"],
                                p["slot_idx"], p["rec_state"], self.out, self.dims, DK ** -0.5,
                                flags=flags, workspace=self.ws,
                                err_flag=self.err if validate else None)

    def step_whole(self):
        """The same call with GDN_FLAG_PREFILL_SEQUENTIAL: one run per (sequence, value head)."""
        self.whole = True
        try:
            self.step()
        finally:
            self.whole = False


def time_graph(torch, graph, per_replay, steps, warmup, min_replays=5):
    """Replay a captured graph of `per_replay` steps (at least `steps` steps and
    `min_replays` replays); per-step ms for each replay."""
    for _ in range(max(1, warmup // per_replay)):
        graph.replay()
    torch.cuda.synchronize()
    n = max(min_replays, -(-steps // per_replay))
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for i in range(n):
        starts[i].record()
        graph.replay()
        ends[i].record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) / per_replay for s, e in zip(starts, ends)]


def time_loop(torch, fn, steps, warmup):
    """Per-launch event timing on the current stream; returns a list of ms."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in zip(starts, ends)]


def time_block(torch, fn, steps, warmup, rounds=3):
    """Average launch duration over a block of back-to-back launches: one event
    pair on the current stream around `steps` launches, divided by `steps`
    (so per-launch event packets do not add to each kernel); returns one mean
    per round."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    out = []
    for _ in range(rounds):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        out.append(s.elapsed_time(e) / steps)
    return out


def host_cpu_counts():
    """(CPUs this process may run on, CPUs the OS reports)."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    return aff, os.cpu_count() or aff


def host_threads():
    """Host threads for the oracle's all-cores leg: the CPUs this process may
    run on, at most 16 -- one GPU's share of the host, the share a one-GPU job
    is granted on the GPU hosts here, whatever the OS reports in total."""
    return max(1, min(16, host_cpu_counts()[0]))


def host_cpu_model():
    """The host CPU's model name (first /proc/cpuinfo entry), or "unknown"."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_oracle_threads(n_threads, budget_s, make_unit):
    """Run independent oracle units on n_threads threads for budget_s seconds.

    make_unit(i) builds thread i's own inputs and caches (untimed) and returns
    (work, units): work() makes one oracle call covering `units` rows or
    tokens.  The oracle is C called through ctypes, which releases the GIL, so
    the threads run in parallel; nothing is shared between them.  Returns
    (units done, wall seconds)."""
    import threading
    works = [make_unit(i) for i in range(n_threads)]
    done = [0] * n_threads
    start = threading.Barrier(n_threads + 1)
    deadline = [0.0]

    def body(i):
        work, units = works[i]
        start.wait()
        while time.perf_counter() < deadline[0]:
            work()
            done[i] += units

    threads = [threading.Thread(target=body, args=(i,)) for i in range(n_threads)]
    for t in threads:
        t.start()
    t0 = time.perf_counter()
    deadline[0] = t0 + budget_s
    start.wait()
    for t in threads:
        t.join()
    return sum(done), time.perf_counter() - t0


def decode_oracle_unit(B, seed):
    """One thread's decode sample: B rows of the batch-256 workload's shapes and
    distributions, with the thread's own fp64 caches."""
    import gdn_inputs as gi
    import oracle
    d = gi.decode_inputs(B, B + 1, seed=seed)
    x = d["mixed_qkv"].double().numpy()
    g = d["g"].double().numpy()
    b = d["beta"].double().numpy()
    slots = d["slot_idx"].numpy()
    cs = d["conv_state"].double().numpy().copy()
    rs = d["rec_state"].double().numpy().copy()
    w = d["conv_weight"].double().numpy()

    def work():
        oracle.decode_step(x, g, b, slots, cs, w, rs, H, HV, DK, DV, DK ** -0.5)
    return work, B


def prefill_oracle_unit(seed):
    """One thread's prefill sample: a 512-token sequence of the prefill
    workload's shapes and distributions (all 32 value heads), own fp64 state."""
    import gdn_inputs as gi
    import oracle
    p = gi.prefill_inputs([512], 2, seed=seed)
    args = [p[k].double().numpy() for k in ("q", "k", "v", "g", "beta")]
    rec = p["rec_state"].double().numpy().copy()
    cu, sl = p["cu_seqlens"].numpy(), p["slot_idx"].numpy()

    def work():
        oracle.prefill(*args, cu, sl, rec, DK ** -0.5)
    return work, 512


def cpu_baseline(budget_s, n_threads):
    """The fp64 oracle, as it stands, on decode rows of the batch-256 workload
    (same shapes and distributions): on n_threads threads over independent row
    samples (the reported figure) and on one thread.  Each leg runs for about
    budget_s seconds of wall time."""
    rows, dt = run_oracle_threads(n_threads, budget_s,
                                  lambda i: decode_oracle_unit(16, 2 + 100 * i))
    gbs = rows * decode_bytes_per_seq() / dt / 1e9
    rows1, dt1 = run_oracle_threads(1, budget_s, lambda i: decode_oracle_unit(64, 2))
    gbs1 = rows1 * decode_bytes_per_seq() / dt1 / 1e9
    aff, ncpu = host_cpu_counts()
    main = {"value": round(gbs, 4), "unit": "GB/s", "cores": n_threads, "kind": "oracle",
            "sample": f"{rows} decode rows (batch-16 steps on {n_threads} threads, each with "
                      f"its own rows and caches; shapes and distributions of the batch-256 "
                      f"workload) in {dt:.1f} s, fp64 C; host CPU '{host_cpu_model()}', "
                      f"nproc {aff} (affinity), {ncpu} CPUs reported by the OS; threads "
                      f"capped at 16, one GPU's share of the host",
            "nproc": aff, "os_cpus": ncpu, "cpu_model": host_cpu_model()}
    one = {"value": round(gbs1, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{rows1} decode rows (steps of batch 64) in {dt1:.1f} s, "
                     "single-threaded fp64 C"}
    return main, one


def cpu_baseline_prefill(budget_s, n_threads):
    """The fp64 oracle prefill on 512-token sequences of the prefill workload's
    shapes (all 32 value heads), one independent sequence per thread."""
    toks, dt = run_oracle_threads(n_threads, budget_s, lambda i: prefill_oracle_unit(3 + 100 * i))
    return {"value": round(toks / dt, 2), "unit": "tokens/s", "cores": n_threads, "kind": "oracle",
            "sample": f"{toks} prefill tokens (512-token sequences, H=16 HV=32 d=128, one per "
                      f"thread on {n_threads} threads) in {dt:.1f} s, fp64 C, token by token"}


def gi_stress(T):
    import gdn_inputs as gi
    return gi.stress_prefill_inputs(T)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the GDN core "
              "implements no cross-GPU step.", file=sys.stderr)
        sys.exit(2)
    import torch
    import gated_deltanet_recurrent_gdn_amd as gdn
    gdn.load_library()                               # raises when not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # decode buckets: batch 1, 2, 4, 8, 16 from a 256-slot cache (seed 1) and
    # batch 256, 1024 from a 2048-slot cache (seed 2); each bucket has its own cache
    buckets = {b: DecodeSetup(b, 256, seed=1, dev="cuda") for b in (1, 2, 4, 8)}
    small = DecodeSetup(16, 256, seed=1, dev="cuda")
    buckets[16] = small
    big = DecodeSetup(256, 2048, seed=2, dev="cuda")
    buckets[256] = big
    pre = PrefillSetup(seed=3, dev="cuda")
    torch.cuda.synchronize()

    # copy calibration for counter runs: one device-to-device copy of 1 GiB
    # (1 GiB read + 1 GiB written by torch's elementwise copy kernel)
    cal_src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    bucket_ms, bucket_sets = {}, {}
    if args.eager:
        r_big = r_small = 1
        ms_big = time_loop(torch, lambda: big.step(args.validate), args.steps, args.warmup)
        ms_small = time_loop(torch, lambda: small.step(args.validate), args.steps, args.warmup)
    else:
        # decode buckets: graph replay of one step per disjoint slot set, at
        # least 5 replays per bucket (mean / min / max / spread over replays)
        for b in (1, 2, 4, 8, 16, 256):
            gph, nsets = buckets[b].capture(args.validate)
            bucket_ms[b] = time_graph(torch, gph, nsets, args.steps, args.warmup)
            bucket_sets[b] = nsets
            del gph
        ms_big, r_big = bucket_ms[256], bucket_sets[256]
        ms_small, r_small = bucket_ms[16], bucket_sets[16]
        for b in (1, 2, 4, 8):
            del buckets[b]
        # batch 1024 (one slot set of the 2048-slot cache: 4 GiB of state per
        # step, far past the Infinity Cache)
        huge = DecodeSetup(1024, 2048, seed=2, dev="cuda")
        gph, nsets = huge.capture(args.validate)
        bucket_ms[1024] = time_graph(torch, gph, nsets, args.steps, args.warmup)
        bucket_sets[1024] = nsets
        del gph, huge
        torch.cuda.synchronize()
    # prefill, eager (one call is milliseconds): the call's own schedule, and
    # whole runs alternating with it
    ms_pre, ms_pre_whole = [], []
    for _ in range(2):
        ms_pre += time_loop(torch, lambda: pre.step(args.validate), max(2, args.steps // 2), args.warmup)
        ms_pre_whole += time_loop(torch, pre.step_whole, max(2, args.steps // 2), args.warmup)
    # the headline step alone (eager launches back to back, one event pair on
    # their stream around each block), and the fused step kernel forced
    ms_step_k = time_block(torch, big.step, args.steps, args.warmup)
    big.extra_flags = gdn.FLAG_STEP_FUSED
    ms_fused_k = time_block(torch, big.step, args.steps, args.warmup)
    big.extra_flags = 0
    # the split path's recurrence kernel alone (post-conv activations in)
    big.prepare_rec()
    ms_rec = time_block(torch, big.rec_step, args.steps, args.warmup)
    torch.cuda.synchronize()
    # gated RMSNorm epilogue on the prefill output (o [T, HV, dv] bf16, z bf16, w fp32)
    zn = torch.randn(pre.T, HV, DV, device=dev).to(torch.bfloat16)
    wn = torch.ones(DV, device=dev)
    yn = torch.empty_like(pre.out)
    ms_norm = time_loop(torch, lambda: gdn.gdn_gated_rmsnorm(pre.out, wn, yn, z=zn),
                        args.steps, args.warmup)
    norm_bytes = pre.T * HV * DV * 2 * 3 + DV * 4
    del zn, yn
    # the varlen conv (gdn_conv_update with cu_seqlens) over the prefill
    # workload's token rows: pre-conv mixed q | k | v bf16 [T, 8192] -> bf16
    # activations, SiLU on, rolling the 8 sequences' conv slots
    cgen = torch.Generator().manual_seed(11)
    cx = torch.randn(pre.T, D, generator=cgen).to(torch.bfloat16).to(dev)
    ccs = torch.randn(16, D, W - 1, generator=cgen).to(torch.bfloat16).to(dev)
    cw = (torch.rand(D, W, generator=cgen) - 0.5).to(torch.bfloat16).to(dev)
    cy = torch.empty(pre.T, D, dtype=torch.bfloat16, device=dev)
    # block timing (one event pair around the steps' back-to-back calls), so the
    # per-call figure holds no event packets between the ~140 us calls
    ms_conv = time_block(torch, lambda: gdn.gdn_conv_update(cx, pre.p["slot_idx"], ccs, cw, cy,
                                                            cu_seqlens=pre.p["cu_seqlens"]),
                         args.steps, args.warmup)
    conv_bytes = pre.T * D * 2 * 2 + 2 * 8 * D * (W - 1) * 2 + D * W * 2
    del cx, ccs, cw, cy
    # the prefill with the Newton-Schulz (4 bf16 rounds) block-inverse variant
    ms_pre_ns4 = time_loop(torch, lambda: gdn.gdn_prefill_chunked(
        pre.p["q"], pre.p["k"], pre.p["v"], pre.p["g"], pre.p["beta"], pre.p["cu_seqlens"],
        pre.p["slot_idx"], pre.p["rec_state"], pre.out, pre.dims, DK ** -0.5,
        flags=gdn.FLAG_QK_L2NORM | gdn.FLAG_PREFILL_NS4), args.steps, args.warmup)
    # one long sequence (the correlated-key stress shape, 16384 tokens): whole-
    # sequence run vs the segment-parallel schedule the call picks by itself
    lp = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
          for k, v in gi_stress(16384).items()}
    lp_out = torch.empty(16384, HV, DV, dtype=torch.bfloat16, device=dev)
    lp_ws = torch.empty(max(1, gdn.gdn_prefill_workspace_size(pre.dims, 1, 16384)),
                        dtype=torch.uint8, device=dev)

    def long_prefill(extra_flags):
        gdn.gdn_prefill_chunked(lp["q"], lp["k"], lp["v"], lp["g"], lp["beta"], lp["cu_seqlens"],
                                lp["slot_idx"], lp["rec_state"], lp_out, pre.dims, DK ** -0.5,
                                flags=gdn.FLAG_QK_L2NORM | extra_flags, workspace=lp_ws)
    lsteps = max(3, args.steps // 4)
    ms_long_seq = time_loop(torch, lambda: long_prefill(gdn.FLAG_PREFILL_SEQUENTIAL), lsteps,
                            max(1, args.warmup // 2))
    ms_long_seg = time_loop(torch, lambda: long_prefill(0), lsteps, max(1, args.warmup // 2))
    del lp, lp_out, lp_ws
    # a mixed step: the batch-256 decode rows plus two 1024-token prefills, with
    # the prefill part overlapped on a second stream and in order on one,
    # alternating so both see the same conditions
    mixed = MixedSetup(big, seed=9, dev="cuda")
    ms_mixed, ms_mixed_serial = [], []
    for _ in range(3):
        ms_mixed += time_loop(torch, mixed.step, max(2, args.steps // 3), args.warmup)
        ms_mixed_serial += time_loop(torch, mixed.step_serial, max(2, args.steps // 3),
                                     args.warmup)
    # the same batch-256 step and prefill with the gating fused in (raw a, b)
    big.use_gating(seed=7)
    pre.use_gating(seed=8)
    if args.eager:
        ms_big_g = time_loop(torch, lambda: big.step(args.validate), args.steps, args.warmup)
    else:
        g_big_g, r_big_g = big.capture(args.validate)
        ms_big_g = time_graph(torch, g_big_g, r_big_g, args.steps, args.warmup)
    ms_pre_g = time_loop(torch, lambda: pre.step(args.validate), args.steps, args.warmup)
    torch.cuda.synchronize()

    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    med = lambda xs: sorted(xs)[len(xs) // 2]  # noqa: E731
    step_bytes_big = 256 * decode_bytes_per_seq() + conv_weight_bytes()
    step_bytes_small = 16 * decode_bytes_per_seq() + conv_weight_bytes()
    # gated step: bf16 a, b (4 B per head) replace fp32 g, beta (8 B), plus A_log, dt_bias
    step_bytes_big_gated = step_bytes_big - 256 * HV * 4 + 2 * HV * 4
    gbs_big = step_bytes_big / (mean(ms_big) * 1e-3) / 1e9
    gbs_small = step_bytes_small / (mean(ms_small) * 1e-3) / 1e9
    rec_ms = mean(ms_rec)
    rec_bytes = 256 * rec_bytes_per_seq()
    rec_gbs = rec_bytes / (rec_ms * 1e-3) / 1e9
    stepk_ms = mean(ms_step_k)
    stepk_gbs = step_bytes_big / (stepk_ms * 1e-3) / 1e9
    fusedk_ms = mean(ms_fused_k)
    fusedk_gbs = step_bytes_big / (fusedk_ms * 1e-3) / 1e9
    big_fused = gdn.gdn_decode_step_fused(big.dims, 256) == 1
    pre_ms = mean(ms_pre)
    pre_flops = prefill_flops(pre.lengths)
    pre_bytes = prefill_bytes(pre.T, len(pre.lengths))
    pre_tps = pre.T / (pre_ms * 1e-3)
    pre_tflops = pre_flops / (pre_ms * 1e-3) / 1e12

    extra = {
        "decode_b256_ms_mean": round(mean(ms_big), 5), "decode_b256_ms_median": round(med(ms_big), 5),
        "decode_b256_ms_min": round(min(ms_big), 5), "decode_b256_ms_max": round(max(ms_big), 5),
        "decode_b256_bytes_per_step": step_bytes_big,
        "decode_b256_pct_hbm_peak": round(100 * gbs_big / HBM_PEAK_GBS, 2),
        "decode_b16_GBps": round(gbs_small, 2),
        "decode_b16_ms_mean": round(mean(ms_small), 5),
        "decode_b16_pct_hbm_peak": round(100 * gbs_small / HBM_PEAK_GBS, 2),
        "decode_timing": ("eager launches with HIP events" if args.eager else
                          "HIP graph replay, one step per disjoint slot set "
                          f"({r_big} sets at batch 256, {r_small} at batch 16)"),
        "prefill_tokens": pre.T, "prefill_lengths": pre.lengths,
        "prefill_ms_mean": round(pre_ms, 4), "prefill_ms_min": round(min(ms_pre), 4),
        "prefill_tokens_per_s": round(pre_tps, 1),
        "prefill_roofline": {
            "bound": "mfma",
            "kernel": "gdn_prefill_chunked call (prefill_seg_map_kernel, prefill_pipe_kernel "
                      "pass 1, prefill_seg_scan_kernel, prefill_pipe_kernel pass 2)",
            "achieved": round(pre_tflops, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4),
            "hbm_frac": round(pre_bytes / (pre_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(PREFILL_TRAFFIC_FILE, PREFILL_SRC, "prefill_sources_sha256"),
            "algorithmic_flops_per_launch": pre_flops, "algorithmic_bytes_per_launch": pre_bytes,
            "note": ("the whole call, event-timed eager calls: on this busy chip the call's own "
                     "schedule is a segment map, pass 1 (each sequence's first 49 chunks, the "
                     "balanced per-CU share, and the P/B runs of longer sequences' tails on CUs "
                     "that short sequences free), a scan and pass 2 (the tails); bound by the "
                     "sequential chunk chain of the longest head and tail")},
        "prefill_whole_ms_mean": round(mean(ms_pre_whole), 4),
        "prefill_whole_note": "the same workload as one run per (sequence, value head), "
                              "GDN_FLAG_PREFILL_SEQUENTIAL, alternating with the timed calls",
        "prefill_TFLOPs": round(pre_tflops, 2),
        "prefill_pct_mfma_peak": round(100 * pre_tflops / BF16_PEAK_TFLOPS, 2),
        "prefill_algorithmic_flops": pre_flops, "prefill_algorithmic_bytes": pre_bytes,
        "prefill_pct_hbm_peak": round(100 * pre_bytes / (pre_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "prefill_ns4_ms_mean": round(mean(ms_pre_ns4), 4),
        "prefill_long_seq_ms_whole": round(mean(ms_long_seq), 4),
        "prefill_long_seq_ms_segmented": round(mean(ms_long_seg), 4),
        "prefill_long_seq_tokens_per_s_segmented": round(16384 / (mean(ms_long_seg) * 1e-3), 1),
        "prefill_long_seq_note": ("one 16384-token sequence (correlated keys, beta 0.9, g 0; "
                                  "H=16 HV=32 d=128): gdn_prefill_chunked with "
                                  "GDN_FLAG_PREFILL_SEQUENTIAL vs the segment-parallel schedule "
                                  "it picks with its workspace"),
        "conv_varlen_ms_mean": round(mean(ms_conv), 4),
        "conv_varlen_roofline": conv_roofline(mean(ms_conv), conv_bytes),
        "conv_varlen_GBps": round(conv_bytes / (mean(ms_conv) * 1e-3) / 1e9, 1),
        "conv_varlen_note": ("gdn_conv_update with cu_seqlens over the prefill workload's "
                             f"{pre.T} token rows: bf16 [T, {D}] in and out, SiLU, 8 conv "
                             "slots rolled (conv + roll kernels)"),
        "gated_rmsnorm_ms_mean": round(mean(ms_norm), 4),
        "gated_rmsnorm_GBps": round(norm_bytes / (mean(ms_norm) * 1e-3) / 1e9, 1),
        "gated_rmsnorm_note": ("gdn_gated_rmsnorm on the prefill output: "
                               f"{pre.T * HV} rows of {DV}, bf16 x, z, out, fp32 weight"),
        "mixed_step_ms_mean": round(mean(ms_mixed), 4),
        "mixed_step_serial_ms_mean": round(mean(ms_mixed_serial), 4),
        "mixed_step_note": ("gdn_mixed_step, eager: the 256 decode rows of the batch-256 "
                            "workload plus two 1024-token prefill sequences (pre-conv input), "
                            "prefill as whole runs; mixed_step: the prefill part on a "
                            "caller-owned second stream (fork / join events), overlapped with "
                            "the decode rows; *_serial: both parts in order on one stream; "
                            "the two alternate in the same run"),
        "decode_step_b256_block_ms_mean": round(stepk_ms, 5),
        "decode_step_b256_block_GBps": round(stepk_gbs, 2),
        "decode_step_b256_path": "fused kernel" if big_fused else "conv kernel + recurrence kernel",
        "decode_fused_kernel_b256_ms_mean": round(fusedk_ms, 5),
        "decode_fused_kernel_b256_GBps": round(fusedk_gbs, 2),
        "decode_fused_kernel_b256_pct_hbm_peak": round(100 * fusedk_gbs / HBM_PEAK_GBS, 2),
        "decode_fused_kernel_note": ("gdn_decode_step at batch 256 with GDN_FLAG_STEP_FUSED (the "
                                     "one-kernel step, bitwise the same results), eager blocks"),
        "decode_rec_kernel_b256_ms_mean": round(rec_ms, 5),
        "decode_rec_kernel_b256_GBps": round(rec_gbs, 2),
        "decode_rec_kernel_b256_pct_hbm_peak": round(100 * rec_gbs / HBM_PEAK_GBS, 2),
        "decode_rec_kernel_note": ("gdn_decode_recurrent alone at batch 256 (fp32 post-conv "
                                   "activations in): the recurrence kernel of the conv + "
                                   "recurrence path"),
        "decode_b256_gated_ms_mean": round(mean(ms_big_g), 5),
        "decode_b256_gated_GBps": round(step_bytes_big_gated / (mean(ms_big_g) * 1e-3) / 1e9, 2),
        "prefill_gated_ms_mean": round(mean(ms_pre_g), 4),
        "gated_note": ("the same steps through gdn_decode_step_gated / gdn_prefill_chunked_gated: "
                       "g and beta computed in-kernel from bf16 a, b and fp32 A_log, dt_bias"),
        "validate": bool(args.validate),
    }

    if bucket_ms:
        # per bucket, as the graph-replay table of the GB10 decode post does:
        # mean / min / max per step over the replays, spread = (max - min) / mean
        tab = {}
        for b, ms in sorted(bucket_ms.items()):
            by = b * decode_bytes_per_seq() + conv_weight_bytes()
            m = mean(ms)
            tab[str(b)] = {"ms_mean": round(m, 5), "ms_min": round(min(ms), 5),
                           "ms_max": round(max(ms), 5),
                           "spread": round((max(ms) - min(ms)) / m, 4),
                           "bytes_per_step": by, "GBps": round(by / (m * 1e-3) / 1e9, 1),
                           "pct_hbm_peak": round(100 * by / (m * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                           "slot_sets": bucket_sets[b], "replays": len(ms)}
        extra["decode_buckets"] = tab
        extra["decode_buckets_note"] = (
            "gdn_decode_step per bucket, HIP graph replay of one step per disjoint slot set "
            "(every set of the cache: batch 1..16 over a 256-slot cache, 256 and 1024 over a "
            "2048-slot cache), per-step time of each replay; bytes = 4325636 per row + the "
            "65536-byte conv weight")

    total_ms = mean(ms_big) + mean(ms_small) + pre_ms

    cpu = None
    if not args.no_cpu_baseline:
        nth = host_threads()
        cpu, extra["cpu_baseline_1thread"] = cpu_baseline(args.cpu_seconds / 2, nth)
        extra["cpu_baseline_prefill"] = cpu_baseline_prefill(max(4.0, args.cpu_seconds / 3), nth)

    if big_fused:
        roof = {"bound": "hbm", "kernel": "decode_step_kernel",
                "achieved": round(stepk_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(stepk_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "avg_launch_ms": round(stepk_ms, 5),
                "algorithmic_bytes_per_launch": step_bytes_big}
    else:
        roof = {"bound": "hbm", "kernel": "decode_rec_kernel",
                "achieved": round(rec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(rec_gbs / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(REC_TRAFFIC_FILE),
                "avg_launch_ms": round(rec_ms, 5),
                "algorithmic_bytes_per_launch": rec_bytes,
                "note": ("the dominant kernel of the batch-256 step (conv_decode_kernel, then "
                         "decode_rec_kernel on the fp32 activations); algorithmic bytes: state "
                         "read + write, activations, g, beta, slot, output")}

    line = {
        "metric": "GDN decode HBM GB/s (% peak) at batch 16/256; prefill tokens/s (% MFMA)",
        "value": round(gbs_big, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "GDN decode step, batch 256 of a 2048-slot cache, H=16 HV=32 "
                               "d=128, conv width 4 (D=8192), bf16 conv cache, fp32 state; "
                               "step also runs decode batch 16 and the 8-sequence varlen "
                               "prefill (see extra)",
                   "global_batch": 256, "seq_len": 1, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
