"""ctypes binding of libgdn.so -- argument marshalling only.

Every function here has the name of the C entry point it calls (see
``include/gdn.h``) and takes torch tensors that already live on the GPU.  It
checks dtypes, shapes and devices, passes raw device pointers and the current
HIP stream, and raises on a non-OK status.  No step of the computation happens
here, and there is no CPU fallback: without the built library every call
raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
FLAG_SILU, FLAG_QK_L2NORM, FLAG_VALIDATE = 1, 2, 4
FLAG_STEP_FUSED, FLAG_STEP_SPLIT = 8, 16
FLAG_PREFILL_NS3, FLAG_PREFILL_NS4 = 32, 64
FLAG_PREFILL_SEQUENTIAL = 128
FLAG_PREFILL_SINGLE_ROLE = 256
NORM_GATE_SIGMOID, NORM_ZERO_CENTRED = 1, 2
EFLAG_SLOT_RANGE, EFLAG_SLOT_REPEAT, EFLAG_SEQLENS = 1, 2, 4
DEFAULT_DECODE_FLAGS = FLAG_SILU | FLAG_QK_L2NORM
DEFAULT_PREFILL_FLAGS = FLAG_QK_L2NORM

_STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_DIMS", 3: "GDN_ERR_DTYPE",
           4: "GDN_ERR_ALIGN", 5: "GDN_ERR_WORKSPACE", 6: "GDN_ERR_LAUNCH", 7: "GDN_ERR_FLAGS"}

EXPORTED = ["gdn_conv_update", "gdn_decode_workspace_size", "gdn_decode_step", "gdn_decode_step_fused",
            "gdn_decode_step_gated", "gdn_decode_step_noalloc", "gdn_decode_recurrent",
            "gdn_prefill_workspace_size", "gdn_prefill_chunked", "gdn_prefill_chunked_gated",
            "gdn_prefill_segmented_workspace_size", "gdn_prefill_segmented",
            "gdn_mixed_workspace_size", "gdn_mixed_step", "gdn_gated_rmsnorm", "gdn_strerror"]


class GDNError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} returned {_STATUS.get(status, status)}: {gdn_strerror(status)}")


class gdn_dims(ctypes.Structure):
    _fields_ = [("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_k_dim", ctypes.c_int32), ("head_v_dim", ctypes.c_int32),
                ("conv_width", ctypes.c_int32)]


class gdn_gate_inputs(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("ab_dt", ctypes.c_int32),
                ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p)]


class GateInputs:
    """Raw gating inputs for the *_gated calls: a, b [rows, HV] (bf16 or fp32,
    the layout of the g / beta they replace), A_log and dt_bias [HV] fp32."""

    def __init__(self, a, b, A_log, dt_bias):
        self.a, self.b, self.A_log, self.dt_bias = a, b, A_log, dt_bias


_lib = None


def load_library(path: str = None):
    """Load libgdn.so; raise if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with "
                          "`python -m gated_deltanet_recurrent_gdn_amd.build`")
    lib = ctypes.CDLL(p)
    P, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    D = ctypes.POINTER(gdn_dims)
    lib.gdn_conv_update.argtypes = [P, i32, P, i32, i32, P, P, i32, i32, P, P, i32, P, i32,
                                    i32, i32, i32, P, P]
    lib.gdn_decode_workspace_size.argtypes = [D, i32]
    lib.gdn_decode_workspace_size.restype = sz
    lib.gdn_decode_step_fused.argtypes = [D, i32]
    lib.gdn_decode_step_fused.restype = i32
    lib.gdn_decode_step.argtypes = [P, i32, P, P, P, i32, P, i32, P, P, i32, P, i32, P, i32,
                                    D, f32, i32, P, sz, P, P]
    lib.gdn_decode_step_noalloc.argtypes = [P, i32, P, P, P, i32, P, i32, P, P, i32, P, i32, P,
                                            i32, D, f32, i32, P, P]
    lib.gdn_decode_recurrent.argtypes = [P, i32, P, P, P, i32, P, i32, P, i32, D, f32, i32,
                                         P, P]
    lib.gdn_prefill_workspace_size.argtypes = [D, i32, i32]
    lib.gdn_prefill_workspace_size.restype = sz
    lib.gdn_prefill_chunked.argtypes = [P, P, P, i32, P, P, P, i32, i32, P, P, i32, P, i32,
                                        D, f32, i32, P, sz, P, P]
    G = ctypes.POINTER(gdn_gate_inputs)
    lib.gdn_decode_step_gated.argtypes = [P, i32, G, P, i32, P, i32, P, P, i32, P, i32, P, i32,
                                          D, f32, i32, P, sz, P, P]
    lib.gdn_prefill_chunked_gated.argtypes = [P, P, P, i32, G, P, i32, i32, P, P, i32, P, i32,
                                              D, f32, i32, P, sz, P, P]
    lib.gdn_prefill_segmented_workspace_size.argtypes = [D, i32, i32, i32]
    lib.gdn_prefill_segmented_workspace_size.restype = sz
    lib.gdn_prefill_segmented.argtypes = [P, P, P, i32, P, P, G, P, i32, i32, P, P, i32, P, i32,
                                          D, f32, i32, i32, i32, P, sz, P, P]
    lib.gdn_mixed_workspace_size.argtypes = [D, i32, i32]
    lib.gdn_mixed_workspace_size.restype = sz
    lib.gdn_mixed_step.argtypes = [P, i32, P, P, i32, P, i32, i32, P, P, i32, P, P, i32, P, i32,
                                   P, i32, D, f32, i32, P, sz, P, P, P, P, P]
    lib.gdn_gated_rmsnorm.argtypes = [P, i32, P, P, i32, ctypes.c_int64, i32, f32, i32, P, i32, P]
    lib.gdn_strerror.argtypes = [i32]
    lib.gdn_strerror.restype = ctypes.c_char_p
    for f in (lib.gdn_conv_update, lib.gdn_decode_step, lib.gdn_decode_step_noalloc,
              lib.gdn_decode_recurrent,
              lib.gdn_prefill_chunked, lib.gdn_decode_step_gated, lib.gdn_prefill_chunked_gated,
              lib.gdn_mixed_step, lib.gdn_gated_rmsnorm, lib.gdn_prefill_segmented):
        f.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def gdn_strerror(status: int) -> str:
    return load_library().gdn_strerror(int(status)).decode()


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GDN_F32
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t, name, dtype=None, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_dims(H, HV, dk, dv, W=4) -> gdn_dims:
    return gdn_dims(H, HV, dk, dv, W)


def _check(fn, status):
    if status != 0:
        raise GDNError(fn, status)


def _gate_struct(gate: GateInputs, rows: int, HV: int) -> gdn_gate_inputs:
    _dev(gate.a, "a", shape=(rows, HV)); _dev(gate.b, "b", gate.a.dtype, (rows, HV))
    _dev(gate.A_log, "A_log", torch.float32, (HV,))
    _dev(gate.dt_bias, "dt_bias", torch.float32, (HV,))
    return gdn_gate_inputs(gate.a.data_ptr(), gate.b.data_ptr(), _dt(gate.a),
                           gate.A_log.data_ptr(), gate.dt_bias.data_ptr())


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------
def gdn_conv_update(x, slot_idx, conv_state, weight, out, bias=None, cu_seqlens=None,
                    flags=FLAG_SILU, err_flag=None, stream=None):
    """Causal conv1d update (gdn.h: gdn_conv_update).  ``x``/``out`` [T, dim],
    ``conv_state`` [num_slots, dim, W-1] rolled in place."""
    lib = load_library()
    T, dim = x.shape
    n = slot_idx.shape[0]
    _dev(x, "x"); _dev(out, "out", shape=(T, dim)); _dev(slot_idx, "slot_idx", torch.int32)
    _dev(conv_state, "conv_state"); _dev(weight, "weight"); _dev(bias, "bias", weight.dtype)
    _dev(cu_seqlens, "cu_seqlens", torch.int32, None if cu_seqlens is None else (n + 1,))
    _dev(err_flag, "err_flag", torch.int32)
    W = weight.shape[1]
    if conv_state.shape[1:] != (dim, W - 1) or weight.shape[0] != dim:
        raise ValueError("conv_state / weight shapes do not match x")
    _check("gdn_conv_update", lib.gdn_conv_update(
        _p(x), _dt(x), _p(cu_seqlens), n, T, _p(slot_idx), _p(conv_state), _dt(conv_state),
        conv_state.shape[0], _p(weight), _p(bias), _dt(weight), _p(out), _dt(out), dim, W,
        flags, _p(err_flag), _stream(stream)))
    return out


def gdn_decode_workspace_size(dims: gdn_dims, batch: int) -> int:
    return int(load_library().gdn_decode_workspace_size(ctypes.byref(dims), int(batch)))


def gdn_decode_step_fused(dims: gdn_dims, batch: int) -> int:
    """1 if gdn_decode_step takes the fused kernel for `batch` rows on this
    device, 0 for the conv + recurrence pair, -1 for invalid arguments."""
    return int(load_library().gdn_decode_step_fused(ctypes.byref(dims), int(batch)))


def _decode_step(fn, mixed_qkv, gb, gate, slot_idx, conv_state, conv_weight, rec_state, out,
                 dims, scale, conv_bias, flags, workspace, err_flag, stream):
    lib = load_library()
    B = mixed_qkv.shape[0]
    HV, dk, dv = dims.num_v_heads, dims.head_k_dim, dims.head_v_dim
    D = 2 * dims.num_k_heads * dk + HV * dv
    _dev(mixed_qkv, "mixed_qkv", shape=(B, D))
    if gate is None:
        _dev(gb[0], "g", torch.float32, (B, HV)); _dev(gb[1], "beta", torch.float32, (B, HV))
    _dev(slot_idx, "slot_idx", torch.int32, (B,))
    _dev(conv_state, "conv_state"); _dev(conv_weight, "conv_weight")
    _dev(conv_bias, "conv_bias", conv_weight.dtype)
    _dev(rec_state, "rec_state", torch.float32)
    _dev(out, "out", shape=(B, HV, dv)); _dev(err_flag, "err_flag", torch.int32)
    ns = rec_state.shape[0]
    if tuple(rec_state.shape[1:]) != (HV, dv, dk):
        raise ValueError("rec_state must be [num_slots, HV, dv, dk]")
    if tuple(conv_state.shape) != (ns, D, dims.conv_width - 1):
        raise ValueError("conv_state must be [num_slots, D, W-1] with the rec_state slot count")
    args = (_p(slot_idx), B, _p(conv_state), _dt(conv_state), _p(conv_weight), _p(conv_bias),
            _dt(conv_weight), _p(rec_state), ns, _p(out), _dt(out), ctypes.byref(dims),
            float(scale), flags)
    if fn == "gdn_decode_step_noalloc":          # no workspace: the library's scratch
        _check(fn, lib.gdn_decode_step_noalloc(_p(mixed_qkv), _dt(mixed_qkv), _p(gb[0]),
                                               _p(gb[1]), *args, _p(err_flag), _stream(stream)))
        return out
    need = gdn_decode_workspace_size(dims, B)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=mixed_qkv.device)
    _dev(workspace, "workspace")
    rest = (*args, _p(workspace), workspace.numel() * workspace.element_size(),
            _p(err_flag), _stream(stream))
    if gate is None:
        status = lib.gdn_decode_step(_p(mixed_qkv), _dt(mixed_qkv), _p(gb[0]), _p(gb[1]), *rest)
    else:
        gs = _gate_struct(gate, B, HV)
        status = lib.gdn_decode_step_gated(_p(mixed_qkv), _dt(mixed_qkv), ctypes.byref(gs), *rest)
    _check(fn, status)
    return out


def gdn_decode_step(mixed_qkv, g, beta, slot_idx, conv_state, conv_weight, rec_state, out,
                    dims: gdn_dims, scale, conv_bias=None, flags=DEFAULT_DECODE_FLAGS,
                    workspace=None, err_flag=None, stream=None):
    """One decode token per row (gdn.h: gdn_decode_step).  Caches in place;
    ``out`` [B, HV, dv] receives o.  A workspace is allocated when not given."""
    return _decode_step("gdn_decode_step", mixed_qkv, (g, beta), None, slot_idx, conv_state,
                        conv_weight, rec_state, out, dims, scale, conv_bias, flags, workspace,
                        err_flag, stream)


def gdn_decode_step_noalloc(mixed_qkv, g, beta, slot_idx, conv_state, conv_weight, rec_state,
                            out, dims: gdn_dims, scale, conv_bias=None,
                            flags=DEFAULT_DECODE_FLAGS, err_flag=None, stream=None):
    """gdn_decode_step without a workspace (gdn.h: gdn_decode_step_noalloc):
    nothing is allocated, here or in the library; the conv + recurrence path
    uses the library's per-device scratch array."""
    return _decode_step("gdn_decode_step_noalloc", mixed_qkv, (g, beta), None, slot_idx,
                        conv_state, conv_weight, rec_state, out, dims, scale, conv_bias, flags,
                        None, err_flag, stream)


def gdn_decode_step_gated(mixed_qkv, gate: GateInputs, slot_idx, conv_state, conv_weight,
                          rec_state, out, dims: gdn_dims, scale, conv_bias=None,
                          flags=DEFAULT_DECODE_FLAGS, workspace=None, err_flag=None, stream=None):
    """gdn_decode_step with the gating fused in (gdn.h: gdn_decode_step_gated)."""
    return _decode_step("gdn_decode_step_gated", mixed_qkv, None, gate, slot_idx, conv_state,
                        conv_weight, rec_state, out, dims, scale, conv_bias, flags, workspace,
                        err_flag, stream)


def gdn_decode_recurrent(qkv, g, beta, slot_idx, rec_state, out, dims: gdn_dims, scale,
                         flags=FLAG_QK_L2NORM, err_flag=None, stream=None):
    """Recurrent half of the decode step on post-conv activations ``qkv`` [B, D]
    (gdn.h: gdn_decode_recurrent).  ``rec_state`` in place; ``out`` [B, HV, dv]."""
    lib = load_library()
    B = qkv.shape[0]
    HV, dk, dv = dims.num_v_heads, dims.head_k_dim, dims.head_v_dim
    D = 2 * dims.num_k_heads * dk + HV * dv
    _dev(qkv, "qkv", shape=(B, D))
    _dev(g, "g", torch.float32, (B, HV)); _dev(beta, "beta", torch.float32, (B, HV))
    _dev(slot_idx, "slot_idx", torch.int32, (B,)); _dev(rec_state, "rec_state", torch.float32)
    _dev(out, "out", shape=(B, HV, dv)); _dev(err_flag, "err_flag", torch.int32)
    if tuple(rec_state.shape[1:]) != (HV, dv, dk):
        raise ValueError("rec_state must be [num_slots, HV, dv, dk]")
    _check("gdn_decode_recurrent", lib.gdn_decode_recurrent(
        _p(qkv), _dt(qkv), _p(g), _p(beta), _p(slot_idx), B, _p(rec_state), rec_state.shape[0],
        _p(out), _dt(out), ctypes.byref(dims), float(scale), flags, _p(err_flag),
        _stream(stream)))
    return out


def gdn_prefill_workspace_size(dims: gdn_dims, n_seqs: int, total_tokens: int) -> int:
    return int(load_library().gdn_prefill_workspace_size(ctypes.byref(dims), int(n_seqs),
                                                          int(total_tokens)))


def gdn_prefill_segmented_workspace_size(dims: gdn_dims, n_seqs: int, total_tokens: int,
                                         seg_len: int) -> int:
    return int(load_library().gdn_prefill_segmented_workspace_size(
        ctypes.byref(dims), int(n_seqs), int(total_tokens), int(seg_len)))


def _prefill(fn, q, k, v, gb, gate, cu_seqlens, slot_idx, rec_state, out, dims, scale, flags,
             workspace, err_flag, stream, seg_len=None, head_len=0):
    lib = load_library()
    T = q.shape[0]
    H, HV, dk, dv = dims.num_k_heads, dims.num_v_heads, dims.head_k_dim, dims.head_v_dim
    n = slot_idx.shape[0]
    _dev(q, "q", shape=(T, H, dk)); _dev(k, "k", q.dtype, (T, H, dk))
    _dev(v, "v", q.dtype, (T, HV, dv))
    if gate is None:
        _dev(gb[0], "g", torch.float32, (T, HV)); _dev(gb[1], "beta", torch.float32, (T, HV))
    _dev(cu_seqlens, "cu_seqlens", torch.int32, (n + 1,))
    _dev(slot_idx, "slot_idx", torch.int32, (n,))
    _dev(rec_state, "rec_state", torch.float32); _dev(out, "out", shape=(T, HV, dv))
    _dev(err_flag, "err_flag", torch.int32)
    if tuple(rec_state.shape[1:]) != (HV, dv, dk):
        raise ValueError("rec_state must be [num_slots, HV, dv, dk]")
    need = (gdn_prefill_workspace_size(dims, n, T) if seg_len is None else
            gdn_prefill_segmented_workspace_size(dims, n, T, seg_len))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    if seg_len is not None:
        gs = None if gate is None else _gate_struct(gate, T, HV)
        status = lib.gdn_prefill_segmented(
            _p(q), _p(k), _p(v), _dt(q), _p(gb[0]) if gate is None else None,
            _p(gb[1]) if gate is None else None, None if gs is None else ctypes.byref(gs),
            _p(cu_seqlens), n, T, _p(slot_idx), _p(rec_state), rec_state.shape[0], _p(out),
            _dt(out), ctypes.byref(dims), float(scale), flags, int(seg_len), int(head_len),
            _p(workspace),
            workspace.numel() * workspace.element_size(), _p(err_flag), _stream(stream))
        _check(fn, status)
        return out
    rest = (_p(cu_seqlens), n, T, _p(slot_idx), _p(rec_state), rec_state.shape[0], _p(out),
            _dt(out), ctypes.byref(dims), float(scale), flags, _p(workspace),
            workspace.numel() * workspace.element_size(), _p(err_flag), _stream(stream))
    if gate is None:
        status = lib.gdn_prefill_chunked(_p(q), _p(k), _p(v), _dt(q), _p(gb[0]), _p(gb[1]), *rest)
    else:
        gs = _gate_struct(gate, T, HV)
        status = lib.gdn_prefill_chunked_gated(_p(q), _p(k), _p(v), _dt(q), ctypes.byref(gs), *rest)
    _check(fn, status)
    return out


def gdn_prefill_chunked(q, k, v, g, beta, cu_seqlens, slot_idx, rec_state, out,
                        dims: gdn_dims, scale, flags=DEFAULT_PREFILL_FLAGS, workspace=None,
                        err_flag=None, stream=None):
    """Varlen chunked prefill (gdn.h: gdn_prefill_chunked).  ``rec_state`` is
    read and written in place; ``out`` [T, HV, dv] receives o."""
    return _prefill("gdn_prefill_chunked", q, k, v, (g, beta), None, cu_seqlens, slot_idx,
                    rec_state, out, dims, scale, flags, workspace, err_flag, stream)


def gdn_prefill_chunked_gated(q, k, v, gate: GateInputs, cu_seqlens, slot_idx, rec_state, out,
                              dims: gdn_dims, scale, flags=DEFAULT_PREFILL_FLAGS, workspace=None,
                              err_flag=None, stream=None):
    """gdn_prefill_chunked with the gating fused in (gdn.h: gdn_prefill_chunked_gated)."""
    return _prefill("gdn_prefill_chunked_gated", q, k, v, None, gate, cu_seqlens, slot_idx,
                    rec_state, out, dims, scale, flags, workspace, err_flag, stream)


def gdn_prefill_segmented(q, k, v, g, beta, cu_seqlens, slot_idx, rec_state, out,
                          dims: gdn_dims, scale, seg_len: int, flags=DEFAULT_PREFILL_FLAGS,
                          gate: GateInputs = None, workspace=None, err_flag=None, stream=None,
                          head_len: int = 0):
    """Segment-parallel prefill (gdn.h: gdn_prefill_segmented): segment 0 of
    head_len tokens (0: seg_len), then seg_len-token segments; with ``gate``
    given, g and beta must be None."""
    if gate is not None and (g is not None or beta is not None):
        raise ValueError("pass either g and beta or gate")
    return _prefill("gdn_prefill_segmented", q, k, v, (g, beta), gate, cu_seqlens, slot_idx,
                    rec_state, out, dims, scale, flags, workspace, err_flag, stream,
                    seg_len=seg_len, head_len=head_len)


def gdn_mixed_workspace_size(dims: gdn_dims, n_dec: int, total_pre: int) -> int:
    return int(load_library().gdn_mixed_workspace_size(ctypes.byref(dims), int(n_dec),
                                                        int(total_pre)))


class MixedStreams:
    """The caller-owned second stream and fork / join events with which
    gdn_mixed_step overlaps its prefill part with its decode rows.  Plain torch
    objects; the library only records and waits on them.  Use one instance per
    host thread."""

    def __init__(self, device=None):
        self.stream = torch.cuda.Stream(device=device)
        self.fork = torch.cuda.Event()
        self.join = torch.cuda.Event()
        # torch creates an event's HIP handle on its first record
        cur = torch.cuda.current_stream(device)
        self.fork.record(cur)
        self.join.record(cur)

    def handles(self):
        return (ctypes.c_void_p(self.stream.cuda_stream), ctypes.c_void_p(self.fork.cuda_event),
                ctypes.c_void_p(self.join.cuda_event))


def gdn_mixed_step(x, g, beta, n_dec, cu_seqlens, slot_idx, conv_state, conv_weight, rec_state,
                   out, dims: gdn_dims, scale, conv_bias=None, flags=DEFAULT_DECODE_FLAGS,
                   workspace=None, err_flag=None, stream=None, streams: MixedStreams = None):
    """One step with ``n_dec`` decode rows followed by prefill sequences
    (gdn.h: gdn_mixed_step).  ``x`` [n_dec + T, D] pre-conv, ``cu_seqlens``
    [n_pre + 1] over the T prefill tokens (or None), ``slot_idx`` [n_dec + n_pre],
    ``out`` [n_dec + T, HV, dv].  Caches updated in place.  Without a
    ``workspace`` the minimal one is allocated (whole prefill runs); a workspace
    of gdn_mixed_workspace_size + gdn_prefill_workspace_size bytes lets the
    prefill part of a step without decode rows take the segment-parallel
    schedule.  ``streams`` (a MixedStreams) overlaps the prefill part with the
    decode rows on its second stream; without it both run in order."""
    lib = load_library()
    rows = x.shape[0]
    HV, dk, dv = dims.num_v_heads, dims.head_k_dim, dims.head_v_dim
    D = 2 * dims.num_k_heads * dk + HV * dv
    n_dec = int(n_dec)
    T = rows - n_dec
    n_pre = 0 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    _dev(x, "x", shape=(rows, D))
    _dev(g, "g", torch.float32, (rows, HV)); _dev(beta, "beta", torch.float32, (rows, HV))
    _dev(cu_seqlens, "cu_seqlens", torch.int32, None if cu_seqlens is None else (n_pre + 1,))
    _dev(slot_idx, "slot_idx", torch.int32, (n_dec + n_pre,))
    _dev(conv_state, "conv_state"); _dev(conv_weight, "conv_weight")
    _dev(conv_bias, "conv_bias", conv_weight.dtype)
    _dev(rec_state, "rec_state", torch.float32)
    _dev(out, "out", shape=(rows, HV, dv)); _dev(err_flag, "err_flag", torch.int32)
    ns = rec_state.shape[0]
    if tuple(rec_state.shape[1:]) != (HV, dv, dk):
        raise ValueError("rec_state must be [num_slots, HV, dv, dk]")
    if tuple(conv_state.shape) != (ns, D, dims.conv_width - 1):
        raise ValueError("conv_state must be [num_slots, D, W-1] with the rec_state slot count")
    need = gdn_mixed_workspace_size(dims, n_dec, T)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace")
    _check("gdn_mixed_step", lib.gdn_mixed_step(
        _p(x), _dt(x), _p(g), _p(beta), n_dec, _p(cu_seqlens), n_pre, T, _p(slot_idx),
        _p(conv_state), _dt(conv_state), _p(conv_weight), _p(conv_bias), _dt(conv_weight),
        _p(rec_state), ns, _p(out), _dt(out), ctypes.byref(dims), float(scale), flags,
        _p(workspace), workspace.numel() * workspace.element_size(), _p(err_flag),
        _stream(stream), *(streams.handles() if streams is not None else (None, None, None))))
    return out


def gdn_gated_rmsnorm(x, weight, out, z=None, eps=1e-6, flags=0, stream=None):
    """Gated RMSNorm over the last axis (gdn.h: gdn_gated_rmsnorm): ``x`` and
    ``z`` [..., dim] (z in x's dtype, or None), ``weight`` [dim]; ``out`` may be x."""
    lib = load_library()
    dim = x.shape[-1]
    rows = x.numel() // dim if dim else 0
    _dev(x, "x"); _dev(z, "z", x.dtype, None if z is None else tuple(x.shape))
    _dev(weight, "weight", shape=(dim,)); _dev(out, "out", shape=tuple(x.shape))
    _check("gdn_gated_rmsnorm", lib.gdn_gated_rmsnorm(
        _p(x), _dt(x), _p(z), _p(weight), _dt(weight), rows, dim, float(eps), flags, _p(out),
        _dt(out), _stream(stream)))
    return out
