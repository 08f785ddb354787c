"""fp64 CPU oracle for the Gated DeltaNet core -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does; the oracle
shares no code with it.  The arithmetic lives in ``oracle.c`` (plain
sequential fp64 loops); this module only marshals numpy arrays.

Entry points mirror the three operations of the product library:
``conv_update``, ``decode_step`` and ``prefill`` (token-by-token, no chunking).
Each raises :class:`OracleError` on a bad slot index or bad ``cu_seqlens``
before any cache is touched, as the goldens of RL-Kernel PR #469 do
(section "State ABI: index validation and the two NULL_BLOCK_ID contracts").
"""
import ctypes
import os

import numpy as np

from . import build as _build

FLAG_SILU = 1
FLAG_QK_L2NORM = 2
NORM_GATE_SIGMOID = 1
NORM_ZERO_CENTRED = 2

ERR_SLOT_RANGE = 1
ERR_SLOT_REPEAT = 2
ERR_SEQLENS = 4
ERR_ARGS = 8

_lib = None


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle rejected the call (error bits {code:#x})")
        self.code = code


def load(path: str = None):
    """Load liboracle.so (building it first only when no build exists)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _build.LIB
    if not os.path.exists(p):
        _build.build(out=p)
    lib = ctypes.CDLL(p)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_conv_update.argtypes = [P, i64, P, i32, P, P, i32, P, P, P, i32, i32, i32]
    lib.oracle_decode_step.argtypes = [P, P, P, P, i32, P, P, P, P, i32, P,
                                       i32, i32, i32, i32, i32, f64, i32]
    lib.oracle_prefill.argtypes = [P, P, P, P, P, P, i32, i64, P, P, i32, P,
                                   i32, i32, i32, i32, f64, i32]
    lib.oracle_gating.argtypes = [P, P, P, P, i64, i32, P, P]
    lib.oracle_gated_rmsnorm.argtypes = [P, P, P, i64, i32, ctypes.c_double, i32, P]
    for f in (lib.oracle_conv_update, lib.oracle_decode_step, lib.oracle_prefill,
              lib.oracle_gating, lib.oracle_gated_rmsnorm):
        f.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check_inplace(a, name):
    if not (isinstance(a, np.ndarray) and a.dtype == np.float64 and a.flags.c_contiguous):
        raise TypeError(f"{name} must be a C-contiguous float64 ndarray (updated in place)")


def conv_update(x, slot_idx, conv_state, weight, bias=None, cu_seqlens=None,
                flags=FLAG_SILU, lib=None):
    """Causal conv1d update; ``conv_state`` [num_slots, dim, W-1] is rolled in place.

    ``x`` is [total_tokens, dim]; with ``cu_seqlens=None`` every row is one
    token of its own sequence.  Returns ``out`` [total_tokens, dim].
    """
    lib = lib or load()
    x = _f64(x)
    _check_inplace(conv_state, "conv_state")
    weight = _f64(weight)
    bias = None if bias is None else _f64(bias)
    slot_idx = _i32(slot_idx)
    T, dim = x.shape
    width = weight.shape[1]
    cu = None if cu_seqlens is None else _i32(cu_seqlens)
    n = slot_idx.shape[0]
    out = np.full_like(x, np.nan)   # the oracle must write every element
    rc = lib.oracle_conv_update(_ptr(x), T, _ptr(cu), n, _ptr(slot_idx),
                                _ptr(conv_state), conv_state.shape[0], _ptr(weight),
                                _ptr(bias), _ptr(out), dim, width, flags)
    if rc:
        raise OracleError(rc)
    return out


def decode_step(mixed_qkv, g, beta, slot_idx, conv_state, conv_weight, rec_state,
                num_k_heads, num_v_heads, head_k_dim, head_v_dim, scale,
                conv_bias=None, flags=FLAG_SILU | FLAG_QK_L2NORM, lib=None):
    """One decode token per row; caches updated in place. Returns o [B, HV, dv]."""
    lib = lib or load()
    x = _f64(mixed_qkv)
    g = _f64(g)
    beta = _f64(beta)
    slot_idx = _i32(slot_idx)
    _check_inplace(conv_state, "conv_state")
    _check_inplace(rec_state, "rec_state")
    w = _f64(conv_weight)
    b = None if conv_bias is None else _f64(conv_bias)
    B = x.shape[0]
    out = np.full((B, num_v_heads, head_v_dim), np.nan)
    rc = lib.oracle_decode_step(_ptr(x), _ptr(g), _ptr(beta), _ptr(slot_idx), B,
                                _ptr(conv_state), _ptr(w), _ptr(b), _ptr(rec_state),
                                rec_state.shape[0], _ptr(out), num_k_heads, num_v_heads,
                                head_k_dim, head_v_dim, w.shape[1], float(scale), flags)
    if rc:
        raise OracleError(rc)
    return out


def prefill(q, k, v, g, beta, cu_seqlens, slot_idx, rec_state, scale,
            flags=FLAG_QK_L2NORM, lib=None):
    """Token-by-token prefill; ``rec_state`` updated in place. Returns o [T, HV, dv]."""
    lib = lib or load()
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    cu = _i32(cu_seqlens)
    slot_idx = _i32(slot_idx)
    _check_inplace(rec_state, "rec_state")
    T, H, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    out = np.full((T, HV, dv), np.nan)
    rc = lib.oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu),
                            slot_idx.shape[0], T, _ptr(slot_idx), _ptr(rec_state),
                            rec_state.shape[0], _ptr(out), H, HV, dk, dv, float(scale), flags)
    if rc:
        raise OracleError(rc)
    return out


def gating(a, b, A_log, dt_bias, lib=None):
    """Fused gating in fp64: returns (g, beta), each shaped like ``a`` [rows, HV]."""
    lib = lib or load()
    a, b, A_log, dt_bias = (_f64(x) for x in (a, b, A_log, dt_bias))
    rows, HV = a.shape
    if b.shape != a.shape or A_log.shape != (HV,) or dt_bias.shape != (HV,):
        raise ValueError("gating shapes: a, b [rows, HV]; A_log, dt_bias [HV]")
    g = np.full(a.shape, np.nan)
    beta = np.full(a.shape, np.nan)
    rc = lib.oracle_gating(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), rows, HV,
                           _ptr(g), _ptr(beta))
    if rc:
        raise OracleError(rc)
    return g, beta


def gated_rmsnorm(x, weight, z=None, eps=1e-6, flags=0, lib=None):
    """Gated RMSNorm over the last axis of ``x`` [..., dim] in fp64."""
    lib = lib or load()
    x = _f64(x)
    shape = x.shape
    dim = shape[-1]
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    w = _f64(weight)
    zz = None if z is None else _f64(z)
    if w.shape != (dim,) or (zz is not None and zz.shape != shape):
        raise ValueError("gated_rmsnorm: weight [dim], z shaped like x")
    out = np.full(shape, np.nan)
    rc = lib.oracle_gated_rmsnorm(_ptr(x), _ptr(zz), _ptr(w), rows, dim, float(eps), flags,
                                  _ptr(out))
    if rc:
        raise OracleError(rc)
    return out
