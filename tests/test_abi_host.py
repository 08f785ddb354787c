"""CPU tests of the C ABI: the library loads, exports every function that
include/gdn.h declares, and rejects bad arguments synchronously (before any
kernel launch, so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import gated_deltanet_recurrent_gdn_amd as gdn
from gated_deltanet_recurrent_gdn_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, ERR_NULL, ERR_DIMS, ERR_DTYPE, ERR_ALIGN, ERR_WS, ERR_LAUNCH, ERR_FLAGS = range(8)


@pytest.fixture(scope="module")
def lib():
    return gdn.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(_abi.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_decode_step_path_query(lib):
    # without a GPU the CU count is the 256 fallback: the fused kernel for
    # 64 .. 256 (row, key head) groups, the conv + recurrence pair outside
    d = gdn.make_dims(16, 32, 128, 128, 4)
    assert [gdn.gdn_decode_step_fused(d, b) for b in (1, 2, 3, 4, 8, 16, 17, 32, 256, 1024)] == \
        [0, 0, 0, 1, 1, 1, 0, 0, 0, 0]
    assert gdn.gdn_decode_step_fused(d, 0) == 0
    assert gdn.gdn_decode_step_fused(gdn.make_dims(16, 32, 256, 256, 4), 8) == 0   # dk > 128
    assert gdn.gdn_decode_step_fused(gdn.make_dims(16, 30, 128, 128, 4), 8) == -1  # HV % H
    assert gdn.gdn_decode_step_fused(d, -1) == -1 and gdn.gdn_decode_step_fused(d, 65536) == -1


def test_strerror(lib):
    for code in range(8):
        assert gdn.gdn_strerror(code)
    assert gdn.gdn_strerror(99) == "unknown status"


def test_workspace_sizes(lib):
    d = gdn.make_dims(16, 32, 128, 128, 4)
    assert gdn.gdn_decode_workspace_size(d, 256) == 256 * 8192 * 4
    assert gdn.gdn_decode_workspace_size(d, 0) == 0
    assert gdn.gdn_decode_workspace_size(gdn.make_dims(16, 32, 100, 128, 4), 4) == 0
    assert gdn.gdn_decode_workspace_size(gdn.make_dims(16, 30, 128, 128, 4), 4) == 0


def _dims(H=16, HV=32, dk=128, dv=128, W=4):
    return ctypes.byref(gdn.make_dims(H, HV, dk, dv, W))


FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced (rejected first)
MISALIGNED = ctypes.c_void_p(0x10004)


def _decode(lib, dims=None, batch=4, flags=3, x=FAKE, rec=FAKE, ws=FAKE, ws_bytes=1 << 30,
            err=None, x_dt=1, out_dt=0):
    return lib.gdn_decode_step(x, x_dt, FAKE, FAKE, FAKE, batch, FAKE, 1, FAKE, None, 1, rec,
                               8, FAKE, out_dt, dims or _dims(), 0.1, flags, ws, ws_bytes, err,
                               None)


@pytest.mark.parametrize("kw,code", [
    (dict(dims=_dims(dk=100)), ERR_DIMS),
    (dict(dims=_dims(HV=24, H=16)), ERR_DIMS),
    (dict(dims=_dims(dv=48)), ERR_DIMS),
    (dict(dims=_dims(W=3)), ERR_DIMS),
    (dict(batch=-1), ERR_DIMS),
    (dict(batch=70000), ERR_DIMS),
    (dict(x_dt=5), ERR_DTYPE),
    (dict(out_dt=2), ERR_DTYPE),
    (dict(flags=64), ERR_FLAGS),
    (dict(flags=7, err=None), ERR_FLAGS),          # VALIDATE without err_flag
    (dict(flags=3 | 8 | 16), ERR_FLAGS),           # both decode-step paths forced
    (dict(flags=3 | 8, dims=_dims(H=1, HV=128, dv=256)), ERR_DIMS),   # fused group > 64 KiB LDS
    (dict(x=None), ERR_NULL),
    (dict(ws=None), ERR_NULL),
    (dict(rec=MISALIGNED), ERR_ALIGN),
    (dict(ws_bytes=16), ERR_WS),
])
def test_decode_step_rejects(lib, kw, code):
    assert _decode(lib, **kw) == code


def test_decode_step_empty_batch_is_ok(lib):
    # batch 0 without validation enqueues nothing at all
    assert _decode(lib, batch=0, x=None, rec=None, ws=None) == OK


def test_conv_update_rejects(lib):
    f = lib.gdn_conv_update
    # width other than 4
    assert f(FAKE, 1, None, 4, 4, FAKE, FAKE, 1, 8, FAKE, None, 1, FAKE, 0, 64, 3, 1, None,
             None) == ERR_DIMS
    # decode form needs total_tokens == n_seqs
    assert f(FAKE, 1, None, 4, 5, FAKE, FAKE, 1, 8, FAKE, None, 1, FAKE, 0, 64, 4, 1, None,
             None) == ERR_DIMS
    # unknown flag (QK norm does not apply to the conv)
    assert f(FAKE, 1, None, 4, 4, FAKE, FAKE, 1, 8, FAKE, None, 1, FAKE, 0, 64, 4, 2, None,
             None) == ERR_FLAGS
    assert f(FAKE, 1, None, 4, 4, None, FAKE, 1, 8, FAKE, None, 1, FAKE, 0, 64, 4, 1, None,
             None) == ERR_NULL
    assert f(FAKE, 7, None, 4, 4, FAKE, FAKE, 1, 8, FAKE, None, 1, FAKE, 0, 64, 4, 1, None,
             None) == ERR_DTYPE


def test_decode_recurrent_rejects(lib):
    f = lib.gdn_decode_recurrent
    assert f(FAKE, 0, FAKE, FAKE, FAKE, 4, FAKE, 8, FAKE, 0, _dims(), 0.1, 1, None,
             None) == ERR_FLAGS                      # SiLU is not part of this call
    assert f(MISALIGNED, 0, FAKE, FAKE, FAKE, 4, FAKE, 8, FAKE, 0, _dims(), 0.1, 2, None,
             None) == ERR_ALIGN
    assert f(FAKE, 0, FAKE, FAKE, FAKE, 4, FAKE, 8, FAKE, 0, _dims(dk=48), 0.1, 2, None,
             None) == ERR_DIMS


def test_binding_refuses_cpu_tensors():
    import torch
    d = gdn.make_dims(2, 4, 32, 32, 4)
    x = torch.zeros(1, 2 * 2 * 32 + 4 * 32)
    with pytest.raises(TypeError):
        gdn.gdn_decode_recurrent(x, torch.zeros(1, 4), torch.zeros(1, 4),
                                 torch.ones(1, dtype=torch.int32), torch.zeros(2, 4, 32, 32),
                                 torch.zeros(1, 4, 32), d, 0.1)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        _abi.load_library(str(tmp_path / "libgdn_missing.so"))


def _gate(a=FAKE, b=FAKE, ab_dt=1, A_log=FAKE, dt_bias=FAKE):
    return ctypes.byref(gdn.gdn_gate_inputs(a, b, ab_dt, A_log, dt_bias))


def _decode_gated(lib, gate, batch=4, flags=3):
    return lib.gdn_decode_step_gated(FAKE, 1, gate, FAKE, batch, FAKE, 1, FAKE, None, 1, FAKE,
                                     8, FAKE, 0, _dims(), 0.1, flags, FAKE, 1 << 30, None, None)


def _prefill_gated(lib, gate, total=64):
    return lib.gdn_prefill_chunked_gated(FAKE, FAKE, FAKE, 1, gate, FAKE, 1, total, FAKE, FAKE,
                                         8, FAKE, 1, _dims(), 0.1, 2, None, 0, None, None)


@pytest.mark.parametrize("gate,code", [
    (None, ERR_NULL),
    ("a", ERR_NULL), ("b", ERR_NULL), ("A_log", ERR_NULL), ("dt_bias", ERR_NULL),
    ("dtype", ERR_DTYPE),
])
def test_gated_calls_reject(lib, gate, code):
    if gate is None:
        g = None
    elif gate == "dtype":
        g = _gate(ab_dt=7)
    else:
        g = _gate(**{gate: None})
    assert _decode_gated(lib, g) == code
    assert _prefill_gated(lib, g) == code


def test_gated_calls_empty_is_ok(lib):
    # nothing to process: the gate arrays are not needed (batch 0 / zero tokens, no sequences)
    g = _gate(a=None, b=None, A_log=None, dt_bias=None)
    assert lib.gdn_decode_step_gated(None, 1, g, None, 0, None, 1, None, None, 1, None, 8, None,
                                     0, _dims(), 0.1, 3, None, 0, None, None) == OK
    assert lib.gdn_prefill_chunked_gated(None, None, None, 1, g, None, 0, 0, None, None, 8, None,
                                         1, _dims(), 0.1, 2, None, 0, None, None) == OK


def _mixed(lib, dims=None, n_dec=2, cu=FAKE, n_pre=1, total=64, flags=3, ws=FAKE,
           ws_bytes=1 << 30, err=None, side=(None, None, None)):
    return lib.gdn_mixed_step(FAKE, 1, FAKE, FAKE, n_dec, cu, n_pre, total, FAKE, FAKE, 1, FAKE,
                              None, 1, FAKE, 8, FAKE, 0, dims or _dims(), 0.1, flags, ws,
                              ws_bytes, err, None, *side)


@pytest.mark.parametrize("kw,code", [
    (dict(flags=3 | 8 | 16), ERR_FLAGS),
    (dict(flags=64), ERR_FLAGS),
    (dict(n_dec=-1), ERR_DIMS),
    (dict(n_pre=-1), ERR_DIMS),
    (dict(dims=_dims(dk=256, dv=256)), ERR_DIMS),      # prefill part needs d <= 128
    (dict(dims=_dims(dk=128, dv=64)), ERR_DIMS),       # and dk == dv
    (dict(cu=None), ERR_NULL),
    (dict(ws=None), ERR_NULL),
    (dict(ws_bytes=16), ERR_WS),
    (dict(side=(FAKE, None, FAKE)), ERR_NULL),         # a prefill stream needs both events
    (dict(side=(FAKE, FAKE, None)), ERR_NULL),
])
def test_mixed_step_rejects(lib, kw, code):
    assert _mixed(lib, **kw) == code


def test_mixed_step_decode_only_dims_ok_without_prefill(lib):
    # d = 256 is fine when the step holds no prefill sequence (rejected later
    # only by the null test pointers, which the empty call never touches)
    assert _mixed(lib, dims=_dims(dk=256, dv=256), n_dec=0, n_pre=0, total=0, cu=None,
                  ws=None) == OK


def test_mixed_step_accepts_sequential_prefill_flag(lib):
    # GDN_FLAG_PREFILL_SEQUENTIAL (128) keeps the prefill part on whole runs; the
    # Newton-Schulz A/B flags stay prefill-call only
    assert _mixed(lib, flags=3 | 128, n_dec=0, n_pre=0, total=0, cu=None, ws=None) == OK
    assert _mixed(lib, flags=3 | 32) == ERR_FLAGS


def test_single_role_prefill_flag(lib):
    # GDN_FLAG_PREFILL_SINGLE_ROLE (256) picks the prefill's chunk-step kernel:
    # prefill calls and the mixed step take it, the decode calls do not
    chunked = (None, None, None, 1, None, None, None, 0, 0, None, None, 8, None, 1, _dims(), 0.1)
    assert lib.gdn_prefill_chunked(*chunked, 2 | 256, None, 0, None, None) == OK
    assert lib.gdn_prefill_chunked(*chunked, 2 | 512, None, 0, None, None) == ERR_FLAGS
    assert lib.gdn_prefill_segmented(None, None, None, 1, None, None, None, None, 0, 0, None,
                                     None, 8, None, 1, _dims(), 0.1, 2 | 256, 128, 0, None, 0,
                                     None, None) == OK
    assert _mixed(lib, flags=3 | 256, n_dec=0, n_pre=0, total=0, cu=None, ws=None) == OK
    assert _decode(lib, flags=3 | 256) == ERR_FLAGS


def test_header_flag_values_match_binding():
    text = open(HEADER).read()
    vals = dict(re.findall(r"\b(GDN_FLAG_[A-Z0-9_]+)\s*=\s*(\d+)", text))
    for name, v in vals.items():
        assert getattr(_abi, name[4:]) == int(v), name
    assert len(vals) == 9


def test_mixed_workspace_size(lib):
    d = _dims()
    D = 2 * 16 * 128 + 32 * 128
    assert lib.gdn_mixed_workspace_size(d, 3, 10) == (
        ((3 * D * 4 + 255) // 256) * 256 + ((10 * D * 2 + 255) // 256) * 256)


@pytest.mark.parametrize("kw,code", [
    (dict(flags=4), ERR_FLAGS),
    (dict(dim=2), ERR_DIMS), (dict(dim=1028), ERR_DIMS), (dict(dim=130), ERR_DIMS),
    (dict(eps=-1.0), ERR_DIMS), (dict(eps=float("nan")), ERR_DIMS), (dict(rows=-1), ERR_DIMS),
    (dict(x_dt=9), ERR_DTYPE),
    (dict(x=None), ERR_NULL),
    (dict(out=MISALIGNED), ERR_ALIGN),
])
def test_gated_rmsnorm_rejects(lib, kw, code):
    a = dict(x=FAKE, x_dt=1, z=None, w=FAKE, w_dt=0, rows=8, dim=128, eps=1e-6, flags=0,
             out=FAKE, out_dt=1)
    a.update(kw)
    assert lib.gdn_gated_rmsnorm(a["x"], a["x_dt"], a["z"], a["w"], a["w_dt"], a["rows"],
                                 a["dim"], a["eps"], a["flags"], a["out"], a["out_dt"],
                                 None) == code


def test_prefill_rejects_both_newton_schulz_variants(lib):
    assert lib.gdn_prefill_chunked(FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 1, 64, FAKE, FAKE, 8,
                                   FAKE, 1, _dims(), 0.1, 2 | 32 | 64, None, 0, None,
                                   None) == ERR_FLAGS


def _segmented(lib, seg_len=128, flags=2, g=FAKE, beta=FAKE, gate=None, ws=FAKE,
               ws_bytes=1 << 34, total=256, head=0):
    return lib.gdn_prefill_segmented(FAKE, FAKE, FAKE, 1, g, beta, gate, FAKE, 1, total, FAKE,
                                     FAKE, 8, FAKE, 1, _dims(), 0.1, flags, seg_len, head, ws,
                                     ws_bytes, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(seg_len=0), ERR_DIMS), (dict(seg_len=-64), ERR_DIMS), (dict(seg_len=100), ERR_DIMS),
    (dict(flags=2 | 128), ERR_FLAGS),              # the sequential flag contradicts the call
    (dict(ws=None), ERR_WS), (dict(ws_bytes=1024), ERR_WS), (dict(ws=MISALIGNED), ERR_ALIGN),
    (dict(g=None), ERR_NULL), (dict(gate="both"), ERR_FLAGS),
    (dict(seg_len=64, total=64 * 32769), ERR_DIMS),   # more than 32768 segments
    # 32768 segments of one sequence at dk = 128: the first pass's separate P
    # and B runs would need 1 + 2 x 32769 grid rows, past 65535
    (dict(seg_len=64, total=64 * 32768), ERR_DIMS),
    (dict(head=64), ERR_DIMS),                     # head shorter than the segments
    (dict(head=200), ERR_DIMS),                    # head not a multiple of 64
    (dict(head=-64), ERR_DIMS),
])
def test_prefill_segmented_rejects(lib, kw, code):
    if kw.get("gate") == "both":
        kw["gate"] = _gate()
    assert _segmented(lib, **kw) == code


def test_prefill_segmented_empty_is_ok(lib):
    # no sequences and no tokens: nothing to run, so no workspace is needed
    assert lib.gdn_prefill_segmented(None, None, None, 1, None, None, None, None, 0, 0, None,
                                     None, 8, None, 1, _dims(), 0.1, 2, 128, 0, None, 0, None,
                                     None) == OK


def test_prefill_workspace_sizes(lib):
    d = gdn.make_dims(16, 32, 128, 128, 4)
    mats = 3 * 32 * 128 * 128 * 4                 # start state, P, B per value head
    maps = 256                                    # the two segment maps, rounded up
    assert gdn.gdn_prefill_segmented_workspace_size(d, 1, 16384, 2048) == (1 + 8 + 1) * mats + maps
    assert gdn.gdn_prefill_segmented_workspace_size(d, 8, 24674, 2048) == (8 + 12 + 1) * mats + maps
    assert gdn.gdn_prefill_segmented_workspace_size(d, 1, 16384, 100) == 0
    assert gdn.gdn_prefill_segmented_workspace_size(gdn.make_dims(16, 32, 256, 256, 4), 1, 64, 64) == 0
    # eight sequences x 32 value heads fill a 256-CU chip (the host fallback
    # count without a GPU): a head of ceil((386 + 4) x 32 / 256) = 49 chunks and
    # tail segments of 13 chunks (832 tokens), 8 + 24674 // 832 + 1 segment ids
    assert gdn.gdn_prefill_workspace_size(d, 8, 24674) == (8 + 29 + 1) * mats + maps
    # a busy chip with short sequences keeps whole runs (head under 8 chunks)
    assert gdn.gdn_prefill_workspace_size(d, 8, 1600) == 0
    # one long sequence leaves most of the chip idle: the call asks for segments.
    # The model (head h, m tails of s chunks, separate P/B runs at dk = 128):
    # m = 8 tails need 2 x 32 x 7 = 448 P/B runs, two rounds on the 224 CUs
    # segment 0 leaves, so s = ceil(256 / (2 + 8)) = 26 chunks (1664 tokens)
    # and h = 256 - 8 x 26 = 48: 1 + 16384 // 1664 + 1 segment ids
    assert gdn.gdn_prefill_workspace_size(d, 1, 16384) == (1 + 9 + 1) * mats + maps
    assert gdn.gdn_prefill_workspace_size(d, 1, 256) == 0     # too short to pay
    assert gdn.gdn_prefill_workspace_size(d, 1, 512) == 0     # 8 chunks: the launches eat the gain
    # 30000 sequences on a busy chip: the segment passes' grids would pass
    # 65535 rows, so the call keeps whole runs
    assert gdn.gdn_prefill_workspace_size(d, 30000, 30000 * 600) == 0
