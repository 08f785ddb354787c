"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each ``pin_*`` function takes a loaded oracle library handle and raises
AssertionError when the oracle disagrees with a closed form, a brute-force
computation, a library routine, or an independent chunked derivation.  They are
run against the real oracle (all must pass) and against textual mutants of its
source (each planted mistake must fail at least one pin).

Page tags: [P1] RL-Kernel PR #469 ("C6: GDN decode-step goldens and
recurrent/conv state contract"); [P4] vLLM PR #53864 (CuteDSL GDN prefill,
Newton-Schulz rounds).
"""
import math

import numpy as np
from scipy.special import expit

import oracle
from chunk_algebra import block_inverse, chunked_prefill, newton_schulz_unit_lower_inverse

NORM = oracle.FLAG_QK_L2NORM


def _one_token(lib, S, q, k, v, g, beta, scale=1.0, flags=0, H=1):
    """Run one token through oracle.prefill for a single key head.

    S [HV, dv, dk] is the initial state (copied); returns (o [HV, dv], S')."""
    HV, dv, dk = S.shape
    rec = np.zeros((2, HV, dv, dk))
    rec[1] = S
    o = oracle.prefill(q.reshape(1, H, dk), k.reshape(1, H, dk), v.reshape(1, HV, dv),
                       np.full((1, HV), g, dtype=np.float64) if np.isscalar(g) else g.reshape(1, HV),
                       np.full((1, HV), beta, dtype=np.float64) if np.isscalar(beta) else beta.reshape(1, HV),
                       [0, 1], [1], rec, scale, flags=flags, lib=lib)
    return o[0], rec[1]


def _unit_half_vector(dk, rng):
    """A vector with exactly four entries of +-1/2 (norm exactly 1, exact in fp)."""
    k = np.zeros(dk)
    idx = rng.choice(dk, 4, replace=False)
    k[idx] = 0.5 * rng.choice([-1.0, 1.0], 4)
    return k


# --- K1: beta = 0, g = 0 leaves the state unchanged and o = S q --------------
def pin_identity_step(lib):
    rng = np.random.default_rng(11)
    dk = dv = 8
    S = rng.standard_normal((1, dv, dk))
    q, k, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
    o, S1 = _one_token(lib, S, q, k, v, 0.0, 0.0, flags=0)
    assert np.array_equal(S1, S), "beta=0, g=0 must leave S unchanged"
    assert np.allclose(o[0], S[0] @ q, rtol=0, atol=1e-14)


# --- K2: beta = 1, unit k: the new state maps k to v exactly (decay first) ---
def pin_delta_rule_unit_key(lib):
    rng = np.random.default_rng(12)
    for dk in (4, 8, 32):
        dv = dk + 3
        S = rng.standard_normal((1, dv, dk))
        for k in (np.eye(dk)[dk // 2], _unit_half_vector(dk, rng)):
            for g in (0.0, math.log(0.5), -3.0):
                for scale in (1.0, 0.37):
                    q, v = rng.standard_normal(dk), rng.standard_normal(dv)
                    _, S1 = _one_token(lib, S, q, k, v, g, 1.0, scale=scale, flags=0)
                    assert np.allclose(S1[0] @ k, v, rtol=0, atol=1e-13), (dk, g, scale)


# --- K3: pure decay; and an overwhelming decay leaves only beta v k^T --------
def pin_decay(lib):
    rng = np.random.default_rng(13)
    H, HV, dk, dv, T = 1, 2, 6, 5, 7
    S0 = rng.standard_normal((HV, dv, dk))
    rec = np.zeros((3, HV, dv, dk)); rec[2] = S0
    g = -rng.random((T, HV))
    oracle.prefill(rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dk)),
                   rng.standard_normal((T, HV, dv)), g, np.zeros((T, HV)), [0, T], [2], rec,
                   1.0, flags=0, lib=lib)
    for hv in range(HV):
        assert np.allclose(rec[2, hv], math.exp(g[:, hv].sum()) * S0[hv], rtol=1e-13, atol=0)
    # g -> -200: exp(g) S is ~1e-87 of S, so S' = beta v k^T and o = beta v (k . q)
    S = rng.standard_normal((1, dv, dk))
    q, k, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
    o, S1 = _one_token(lib, S, q, k, v, -200.0, 0.7, flags=0)
    assert np.allclose(S1[0], 0.7 * np.outer(v, k), rtol=1e-13, atol=1e-80)
    assert np.allclose(o[0], 0.7 * v * np.dot(k, q), rtol=1e-12, atol=1e-80)


# --- K4: repeated unit key with beta = 1 overwrites: o_t = S_t k = v_t --------
def pin_overwrite(lib):
    rng = np.random.default_rng(14)
    H, HV, d, T = 1, 1, 16, 9
    k = _unit_half_vector(d, rng)
    K = np.tile(k, (T, H, 1))
    V = rng.standard_normal((T, HV, d))
    rec = np.zeros((2, HV, d, d)); rec[1] = rng.standard_normal((HV, d, d))
    o = oracle.prefill(K.copy(), K, V, np.zeros((T, HV)), np.ones((T, HV)), [0, T], [1], rec,
                       1.0, flags=0, lib=lib)
    assert np.allclose(o[:, 0], V[:, 0], rtol=0, atol=1e-13)
    assert np.allclose(rec[1, 0] @ k, V[-1, 0], rtol=0, atol=1e-13)


# --- K5: brute force with full matrices: exp(g) S (I - b k k^T) + b v k^T -----
def pin_brute_force_matrix_form(lib):
    rng = np.random.default_rng(15)
    for d in (2, 3, 4):
        H, HV, T = 2, 4, 6
        q = rng.standard_normal((T, H, d)); k = rng.standard_normal((T, H, d))
        v = rng.standard_normal((T, HV, d))
        g = -rng.random((T, HV)); beta = rng.random((T, HV))
        S0 = rng.standard_normal((HV, d, d))
        rec = np.zeros((2, HV, d, d)); rec[1] = S0
        o = oracle.prefill(q, k, v, g, beta, [0, T], [1], rec, 0.5, flags=0, lib=lib)
        for hv in range(HV):
            h = hv // (HV // H)
            S = S0[hv].copy()
            for t in range(T):
                kk = k[t, h]
                S = math.exp(g[t, hv]) * S @ (np.eye(d) - beta[t, hv] * np.outer(kk, kk)) \
                    + beta[t, hv] * np.outer(v[t, hv], kk)
                assert np.allclose(o[t, hv], S @ (0.5 * q[t, h]), rtol=1e-12, atol=1e-13)
            assert np.allclose(rec[1, hv], S, rtol=1e-12, atol=1e-13)


# --- QK norm: x / sqrt(sum x^2 + 1e-6), scale on q only ([P1] QK norm) -------
def pin_qk_norm(lib):
    d = 8
    q = np.zeros(d); q[0], q[1] = 3.0, 4.0
    k = np.zeros(d); k[2] = 1.0
    S = np.eye(d)[None]                              # o = S q_hat = q_hat
    o, S1 = _one_token(lib, S, q, k, np.zeros(d), 0.0, 0.0, scale=0.25, flags=NORM)
    expect = np.zeros(d); expect[0], expect[1] = 3.0, 4.0
    expect = expect / math.sqrt(25.0 + 1e-6) * 0.25
    assert np.allclose(o[0], expect, rtol=0, atol=1e-15)
    # k normalised (not scaled): beta = 1, g = 0 writes v along k_hat; with S = 0,
    # S' = v k_hat^T with k_hat = k / sqrt(|k|^2 + 1e-6)
    k2 = np.zeros(d); k2[3] = 2.0
    v = np.arange(d, dtype=np.float64)
    _, S2 = _one_token(lib, np.zeros((1, d, d)), np.ones(d), k2, v, 0.0, 1.0, scale=0.25,
                       flags=NORM)
    khat = k2 / math.sqrt(4.0 + 1e-6)
    u = 0.0
    assert np.allclose(S2[0], np.outer(v - u, khat), rtol=0, atol=1e-15)


# --- GQA map: key head j drives value heads j*grp .. j*grp+grp-1 --------------
def pin_gqa_map(lib):
    rng = np.random.default_rng(16)
    H, HV, d, T = 4, 8, 6, 3
    q = rng.standard_normal((T, H, d)); k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, HV, d)); g = -rng.random((T, HV)); b = rng.random((T, HV))
    S0 = rng.standard_normal((2, HV, d, d))
    base = oracle.prefill(q, k, v, g, b, [0, T], [1], S0.copy(), 1.0, flags=NORM, lib=lib)
    grp = HV // H
    for j in range(H):
        k2 = k.copy(); k2[:, j] += 0.5
        o = oracle.prefill(q, k2, v, g, b, [0, T], [1], S0.copy(), 1.0, flags=NORM, lib=lib)
        changed = [hv for hv in range(HV) if not np.array_equal(o[:, hv], base[:, hv])]
        assert changed == list(range(j * grp, (j + 1) * grp)), (j, changed)


# --- conv: varlen == token-by-token == direct sliding window; roll exact ------
def pin_conv_sliding_window(lib):
    rng = np.random.default_rng(17)
    dim, W, num_slots = 5, 4, 6
    weight = rng.standard_normal((dim, W)); bias = rng.standard_normal(dim)
    for L in (1, 2, 3, 4, 9):
        for use_bias in (False, True):
            st = rng.standard_normal((num_slots, dim, W - 1))
            x = rng.standard_normal((L, dim))
            st_a = st.copy()
            out = oracle.conv_update(x, [3], st_a, weight, bias if use_bias else None,
                                     cu_seqlens=[0, L], flags=0, lib=lib)
            X = np.concatenate([st[3].T, x], axis=0)          # [W-1+L, dim], oldest first
            for c in range(dim):
                ref = np.correlate(X[:, c], weight[c], mode="valid")  # sum_j X[t+j] w[j]
                if use_bias:
                    ref = ref + bias[c]
                assert np.allclose(out[:, c], ref, rtol=1e-14, atol=1e-14), (L, c)
            assert np.array_equal(st_a[3], X[-(W - 1):].T), "state must be the last W-1 inputs"
            others = [s for s in range(num_slots) if s != 3]
            assert np.array_equal(st_a[others], st[others])
            # token-by-token calls give the same numbers
            st_b = st.copy()
            outs = [oracle.conv_update(x[t:t + 1], [3], st_b, weight,
                                       bias if use_bias else None, flags=0, lib=lib)
                    for t in range(L)]
            assert np.array_equal(np.concatenate(outs), out)
            assert np.array_equal(st_b, st_a)


def pin_silu(lib):
    rng = np.random.default_rng(18)
    dim, W = 7, 4
    x = rng.standard_normal((1, dim)) * 4
    st = np.zeros((2, dim, W - 1))
    weight = np.zeros((dim, W)); weight[:, W - 1] = 1.0       # identity tap
    out = oracle.conv_update(x, [1], st, weight, flags=oracle.FLAG_SILU, lib=lib)
    assert np.allclose(out[0], x[0] * expit(x[0]), rtol=1e-15, atol=1e-15)


# --- decode entry point == conv + [q|k|v] split + one prefill token ----------
def pin_decode_split(lib):
    rng = np.random.default_rng(19)
    H, HV, dk, dv, W, B, ns = 2, 4, 4, 3, 4, 3, 5
    D = 2 * H * dk + HV * dv
    x = rng.standard_normal((B, D)); g = -rng.random((B, HV)); b = rng.random((B, HV))
    weight = np.zeros((D, W)); weight[:, W - 1] = 1.0          # conv = identity
    cs = rng.standard_normal((ns, D, W - 1)); rs = rng.standard_normal((ns, HV, dv, dk))
    slots = np.array([4, 1, 2], dtype=np.int32)
    rs_a = rs.copy()
    o = oracle.decode_step(x, g, b, slots, cs.copy(), weight, rs_a, H, HV, dk, dv, 0.3,
                           flags=NORM, lib=lib)
    for r in range(B):
        q = x[r, :H * dk].reshape(1, H, dk)
        k = x[r, H * dk:2 * H * dk].reshape(1, H, dk)
        v = x[r, 2 * H * dk:].reshape(1, HV, dv)
        rs_b = rs.copy()
        ob = oracle.prefill(q, k, v, g[r:r + 1], b[r:r + 1], [0, 1], [slots[r]], rs_b, 0.3,
                            flags=NORM, lib=lib)
        assert np.allclose(o[r], ob[0], rtol=1e-14, atol=1e-14)
        assert np.allclose(rs_a[slots[r]], rs_b[slots[r]], rtol=1e-14, atol=1e-14)


# --- chunked WY/UT form (independent route) == token-by-token oracle ---------
def pin_chunked_equals_token(lib, lengths_sets=((1,), (15, 16, 17), (63, 64, 65), (128, 130))):
    rng = np.random.default_rng(20)
    H, HV, d = 2, 4, 8
    for lengths in lengths_sets:
        for init in (False, True):
            T = sum(lengths)
            cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
            q = rng.standard_normal((T, H, d)); k = rng.standard_normal((T, H, d))
            v = rng.standard_normal((T, HV, d))
            g = -rng.random((T, HV)); b = rng.random((T, HV))
            ns = len(lengths) + 2
            rec = rng.standard_normal((ns, HV, d, d)) if init else np.zeros((ns, HV, d, d))
            slots = np.arange(len(lengths), 0, -1, dtype=np.int32) + 1
            r1, r2 = rec.copy(), rec.copy()
            o1 = oracle.prefill(q, k, v, g, b, cu, slots, r1, 0.35, flags=NORM, lib=lib)
            o2 = chunked_prefill(q, k, v, g, b, cu, slots, r2, 0.35, qk_l2norm=True)
            so = max(1.0, np.abs(o1).max()); ss = max(1.0, np.abs(r1).max())
            assert np.abs(o1 - o2).max() / so < 1e-12, (lengths, init)
            assert np.abs(r1 - r2).max() / ss < 1e-12, (lengths, init)


# --- indices: inactive rows zero + caches untouched; bad indices raise -------
def pin_slot_contract(lib):
    rng = np.random.default_rng(21)
    H, HV, dk, dv, W, ns = 1, 2, 4, 4, 4, 6
    D = 2 * H * dk + HV * dv
    x = rng.standard_normal((4, D)); g = -rng.random((4, HV)); b = rng.random((4, HV))
    w = rng.standard_normal((D, W))
    cs = rng.standard_normal((ns, D, W - 1)); rs = rng.standard_normal((ns, HV, dv, dk))
    cs0, rs0 = cs.copy(), rs.copy()
    slots = np.array([0, 3, -1, 5], dtype=np.int32)
    o = oracle.decode_step(x, g, b, slots, cs, w, rs, H, HV, dk, dv, 0.5, lib=lib)
    assert np.array_equal(o[0], np.zeros_like(o[0])) and np.array_equal(o[2], np.zeros_like(o[2]))
    # several padded rows may share the null slot (or the same negative value)
    o2 = oracle.decode_step(x, g, b, np.array([0, 0, -1, -1], dtype=np.int32), cs.copy(), w,
                            rs.copy(), H, HV, dk, dv, 0.5, lib=lib)
    assert np.array_equal(o2, np.zeros_like(o2))
    assert np.abs(o[1]).max() > 0 and np.abs(o[3]).max() > 0
    untouched = [0, 1, 2, 4]
    assert np.array_equal(cs[untouched], cs0[untouched]) and np.array_equal(rs[untouched], rs0[untouched])
    for bad, code in (([1, 6, 2, 3], oracle.ERR_SLOT_RANGE), ([1, 2, 2, 3], oracle.ERR_SLOT_REPEAT)):
        cs1, rs1 = cs0.copy(), rs0.copy()
        try:
            oracle.decode_step(x, g, b, np.array(bad, dtype=np.int32), cs1, w, rs1, H, HV, dk, dv,
                               0.5, lib=lib)
        except oracle.OracleError as e:
            assert e.code & code
        else:
            raise AssertionError(f"bad slots {bad} accepted")
        assert np.array_equal(cs1, cs0) and np.array_equal(rs1, rs0)
    # prefill: bad cu_seqlens raises, inactive sequence -> zeros
    q = rng.standard_normal((5, H, dk)); kk = rng.standard_normal((5, H, dk))
    v = rng.standard_normal((5, HV, dv)); gg = -rng.random((5, HV)); bb = rng.random((5, HV))
    rs1 = rs0.copy()
    o = oracle.prefill(q, kk, v, gg, bb, [0, 2, 5], [0, 4], rs1, 1.0, lib=lib)
    assert np.array_equal(o[:2], np.zeros_like(o[:2])) and np.abs(o[2:]).max() > 0
    for cu in ([0, 3, 2], [0, 2, 4], [1, 2, 5]):
        try:
            oracle.prefill(q, kk, v, gg, bb, cu, [1, 4], rs0.copy(), 1.0, lib=lib)
        except oracle.OracleError as e:
            assert e.code & oracle.ERR_SEQLENS
        else:
            raise AssertionError(f"bad cu_seqlens {cu} accepted")


# --- G6: fused gating ([P1] "How the golden relates to the kernel", item 1) --
def pin_gating(lib):
    """beta against scipy's expit; softplus against numpy's logaddexp(0, x)
    below the threshold and the identity above it; g's closed forms at
    a + dt_bias = 0 (-exp(A_log) ln 2); per-head A_log / dt_bias indexing;
    dt_bias enters additively (shifting a by c and dt_bias by -c changes
    nothing)."""
    rng = np.random.default_rng(41)
    rows, HV = 7, 5
    a = rng.standard_normal((rows, HV)) * 4.0
    a[0, :] = [-30.0, -1.0, 19.5, 20.5, 40.0]
    b = rng.standard_normal((rows, HV)) * 3.0
    b[1, :] = [0.0, -50.0, 50.0, 1.0, -1.0]
    A_log = rng.standard_normal(HV)
    dt_bias = np.array([0.0, 0.5, 0.5, 0.5, -0.25])
    a[0, :] -= dt_bias                       # row 0 probes x = a + dt_bias exactly
    g, beta = oracle.gating(a, b, A_log, dt_bias, lib=lib)
    assert np.allclose(beta, expit(b), rtol=1e-15, atol=0), "beta must be sigmoid(b)"
    x = a + dt_bias[None, :]
    sp = np.where(x <= 20.0, np.logaddexp(0.0, x), x)
    assert np.allclose(g, -np.exp(A_log)[None, :] * sp, rtol=1e-14, atol=0)
    # threshold branch: identity above 20 (exactly), log1p(exp) at and below
    assert g[0, 3] == -math.exp(A_log[3]) * x[0, 3]
    assert g[0, 4] == -math.exp(A_log[4]) * x[0, 4]
    assert abs(g[0, 2] / -math.exp(A_log[2]) - (19.5 + math.log1p(math.exp(-19.5)))) < 1e-13
    # closed form at x = 0 and A_log = log 3
    g0, _ = oracle.gating(np.zeros((1, 2)), np.zeros((1, 2)), np.array([0.0, math.log(3.0)]),
                          np.zeros(2), lib=lib)
    assert abs(g0[0, 0] + math.log(2.0)) < 1e-15 and abs(g0[0, 1] + 3 * math.log(2.0)) < 1e-14
    # additive dt_bias
    g1, _ = oracle.gating(a + 0.75, b, A_log, dt_bias - 0.75, lib=lib)
    assert np.allclose(g1, g, rtol=1e-13, atol=0)
    assert np.all(g <= 0.0) and np.all((beta >= 0.0) & (beta <= 1.0))


# --- gated RMSNorm epilogue (plain definition; [P1] "Latest Status") ------------
def pin_gated_rmsnorm(lib):
    """Facts about an RMS normalisation that do not restate the formula:
    with eps = 0 and unit weights the normalised row has sum of squares
    exactly dim (catches sum-vs-mean, a missing sqrt) and is invariant to
    scaling the row; SiLU(0) = 0 and sigmoid(0) = 1/2 fix the gate forms; a
    weight of -1 under the zero-centred offset gives zeros; a zero row stays
    zero; rows are independent (each row alone equals the row in a batch);
    large gate inputs make SiLU the identity and sigmoid 1."""
    rng = np.random.default_rng(51)
    rows, dim = 6, 48
    x = rng.standard_normal((rows, dim)) * rng.uniform(0.1, 10.0, (rows, 1))
    ones = np.ones(dim)
    y = oracle.gated_rmsnorm(x, ones, eps=0.0, lib=lib)
    assert np.allclose((y ** 2).sum(axis=1), dim, rtol=1e-13, atol=0)
    y7 = oracle.gated_rmsnorm(7.5 * x, ones, eps=0.0, lib=lib)
    assert np.allclose(y7, y, rtol=1e-13, atol=0)
    w = rng.standard_normal(dim)
    yw = oracle.gated_rmsnorm(x, w, eps=0.0, lib=lib)
    assert np.allclose(yw, y * w[None, :], rtol=1e-13, atol=1e-15)
    z0 = np.zeros_like(x)
    assert np.all(oracle.gated_rmsnorm(x, w, z=z0, eps=0.0, lib=lib) == 0.0)        # SiLU(0) = 0
    ys = oracle.gated_rmsnorm(x, w, z=z0, eps=0.0, flags=oracle.NORM_GATE_SIGMOID, lib=lib)
    assert np.allclose(ys, 0.5 * yw, rtol=1e-15, atol=0)                             # sigmoid(0)
    zbig = np.full_like(x, 60.0)
    assert np.allclose(oracle.gated_rmsnorm(x, w, z=zbig, eps=0.0, lib=lib), 60.0 * yw,
                       rtol=1e-13, atol=1e-13)                                       # SiLU ~ id
    assert np.allclose(oracle.gated_rmsnorm(x, w, z=zbig, eps=0.0,
                                            flags=oracle.NORM_GATE_SIGMOID, lib=lib), yw,
                       rtol=1e-13, atol=1e-15)                                        # sigmoid ~ 1
    assert np.all(oracle.gated_rmsnorm(x, -ones, eps=1e-6, flags=oracle.NORM_ZERO_CENTRED,
                                       lib=lib) == 0.0)
    xz = x.copy(); xz[2] = 0.0
    assert np.all(oracle.gated_rmsnorm(xz, w, eps=1e-6, lib=lib)[2] == 0.0)
    z = rng.standard_normal(x.shape)
    full = oracle.gated_rmsnorm(x, w, z=z, eps=1e-5, lib=lib)
    for r in range(rows):
        one = oracle.gated_rmsnorm(x[r:r + 1], w, z=z[r:r + 1], eps=1e-5, lib=lib)
        assert np.array_equal(one[0], full[r])
    # eps enters under the root: for a row of equal values c, y = c / sqrt(c^2 + eps)
    c = np.full((1, dim), 0.01)
    assert abs(oracle.gated_rmsnorm(c, ones, eps=1e-4, lib=lib)[0, 0] - 0.01 / math.sqrt(1e-4 + 1e-4)) < 1e-15


ALL_PINS = [pin_identity_step, pin_delta_rule_unit_key, pin_decay, pin_overwrite,
            pin_brute_force_matrix_form, pin_qk_norm, pin_gqa_map, pin_conv_sliding_window,
            pin_silu, pin_decode_split, pin_chunked_equals_token, pin_slot_contract,
            pin_gating, pin_gated_rmsnorm]


def run_all(lib):
    """Run every pin; return the names of those that failed (or raised)."""
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except Exception:  # noqa: BLE001 -- a mutant may fail in any way
            failed.append(pin.__name__)
    return failed


def check_inverse_and_newton_schulz():
    """The block inverse is exact to fp64 eps; NS from X0 = I - N is exact after
    3 rounds on a 16x16 block in exact arithmetic ([P4] root cause), and a
    bf16-stored NS is not, on correlated keys."""
    rng = np.random.default_rng(22)
    base = rng.standard_normal(32)
    K = base + 0.05 * rng.standard_normal((64, 32))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    A = 0.9 * np.tril(K @ K.T, -1)
    IA = np.eye(64) + A
    T = block_inverse(IA, 16)
    assert np.abs(IA @ T - np.eye(64)).max() < 1e-9
    assert np.abs(T - np.linalg.inv(IA)).max() < 1e-9 * max(1.0, np.abs(T).max())
    L16 = IA[:16, :16]
    N = L16 - np.eye(16)
    # residual I - L X_k = N^(2^(k+1)); nilpotent of index <= 16 -> 0 after 3 rounds
    assert np.allclose(np.linalg.matrix_power(N, 16), 0, atol=1e-300)
    X3 = newton_schulz_unit_lower_inverse(L16, 3)
    X2 = newton_schulz_unit_lower_inverse(L16, 2)
    ex = np.linalg.inv(L16)
    err3 = np.abs(X3 - ex).max(); err2 = np.abs(X2 - ex).max()
    assert err3 < 1e-9 * np.abs(ex).max(), err3
    assert err2 > 1e3 * err3
    return err2, err3
