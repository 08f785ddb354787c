"""Test-only fp64 chunked (WY / UT) formulation of the gated delta rule.

This is NOT the oracle and not the product path: it is a second, independent
route to the same numbers, used to pin the token-by-token oracle (the chunked
form must equal it to rounding) and to check the chunk algebra before any
kernel relies on it.

Per value head, for one chunk of L tokens with state S0 [dv, dk] at its start
(o = S q convention, S[v, k]) and cumulative log-decay gamma_r = sum_{i<=r} g_i:

    A[r, i] = beta_r * exp(gamma_r - gamma_i) * (k_r . k_i)      for i < r
    T       = (I + A)^-1                       (unit lower triangular)
    W       = T diag(beta * exp(gamma)) K       Ut = T diag(beta) V
    U       = Ut - W S0^T                       (rows: beta_r times the delta)
    O       = diag(exp(gamma)) Q S0^T + (M o P) U,
              P[r, i] = q_r . k_i,  M[r, i] = exp(gamma_r - gamma_i) for i <= r
    S_L     = exp(gamma_L) S0 + U^T diag(exp(gamma_L - gamma)) K

T is formed the way vLLM PR #53864 ("Numerical root cause and fix")
describes the structure: inverses of the 16x16 diagonal blocks of the
lower-triangular KK^T matrix, here by exact forward substitution, then merged
16 -> 32 -> 64 with T21 = -T22 A21 T11.  The 64-token chunk is the grid of
RL-Kernel PR #469 (mixed-step notes on 64-token scheduler alignment).
"""
import numpy as np


def l2norm(x, eps=1e-6):
    """x / sqrt(sum(x*x) + eps) over the last axis (RL-Kernel PR #469, QK norm)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def forward_subst_unit_lower_inverse(Lm):
    """Inverse of a unit lower-triangular matrix, column by column."""
    n = Lm.shape[0]
    T = np.zeros_like(Lm)
    for c in range(n):
        T[c, c] = 1.0
        for r in range(c + 1, n):
            T[r, c] = -np.dot(Lm[r, c:r], T[c:r, c])
    return T


def block_inverse(IA, block=16):
    """(I + A)^-1 from diagonal-block inverses merged pairwise (16 -> 32 -> 64)."""
    n = IA.shape[0]
    T = np.zeros_like(IA)
    for b0 in range(0, n, block):
        b1 = min(n, b0 + block)
        T[b0:b1, b0:b1] = forward_subst_unit_lower_inverse(IA[b0:b1, b0:b1])
    size = block
    while size < n:
        for b0 in range(0, n, 2 * size):
            m = b0 + size
            e = min(n, b0 + 2 * size)
            if m >= n:
                continue
            T11 = T[b0:m, b0:m]
            T22 = T[m:e, m:e]
            A21 = IA[m:e, b0:m]
            T[m:e, b0:m] = -T22 @ A21 @ T11
        size *= 2
    return T


def newton_schulz_unit_lower_inverse(Lm, rounds, x0="first_order", store=None):
    """Newton-Schulz X <- X (2I - L X) for a unit lower-triangular L.

    Starting from X0 = I - N (N the strict lower part), the residual after k
    rounds is N^(2^(k+1)), so 16x16 blocks are exact after 3 rounds in exact
    arithmetic (the statement of vLLM PR #53864).  ``store`` optionally rounds
    X after every round (to emulate a low-precision intermediate).
    """
    n = Lm.shape[0]
    eye = np.eye(n)
    X = eye - (Lm - eye) if x0 == "first_order" else eye.copy()
    for _ in range(rounds):
        X = X @ (2 * eye - Lm @ X)
        if store is not None:
            X = store(X)
    return X


def chunked_prefill(q, k, v, g, beta, cu_seqlens, slot_idx, rec_state, scale,
                    qk_l2norm=True, chunk=64, block=16):
    """Chunked fp64 prefill; same contract as the oracle's ``prefill``."""
    T_, H, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    grp = HV // H
    out = np.zeros((T_, HV, dv))
    for n in range(len(slot_idx)):
        s0, s1 = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        slot = int(slot_idx[n])
        if slot <= 0:
            continue
        for hv in range(HV):
            h = hv // grp
            S = rec_state[slot, hv].copy()
            for c0 in range(s0, s1, chunk):
                c1 = min(s1, c0 + chunk)
                Q = q[c0:c1, h].astype(np.float64)
                K = k[c0:c1, h].astype(np.float64)
                if qk_l2norm:
                    Q, K = l2norm(Q), l2norm(K)
                Q = Q * scale
                V = v[c0:c1, hv].astype(np.float64)
                gg = g[c0:c1, hv].astype(np.float64)
                bb = beta[c0:c1, hv].astype(np.float64)
                L = c1 - c0
                gam = np.cumsum(gg)
                D = gam[:, None] - gam[None, :]
                lower_strict = np.tril(np.ones((L, L)), -1)
                lower = np.tril(np.ones((L, L)))
                Dm = np.where(lower > 0, D, -np.inf)
                decay = np.exp(Dm)                      # exp(gamma_r - gamma_i), i <= r
                G = K @ K.T
                A = bb[:, None] * decay * G * lower_strict
                Tm = block_inverse(np.eye(L) + A, block)
                W = Tm @ ((bb * np.exp(gam))[:, None] * K)
                Ut = Tm @ (bb[:, None] * V)
                U = Ut - W @ S.T
                P = Q @ K.T
                O = np.exp(gam)[:, None] * (Q @ S.T) + (decay * P) @ U
                out[c0:c1, hv] = O
                S = np.exp(gam[-1]) * S + U.T @ (np.exp(gam[-1] - gam)[:, None] * K)
            rec_state[slot, hv] = S
    return out
