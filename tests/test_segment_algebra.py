"""The segment map that the segment-parallel prefill relies on, checked on the
fp64 oracle (CPU).

The token update S <- exp(g) S (I - beta k k^T) + beta v k^T (o = S q, state
S[v, k]) is affine in S, so a run over any token range maps its start state S
to S P + B, where P is the run from the identity with v = 0 and B the run from
the zero state.  Cutting a sequence into segments, composing the segment maps
in order and rerunning each segment from its composed start state reproduces
the whole run.  These checks exercise the oracle alone; the GPU schedule is
compared with the oracle in the GPU tests.
"""
import numpy as np

import oracle


def _inputs(T, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, 1, d))
    k = rng.standard_normal((T, 1, d))
    v = rng.standard_normal((T, 1, d))
    g = -rng.uniform(0.0, 1.0, (T, 1))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, 1))))
    S0 = 0.3 * rng.standard_normal((d, d))
    return q, k, v, g, b, S0


def _run(q, k, v, g, b, S, scale):
    """One sequence over all rows given, from state S; returns (o [T, dv], end state)."""
    d = q.shape[2]
    rec = np.zeros((2, 1, d, d))
    rec[1, 0] = S
    o = oracle.prefill(q, k, v, g, b, np.array([0, q.shape[0]], np.int32),
                       np.array([1], np.int32), rec, scale)
    return o[:, 0], rec[1, 0].copy()


def test_run_is_affine_in_its_start_state():
    d, T = 8, 150
    q, k, v, g, b, S0 = _inputs(T, d, 5)
    scale = d ** -0.5
    _, S_end = _run(q, k, v, g, b, S0, scale)
    _, P = _run(q, k, np.zeros_like(v), g, b, np.eye(d), scale)
    _, B = _run(q, k, v, g, b, np.zeros((d, d)), scale)
    assert np.max(np.abs(S_end - (S0 @ P + B))) < 1e-12
    # and not trivially: P is far from the identity, B from zero
    assert np.max(np.abs(P - np.eye(d))) > 0.1 and np.max(np.abs(B)) > 0.1


def test_segment_maps_compose_to_the_whole_run():
    d, T, seg = 8, 230, 64
    q, k, v, g, b, S0 = _inputs(T, d, 6)
    scale = d ** -0.5
    o_ref, S_ref = _run(q, k, v, g, b, S0, scale)
    bounds = list(range(0, T, seg)) + [T]
    start = S0
    o = np.full_like(o_ref, np.nan)
    for a, e in zip(bounds[:-1], bounds[1:]):
        sl = slice(a, e)
        # rerun the segment from its composed start state (outputs), then
        # advance the start state by the segment's map S P + B
        o[sl], _ = _run(q[sl], k[sl], v[sl], g[sl], b[sl], start, scale)
        _, P = _run(q[sl], k[sl], np.zeros_like(v[sl]), g[sl], b[sl], np.eye(d), scale)
        _, B = _run(q[sl], k[sl], v[sl], g[sl], b[sl], np.zeros((d, d)), scale)
        start = start @ P + B
    assert np.max(np.abs(o - o_ref)) < 1e-11
    assert np.max(np.abs(start - S_ref)) < 1e-11
