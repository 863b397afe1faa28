"""The process-pool helper that runs the oracle's wrappers over all heads of
the large workloads returns what one direct call of the same wrapper returns
(CPU only)."""

import numpy as np

import oracle
import oracle_pool as OP


def _close(a, b):
    assert a.shape == b.shape
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


def test_pool_gdr_forward_and_backward_match_direct_calls():
    r = np.random.default_rng(3)
    lengths, H, DK, DV = [70, 0, 5, 129], 5, 4, 3
    T = sum(lengths)
    q, k = r.standard_normal((1, T, H, DK)), r.standard_normal((1, T, H, DK)) / 2
    v, do = r.standard_normal((1, T, H, DV)), r.standard_normal((1, T, H, DV))
    g, beta = -np.abs(r.standard_normal((1, T, H))) * 0.1, r.uniform(0, 1, (1, T, H))
    h0, dhT = r.standard_normal((4, H, DK, DV)), r.standard_normal((4, H, DK, DV))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    a = OP.gdr_forward_all_heads(q, k, v, g, beta, h0, cu, 0.5)
    b = oracle.gdr_recurrent_fp64(q, k, v, g, beta, h0, cu, 0.5)
    for key in ("o", "v_new", "h", "hT"):
        _close(a[key], b[key])
    a = OP.gdr_backward_all_heads(q, k, g, beta, do, dhT, cu, 0.5)
    b = oracle.gdr_backward_fp64(q, k, g, beta, do, dhT, cu, 0.5)
    for key in ("dh", "dh0", "dv_new"):
        _close(a[key], b[key])


def test_pool_abc_matches_direct_calls():
    r = np.random.default_rng(4)
    B, T, H, K, M, V = 2, 70, 3, 4, 2, 5
    q, k, v, s = (r.standard_normal((B, T, H, x)) for x in (K, K, V, M))
    p, ds, do = r.uniform(0, 1, (B, T, H, M)), r.standard_normal((B, T, H, M)), r.standard_normal((B, T, H, V))
    ek, ev = r.standard_normal((B, H, K, M)), r.standard_normal((B, H, M, V))
    a, b = OP.abc_states_all(k, v, s), oracle.abc_recurrent_fp64(k, v, s)
    for key in ("z", "hk", "hv", "hk_final", "hv_final"):
        _close(a[key], b[key])
    a, b = OP.abc_read_all(q, k, v, s, 0.3), oracle.abc_forward_fp64(q, k, v, s, 0.3)
    for key in ("o", "p"):
        _close(a[key], b[key])
    a = OP.abc_backward_all(q, s, p, ds, do, ek, ev, 0.3)
    b = oracle.abc_backward_fp64(q, s, p, ds, do, ek, ev, 0.3)
    for key in ("dhk", "dhv"):
        _close(a[key], b[key])
