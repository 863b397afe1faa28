"""Pins of the FP64 oracle against facts that do not come from the oracle itself.

Each ``check_*`` takes the oracle module(s) as arguments so the mutation tests
can run the very same checks against deliberately broken copies of the
oracle source.  A check raises AssertionError when the oracle disagrees with
the independent fact it encodes:

* brute force: dense transition matrices a_t (I - b_t k_t k_t^T) multiplied out
  explicitly for short sequences;
* exact rationals: the same products in ``fractions.Fraction`` arithmetic;
* closed forms: pure decay when b = 0, exact recall of orthonormal keys when
  a = b = 1, the ABC normaliser as a prefix log-sum-exp and the normalised
  states as explicit weighted sums;
* invariants: linearity in (S0, v), independence of packed sequences, linear
  output scale, slot weights summing to one;
* for the reverse recurrence: central finite differences of the (pinned)
  forward oracles, which are exact here because the loss is linear in the
  perturbed state or write vector, the pure-decay closed form, and the
  reverse chunk relation the GPU kernel uses.
"""

from __future__ import annotations

from fractions import Fraction as Fr

import numpy as np

TOL = 1e-12


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def _assert_close(a, b, tol=TOL, what=""):
    r = rel(a, b)
    assert r <= tol, f"{what}: relative L2 {r:.3e} > {tol:.1e}"


def rand_problem(seed, L, H, DK, DV, contract=True):
    """Small random float64 problem (one sequence): q, k unit rows, v normal,
    a in (0, 1], b in (0, 1)."""
    r = np.random.default_rng(seed)
    q = r.standard_normal((L, H, DK))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = r.standard_normal((L, H, DK))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((L, H, DV))
    a = 1.0 / (1.0 + np.exp(-r.normal(3.0, 1.0, (L, H)))) if contract else np.ones((L, H))
    b = 1.0 / (1.0 + np.exp(-r.standard_normal((L, H))))
    S0 = 0.3 * r.standard_normal((H, DK, DV))
    return q, k, v, a, b, S0


# --------------------------------------------------------------------------- brute force
def brute_force_states(k, v, a, b, S0):
    """One head: explicit dense transitions.  Returns the list S_1..S_L where
    S_t = P(t,1) S0 + sum_{i<=t} P(t,i+1) b_i k_i v_i^T and P(t,j) = A_t...A_j."""
    L, DK = k.shape
    A = [a[t] * (np.eye(DK) - b[t] * np.outer(k[t], k[t])) for t in range(L)]
    out = []
    for t in range(L):
        # P(t, 1) = A_t ... A_1, built by left-multiplying in token order
        P_all = np.eye(DK)
        for j in range(0, t + 1):
            P_all = A[j] @ P_all
        S = P_all @ S0
        for i in range(t + 1):
            Pi = np.eye(DK)
            for j in range(i + 1, t + 1):
                Pi = A[j] @ Pi
            S = S + Pi @ (b[i] * np.outer(k[i], v[i]))
        out.append(S)
    return out


def check_brute_force(gdr_ref):
    L, H, DK, DV, C = 13, 2, 5, 3, 4
    q, k, v, a, b, S0 = rand_problem(11, L, H, DK, DV)
    o, pre, ST = gdr_ref.gdr_scan_sequence(q, k, v, a, b, S0, 1.0, C)
    for h in range(H):
        Ss = brute_force_states(k[:, h], v[:, h], a[:, h], b[:, h], S0[h])
        _assert_close(ST[h], Ss[-1], what="final state vs dense products")
        o_bf = np.stack([Ss[t].T @ q[t, h] for t in range(L)])
        _assert_close(o[:, h], o_bf, what="outputs vs dense products")
        starts = list(range(0, L, C))
        assert pre.shape[0] == len(starts), "one pre-chunk state per chunk"
        for c, t0 in enumerate(starts):
            ref = S0[h] if t0 == 0 else Ss[t0 - 1]
            _assert_close(pre[c, h], ref, what=f"pre-chunk state {c}")


# --------------------------------------------------------------------------- exact rationals
def _fr_matmul(A, B):
    n, m = len(A), len(B[0])
    kk = len(B)
    return [[sum((A[i][x] * B[x][j] for x in range(kk)), Fr(0)) for j in range(m)] for i in range(n)]


def check_rationals(gdr_ref):
    """dk = dv = 3, T = 5, one head, every input a small rational: exact equality."""
    r = np.random.default_rng(5)
    L, D = 5, 3

    def fr(x, den=8):
        return Fr(int(round(x * den)), den)

    q = [[fr(x) for x in r.standard_normal(D)] for _ in range(L)]
    k = [[fr(x) for x in r.standard_normal(D)] for _ in range(L)]
    v = [[fr(x) for x in r.standard_normal(D)] for _ in range(L)]
    a = [Fr(int(r.integers(5, 16)), 16) for _ in range(L)]
    b = [Fr(int(r.integers(1, 8)), 8) for _ in range(L)]
    S0 = [[fr(x, 4) for x in r.standard_normal(D)] for _ in range(D)]
    # dense transition products in exact arithmetic
    S = S0
    o_ref, pre_ref = [], []
    for t in range(L):
        if t % 2 == 0:
            pre_ref.append(S)
        A = [[a[t] * ((Fr(1) if i == j else Fr(0)) - b[t] * k[t][i] * k[t][j]) for j in range(D)]
             for i in range(D)]
        S = _fr_matmul(A, S)
        S = [[S[i][j] + b[t] * k[t][i] * v[t][j] for j in range(D)] for i in range(D)]
        o_ref.append([sum((S[i][j] * q[t][i] for i in range(D)), Fr(0)) for j in range(D)])

    def obj(x, shape):
        arr = np.empty(shape, dtype=object)
        arr[...] = np.array(x, dtype=object).reshape(shape)
        return arr

    o, pre, ST = gdr_ref.gdr_scan_sequence(
        obj(q, (L, 1, D)), obj(k, (L, 1, D)), obj(v, (L, 1, D)), obj(a, (L, 1)), obj(b, (L, 1)),
        obj(S0, (1, D, D)), Fr(1), 2)
    assert all(ST[0, i, j] == S[i][j] for i in range(D) for j in range(D)), "final state not exact"
    assert all(o[t, 0, j] == o_ref[t][j] for t in range(L) for j in range(D)), "outputs not exact"
    assert len(pre) == len(pre_ref)
    for c in range(len(pre_ref)):
        assert all(pre[c, 0, i, j] == pre_ref[c][i][j] for i in range(D) for j in range(D)), \
            f"pre-chunk state {c} not exact"


# --------------------------------------------------------------------------- closed forms
def check_pure_decay(gdr_ref):
    L, H, DK, DV, C = 40, 3, 6, 4, 16
    q, k, v, a, b, S0 = rand_problem(21, L, H, DK, DV)
    b = np.zeros_like(b)
    o, pre, ST = gdr_ref.gdr_scan_sequence(q, k, v, a, b, S0, 1.0, C)
    cum = np.cumprod(a, axis=0)                              # prod_{s<=t} a_s
    _assert_close(ST, cum[-1][:, None, None] * S0, what="b=0 final state")
    o_cf = cum[:, :, None] * np.einsum("hkv,thk->thv", S0, q)
    _assert_close(o, o_cf, what="b=0 outputs")
    for c, t0 in enumerate(range(0, L, C)):
        f = np.ones(H) if t0 == 0 else cum[t0 - 1]
        _assert_close(pre[c], f[:, None, None] * S0, what=f"b=0 pre-chunk {c}")


def check_exact_recall(gdr_ref):
    DK, DV, L = 8, 5, 6
    r = np.random.default_rng(31)
    Qm, _ = np.linalg.qr(r.standard_normal((DK, DK)))
    K = Qm[:L]                                              # orthonormal keys
    V = r.standard_normal((L, DV))
    S0 = r.standard_normal((DK, DV))
    o, pre, ST = gdr_ref.gdr_scan_sequence(K[:, None], K[:, None], V[:, None], np.ones((L, 1)),
                                           np.ones((L, 1)), S0[None], 1.0, 64)
    _assert_close(ST[0], (np.eye(DK) - K.T @ K) @ S0 + K.T @ V, TOL, "recall closed form")
    for t in range(L):
        _assert_close(ST[0].T @ K[t], V[t], TOL, f"recall of key {t}")
    # overwrite: the same key twice keeps only the second value
    k1 = K[0]
    kk = np.stack([k1, k1])[:, None]
    vv = np.stack([V[0], V[1]])[:, None]
    _, _, S2 = gdr_ref.gdr_scan_sequence(kk, kk, vv, np.ones((2, 1)), np.ones((2, 1)), S0[None], 1.0, 64)
    _assert_close(S2[0].T @ k1, V[1], TOL, "overwrite")
    _assert_close(S2[0], (np.eye(DK) - np.outer(k1, k1)) @ S0 + np.outer(k1, V[1]), TOL, "overwrite state")


# --------------------------------------------------------------------------- invariants
def check_linearity(gdr_ref):
    L, H, DK, DV = 20, 2, 6, 5
    q, k, v, a, b, S0 = rand_problem(41, L, H, DK, DV)
    _, _, v2, _, _, S02 = rand_problem(42, L, H, DK, DV)
    al, be = 0.7, -1.3
    o1, p1, T1 = gdr_ref.gdr_scan_sequence(q, k, v, a, b, S0, 1.0, 8)
    o2, p2, T2 = gdr_ref.gdr_scan_sequence(q, k, v2, a, b, S02, 1.0, 8)
    o3, p3, T3 = gdr_ref.gdr_scan_sequence(q, k, al * v + be * v2, a, b, al * S0 + be * S02, 1.0, 8)
    _assert_close(o3, al * o1 + be * o2, 1e-11, "linearity of outputs")
    _assert_close(T3, al * T1 + be * T2, 1e-11, "linearity of final state")
    _assert_close(p3, al * p1 + be * p2, 1e-11, "linearity of pre-chunk states")
    o4, _, _ = gdr_ref.gdr_scan_sequence(q, k, v, a, b, S0, 0.25, 8)
    _assert_close(o4, 0.25 * o1, 1e-14, "output scale")


def check_sequence_independence(gdr_ref):
    lengths = [5, 70, 1, 64, 0, 130]
    H, DK, DV = 2, 6, 4
    r = np.random.default_rng(51)
    Ttot = sum(lengths)
    q = r.standard_normal((1, Ttot, H, DK))
    k = r.standard_normal((1, Ttot, H, DK)) / 3
    v = r.standard_normal((1, Ttot, H, DV))
    g = -np.abs(r.standard_normal((1, Ttot, H))) * 0.05
    beta = r.uniform(0, 1, (1, Ttot, H))
    h0 = r.standard_normal((len(lengths), H, DK, DV))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    full = gdr_ref.gdr_recurrent_fp64(q, k, v, g, beta, h0, cu, 1.0)
    offs = full["chunk_offsets"]
    assert list(np.diff(offs)) == [(x + 63) // 64 for x in lengths], "chunk counts"
    for n, L in enumerate(lengths):
        s, e = cu[n], cu[n + 1]
        one = gdr_ref.gdr_recurrent_fp64(q[:, s:e], k[:, s:e], v[:, s:e], g[:, s:e], beta[:, s:e],
                                         h0[n:n + 1], None, 1.0)
        _assert_close(full["o"][:, s:e], one["o"], 1e-15, f"seq {n} outputs")
        _assert_close(full["hT"][n], one["hT"][0], 1e-15, f"seq {n} final")
        _assert_close(full["h"][offs[n]:offs[n + 1]], one["h"], 1e-15, f"seq {n} pre-chunk")
        if L == 0:
            _assert_close(full["hT"][n], h0[n], 0.0, "empty sequence keeps h0")


def check_delta_definition(gdr_ref):
    """The recorded write vectors satisfy delta_t = b_t (v_t - a_t S_{t-1}^T k_t)."""
    L, H, DK, DV = 9, 2, 5, 3
    q, k, v, a, b, S0 = rand_problem(61, L, H, DK, DV)
    _, _, _, d = gdr_ref.gdr_scan_sequence(q, k, v, a, b, S0, 1.0, 64, return_delta=True)
    for h in range(H):
        Ss = [S0[h]] + brute_force_states(k[:, h], v[:, h], a[:, h], b[:, h], S0[h])
        for t in range(L):
            ref = b[t, h] * (v[t, h] - a[t, h] * Ss[t].T @ k[t, h])
            _assert_close(d[t, h], ref, TOL, f"delta_{t}")


def check_chunk_algebra(gdr_ref, chunked_ref):
    """The chunked WY form equals the token recurrence at several chunk sizes."""
    lengths = [1, 63, 64, 65, 150]
    H, DK, DV = 2, 8, 6
    r = np.random.default_rng(71)
    Ttot = sum(lengths)
    q = r.standard_normal((1, Ttot, H, DK))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = r.standard_normal((1, Ttot, H, DK))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((1, Ttot, H, DV))
    g = np.log(1 / (1 + np.exp(-r.normal(4, 1, (1, Ttot, H)))))
    beta = 1 / (1 + np.exp(-r.standard_normal((1, Ttot, H))))
    h0 = 0.1 * r.standard_normal((len(lengths), H, DK, DV))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    for C in (1, 2, 7, 16, 64):
        a = gdr_ref.gdr_recurrent_fp64(q, k, v, g, beta, h0, cu, 0.5, chunk=C)
        c = chunked_ref.gdr_chunked_fp64(q, k, v, g, beta, h0, cu, 0.5, chunk=C)
        for key in ("o", "v_new", "h", "hT"):
            _assert_close(c[key], a[key], 1e-12, f"chunk {C} {key}")


def check_segment_algebra(gdr_ref):
    L, H, DK, DV, P = 600, 2, 6, 4, 4
    q, k, v, a, b, S0 = rand_problem(81, L, H, DK, DV)
    g = np.log(a)
    bounds = gdr_ref.segment_bounds(L, P)
    assert bounds[0][0] == 0 and bounds[-1][1] == L
    assert all(bounds[i][1] == bounds[i + 1][0] for i in range(P - 1))
    assert all(t0 % 64 == 0 for t0, _ in bounds)
    S_loc, M = gdr_ref.gdr_segment_summaries_fp64(k, v, g, b, bounds)
    # transition products against dense matrices
    for s, (t0, t1) in enumerate(bounds):
        for h in range(H):
            D = np.eye(DK)
            for t in range(t0, t1):
                D = a[t, h] * (np.eye(DK) - b[t, h] * np.outer(k[t, h], k[t, h])) @ D
            _assert_close(M[s, h], D, 1e-12, f"M_{s}")
    inits, SP = gdr_ref.gdr_segment_compose_fp64(S_loc, M, S0)
    serial = gdr_ref.gdr_recurrent_fp64(q[None], k[None], v[None], g[None], b[None], S0[None], None)
    _assert_close(SP, serial["hT"][0], 1e-12, "composed final state")
    for s, (t0, _) in enumerate(bounds):
        _assert_close(inits[s], serial["h"][t0 // 64], 1e-12, f"segment {s} initial state")
    # one segment: S_T = M S0 + S_loc
    S_loc1, M1 = gdr_ref.gdr_segment_summaries_fp64(k, v, g, b, [(0, L)])
    _assert_close(np.matmul(M1[0], S0) + S_loc1[0], serial["hT"][0], 1e-12, "affine summary")


def check_segment_bounds(gdr_ref):
    """The even chunk split: 1024 chunks over 16 segments, a ragged split, and
    more segments than chunks."""
    b = gdr_ref.segment_bounds(65536, 16)
    assert b == [(64 * 64 * s, 64 * 64 * (s + 1)) for s in range(16)]
    # 10 chunks over 4 segments -> 3, 3, 2, 2 chunks; the tail ends at L
    b = gdr_ref.segment_bounds(600, 4)
    assert b == [(0, 192), (192, 384), (384, 512), (512, 600)], b
    b = gdr_ref.segment_bounds(100, 4)
    assert b == [(0, 64), (64, 100), (100, 100), (100, 100)], b


GDR_CHECKS = [check_segment_bounds, check_brute_force, check_rationals, check_pure_decay, check_exact_recall,
              check_linearity, check_sequence_independence, check_delta_definition,
              check_segment_algebra]


# --------------------------------------------------------------------------- ABC
def _cum_lse(s):
    """log sum_{i<=t} exp(s_i) along axis 0, computed by explicit prefix sums of
    exp(s - max) (a different route from the oracle's pairwise logaddexp)."""
    m = np.max(s, axis=0, keepdims=True)
    return np.log(np.cumsum(np.exp(s - m), axis=0)) + m


def check_abc_closed_form(abc_ref):
    T, H, K, M, V = 150, 2, 5, 4, 3
    r = np.random.default_rng(91)
    k = r.standard_normal((T, H, K))
    v = r.standard_normal((T, H, V))
    s = r.standard_normal((T, H, M)) * 2
    z, hk_pre, hv_pre, hk, hv = abc_ref.abc_scan_sequence(k, v, s, 64)
    zc = _cum_lse(s)
    _assert_close(z, zc, 1e-13, "normaliser = prefix log-sum-exp")
    for c, t0 in enumerate(range(0, T, 64)):
        if t0 == 0:
            assert np.all(hk_pre[0] == 0) and np.all(hv_pre[0] == 0)
            continue
        wts = np.exp(s[:t0] - zc[t0 - 1][None])              # [t0, H, M]
        _assert_close(hk_pre[c], np.einsum("thk,thm->hkm", k[:t0], wts), 1e-12, f"Hk pre {c}")
        _assert_close(hv_pre[c], np.einsum("thm,thv->hmv", wts, v[:t0]), 1e-12, f"Hv pre {c}")
    wts = np.exp(s - zc[-1][None])
    _assert_close(hk, np.einsum("thk,thm->hkm", k, wts), 1e-12, "Hk final")
    _assert_close(hv, np.einsum("thm,thv->hmv", wts, v), 1e-12, "Hv final")


def check_abc_ones(abc_ref):
    T, H, K, M, V = 130, 2, 3, 4, 5
    r = np.random.default_rng(92)
    s = r.standard_normal((T, H, M)) * 3
    _, hk_pre, hv_pre, hk, hv = abc_ref.abc_scan_sequence(np.ones((T, H, K)), np.ones((T, H, V)), s, 64)
    _assert_close(hk, np.ones_like(hk), 1e-14, "weights sum to one (Hk)")
    _assert_close(hv, np.ones_like(hv), 1e-14, "weights sum to one (Hv)")
    _assert_close(hk_pre[1:], np.ones_like(hk_pre[1:]), 1e-14, "pre-chunk Hk")


def check_abc_constant_logits(abc_ref):
    T, H, K, M, V = 100, 1, 4, 3, 2
    r = np.random.default_rng(93)
    k = r.standard_normal((T, H, K))
    v = r.standard_normal((T, H, V))
    s = np.broadcast_to(r.standard_normal((1, H, M)), (T, H, M)).copy()
    _, _, _, hk, hv = abc_ref.abc_scan_sequence(k, v, s, 64)
    mk = k.mean(axis=0)                                       # [H, K]
    mv = v.mean(axis=0)
    _assert_close(hk, np.broadcast_to(mk[:, :, None], hk.shape), 1e-13, "running mean (Hk)")
    _assert_close(hv, np.broadcast_to(mv[:, None, :], hv.shape), 1e-13, "running mean (Hv)")


def check_abc_rationals(abc_ref):
    """Weights given directly as rationals: exact match with the explicit sum
    H_T = sum_t x_t (x) w_t prod_{u>t} r_u."""
    T, K, M, V = 6, 2, 3, 2
    r = np.random.default_rng(94)

    def fr(x):
        return Fr(int(round(x * 8)), 8)

    def obj(a):
        o = np.empty(a.shape, dtype=object)
        o[...] = a
        return o

    k = obj(np.array([[fr(x) for x in r.standard_normal(K)] for _ in range(T)], dtype=object))
    v = obj(np.array([[fr(x) for x in r.standard_normal(V)] for _ in range(T)], dtype=object))
    w = obj(np.array([[Fr(int(r.integers(1, 9)), 8) for _ in range(M)] for _ in range(T)], dtype=object))
    rr = obj(np.array([[Fr(int(r.integers(1, 9)), 9) for _ in range(M)] for _ in range(T)], dtype=object))
    hk, hv = abc_ref.abc_weighted_scan(k, v, w, rr)
    for i in range(K):
        for m in range(M):
            ref = Fr(0)
            for t in range(T):
                f = Fr(1)
                for u in range(t + 1, T):
                    f *= rr[u, m]
                ref += k[t, i] * w[t, m] * f
            assert hk[i, m] == ref, "Hk not exact"
    for m in range(M):
        for j in range(V):
            ref = Fr(0)
            for t in range(T):
                f = Fr(1)
                for u in range(t + 1, T):
                    f *= rr[u, m]
                ref += w[t, m] * v[t, j] * f
            assert hv[m, j] == ref, "Hv not exact"


def check_abc_chunk_affine(abc_ref):
    """Chaining S_out = S_in * r_c + c_c per 64-token chunk reproduces the states."""
    T, H, K, M, V = 200, 2, 4, 3, 5
    r = np.random.default_rng(95)
    k = r.standard_normal((T, H, K))
    v = r.standard_normal((T, H, V))
    s = r.standard_normal((T, H, M))
    z, hk_pre, hv_pre, hk, hv = abc_ref.abc_scan_sequence(k, v, s, 64)
    zc = _cum_lse(s)
    Sk = np.zeros((H, K, M))
    Sv = np.zeros((H, M, V))
    zprev = np.full((H, M), -np.inf)
    for c, t0 in enumerate(range(0, T, 64)):
        t1 = min(t0 + 64, T)
        _assert_close(hk_pre[c], Sk, 1e-12, f"affine Hk {c}")
        _assert_close(hv_pre[c], Sv, 1e-12, f"affine Hv {c}")
        zl = zc[t1 - 1]
        E = np.exp(s[t0:t1] - zl[None])
        rc = np.exp(zprev - zl)
        Sk = Sk * rc[:, None, :] + np.einsum("thk,thm->hkm", k[t0:t1], E)
        Sv = Sv * rc[:, :, None] + np.einsum("thm,thv->hmv", E, v[t0:t1])
        zprev = zl
    _assert_close(hk, Sk, 1e-12, "affine Hk final")
    _assert_close(hv, Sv, 1e-12, "affine Hv final")


ABC_CHECKS = [check_abc_closed_form, check_abc_ones, check_abc_constant_logits,
              check_abc_rationals, check_abc_chunk_affine]


# --------------------------------------------------------------------------- reverse recurrence
def _bwd_problem(seed, L=8, H=2, DK=3, DV=2):
    q, k, v, a, b, S0 = rand_problem(seed, L, H, DK, DV)
    r = np.random.default_rng(seed + 1)
    do = r.standard_normal((L, H, DV))
    dS_end = r.standard_normal((H, DK, DV))
    return q, k, v, np.log(a), b, S0, do, dS_end


def _loss(gdr_ref, q, k, v, g, b, S0, do, dS_end, scale, chunk):
    o, _, Sf = gdr_ref.gdr_scan_sequence(q, k, v, np.exp(g), b, S0, scale, chunk)
    return float(np.sum(o * do) + np.sum(Sf * dS_end))


def _fd(f, x, eps=1e-6):
    """Central differences of a scalar function of an array."""
    grad = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[i] += eps
        xm[i] -= eps
        grad[i] = (f(xp) - f(xm)) / (2 * eps)
    return grad


def check_bwd_initial_state(bwd_ref, gdr_ref):
    """dh0 = dL/dS0 of L = sum <do, o> + <dS_end, S_final> (finite differences)."""
    q, k, v, g, b, S0, do, dS_end = _bwd_problem(91)
    _, dh0, _ = bwd_ref.gdr_backward_sequence(q, k, g, b, do, dS_end, 0.7, chunk=3)
    fd = _fd(lambda S: _loss(gdr_ref, q, k, v, g, b, S, do, dS_end, 0.7, 3), S0)
    _assert_close(dh0, fd, 1e-7, "dh0 vs finite differences")


def check_bwd_boundaries(bwd_ref, gdr_ref):
    """dh[c] = gradient of the loss of the tokens after chunk c with respect to
    the state they start from (finite differences on a restarted forward)."""
    chunk = 3
    q, k, v, g, b, S0, do, dS_end = _bwd_problem(92, L=8)
    dh, _, _ = bwd_ref.gdr_backward_sequence(q, k, g, b, do, dS_end, 0.7, chunk=chunk)
    L = q.shape[0]
    for c in range(dh.shape[0]):
        t0 = (c + 1) * chunk
        if t0 >= L:
            _assert_close(dh[c], dS_end, 1e-12, f"dh[{c}] after the last chunk")
            continue
        sl = slice(t0, L)
        fd = _fd(lambda S: _loss(gdr_ref, q[sl], k[sl], v[sl], g[sl], b[sl], S, do[sl], dS_end, 0.7, chunk),
                 np.zeros_like(S0))
        _assert_close(dh[c], fd, 1e-7, f"dh[{c}] vs finite differences")


def check_bwd_write_vectors(bwd_ref, chunked_ref):
    """dv_new = dL/dDelta of the chunk form (finite differences on Delta)."""
    chunk = 3
    q, k, v, g, b, S0, do, dS_end = _bwd_problem(93, L=8)
    _, _, dv = bwd_ref.gdr_backward_sequence(q, k, g, b, do, dS_end, 0.7, chunk=chunk)

    def loss(shift):
        r = chunked_ref.chunked_scan_sequence(q, k, v, g, b, S0, 0.7, chunk, delta_shift=shift)
        return float(np.sum(r["o"] * do) + np.sum(r["hT"] * dS_end))

    fd = _fd(loss, np.zeros_like(do))
    _assert_close(dv, fd, 1e-7, "dv_new vs finite differences")


def check_bwd_pure_decay(bwd_ref):
    """b = 0: dh0 = sum_t scale exp(g_1 + .. + g_t) q_t do_t^T + exp(sum g) dS_end."""
    q, k, v, g, b, S0, do, dS_end = _bwd_problem(94, L=9)
    b = np.zeros_like(b)
    _, dh0, _ = bwd_ref.gdr_backward_sequence(q, k, g, b, do, dS_end, 0.5, chunk=4)
    cg = np.cumsum(g, axis=0)
    ref = np.exp(cg[-1])[:, None, None] * dS_end
    for t in range(q.shape[0]):
        ref = ref + 0.5 * np.exp(cg[t])[:, None, None] * q[t][:, :, None] * do[t][:, None, :]
    _assert_close(dh0, ref, 1e-12, "pure decay dh0")


def check_bwd_chunk_relation(bwd_ref, chunked_ref):
    """The reverse chunk step the kernel runs:
    dS_c = e^{gamma_C} dh[c] + scale Q_c^T diag(e^gamma) dO_c - W_c^T dv_new_c,
    with dS_c = dh[c-1] (dh0 for the first chunk), W from the chunk form."""
    L, H, DK, DV, C = 150, 2, 8, 6, 64
    q, k, v, a, b, S0 = rand_problem(95, L, H, DK, DV)
    g = np.log(a)
    r = np.random.default_rng(96)
    do = r.standard_normal((L, H, DV))
    dS_end = r.standard_normal((H, DK, DV))
    dh, dh0, dv = bwd_ref.gdr_backward_sequence(q, k, g, b, do, dS_end, 0.7, chunk=C)
    fw = chunked_ref.chunked_scan_sequence(q, k, v, g, b, S0, 0.7, C)
    W, gam = fw["w"], fw["g_cum"]
    for c in range(dh.shape[0]):
        c0, c1 = c * C, min(L, (c + 1) * C)
        for hh in range(H):
            ga = gam[c0:c1, hh]
            lhs = (np.exp(ga[-1]) * dh[c, hh] + 0.7 * q[c0:c1, hh].T @ (np.exp(ga)[:, None] * do[c0:c1, hh])
                   - W[c0:c1, hh].T @ dv[c0:c1, hh])
            prev = dh0[hh] if c == 0 else dh[c - 1, hh]
            _assert_close(lhs, prev, 1e-10, f"reverse chunk step {c}")


BWD_CHECKS = [check_bwd_initial_state, check_bwd_boundaries, check_bwd_write_vectors, check_bwd_pure_decay,
              check_bwd_chunk_relation]


def run_bwd_check(check, bwd_ref, gdr_ref, chunked_ref):
    if check.__name__ == "check_bwd_wrapper_packed":
        return check(bwd_ref, gdr_ref, chunked_ref)
    if check in (check_bwd_initial_state, check_bwd_boundaries):
        return check(bwd_ref, gdr_ref)
    if check in (check_bwd_write_vectors, check_bwd_chunk_relation):
        return check(bwd_ref, chunked_ref)
    return check(bwd_ref)


# --------------------------------------------------------------------------- ABC reads and reverse recurrence
def check_abc_resume(abc_ref):
    """Resuming from the carried states and normaliser reproduces the whole run."""
    T, H, K, M, V = 150, 2, 3, 4, 2
    r = np.random.default_rng(97)
    k = r.standard_normal((T, H, K))
    v = r.standard_normal((T, H, V))
    s = r.standard_normal((T, H, M)) * 2
    z, hk_pre, hv_pre, hk, hv = abc_ref.abc_scan_sequence(k, v, s, 64)
    t1 = 64
    za, _, _, hka, hva = abc_ref.abc_scan_sequence(k[:t1], v[:t1], s[:t1], 64)
    zb, hk_preb, hv_preb, hkb, hvb = abc_ref.abc_scan_sequence(k[t1:], v[t1:], s[t1:], 64, hka, hva, za[-1])
    _assert_close(np.concatenate([za, zb]), z, 1e-13, "resumed normaliser")
    _assert_close(hk_preb, hk_pre[1:], 1e-12, "resumed pre-chunk Hk")
    _assert_close(hv_preb, hv_pre[1:], 1e-12, "resumed pre-chunk Hv")
    _assert_close(hkb, hk, 1e-12, "resumed Hk")
    _assert_close(hvb, hv, 1e-12, "resumed Hv")


def check_abc_readout(abc_ref):
    """The reads against the explicit weighted sums, and the softmax read with
    constant logits: every slot holds the running mean, so the weights are
    uniform and o_t is the running mean of v."""
    T, H, K, M, V = 70, 2, 3, 4, 5
    r = np.random.default_rng(98)
    q = r.standard_normal((T, H, K))
    k = r.standard_normal((T, H, K))
    v = r.standard_normal((T, H, V))
    s = r.standard_normal((T, H, M))
    p = r.uniform(0.0, 1.0, (T, H, M))
    out = abc_ref.abc_readout_sequence(q, k, v, s, p, 0.6)
    zc = _cum_lse(s)
    for t in (0, 1, 33, T - 1):
        wts = np.exp(s[: t + 1] - zc[t][None])
        hk = np.einsum("thk,thm->hkm", k[: t + 1], wts)
        hv = np.einsum("thm,thv->hmv", wts, v[: t + 1])
        _assert_close(out["score"][t], 0.6 * np.einsum("hkm,hk->hm", hk, q[t]), 1e-12, f"score {t}")
        _assert_close(out["o"][t], np.einsum("hmv,hm->hv", hv, p[t]), 1e-12, f"o {t}")
    sc = np.broadcast_to(r.standard_normal((1, H, M)), (T, H, M)).copy()
    out = abc_ref.abc_readout_sequence(q, k, v, sc, None, 0.6)
    n = np.arange(1, T + 1)[:, None, None]
    mk = np.cumsum(k, axis=0) / n
    mv = np.cumsum(v, axis=0) / n
    _assert_close(out["score"], 0.6 * np.broadcast_to(np.einsum("thk,thk->th", mk, q)[:, :, None], (T, H, M)),
                  1e-12, "running-mean scores")
    _assert_close(out["p"], np.full((T, H, M), 1.0 / M), 1e-12, "uniform slot weights")
    _assert_close(out["o"], mv, 1e-12, "running-mean output")


def _abc_bwd_problem(seed, T, H=1, K=2, M=3, V=2):
    r = np.random.default_rng(seed)
    q = r.standard_normal((T, H, K))
    k = r.standard_normal((T, H, K))
    v = r.standard_normal((T, H, V))
    s = r.standard_normal((T, H, M))
    p = r.uniform(0.0, 1.0, (T, H, M))
    dscore = r.standard_normal((T, H, M))
    do = r.standard_normal((T, H, V))
    ek = r.standard_normal((H, K, M))
    ev = r.standard_normal((H, M, V))
    return q, k, v, s, p, dscore, do, ek, ev


def check_abc_bwd_boundaries(abc_bwd_ref, abc_ref):
    """dhk[c], dhv[c] = gradients of the reads after chunk c (and of the final
    states) with respect to the states they start from: finite differences of
    the resumed forward read."""
    chunk, T, scale = 3, 10, 0.6
    q, k, v, s, p, dscore, do, ek, ev = _abc_bwd_problem(99, T)
    dhk, dhv = abc_bwd_ref.abc_backward_sequence(q, s, p, dscore, do, ek, ev, scale, chunk)
    zc = _cum_lse(s)
    for c in range(dhk.shape[0]):
        t0 = (c + 1) * chunk
        if t0 >= T:
            _assert_close(dhk[c], ek, 1e-12, "dhk after the last chunk")
            _assert_close(dhv[c], ev, 1e-12, "dhv after the last chunk")
            continue
        sl = slice(t0, T)

        def loss(xk, xv):
            o = abc_ref.abc_readout_sequence(q[sl], k[sl], v[sl], s[sl], p[sl], scale, xk, xv, zc[t0 - 1])
            return float(np.sum(o["score"] * dscore[sl]) + np.sum(o["o"] * do[sl])
                         + np.sum(o["hk_final"] * ek) + np.sum(o["hv_final"] * ev))

        zk, zv = np.zeros_like(ek), np.zeros_like(ev)
        _assert_close(dhk[c], _fd(lambda x: loss(x, zv), zk), 1e-7, f"dhk[{c}] vs finite differences")
        _assert_close(dhv[c], _fd(lambda x: loss(zk, x), zv), 1e-7, f"dhv[{c}] vs finite differences")


def check_abc_bwd_running_mean(abc_bwd_ref):
    """Constant logits: r_t = (t-1)/t (tokens counted from 1), so the state
    after token e reaches token t > e scaled by e/t:
    dhk after e = sum_{t>e} scale q_t dscore_t^T e/t + dhk_end e/T (and the
    same with p_t do_t^T for dhv)."""
    chunk, T, scale = 4, 11, 0.8
    q, k, v, s, p, dscore, do, ek, ev = _abc_bwd_problem(100, T, H=2, K=3, M=2, V=4)
    s = np.broadcast_to(s[:1], s.shape).copy()
    dhk, dhv = abc_bwd_ref.abc_backward_sequence(q, s, p, dscore, do, ek, ev, scale, chunk)
    for c in range(dhk.shape[0]):
        e = min(T, (c + 1) * chunk)
        rk = ek * e / T
        rv = ev * e / T
        for t in range(e + 1, T + 1):
            rk = rk + scale * q[t - 1][:, :, None] * dscore[t - 1][:, None, :] * e / t
            rv = rv + p[t - 1][:, :, None] * do[t - 1][:, None, :] * e / t
        _assert_close(dhk[c], rk, 1e-12, f"running-mean dhk[{c}]")
        _assert_close(dhv[c], rv, 1e-12, f"running-mean dhv[{c}]")


def check_abc_bwd_chunk_relation(abc_bwd_ref):
    """The reverse chunk step of the state walk, with zc the normaliser at
    chunk ends:
      dhk[c-1] = dhk[c] * exp(zc[c-1] - zc[c])[None, :] + scale Q_c^T (dscore_c * exp(zc[c-1] - z_t))
      dhv[c-1] = exp(zc[c-1] - zc[c])[:, None] * dhv[c] + (p_c * exp(zc[c-1] - z_t))^T dO_c"""
    C, T, scale = 64, 150, 0.7
    q, k, v, s, p, dscore, do, ek, ev = _abc_bwd_problem(101, T, H=2, K=5, M=4, V=3)
    dhk, dhv = abc_bwd_ref.abc_backward_sequence(q, s, p, dscore, do, ek, ev, scale, C)
    z = _cum_lse(s)
    for c in range(1, dhk.shape[0]):
        c0, c1 = c * C, min(T, (c + 1) * C)
        zp, zl = z[c0 - 1], z[c1 - 1]
        x = np.exp(zp[None] - z[c0:c1])                          # [n, H, M]
        rk = dhk[c] * np.exp(zp - zl)[:, None, :] + scale * np.einsum("thk,thm->hkm", q[c0:c1], dscore[c0:c1] * x)
        rv = np.exp(zp - zl)[:, :, None] * dhv[c] + np.einsum("thm,thv->hmv", p[c0:c1] * x, do[c0:c1])
        _assert_close(dhk[c - 1], rk, 1e-12, f"reverse chunk step dhk {c}")
        _assert_close(dhv[c - 1], rv, 1e-12, f"reverse chunk step dhv {c}")


ABC_READ_CHECKS = [check_abc_resume, check_abc_readout]
ABC_BWD_CHECKS = [check_abc_bwd_boundaries, check_abc_bwd_running_mean, check_abc_bwd_chunk_relation]


def run_abc_bwd_check(check, abc_bwd_ref, abc_ref):
    if check.__name__ in ("check_abc_bwd_boundaries", "check_abc_bwd_wrapper_sampled"):
        return check(abc_bwd_ref, abc_ref)
    return check(abc_bwd_ref)


# --------------------------------------------------------------------------- per-channel decay (KDA-style)
def _kda_problem(seed, L, H, DK, DV):
    """Small float64 problem: unit q, k rows, per-channel decays in (0, 1]."""
    q, k, v, _, b, S0 = rand_problem(seed, L, H, DK, DV)
    r = np.random.default_rng(seed + 1000)
    a = 1.0 / (1.0 + np.exp(-r.normal(2.0, 1.0, (L, H, DK))))
    return q, k, v, a, b, S0


def check_kda_brute_force(kda_ref):
    """Dense transitions (I - b_t k_t k_t^T) diag(a_t) multiplied out explicitly."""
    L, H, DK, DV, C = 11, 2, 5, 3, 4
    q, k, v, a, b, S0 = _kda_problem(41, L, H, DK, DV)
    o, pre, ST = kda_ref.kda_scan_sequence(q, k, v, a, b, S0, 0.7, C)
    for h in range(H):
        S = S0[h]
        states = []
        for t in range(L):
            A = (np.eye(DK) - b[t, h] * np.outer(k[t, h], k[t, h])) @ np.diag(a[t, h])
            S = A @ S + b[t, h] * np.outer(k[t, h], v[t, h])
            states.append(S)
        _assert_close(ST[h], states[-1], what="final state vs dense products")
        _assert_close(o[:, h], 0.7 * np.stack([states[t].T @ q[t, h] for t in range(L)]), what="outputs vs dense")
        for c, t0 in enumerate(range(0, L, C)):
            _assert_close(pre[c, h], S0[h] if t0 == 0 else states[t0 - 1], what=f"pre-chunk state {c}")


def check_kda_rationals(kda_ref):
    """DK = DV = 3, T = 5, per-channel rational decays: exact equality with the
    dense products (I - b k k^T) diag(a) in Fraction arithmetic."""
    r = np.random.default_rng(6)
    L, D = 5, 3

    def fr(x, den=8):
        return Fr(int(round(x * den)), den)

    q = [[fr(x) for x in r.standard_normal(D)] for _ in range(L)]
    k = [[fr(x) for x in r.standard_normal(D)] for _ in range(L)]
    v = [[fr(x) for x in r.standard_normal(D)] for _ in range(L)]
    a = [[Fr(int(r.integers(5, 16)), 16) for _ in range(D)] for _ in range(L)]
    b = [Fr(int(r.integers(1, 8)), 8) for _ in range(L)]
    S0 = [[fr(x, 4) for x in r.standard_normal(D)] for _ in range(D)]
    S = S0
    o_ref, pre_ref = [], []
    for t in range(L):
        if t % 2 == 0:
            pre_ref.append(S)
        A = [[((Fr(1) if i == j else Fr(0)) - b[t] * k[t][i] * k[t][j]) * a[t][j] for j in range(D)]
             for i in range(D)]
        S = _fr_matmul(A, S)
        S = [[S[i][j] + b[t] * k[t][i] * v[t][j] for j in range(D)] for i in range(D)]
        o_ref.append([sum((S[i][j] * q[t][i] for i in range(D)), Fr(0)) for j in range(D)])

    def obj(x, shape):
        arr = np.empty(shape, dtype=object)
        arr[...] = np.array(x, dtype=object).reshape(shape)
        return arr

    o, pre, ST = kda_ref.kda_scan_sequence(obj(q, (L, 1, D)), obj(k, (L, 1, D)), obj(v, (L, 1, D)),
                                           obj(a, (L, 1, D)), obj(b, (L, 1)), obj(S0, (1, D, D)), Fr(1), 2)
    assert all(ST[0, i, j] == S[i][j] for i in range(D) for j in range(D)), "final state not exact"
    assert all(o[t, 0, j] == o_ref[t][j] for t in range(L) for j in range(D)), "outputs not exact"
    for c in range(len(pre_ref)):
        assert all(pre[c, 0, i, j] == pre_ref[c][i][j] for i in range(D) for j in range(D)), \
            f"pre-chunk state {c} not exact"


def check_kda_scalar_reduction(kda_ref, gdr_ref):
    """Every channel decaying alike is the scalar gated delta rule (itself pinned)."""
    L, H, DK, DV, C = 70, 2, 6, 4, 16
    q, k, v, a, b, S0 = rand_problem(51, L, H, DK, DV)
    ak = np.repeat(a[:, :, None], DK, axis=2)
    o1, p1, s1 = kda_ref.kda_scan_sequence(q, k, v, ak, b, S0, 0.5, C)
    o2, p2, s2 = gdr_ref.gdr_scan_sequence(q, k, v, a, b, S0, 0.5, C)
    _assert_close(o1, o2, 1e-13, "outputs")
    _assert_close(p1, p2, 1e-13, "pre-chunk states")
    _assert_close(s1, s2, 1e-13, "final state")


def check_kda_pure_decay(kda_ref):
    """b = 0: every key row keeps its own running product of decays."""
    L, H, DK, DV, C = 40, 2, 6, 4, 16
    q, k, v, a, b, S0 = _kda_problem(61, L, H, DK, DV)
    b = np.zeros_like(b)
    o, pre, ST = kda_ref.kda_scan_sequence(q, k, v, a, b, S0, 1.0, C)
    cum = np.cumprod(a, axis=0)                              # [L, H, DK]
    _assert_close(ST, cum[-1][:, :, None] * S0, what="b=0 final state")
    _assert_close(o, np.einsum("thk,hkv,thk->thv", cum, S0, q), what="b=0 outputs")
    for c, t0 in enumerate(range(0, L, C)):
        f = np.ones((H, DK)) if t0 == 0 else cum[t0 - 1]
        _assert_close(pre[c], f[:, :, None] * S0, what=f"b=0 pre-chunk {c}")


def check_kda_recall(kda_ref):
    """a = 1, b = 1, orthonormal keys: exact recall; a channel decayed to zero
    forgets its row of the state before the write."""
    DK, DV, L = 8, 5, 6
    r = np.random.default_rng(71)
    Qm, _ = np.linalg.qr(r.standard_normal((DK, DK)))
    K = Qm[:L]
    V = r.standard_normal((L, DV))
    S0 = r.standard_normal((DK, DV))
    o, pre, ST = kda_ref.kda_scan_sequence(K[:, None], K[:, None], V[:, None], np.ones((L, 1, DK)),
                                           np.ones((L, 1)), S0[None], 1.0, 64)
    _assert_close(ST[0], (np.eye(DK) - K.T @ K) @ S0 + K.T @ V, TOL, "recall closed form")
    a = np.ones((1, 1, DK))
    a[0, 0, 2] = 0.0
    _, _, S1 = kda_ref.kda_scan_sequence(K[:1, None], K[:1, None], V[:1, None], a, np.zeros((1, 1)), S0[None],
                                         1.0, 64)
    ref = S0.copy()
    ref[2] = 0.0
    _assert_close(S1[0], ref, TOL, "zeroed channel")


def check_kda_chunk_algebra(kda_ref):
    """The chunk (WY) form equals the token recurrence at several chunk sizes,
    packed sequences with ragged tails, initial states and an output scale."""
    lengths = [1, 63, 64, 65, 150]
    H, DK, DV = 2, 8, 6
    r = np.random.default_rng(81)
    Ttot = sum(lengths)
    q = r.standard_normal((1, Ttot, H, DK))
    k = r.standard_normal((1, Ttot, H, DK))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((1, Ttot, H, DV))
    g = np.log(1.0 / (1.0 + np.exp(-r.normal(2.0, 1.0, (1, Ttot, H, DK)))))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((1, Ttot, H))))
    h0 = 0.2 * r.standard_normal((len(lengths), H, DK, DV))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    for C in (1, 2, 7, 16, 64):
        ref = kda_ref.kda_recurrent_fp64(q, k, v, g, beta, h0, cu, 0.5, C)
        got = kda_ref.kda_chunked_fp64(q, k, v, g, beta, h0, cu, 0.5, C)
        for key in ("o", "v_new", "h", "hT"):
            _assert_close(got[key], ref[key], 1e-11, f"chunk {C}: {key}")


KDA_CHECKS = [check_kda_brute_force, check_kda_rationals, check_kda_pure_decay, check_kda_recall]


# --------------------------------------------------------------------------- batch wrappers
# The GPU parity tests compare against the oracle's whole-problem wrappers
# (packed sequences, sampled heads / batch rows).  These pins hold each
# wrapper's packing and sampling against facts computed here, sequence by
# sequence and head by head, from the raw inputs: dense transition products,
# closed-form weighted sums and finite differences.
def _packed_problem(seed, lengths, H, DK, DV):
    r = np.random.default_rng(seed)
    T = sum(lengths)
    q = r.standard_normal((1, T, H, DK))
    k = r.standard_normal((1, T, H, DK))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((1, T, H, DV))
    g = np.log(1.0 / (1.0 + np.exp(-r.normal(2.0, 1.0, (1, T, H)))))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((1, T, H))))
    h0 = 0.3 * r.standard_normal((len(lengths), H, DK, DV))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return q, k, v, g, beta, h0, cu


def check_wrapper_packed_heads(gdr_ref):
    """gdr_recurrent_fp64 on packed sequences with a head sample: every
    sampled head of every sequence equals the dense transition products of
    that head alone, started from that sequence's and head's h0 (outputs,
    write vectors, pre-chunk rows at the packed chunk offsets, final state)."""
    lengths, H, DK, DV, C, scale = [9, 4, 0, 6, 11], 3, 3, 2, 4, 0.7
    hs = [2, 0]
    q, k, v, g, beta, h0, cu = _packed_problem(71, lengths, H, DK, DV)
    out = gdr_ref.gdr_recurrent_fp64(q, k, v, g, beta, h0, cu, scale, chunk=C, heads=hs)
    counts = [(L + C - 1) // C for L in lengths]
    offs = np.concatenate([[0], np.cumsum(counts)])
    assert list(out["chunk_offsets"]) == list(offs), "chunk offsets"
    assert out["h"].shape == (offs[-1], len(hs), DK, DV) and out["hT"].shape == (len(lengths), len(hs), DK, DV)
    a = np.exp(g)
    for n, L in enumerate(lengths):
        s = int(cu[n])
        for j, hh in enumerate(hs):
            kk, vv, aa, bb = k[0, s:s + L, hh], v[0, s:s + L, hh], a[0, s:s + L, hh], beta[0, s:s + L, hh]
            Ss = brute_force_states(kk, vv, aa, bb, h0[n, hh])
            fin = Ss[-1] if L else h0[n, hh]
            _assert_close(out["hT"][n, j], fin, 1e-12, f"seq {n} head {hh} final")
            for t in range(L):
                prev = h0[n, hh] if t == 0 else Ss[t - 1]
                _assert_close(out["o"][0, s + t, j], scale * Ss[t].T @ q[0, s + t, hh], 1e-12,
                              f"seq {n} head {hh} o_{t}")
                _assert_close(out["v_new"][0, s + t, j], bb[t] * (vv[t] - aa[t] * prev.T @ kk[t]), 1e-12,
                              f"seq {n} head {hh} delta_{t}")
            for c in range(counts[n]):
                ref = h0[n, hh] if c == 0 else Ss[c * C - 1]
                _assert_close(out["h"][offs[n] + c, j], ref, 1e-12, f"seq {n} head {hh} pre-chunk {c}")


def check_bwd_wrapper_packed(bwd_ref, gdr_ref, chunked_ref):
    """gdr_backward_fp64 on packed sequences with a head sample, against
    finite differences of a linear loss (upstream dO on every output, dhT on
    every final state) of the packed forward of each sampled head: dh0[n] by
    perturbing h0[n], dh[row] by restarting sequence n after that chunk, and
    the write-vector gradient through the chunk form's write vectors."""
    lengths, H, DK, DV, C, scale = [7, 0, 3, 5], 2, 3, 2, 3, 0.6
    hs = [1]
    q, k, v, g, beta, h0, cu = _packed_problem(72, lengths, H, DK, DV)
    r = np.random.default_rng(73)
    do = r.standard_normal((1, sum(lengths), H, DV))
    dhT = r.standard_normal((len(lengths), H, DK, DV))
    out = bwd_ref.gdr_backward_fp64(q, k, g, beta, do, dhT, cu, scale, chunk=C, heads=hs)
    counts = [(L + C - 1) // C for L in lengths]
    offs = np.concatenate([[0], np.cumsum(counts)])
    assert list(out["chunk_offsets"]) == list(offs), "chunk offsets"
    hh = hs[0]

    def loss_tail(n, t0, S):
        """Loss of sequence n's tokens from t0 on, started from S (head hh)."""
        s, e = int(cu[n]), int(cu[n + 1])
        sl = slice(s + t0, e)
        o, _, Sf = gdr_ref.gdr_scan_sequence(q[0, sl][:, [hh]], k[0, sl][:, [hh]], v[0, sl][:, [hh]],
                                             np.exp(g[0, sl][:, [hh]]), beta[0, sl][:, [hh]], S[None], scale, C)
        return float(np.sum(o[:, 0] * do[0, sl, hh]) + np.sum(Sf[0] * dhT[n, hh]))

    for n, L in enumerate(lengths):
        fd0 = _fd(lambda S: loss_tail(n, 0, S), h0[n, hh].copy())
        _assert_close(out["dh0"][n, 0], fd0, 1e-7, f"seq {n} dh0")
        for c in range(counts[n]):
            t0 = (c + 1) * C
            if t0 >= L:
                _assert_close(out["dh"][offs[n] + c, 0], dhT[n, hh], 1e-12, f"seq {n} last dh row")
                continue
            fd = _fd(lambda S: loss_tail(n, t0, S), np.zeros((DK, DV)))
            _assert_close(out["dh"][offs[n] + c, 0], fd, 1e-7, f"seq {n} dh row {c}")
        if L:
            s, e = int(cu[n]), int(cu[n + 1])

            def loss_shift(shift):
                rr = chunked_ref.chunked_scan_sequence(q[0, s:e][:, [hh]], k[0, s:e][:, [hh]], v[0, s:e][:, [hh]],
                                                       g[0, s:e][:, [hh]], beta[0, s:e][:, [hh]], h0[n][[hh]],
                                                       scale, C, delta_shift=shift)
                return float(np.sum(rr["o"][:, 0] * do[0, s:e, hh]) + np.sum(rr["hT"][0] * dhT[n, hh]))

            fdv = _fd(loss_shift, np.zeros((L, 1, DV)))
            _assert_close(out["dv_new"][0, s:e, 0], fdv[:, 0], 1e-7, f"seq {n} dv_new")


def _abc_batch(seed, B, T, H, K, M, V):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, K))
    k = r.standard_normal((B, T, H, K))
    v = r.standard_normal((B, T, H, V))
    s = 1.5 * r.standard_normal((B, T, H, M))
    return q, k, v, s


def check_abc_wrapper_sampled(abc_ref):
    """abc_recurrent_fp64 and abc_forward_fp64 on a batch-row and head sample:
    every sampled (row, head) equals the closed-form weighted sums of that
    row's and head's own inputs (normaliser, pre-chunk and final states, the
    score / softmax / value reads, and the value read with given weights)."""
    B, T, H, K, M, V, C, scale = 2, 9, 3, 3, 2, 2, 4, 0.8
    bs, hs = [1, 0], [2, 0]
    q, k, v, s = _abc_batch(74, B, T, H, K, M, V)
    p = np.random.default_rng(75).uniform(0.0, 1.0, (B, T, H, M))
    rec = abc_ref.abc_recurrent_fp64(k, v, s, C, batches=bs, heads=hs)
    fwd = abc_ref.abc_forward_fp64(q, k, v, s, scale, batches=bs, heads=hs)
    fwp = abc_ref.abc_forward_fp64(q, k, v, s, scale, p=p, batches=bs, heads=hs)
    for i, b in enumerate(bs):
        for j, hh in enumerate(hs):
            kk, vv, ss, qq = k[b, :, hh], v[b, :, hh], s[b, :, hh], q[b, :, hh]
            zc = _cum_lse(ss)
            _assert_close(rec["z"][i, :, j], zc, 1e-13, f"({b},{hh}) z")
            for c, t0 in enumerate(range(0, T, C)):
                if t0 == 0:
                    assert np.all(rec["hk"][i, 0, j] == 0) and np.all(rec["hv"][i, 0, j] == 0)
                    continue
                wts = np.exp(ss[:t0] - zc[t0 - 1][None])
                _assert_close(rec["hk"][i, c, j], kk[:t0].T @ wts, 1e-12, f"({b},{hh}) Hk pre {c}")
                _assert_close(rec["hv"][i, c, j], wts.T @ vv[:t0], 1e-12, f"({b},{hh}) Hv pre {c}")
            wts = np.exp(ss - zc[-1][None])
            _assert_close(rec["hk_final"][i, j], kk.T @ wts, 1e-12, f"({b},{hh}) Hk final")
            _assert_close(rec["hv_final"][i, j], wts.T @ vv, 1e-12, f"({b},{hh}) Hv final")
            for t in range(T):
                wt = np.exp(ss[:t + 1] - zc[t][None])                  # [t+1, M]
                hk_t, hv_t = kk[:t + 1].T @ wt, wt.T @ vv[:t + 1]
                sc = scale * hk_t.T @ qq[t]
                e = np.exp(sc - sc.max())
                pt = e / e.sum()
                _assert_close(fwd["p"][i, t, j], pt, 1e-12, f"({b},{hh}) p_{t}")
                _assert_close(fwd["o"][i, t, j], hv_t.T @ pt, 1e-12, f"({b},{hh}) o_{t}")
                _assert_close(fwp["o"][i, t, j], hv_t.T @ p[b, t, hh], 1e-12, f"({b},{hh}) o_{t} (given p)")


def check_abc_bwd_wrapper_sampled(abc_bwd_ref, abc_ref):
    """abc_backward_fp64 on a batch-row and head sample: the gradient rows of
    every sampled (row, head) against finite differences of that row's and
    head's read-out, resumed after each chunk from a perturbed state
    (loss: dscore on the scores, dO on the outputs, the final-state gradients
    on the final states)."""
    B, T, H, K, M, V, C, scale = 2, 7, 3, 2, 2, 2, 3, 0.7
    bs, hs = [1, 0], [2]
    q, k, v, s = _abc_batch(76, B, T, H, K, M, V)
    r = np.random.default_rng(77)
    p = r.uniform(0.0, 1.0, (B, T, H, M))
    dscore = r.standard_normal((B, T, H, M))
    do = r.standard_normal((B, T, H, V))
    ek = r.standard_normal((B, H, K, M))
    ev = r.standard_normal((B, H, M, V))
    out = abc_bwd_ref.abc_backward_fp64(q, s, p, dscore, do, ek, ev, scale, C, batches=bs, heads=hs)
    nc = (T + C - 1) // C
    assert out["dhk"].shape == (len(bs), nc, len(hs), K, M)
    for i, b in enumerate(bs):
        for j, hh in enumerate(hs):
            zc = _cum_lse(s[b, :, [hh]].transpose(1, 0, 2))           # [T, 1, M]
            for c in range(nc):
                t0 = (c + 1) * C
                if t0 >= T:
                    _assert_close(out["dhk"][i, c, j], ek[b, hh], 1e-12, f"({b},{hh}) dhk after the last chunk")
                    _assert_close(out["dhv"][i, c, j], ev[b, hh], 1e-12, f"({b},{hh}) dhv after the last chunk")
                    continue
                sl = slice(t0, T)
                sel = lambda x: x[b, sl][:, [hh]]

                def loss(xk, xv):
                    o = abc_ref.abc_readout_sequence(sel(q), sel(k), sel(v), sel(s), sel(p), scale,
                                                     xk[None], xv[None], zc[t0 - 1])
                    return float(np.sum(o["score"] * sel(dscore)) + np.sum(o["o"] * sel(do))
                                 + np.sum(o["hk_final"][0] * ek[b, hh]) + np.sum(o["hv_final"][0] * ev[b, hh]))

                zk, zv = np.zeros((K, M)), np.zeros((M, V))
                _assert_close(out["dhk"][i, c, j], _fd(lambda x: loss(x, zv), zk), 1e-7, f"({b},{hh}) dhk[{c}]")
                _assert_close(out["dhv"][i, c, j], _fd(lambda x: loss(zk, x), zv), 1e-7, f"({b},{hh}) dhv[{c}]")


GDR_CHECKS.append(check_wrapper_packed_heads)
ABC_CHECKS.append(check_abc_wrapper_sampled)
BWD_CHECKS.append(check_bwd_wrapper_packed)
ABC_BWD_CHECKS.append(check_abc_bwd_wrapper_sampled)
