"""FP64 chunked (WY) form of the gated delta rule — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module; the HIP product path never does.

The kev page's state-scan kernel (kev pull request #259, opening section)
works per 64-token chunk on factors w and u prepared from k, v, g and beta.
The pages do not print that algebra, so it is derived here from the
token recurrence in ``gdr_ref`` (S_t = a_t S_{t-1} + k_t delta_t^T with
delta_t = b_t (v_t - a_t S_{t-1}^T k_t)).  Unrolled inside one chunk that
starts from state S0, with gamma = the chunk-local cumulative sum of g and
Gamma_t = exp(gamma_t):

    A[t, i] = b_t exp(gamma_t - gamma_i) (k_t . k_i)        for i < t, else 0
    (I + A) Delta = diag(b) V - diag(b Gamma) K S0
    T = (I + A)^-1,   W = T diag(b Gamma) K,   U = T diag(b) V
    Delta = U - W S0                                   (= the write vectors)
    S_end = Gamma_last S0 + K^T diag(exp(gamma_last - gamma)) Delta
    O = scale (diag(Gamma) Q S0 + (tril(Q K^T) * exp(gamma_t - gamma_i)) Delta)

(the lower-triangular mask in O includes the diagonal).  A partial last chunk
simply has fewer rows.  This module evaluates those formulas with dense numpy
linear algebra, chunk by chunk, and is pinned to ``gdr_ref`` by the tests at
several chunk sizes; it also supplies the prepared factors (g_cum, w, u) that
the chunk-preparation step produces, for element-wise checks.
"""

from __future__ import annotations

import numpy as np

from .gdr_ref import _sequences, chunk_counts

CHUNK = 64


def chunk_factors(k, v, g, beta):
    """One chunk, one head: k [n, DK], v [n, DV], g, beta [n] (float64).

    Returns (gamma [n], W [n, DK], U [n, DV]).
    """
    n = k.shape[0]
    gamma = np.cumsum(g)
    Gam = np.exp(gamma)
    decay = np.exp(gamma[:, None] - gamma[None, :])
    A = np.tril(beta[:, None] * decay * (k @ k.T), -1)
    T = np.linalg.inv(np.eye(n) + A)
    W = T @ ((beta * Gam)[:, None] * k)
    U = T @ (beta[:, None] * v)
    return gamma, W, U


def chunked_scan_sequence(q, k, v, g, beta, S0, scale=1.0, chunk: int = CHUNK, delta_shift=None):
    """One sequence: q, k [L, H, DK], v [L, H, DV], g, beta [L, H], S0 [H, DK, DV].

    Returns dict with o, v_new (Delta), w, u, g_cum [L, H, ...], h (pre-chunk
    states) [nc, H, DK, DV] and hT [H, DK, DV].  ``delta_shift`` [L, H, DV], if
    given, is added to each chunk's Delta right after it is formed (the tests
    differentiate the chunk form with respect to Delta by finite differences).
    """
    L, H, DK = k.shape
    DV = v.shape[-1]
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((L, H, DV))
    vnew = np.zeros((L, H, DV))
    w = np.zeros((L, H, DK))
    u = np.zeros((L, H, DV))
    gcum = np.zeros((L, H))
    pre = []
    for c0 in range(0, L, chunk):
        c1 = min(c0 + chunk, L)
        pre.append(S.copy())
        for hh in range(H):
            kk, vv, qq = k[c0:c1, hh], v[c0:c1, hh], q[c0:c1, hh]
            gamma, W, U = chunk_factors(kk, vv, g[c0:c1, hh], beta[c0:c1, hh])
            S0h = S[hh]
            D = U - W @ S0h
            if delta_shift is not None:
                D = D + delta_shift[c0:c1, hh]
            P = np.tril(qq @ kk.T) * np.exp(gamma[:, None] - gamma[None, :])
            o[c0:c1, hh] = scale * (np.exp(gamma)[:, None] * (qq @ S0h) + P @ D)
            S[hh] = np.exp(gamma[-1]) * S0h + kk.T @ (np.exp(gamma[-1] - gamma)[:, None] * D)
            vnew[c0:c1, hh] = D
            w[c0:c1, hh] = W
            u[c0:c1, hh] = U
            gcum[c0:c1, hh] = gamma
    h = np.stack(pre) if pre else np.zeros((0, H, DK, DV))
    return {"o": o, "v_new": vnew, "w": w, "u": u, "g_cum": gcum, "h": h, "hT": S}


def gdr_chunked_fp64(q, k, v, g, beta, h0=None, cu_seqlens=None, scale: float = 1.0,
                     chunk: int = CHUNK, heads=None) -> dict:
    """Whole problem in the chunked form; same layouts as ``gdr_recurrent_fp64``
    plus w, u [B, T, H', D] and g_cum [B, T, H']."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, DK = k.shape
    DV = v.shape[-1]
    hs = list(range(H)) if heads is None else list(heads)
    Hs = len(hs)
    seqs = _sequences(B, T, cu_seqlens)
    counts = chunk_counts([e - s for _, s, e in seqs], chunk)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    out = {
        "o": np.zeros((B, T, Hs, DV)), "v_new": np.zeros((B, T, Hs, DV)),
        "w": np.zeros((B, T, Hs, DK)), "u": np.zeros((B, T, Hs, DV)),
        "g_cum": np.zeros((B, T, Hs)), "h": np.zeros((int(offsets[-1]), Hs, DK, DV)),
        "hT": np.zeros((len(seqs), Hs, DK, DV)), "chunk_offsets": offsets,
    }
    for n, (b, s, e) in enumerate(seqs):
        S0 = np.zeros((Hs, DK, DV)) if h0 is None else np.array(h0[n][hs], dtype=np.float64)
        r = chunked_scan_sequence(q[b, s:e][:, hs], k[b, s:e][:, hs], v[b, s:e][:, hs],
                                  g[b, s:e][:, hs], beta[b, s:e][:, hs], S0, scale, chunk)
        for key in ("o", "v_new", "w", "u", "g_cum"):
            out[key][b, s:e] = r[key]
        out["h"][offsets[n]:offsets[n + 1]] = r["h"]
        out["hT"][n] = r["hT"]
    return out
