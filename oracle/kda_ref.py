"""FP64 oracle of the gated delta rule with a per-key-channel decay — test
infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module; the HIP product path never does.

What it computes
----------------
The cuLA pull request #127 ("Summary"; "Root cause and implementation")
builds its context-parallel pre-scan around the serial FlashKDA kernel, whose
gate decays every key channel by its own factor; the pages name that path
but print no recurrence.  The plainest reading that agrees with the scalar
gated delta rule of ``gdr_ref`` (which it must reduce to when every channel
decays alike) is, per token t of one sequence and one head, with per-channel
decay a_t = exp(g_t) in R^DK and write strength b_t = beta_t:

    S_t = (I - b_t k_t k_t^T) diag(a_t) S_{t-1} + b_t k_t v_t^T      (DK x DV)
    o_t = scale * S_t^T q_t

evaluated token by token as the decay of every key row of the state by its
own factor (S <- diag(a_t) S), then the delta-rule write on the decayed state
(S <- S + b_t k_t (v_t - S^T k_t)^T).  The output reads the updated state; the
state before every 64-token chunk of a sequence is recorded; sequences
restart at each ``cu_seqlens`` boundary.

``kda_chunk_factors`` / ``kda_chunked_scan_sequence`` write the same thing in
the per-chunk (WY) form, derived here from the token recurrence (the pages do
not print it).  Inside a chunk starting from S0, with Gam = the chunk-local
cumulative sum of g per channel (Gam_t in R^DK):

    A[t, i] = b_t sum_d k_td k_id exp(Gam_td - Gam_id)          (i < t)
    T = (I + A)^-1,   W = T diag(b) (K * exp(Gam)),   U = T diag(b) V
    Delta = U - W S0                                   (the write vectors)
    S_end = diag(exp(Gam_last)) S0 + Kg^T Delta,   Kg = K * exp(Gam_last - Gam)
    O = scale ((Q * exp(Gam)) S0 + P Delta),
        P[t, i] = sum_d q_td k_id exp(Gam_td - Gam_id)          (i <= t)

Every exponent exp(Gam_td - Gam_id) with i <= t is evaluated for the pair
itself, so nothing here can overflow.  Works on float64 arrays; the token
form also on numpy object arrays of ``fractions.Fraction``.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .gdr_ref import _sequences, chunk_counts

CHUNK = 64


def kda_scan_sequence(q, k, v, a, b, S0, scale=1.0, chunk: int = CHUNK, return_delta=False):
    """Token-serial per-channel-decay delta rule over one sequence, all heads.

    q, k: [L, H, DK]; v: [L, H, DV]; a (per-channel decay multipliers) [L, H, DK];
    b (beta) [L, H]; S0 [H, DK, DV].  Returns (o [L, H, DV], pre-chunk states
    [nc, H, DK, DV], final state [H, DK, DV]) and, with ``return_delta``, the
    write vectors delta [L, H, DV].
    """
    L = k.shape[0]
    H, DK, DV = S0.shape
    dt = S0.dtype
    S = S0.copy()
    o = np.zeros((L, H, DV), dtype=dt) if dt != object else np.empty((L, H, DV), dtype=object)
    vnew = np.zeros((L, H, DV), dtype=dt) if dt != object else np.empty((L, H, DV), dtype=object)
    pre = []
    for t in range(L):
        if t % chunk == 0:
            pre.append(S.copy())
        # every key row of the state decays by its own channel's factor ...
        S = a[t][:, :, None] * S
        # ... then the delta-rule write on the decayed state
        kt = k[t]
        pred = np.einsum("hk,hkv->hv", kt, S)
        delta = b[t][:, None] * (v[t] - pred)
        S = S + kt[:, :, None] * delta[:, None, :]
        vnew[t] = delta
        o[t] = scale * np.einsum("hk,hkv->hv", q[t], S)
    pre_arr = np.stack(pre) if pre else np.zeros((0, H, DK, DV), dtype=dt)
    if return_delta:
        return o, pre_arr, S, vnew
    return o, pre_arr, S


def kda_recurrent_fp64(q, k, v, g, beta, h0=None, cu_seqlens=None, scale: float = 1.0,
                       chunk: int = CHUNK, heads: Optional[Sequence[int]] = None) -> dict:
    """Whole problem, dense [B, T, H, D] rows or packed sequences (B = 1, cu_seqlens).

    g [B, T, H, DK] is the per-token, per-channel log decay.  Returns float64
    o, v_new [B, T, H', DV], h [NT_total, H', DK, DV] (state before each chunk,
    sequences packed in order), hT [N, H', DK, DV] and chunk_offsets [N + 1].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, DK = k.shape
    DV = v.shape[-1]
    hs = list(range(H)) if heads is None else list(heads)
    seqs = _sequences(B, T, cu_seqlens)
    N = len(seqs)
    counts = chunk_counts([e - s for _, s, e in seqs], chunk)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    Hs = len(hs)
    o = np.zeros((B, T, Hs, DV))
    vnew = np.zeros((B, T, Hs, DV))
    h = np.zeros((int(offsets[-1]), Hs, DK, DV))
    hT = np.zeros((N, Hs, DK, DV))
    a_all = np.exp(g)
    for n, (b, s, e) in enumerate(seqs):
        S0 = np.zeros((Hs, DK, DV)) if h0 is None else np.array(h0[n][hs], dtype=np.float64)
        on, pre, Sf, dn = kda_scan_sequence(q[b, s:e][:, hs], k[b, s:e][:, hs], v[b, s:e][:, hs],
                                            a_all[b, s:e][:, hs], beta[b, s:e][:, hs], S0, scale, chunk,
                                            return_delta=True)
        o[b, s:e] = on
        vnew[b, s:e] = dn
        h[offsets[n]:offsets[n + 1]] = pre
        hT[n] = Sf
    return {"o": o, "v_new": vnew, "h": h, "hT": hT, "chunk_offsets": offsets}


def _pair_decay(Gam):
    """exp(Gam_t - Gam_i) per channel for every pair i <= t of one chunk, and 0
    for i > t (those exponents are never evaluated).  Gam [n, DK] -> [n, n, DK]."""
    n = Gam.shape[0]
    causal = np.tril(np.ones((n, n), dtype=bool))[:, :, None]
    return np.exp(np.where(causal, Gam[:, None, :] - Gam[None, :, :], -np.inf))


def kda_chunk_factors(k, v, g, beta):
    """One chunk, one head: k [n, DK], v [n, DV], g [n, DK], beta [n] (float64).

    Returns (Gam [n, DK], W [n, DK], U [n, DV], Kg [n, DK], decay [DK]) with
    Kg = K * exp(Gam_last - Gam) and decay = exp(Gam_last).
    """
    n = k.shape[0]
    Gam = np.cumsum(g, axis=0)
    dec = _pair_decay(Gam)
    A = np.tril(beta[:, None] * np.einsum("td,id,tid->ti", k, k, dec), -1)
    T = np.linalg.inv(np.eye(n) + A)
    W = T @ (beta[:, None] * k * np.exp(Gam))
    U = T @ (beta[:, None] * v)
    Kg = k * np.exp(Gam[-1][None, :] - Gam)
    return Gam, W, U, Kg, np.exp(Gam[-1])


def kda_chunked_scan_sequence(q, k, v, g, beta, S0, scale=1.0, chunk: int = CHUNK):
    """One sequence in the chunk form: q, k [L, H, DK], v [L, H, DV], g [L, H, DK],
    beta [L, H], S0 [H, DK, DV].  Returns dict with o, v_new, w, u, kg, g_cum
    [L, H, .], decay [nc, H, DK], h [nc, H, DK, DV] and hT [H, DK, DV]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    L, H, DK = k.shape
    DV = v.shape[-1]
    nc = (L + chunk - 1) // chunk
    out = {key: np.zeros((L, H, d)) for key, d in (("o", DV), ("v_new", DV), ("w", DK), ("u", DV), ("kg", DK),
                                                     ("g_cum", DK))}
    out["decay"] = np.zeros((nc, H, DK))
    out["h"] = np.zeros((nc, H, DK, DV))
    S = np.array(S0, dtype=np.float64)
    for c in range(nc):
        t0, t1 = c * chunk, min((c + 1) * chunk, L)
        out["h"][c] = S
        for hd in range(H):
            Gam, W, U, Kg, dec = kda_chunk_factors(k[t0:t1, hd], v[t0:t1, hd], g[t0:t1, hd], beta[t0:t1, hd])
            Delta = U - W @ S[hd]
            qq, kk = q[t0:t1, hd], k[t0:t1, hd]
            P = np.einsum("td,id,tid->ti", qq, kk, _pair_decay(Gam))
            out["o"][t0:t1, hd] = scale * ((qq * np.exp(Gam)) @ S[hd] + P @ Delta)
            out["v_new"][t0:t1, hd] = Delta
            out["w"][t0:t1, hd] = W
            out["u"][t0:t1, hd] = U
            out["kg"][t0:t1, hd] = Kg
            out["g_cum"][t0:t1, hd] = Gam
            out["decay"][c, hd] = dec
            S[hd] = dec[:, None] * S[hd] + Kg.T @ Delta
    out["hT"] = S
    return out


def kda_chunked_fp64(q, k, v, g, beta, h0=None, cu_seqlens=None, scale: float = 1.0,
                     chunk: int = CHUNK, heads: Optional[Sequence[int]] = None) -> dict:
    """Whole problem in the chunk form (same layout as ``kda_recurrent_fp64``),
    plus the prepared factors w, u, kg, g_cum [B, T, H', .] and the per-chunk
    channel decays [NT_total, H', DK]."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, DK = k.shape
    DV = v.shape[-1]
    hs = list(range(H)) if heads is None else list(heads)
    seqs = _sequences(B, T, cu_seqlens)
    N = len(seqs)
    counts = chunk_counts([e - s for _, s, e in seqs], chunk)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    Hs = len(hs)
    res = {key: np.zeros((B, T, Hs, d)) for key, d in (("o", DV), ("v_new", DV), ("w", DK), ("u", DV),
                                                         ("kg", DK), ("g_cum", DK))}
    res["decay"] = np.zeros((int(offsets[-1]), Hs, DK))
    res["h"] = np.zeros((int(offsets[-1]), Hs, DK, DV))
    res["hT"] = np.zeros((N, Hs, DK, DV))
    for n, (b, s, e) in enumerate(seqs):
        S0 = np.zeros((Hs, DK, DV)) if h0 is None else np.array(h0[n][hs], dtype=np.float64)
        r = kda_chunked_scan_sequence(np.asarray(q)[b, s:e][:, hs], k[b, s:e][:, hs], v[b, s:e][:, hs],
                                      np.asarray(g)[b, s:e][:, hs], np.asarray(beta)[b, s:e][:, hs], S0, scale,
                                      chunk)
        for key in ("o", "v_new", "w", "u", "kg", "g_cum"):
            res[key][b, s:e] = r[key]
        res["decay"][offsets[n]:offsets[n + 1]] = r["decay"]
        res["h"][offsets[n]:offsets[n + 1]] = r["h"]
        res["hT"][n] = r["hT"]
    res["chunk_offsets"] = offsets
    return res
