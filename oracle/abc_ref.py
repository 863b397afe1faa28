"""FP64 oracle of the ABC normalised slot recurrence — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module; the HIP product path never does.

What it computes (flash-linear-attention fork issue #23, "[Perf][B300]
Parallelize ABC chunk state construction with affine summaries", sections
"Problem" and "Proposed Dataflow"): for each batch row and head, with slot
logits s_t in R^M, the running normaliser

    z_t = log(exp(z_{t-1}) + exp(s_t))          (elementwise over slots, z_0 = -inf)

and the two slot states, key-side Hk [K x M] and value-side Hv [M x V],
advanced per token t by

    w_t = exp(s_t - z_t)            r_t = exp(z_{t-1} - z_t)
    Hk_t = Hk_{t-1} * r_t[None, :] + outer(k_t, w_t)
    Hv_t = Hv_{t-1} * r_t[:, None] + outer(w_t, v_t)

i.e. H_t = H_{t-1} exp(z_{t-1} - z_t) + outer(x_t, exp(s_t - z_t)) with the slot
axis carrying the normaliser.  The issue's page describes calls without an
initial state (its dense, state-free path), so the recurrence starts from zero
states with z_0 = -inf, which makes r_1 = 0.  The state before each 64-token
chunk (offsets 0, 64, ...) is recorded, as is the state after the last token.

``abc_scan_sequence`` also accepts numpy object arrays (the pins use exact
``fractions.Fraction`` weights by handing in w and r directly).
"""

from __future__ import annotations

import numpy as np

CHUNK = 64


def abc_scan_sequence(k, v, s, chunk: int = CHUNK, hk0=None, hv0=None, z0=None):
    """One sequence, all heads: k [T, H, K], v [T, H, V], s [T, H, M] (float64).

    Returns (z [T, H, M], hk_pre [NC, H, K, M], hv_pre [NC, H, M, V],
    hk_final [H, K, M], hv_final [H, M, V]).  ``hk0``, ``hv0``, ``z0`` resume a
    sequence from a carried state and normaliser (default: zero states,
    z0 = -inf, the page's state-free start).
    """
    T, H, K = k.shape
    V = v.shape[-1]
    M = s.shape[-1]
    z_prev = np.full((H, M), -np.inf) if z0 is None else np.array(z0, dtype=np.float64)
    Hk = np.zeros((H, K, M)) if hk0 is None else np.array(hk0, dtype=np.float64)
    Hv = np.zeros((H, M, V)) if hv0 is None else np.array(hv0, dtype=np.float64)
    z = np.zeros((T, H, M))
    hk_pre, hv_pre = [], []
    for t in range(T):
        if t % chunk == 0:
            hk_pre.append(Hk.copy())
            hv_pre.append(Hv.copy())
        zt = np.logaddexp(z_prev, s[t])
        w = np.exp(s[t] - zt)                 # [H, M]
        r = np.exp(z_prev - zt)               # [H, M]; 0 at the first token
        Hk = Hk * r[:, None, :] + k[t][:, :, None] * w[:, None, :]
        Hv = Hv * r[:, :, None] + w[:, :, None] * v[t][:, None, :]
        z[t] = zt
        z_prev = zt
    nc = len(hk_pre)
    hk_pre = np.stack(hk_pre) if nc else np.zeros((0, H, K, M))
    hv_pre = np.stack(hv_pre) if nc else np.zeros((0, H, M, V))
    return z, hk_pre, hv_pre, Hk, Hv


def abc_readout_sequence(q, k, v, s, p=None, scale: float = 1.0, hk0=None, hv0=None, z0=None):
    """The two reads of the slot states, token by token, one sequence, all heads.

    q [T, H, K], k [T, H, K], v [T, H, V], s [T, H, M].  After token t's update:

        score_t = scale * Hk_t^T q_t          (M slot scores)
        o_t     = Hv_t^T p_t                  (V outputs)

    with p_t the given slot weights ``p`` [T, H, M], or softmax over the slots
    of score_t when ``p`` is None (the full ABC read: scores, a softmax over
    the M slots, then the value read).  Returns a dict of float64 arrays:
    score [T, H, M], p [T, H, M], o [T, H, V], z [T, H, M], hk_final, hv_final.
    """
    T, H, K = k.shape
    V = v.shape[-1]
    M = s.shape[-1]
    z_prev = np.full((H, M), -np.inf) if z0 is None else np.array(z0, dtype=np.float64)
    Hk = np.zeros((H, K, M)) if hk0 is None else np.array(hk0, dtype=np.float64)
    Hv = np.zeros((H, M, V)) if hv0 is None else np.array(hv0, dtype=np.float64)
    score = np.zeros((T, H, M))
    pw = np.zeros((T, H, M))
    o = np.zeros((T, H, V))
    z = np.zeros((T, H, M))
    for t in range(T):
        zt = np.logaddexp(z_prev, s[t])
        w = np.exp(s[t] - zt)
        r = np.exp(z_prev - zt)
        Hk = Hk * r[:, None, :] + k[t][:, :, None] * w[:, None, :]
        Hv = Hv * r[:, :, None] + w[:, :, None] * v[t][:, None, :]
        score[t] = scale * np.einsum("hkm,hk->hm", Hk, q[t])
        if p is None:
            e = np.exp(score[t] - score[t].max(axis=-1, keepdims=True))
            pw[t] = e / e.sum(axis=-1, keepdims=True)
        else:
            pw[t] = p[t]
        o[t] = np.einsum("hmv,hm->hv", Hv, pw[t])
        z[t] = zt
        z_prev = zt
    return {"score": score, "p": pw, "o": o, "z": z, "hk_final": Hk, "hv_final": Hv}


def abc_recurrent_fp64(k, v, s, chunk: int = CHUNK, batches=None, heads=None) -> dict:
    """Dense [B, T, H, *] problem.  ``batches`` / ``heads`` restrict to a sample.

    Returns float64 arrays z [B', T, H', M], hk [B', NC, H', K, M],
    hv [B', NC, H', M, V], hk_final [B', H', K, M], hv_final [B', H', M, V].
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    B = k.shape[0]
    bs = list(range(B)) if batches is None else list(batches)
    hs = list(range(k.shape[2])) if heads is None else list(heads)
    outs = [abc_scan_sequence(k[b][:, hs], v[b][:, hs], s[b][:, hs], chunk) for b in bs]
    return {
        "z": np.stack([o[0] for o in outs]),
        "hk": np.stack([o[1] for o in outs]),
        "hv": np.stack([o[2] for o in outs]),
        "hk_final": np.stack([o[3] for o in outs]),
        "hv_final": np.stack([o[4] for o in outs]),
    }


def abc_forward_fp64(q, k, v, s, scale: float = 1.0, p=None, batches=None, heads=None) -> dict:
    """The ABC read over a dense [B, T, H, *] problem (``abc_readout_sequence``
    per batch row; softmax slot weights unless ``p`` is given).  ``batches`` /
    ``heads`` restrict to a sample.  Returns float64 o [B', T, H', V] and
    p [B', T, H', M]."""
    q, k, v, s = (np.asarray(x, dtype=np.float64) for x in (q, k, v, s))
    B = k.shape[0]
    bs = list(range(B)) if batches is None else list(batches)
    hs = list(range(k.shape[2])) if heads is None else list(heads)
    outs = [abc_readout_sequence(q[b][:, hs], k[b][:, hs], v[b][:, hs], s[b][:, hs],
                                 None if p is None else np.asarray(p[b], dtype=np.float64)[:, hs], scale)
            for b in bs]
    return {"o": np.stack([x["o"] for x in outs]), "p": np.stack([x["p"] for x in outs])}


def abc_weighted_scan(k, v, w, r, chunk: int = CHUNK):
    """The same state update with the weights given directly (no exp/log).

    k [T, K], v [T, V], w, r [T, M], one head; any numeric dtype (e.g. Fraction
    object arrays).  Returns (hk_final [K, M], hv_final [M, V]).
    """
    T, K = k.shape
    V = v.shape[-1]
    M = w.shape[-1]
    dt = np.asarray(w).dtype
    Hk = np.zeros((K, M), dtype=dt) if dt != object else np.full((K, M), 0, dtype=object)
    Hv = np.zeros((M, V), dtype=dt) if dt != object else np.full((M, V), 0, dtype=object)
    for t in range(T):
        Hk = Hk * r[t][None, :] + np.outer(k[t], w[t])
        Hv = Hv * r[t][:, None] + np.outer(w[t], v[t])
    return Hk, Hv
