"""FP64 oracle of the reverse (gradient) state recurrence — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module; the HIP product path never does.

What it computes
----------------
The flash-linear-attention fork issue #23 ("Problem": the reverse kernel
that walks the state tiles chunk by chunk; "Proposed Dataflow", item 4: the
reverse dH recurrence is the next thing to carry over) names the reverse pass
of the chunked state scan without printing it.  For the gated delta rule it
is the adjoint of the forward recurrence, derived here.

Forward, per token t of one sequence and one head (``gdr_ref``):

    S_t = J_t S_{t-1} + b_t k_t v_t^T,   J_t = a_t (I - b_t k_t k_t^T)   (symmetric)
    o_t = scale * S_t^T q_t

Given upstream gradients do_t = dL/do_t and dS_end = dL/dS_{L-1} (the final
state's gradient), the total gradient with respect to the state after token
t is

    G_{L-1} = scale q_{L-1} do_{L-1}^T + dS_end
    G_t     = scale q_t do_t^T + J_{t+1} G_{t+1}

which needs no forward state: the recurrence is linear in S.  Reported:

    dh[c]  the gradient carried from chunk c+1 back into chunk c: the
           gradient with respect to the state after chunk c as the input of
           the rest of the sequence, J_{e+1} G_{e+1} for chunk c ending at
           token e, and dS_end after the sequence's last chunk;
    dh0    J_0 G_0, the gradient with respect to the initial state;
    dv_new the gradient with respect to the chunk form's write vectors
           Delta (the forward scan's v_new).  Inside chunk c the chunk form
           writes S = e^{gamma_t} S_c + sum_{i<=t} e^{gamma_t - gamma_i} k_i Delta_i^T
           (gamma = the chunk-local inclusive cumsum of g), so Delta_i reaches
           the outputs o_t (t >= i in the chunk) and the chunk's end state:
              dv_new_i = scale sum_{t>=i} e^{gamma_t - gamma_i} (q_t . k_i) do_t
                         + e^{gamma_C - gamma_i} dh[c]^T k_i
           (gamma_C: the chunk's last valid token).

Layouts follow ``gdr_recurrent_fp64``: dh [NT, H', DK, DV] (one row per
chunk, sequences packed in order), dh0 [N, H', DK, DV], dv_new [B, T, H', DV].
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .gdr_ref import CHUNK, _sequences, chunk_counts


def gdr_backward_sequence(q, k, g, beta, do, dS_end, scale=1.0, chunk: int = CHUNK):
    """One sequence, all heads: q, k [L, H, DK]; g, beta [L, H]; do [L, H, DV];
    dS_end [H, DK, DV].  Returns (dh [nc, H, DK, DV], dh0 [H, DK, DV],
    dv_new [L, H, DV]) in float64."""
    L, H, DK = k.shape
    DV = do.shape[-1]
    a = np.exp(g)
    nc = (L + chunk - 1) // chunk
    dh = np.zeros((nc, H, DK, DV))
    dv = np.zeros((L, H, DV))

    def J(t, X):  # J_t X = a_t (X - b_t k_t (k_t^T X)), per head
        kt = k[t]
        return a[t][:, None, None] * (X - beta[t][:, None, None] * kt[:, :, None]
                                      * np.einsum("hk,hkv->hv", kt, X)[:, None, :])

    carry = np.array(dS_end, dtype=np.float64)   # gradient entering the state after token t from later tokens
    for t in range(L - 1, -1, -1):
        if t % chunk == chunk - 1 or t == L - 1:
            dh[t // chunk] = carry               # the state after chunk t // chunk
        G = carry + scale * q[t][:, :, None] * do[t][:, None, :]
        carry = J(t, G)
    dh0 = carry

    # gradient of the chunk form's write vectors
    for c in range(nc):
        c0, c1 = c * chunk, min(L, (c + 1) * chunk)
        gam = np.cumsum(g[c0:c1], axis=0)                       # [n, H]
        for hh in range(H):
            qq, kk, dd = q[c0:c1, hh], k[c0:c1, hh], do[c0:c1, hh]
            ga = gam[:, hh]
            P = np.tril(qq @ kk.T) * np.exp(ga[:, None] - ga[None, :])   # P[t, i], i <= t
            dv[c0:c1, hh] = scale * (P.T @ dd) + np.exp(ga[-1] - ga)[:, None] * (kk @ dh[c, hh])
    return dh, dh0, dv


def gdr_backward_fp64(q, k, g, beta, do, dhT=None, cu_seqlens=None, scale: float = 1.0,
                      chunk: int = CHUNK, heads: Optional[Sequence[int]] = None) -> dict:
    """Whole problem (dense rows or packed sequences), float64 results:
    dh [NT, H', DK, DV], dh0 [N, H', DK, DV], dv_new [B, T, H', DV].
    ``dhT`` [N, H, DK, DV] is the final states' gradient (zero when None)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, T, H, DK = k.shape
    DV = do.shape[-1]
    hs = list(range(H)) if heads is None else list(heads)
    Hs = len(hs)
    seqs = _sequences(B, T, cu_seqlens)
    counts = chunk_counts([e - s for _, s, e in seqs], chunk)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    out = {"dh": np.zeros((int(offsets[-1]), Hs, DK, DV)), "dh0": np.zeros((len(seqs), Hs, DK, DV)),
           "dv_new": np.zeros((B, T, Hs, DV)), "chunk_offsets": offsets}
    for n, (b, s, e) in enumerate(seqs):
        dS_end = np.zeros((Hs, DK, DV)) if dhT is None else np.array(dhT[n][hs], dtype=np.float64)
        dh, dh0, dv = gdr_backward_sequence(q[b, s:e][:, hs], k[b, s:e][:, hs], g[b, s:e][:, hs],
                                            beta[b, s:e][:, hs], do[b, s:e][:, hs], dS_end, scale, chunk)
        out["dh"][offsets[n]:offsets[n + 1]] = dh
        out["dh0"][n] = dh0
        out["dv_new"][b, s:e] = dv
    return out
