"""FP64 oracle of the ABC reverse (dH) slot-state recurrence — test
infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module; the HIP product path never does.

What it computes
----------------
The flash-linear-attention fork issue #23 ("Problem": the reverse kernel
that walks every state tile chunk by chunk; "Proposed Dataflow", item 4: the
reverse dH recurrence is to take the same producer / ordered-scan split)
names this pass without printing it; it is the adjoint of the forward slot
recurrence in ``abc_ref``:

    Hk_t = Hk_{t-1} * r_t[None, :] + k_t (x) w_t      (r over slot columns)
    Hv_t = Hv_{t-1} * r_t[:, None] + w_t (x) v_t      (r over slot rows)
    r_t = exp(z_{t-1} - z_t),  w_t = exp(s_t - z_t)

read after every update as score_t = scale Hk_t^T q_t and o_t = Hv_t^T p_t
(``abc_readout_sequence``).  Given upstream gradients dscore_t, do_t and the
final states' gradients, the total gradient with respect to the states
after token t is

    Gk_t = scale q_t (x) dscore_t + Gk_{t+1} * r_{t+1}[None, :]
    Gv_t = p_t (x) do_t           + r_{t+1}[:, None] * Gv_{t+1}

(the gradient of the final states enters as Gk_T, Gv_T's carry).  The
recurrence is linear in the states, so it needs none of them; it needs the
normaliser z, which it computes from s exactly as the forward does.

Reported per chunk c (tokens c*chunk .. e): dhk[c], dhv[c] = the gradient
with respect to the state after chunk c as the input of the rest of the
sequence, i.e. the carry Gk_{e+1} * r_{e+1} (the final states' gradient after
the last chunk).  The states before the first chunk are zero by construction
(no initial state), so nothing is reported for them.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

CHUNK = 64


def abc_backward_sequence(q, s, p, dscore, do, dhk_end=None, dhv_end=None, scale: float = 1.0,
                          chunk: int = CHUNK, z0=None):
    """One sequence, all heads: q [T, H, K], s, p, dscore [T, H, M], do [T, H, V];
    dhk_end [H, K, M], dhv_end [H, M, V] (zero when None).  ``z0`` is the
    normaliser carried in when the sequence resumes (default -inf).
    Returns (dhk [NC, H, K, M], dhv [NC, H, M, V]) in float64."""
    T, H, K = q.shape
    M = s.shape[-1]
    V = do.shape[-1]
    z = np.zeros((T, H, M))
    z_prev = np.full((H, M), -np.inf) if z0 is None else np.array(z0, dtype=np.float64)
    for t in range(T):
        z_prev = np.logaddexp(z_prev, s[t])
        z[t] = z_prev
    nc = (T + chunk - 1) // chunk
    dhk = np.zeros((nc, H, K, M))
    dhv = np.zeros((nc, H, M, V))
    ck = np.zeros((H, K, M)) if dhk_end is None else np.array(dhk_end, dtype=np.float64)
    cv = np.zeros((H, M, V)) if dhv_end is None else np.array(dhv_end, dtype=np.float64)
    z_before = np.full((H, M), -np.inf) if z0 is None else np.array(z0, dtype=np.float64)
    for t in range(T - 1, -1, -1):
        if t % chunk == chunk - 1 or t == T - 1:
            dhk[t // chunk] = ck                 # the state after chunk t // chunk
            dhv[t // chunk] = cv
        Gk = ck + scale * q[t][:, :, None] * dscore[t][:, None, :]
        Gv = cv + p[t][:, :, None] * do[t][:, None, :]
        zp = z[t - 1] if t > 0 else z_before
        r = np.exp(zp - z[t])                    # r_t; 0 at the first token of a fresh sequence
        ck = Gk * r[:, None, :]
        cv = Gv * r[:, :, None]
    return dhk, dhv


def abc_backward_fp64(q, s, p, dscore, do, dhk_final=None, dhv_final=None, scale: float = 1.0,
                      chunk: int = CHUNK, batches: Optional[Sequence[int]] = None,
                      heads: Optional[Sequence[int]] = None) -> dict:
    """Dense [B, T, H, *] problem.  dhk_final [B, H, K, M], dhv_final [B, H, M, V]
    (zero when None).  ``batches`` / ``heads`` restrict to a sample.
    Returns float64 dhk [B', NC, H', K, M], dhv [B', NC, H', M, V]."""
    q, s, p, dscore, do = (np.asarray(x, dtype=np.float64) for x in (q, s, p, dscore, do))
    B = q.shape[0]
    bs = list(range(B)) if batches is None else list(batches)
    hs = list(range(q.shape[2])) if heads is None else list(heads)
    outs = []
    for b in bs:
        ek = None if dhk_final is None else np.asarray(dhk_final[b], dtype=np.float64)[hs]
        ev = None if dhv_final is None else np.asarray(dhv_final[b], dtype=np.float64)[hs]
        outs.append(abc_backward_sequence(q[b][:, hs], s[b][:, hs], p[b][:, hs], dscore[b][:, hs], do[b][:, hs],
                                          ek, ev, scale, chunk))
    return {"dhk": np.stack([o[0] for o in outs]), "dhv": np.stack([o[1] for o in outs])}
