"""FP64 oracle of the gated delta rule — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module; the HIP product path never does.

What it computes
----------------
The pages name the recurrence but never print it: the state-scan kernel that
the kev page runs inside each DeltaNet layer (kev pull request #259, opening
section) is the chunked form of the gated delta rule, and its per-chunk step
emits the state before each 64-token chunk.  Written out per token t of one sequence and one
head, with decay a_t = exp(g_t) and write strength b_t = beta_t::

    S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T          (dk x dv)
    o_t = scale * S_t^T q_t

This module evaluates exactly that, one token at a time: first the decay
S <- a_t S, then the delta-rule write S <- S + b_t k_t (v_t - S^T k_t)^T on
the decayed state, which is the same matrix product expanded.  The output uses
the state after token t's update.  Sequences restart at each ``cu_seqlens``
boundary (kev pull request #259, opening section: the sequence count of a
packed pass is ``len(cu_seqlens) - 1``), and the state before every 64-token
chunk of a sequence (offsets 0, 64, ... from the sequence start) is recorded.

Segment summaries (cuLA pull request #127, "Root cause and implementation"):
a segment of a long sequence maps its incoming state S_in to
``M S_in + S_loc`` where M is the product of the segment's per-token
transitions a_t (I - b_t k_t k_t^T) and S_loc is the state the segment reaches
from zero.  ``gdr_segment_summaries_fp64`` applies the transitions one token at
a time to the identity (M) and runs the recurrence from zero (S_loc);
``gdr_segment_compose_fp64`` chains S_init(s+1) = M_s S_init(s) + S_loc(s).

The core step works on float64 arrays and also on numpy object arrays of
``fractions.Fraction`` (exact arithmetic), which the pin tests use.
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

CHUNK = 64


def chunk_counts(lengths: Sequence[int], chunk: int = CHUNK) -> List[int]:
    """Number of chunks of each sequence: ceil(L / chunk) (0 for an empty one)."""
    return [(int(L) + chunk - 1) // chunk for L in lengths]


def gdr_scan_sequence(q, k, v, a, b, S0, scale=1.0, chunk: int = CHUNK, return_delta=False):
    """Token-serial gated delta rule over one sequence, all heads at once.

    q, k: [L, H, DK]; v: [L, H, DV]; a (decay multiplier), b (beta): [L, H];
    S0: [H, DK, DV].  Returns (o [L, H, DV], pre-chunk states [nc, H, DK, DV],
    final state [H, DK, DV]) and, with ``return_delta``, the per-token write
    vectors delta [L, H, DV].  Works for float64 and for Fraction object arrays.
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
        # decay first ...
        S = a[t][:, None, None] * S
        # ... then the delta-rule write on the decayed state: S += b k (v - S^T k)^T
        kt = k[t]                                        # [H, DK]
        pred = np.einsum("hk,hkv->hv", kt, S)            # S^T k  -> [H, DV]
        err = v[t] - pred
        # the value-side vector written along k_t: delta_t = b_t (v_t - a_t S_{t-1}^T k_t)
        delta = b[t][:, None] * err
        S = S + kt[:, :, None] * delta[:, None, :]
        vnew[t] = delta
        # output reads the updated state: o_t = scale * S_t^T q_t
        o[t] = scale * np.einsum("hk,hkv->hv", q[t], S)
    if pre:
        pre_arr = np.stack(pre)
    else:
        pre_arr = np.zeros((0, H, DK, DV), dtype=dt)
    if return_delta:
        return o, pre_arr, S, vnew
    return o, pre_arr, S


def _sequences(B: int, T: int, cu_seqlens) -> List[Tuple[int, int, int]]:
    """(batch row, start, end) of every sequence."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    if B != 1:
        raise ValueError("packed sequences need B == 1")
    return [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def gdr_recurrent_fp64(q, k, v, g, beta, h0=None, cu_seqlens=None, scale: float = 1.0,
                       chunk: int = CHUNK, heads: Optional[Sequence[int]] = None) -> dict:
    """Whole problem: dense [B, T, H, D] rows or packed sequences (B = 1, cu_seqlens).

    g is the per-token log decay (a_t = exp(g_t)).  ``heads`` restricts the work
    to a subset of heads (heads are independent), for sampled checks of large
    problems.  Returns float64 arrays:

      o   [B, T, H', DV]
      v_new [B, T, H', DV]         delta_t = b_t (v_t - a_t S_{t-1}^T k_t), the write vectors
      h   [NT_total, H', DK, DV]   state before each chunk, sequences packed in order
      hT  [N, H', DK, DV]          state after each sequence's last token
      chunk_offsets [N + 1]        first row of each sequence in ``h``
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
        on, pre, Sf, dn = gdr_scan_sequence(q[b, s:e][:, hs], k[b, s:e][:, hs], v[b, s:e][:, hs],
                                            a_all[b, s:e][:, hs], beta[b, s:e][:, hs], S0, scale,
                                            chunk, return_delta=True)
        o[b, s:e] = on
        vnew[b, s:e] = dn
        h[offsets[n]:offsets[n + 1]] = pre
        hT[n] = Sf
    return {"o": o, "v_new": vnew, "h": h, "hT": hT, "chunk_offsets": offsets}


def segment_bounds(L: int, n_segments: int, chunk: int = CHUNK) -> List[Tuple[int, int]]:
    """Token ranges of the chunk-aligned segments of one sequence of length L.

    The NT = ceil(L / chunk) chunks are dealt out as evenly as possible: every
    segment gets floor(NT / P) chunks and the first NT mod P segments one more.
    (The pages fix a sixteen-way split of a 64K-token sequence, not the rule;
    this is the plainest even split.)  A segment may be empty when P > NT.
    """
    nt = (L + chunk - 1) // chunk
    base, extra = divmod(nt, n_segments)
    out = []
    c = 0
    for s in range(n_segments):
        nc = base + (1 if s < extra else 0)
        t0 = min(c * chunk, L)
        t1 = min((c + nc) * chunk, L)
        out.append((t0, t1))
        c += nc
    return out


def gdr_segment_summaries_fp64(k, v, g, beta, bounds: Sequence[Tuple[int, int]],
                               heads: Optional[Sequence[int]] = None):
    """Per-segment (S_loc, M) of one sequence: k [L, H, DK], v [L, H, DV], g, beta [L, H].

    S_loc(s): the recurrence over the segment's tokens from a zero state.
    M_s: the per-token transitions a_t (I - b_t k_t k_t^T) applied, in order, to
    the identity (a zero value stream leaves exactly that product).
    Returns (S_loc [P, H', DK, DV], M [P, H', DK, DK]).
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    a = np.exp(np.asarray(g, dtype=np.float64))
    beta = np.asarray(beta, dtype=np.float64)
    L, H, DK = k.shape
    DV = v.shape[-1]
    hs = list(range(H)) if heads is None else list(heads)
    Hs = len(hs)
    S_loc = np.zeros((len(bounds), Hs, DK, DV))
    M = np.zeros((len(bounds), Hs, DK, DK))
    eye = np.broadcast_to(np.eye(DK), (Hs, DK, DK)).copy()
    for s, (t0, t1) in enumerate(bounds):
        kk = k[t0:t1][:, hs]
        aa = a[t0:t1][:, hs]
        bb = beta[t0:t1][:, hs]
        qz = np.zeros_like(kk)
        _, _, S_loc[s] = gdr_scan_sequence(qz, kk, v[t0:t1][:, hs], aa, bb,
                                           np.zeros((Hs, DK, DV)), 1.0, max(t1 - t0, 1))
        _, _, M[s] = gdr_scan_sequence(qz, kk, np.zeros((t1 - t0, Hs, DK)), aa, bb,
                                       eye, 1.0, max(t1 - t0, 1))
    return S_loc, M


def gdr_segment_compose_fp64(S_loc, M, h0=None):
    """Serial composition: S_init(0) = h0 (or 0); S_init(s+1) = M_s S_init(s) + S_loc(s).

    Returns (S_init [P, H, DK, DV], state after the last segment [H, DK, DV]).
    """
    P, H, DK, DV = S_loc.shape
    S = np.zeros((H, DK, DV)) if h0 is None else np.array(h0, dtype=np.float64)
    inits = np.zeros_like(S_loc)
    for s in range(P):
        inits[s] = S
        S = np.matmul(M[s], S) + S_loc[s]
    return inits, S


def decay_product(g) -> float:
    """exp(sum g): the pure-decay factor of a token range (used by the b = 0 pin)."""
    return math.exp(float(np.sum(np.asarray(g, dtype=np.float64))))
