"""Error measures of the GPU parity tests (relative L2 against the FP64
oracle), over whole tensors and per (sequence, head) slice."""

from __future__ import annotations

import numpy as np


def rel(a, b):
    """||a - b|| / ||b|| in float64 (b the oracle)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def sequences(B, T, cu, offsets):
    """(b, s, e, first chunk row, end chunk row, n) of every non-empty
    sequence: packed (cu given, B = 1) or dense rows."""
    if cu is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        cu = [int(x) for x in np.asarray(cu)]
        seqs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    return [(b, s, e, int(offsets[n]), int(offsets[n + 1]), n) for n, (b, s, e) in enumerate(seqs) if e > s]


def per_sequence_max(pairs, cu, offsets):
    """Largest relative L2 over the (sequence, head) slices of each tensor.

    ``pairs``: name -> (got, ref, kind) with numpy arrays in the oracle's
    layout; kind "token" = [B, T, H, ...], "chunk" = [NT, H, ...] (rows packed
    by ``offsets``), "seq" = [N, H, ...].  Slices whose reference is all zero
    are skipped.  Returns name -> (error, sequence, head)."""
    any_tok = next(p for p in pairs.values() if p[2] == "token")[1]
    B, T, H = any_tok.shape[:3]
    worst = {}
    for b, s, e, c0, c1, n in sequences(B, T, cu, offsets):
        for j in range(H):
            for name, (got, ref, kind) in pairs.items():
                if kind == "token":
                    gx, rx = got[b, s:e, j], ref[b, s:e, j]
                elif kind == "chunk":
                    gx, rx = got[c0:c1, j], ref[c0:c1, j]
                else:
                    gx, rx = got[n, j], ref[n, j]
                if np.linalg.norm(rx) == 0:
                    continue
                err = rel(gx, rx)
                if err > worst.get(name, (-1.0,))[0]:
                    worst[name] = (err, n, j)
    return worst


def per_row_head_max(pairs):
    """Largest relative L2 over the (batch row, head) slices of dense ABC
    tensors.  ``pairs``: name -> (got, ref, head_axis).  Returns
    name -> (error, row, head)."""
    worst = {}
    for name, (got, ref, hax) in pairs.items():
        B, H = ref.shape[0], ref.shape[hax]
        for b in range(B):
            for h in range(H):
                rx = np.take(ref[b], h, axis=hax - 1)
                if np.linalg.norm(rx) == 0:
                    continue
                err = rel(np.take(got[b], h, axis=hax - 1), rx)
                if err > worst.get(name, (-1.0,))[0]:
                    worst[name] = (err, b, h)
    return worst


def gate(errs, worst, tol, what):
    """Print both figures and assert each is within ``tol``."""
    print(what, " ".join(f"{k}={v:.3e}" for k, v in errs.items()), "| per slice max:",
          " ".join(f"{k}={v[0]:.3e}@{v[1:]}" for k, v in worst.items()), flush=True)
    for k, e in errs.items():
        assert e <= tol, f"{what} {k}: rel-L2 {e:.3e} > {tol:.1e}"
    for k, (e, a, b) in worst.items():
        assert e <= tol, f"{what} {k}: rel-L2 {e:.3e} > {tol:.1e} on slice ({a}, {b})"
