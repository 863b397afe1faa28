"""Run the FP64 oracle's whole-problem wrappers over all heads of a large
problem in a pool of worker processes — test infrastructure only.

Heads (and, for ABC, batch rows) are independent in every recurrence, and
each wrapper takes a ``heads`` (``batches``) sample; the CPU pins hold that
sampling against per-head dense products, closed forms and finite
differences.  This module only splits the inputs by head, calls the wrapper
on each part in a separate process (spawned: the workers import numpy and the
oracle, never torch or the GPU library) and concatenates the parts along the
head axis.  It does no arithmetic of the method.
"""

from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np


def workers() -> int:
    """Worker processes: the host's cores, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _groups(n: int, parts: int):
    parts = max(1, min(parts, n))
    edges = np.linspace(0, n, parts + 1).round().astype(int)
    return [list(range(edges[i], edges[i + 1])) for i in range(parts) if edges[i + 1] > edges[i]]


def _gdr_part(args):
    import oracle

    kind, arrays, kw = args
    fn = {"fwd": oracle.gdr_recurrent_fp64, "bwd": oracle.gdr_backward_fp64, "kda": oracle.kda_recurrent_fp64}[kind]
    return fn(*arrays, **kw)


def _run(fn, jobs):
    if len(jobs) == 1:
        return [fn(jobs[0])]
    ctx = mp.get_context("spawn")
    with ctx.Pool(len(jobs)) as pool:
        return pool.map(fn, jobs)


def _cat(parts, axes):
    return {key: (np.concatenate([p[key] for p in parts], axis=ax) if ax is not None else parts[0][key])
            for key, ax in axes.items()}


def gdr_forward_all_heads(q, k, v, g, beta, h0, cu_seqlens, scale, kind="fwd"):
    """oracle.gdr_recurrent_fp64 (or kda_recurrent_fp64 with kind="kda") over
    every head: o, v_new [B, T, H, DV], h [NT, H, DK, DV], hT [N, H, DK, DV]."""
    H = k.shape[2]
    jobs = []
    for hs in _groups(H, workers()):
        arrays = (q[:, :, hs], k[:, :, hs], v[:, :, hs], g[:, :, hs], beta[:, :, hs],
                  None if h0 is None else h0[:, hs], cu_seqlens, scale)
        jobs.append((kind, arrays, {}))
    parts = _run(_gdr_part, jobs)
    return _cat(parts, {"o": 2, "v_new": 2, "h": 1, "hT": 1, "chunk_offsets": None})


def gdr_backward_all_heads(q, k, g, beta, do, dhT, cu_seqlens, scale):
    """oracle.gdr_backward_fp64 over every head: dh [NT, H, DK, DV],
    dh0 [N, H, DK, DV], dv_new [B, T, H, DV]."""
    H = k.shape[2]
    jobs = []
    for hs in _groups(H, workers()):
        arrays = (q[:, :, hs], k[:, :, hs], g[:, :, hs], beta[:, :, hs], do[:, :, hs],
                  None if dhT is None else dhT[:, hs], cu_seqlens, scale)
        jobs.append(("bwd", arrays, {}))
    parts = _run(_gdr_part, jobs)
    return _cat(parts, {"dh": 1, "dh0": 1, "dv_new": 2, "chunk_offsets": None})


def _abc_part(args):
    import oracle

    kind, arrays, kw = args
    fn = {"rec": oracle.abc_recurrent_fp64, "fwd": oracle.abc_forward_fp64, "bwd": oracle.abc_backward_fp64}[kind]
    return fn(*arrays, **kw)


def _abc_all(kind, arrays, head_axes, kw, B, H, axes):
    """One job per (batch row, head), each on its own slice of the inputs:
    batch rows on axis 0, heads on ``head_axes[i]`` of input i (2 for the
    [B, T, H, *] inputs, 1 for the [B, H, *, *] final-state gradients, None
    for an absent input).  The parts are reassembled along ``axes``."""
    def part(x, ax, b, h):
        if x is None:
            return None
        x = x[b:b + 1]
        return x[:, h:h + 1] if ax == 1 else x[:, :, h:h + 1]

    jobs = [(kind, tuple(part(x, ax, b, h) for x, ax in zip(arrays, head_axes)), kw)
            for b in range(B) for h in range(H)]
    parts = _run(_abc_part, jobs)
    out = {}
    for key, hax in axes.items():
        rows = [np.concatenate([parts[b * H + h][key] for h in range(H)], axis=hax) for b in range(B)]
        out[key] = np.concatenate(rows, axis=0)
    return out


def abc_states_all(k, v, s):
    """oracle.abc_recurrent_fp64 over every (batch row, head)."""
    B, _, H, _ = k.shape
    return _abc_all("rec", (k, v, s), (2, 2, 2), {}, B, H,
                    {"z": 2, "hk": 2, "hv": 2, "hk_final": 1, "hv_final": 1})


def abc_read_all(q, k, v, s, scale):
    """oracle.abc_forward_fp64 (softmax slot weights) over every (batch row, head)."""
    B, _, H, _ = k.shape
    return _abc_all("fwd", (q, k, v, s), (2, 2, 2, 2), {"scale": scale}, B, H, {"o": 2, "p": 2})


def abc_backward_all(q, s, p, dscore, do, dhk_final, dhv_final, scale):
    """oracle.abc_backward_fp64 over every (batch row, head)."""
    B, _, H, _ = q.shape
    return _abc_all("bwd", (q, s, p, dscore, do, dhk_final, dhv_final), (2, 2, 2, 2, 2, 1, 1),
                    {"scale": scale}, B, H, {"dhk": 2, "dhv": 2})
