"""Seeded synthetic input recipes (no scan arithmetic lives here).

Every workload draws from ``numpy.random.default_rng(seed)`` (PCG64, stable
across platforms) in a fixed order:

    lengths -> q -> k -> v -> beta pre-activation -> g pre-activation -> h0

for the gated delta rule, and ``k -> v -> s`` for the ABC slot recurrence.
Normal draws are float64; q and k are L2-normalised per token and head in
float64; every tensor is then rounded to float32 and, for bfloat16 storage,
rounded again by torch's round-to-nearest-even cast.  The consumers (the FP64
oracle and the HIP path) both read the stored values, so the rounding is part
of the input, not of either side's arithmetic.

Gate recipes
------------
``logsigmoid``   beta = sigmoid(N(0,1)), g = log(sigmoid(N(4,1)))  (decay close
                 to 1 but clearly contracting: a = sigmoid(x) with x ~ N(4,1)).
``logsigmoid_mid``  beta as above, g = log(sigmoid(N(2.5, 0.3))) (about -0.08
                 per token: the state shrinks by e^-40 over 500 tokens).
``logsigmoid_fast`` beta as above, g = log(sigmoid(N(-1, 1))) (about -1.4 per
                 token: a chunk's total decay underflows float32).
``near_one``     a = 1 - 1e-4 * U(0,1), g = log(a) evaluated as log1p in
                 float64, and beta = U(0.01, 0.05): the transition-sensitive,
                 nearly non-contracting long-context regime.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

__all__ = [
    "GdrInputs",
    "AbcInputs",
    "CONFIGS",
    "make_gdr",
    "make_abc",
    "make_config",
    "random_lengths",
]


def _to_storage(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Round a float64 array into the storage dtype (via float32, RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype) if dtype != torch.float32 else t


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def random_lengths(rng: np.random.Generator, n: int, lo: int, hi: int,
                   avoid_multiple: Optional[int] = None) -> List[int]:
    """n lengths uniform in [lo, hi]; optionally redraw multiples of a chunk size."""
    if avoid_multiple is None:
        return [int(x) for x in rng.integers(lo, hi + 1, n)]
    out: List[int] = []
    while len(out) < n:
        x = int(rng.integers(lo, hi + 1))
        if x % avoid_multiple:
            out.append(x)
    return out


@dataclass
class GdrInputs:
    """Inputs of one gated-delta-rule problem, stored on the CPU.

    q, k: [B, T, H, DK]; v: [B, T, H, DV] in ``dtype``.  g (per-token log decay)
    and beta: [B, T, H] float32 (per-channel gates: g [B, T, H, DK]).  Packed variable-length batches use B = 1 with
    ``cu_seqlens`` (int32, N+1 entries).  h0: [N, H, DK, DV] float32 or None.
    """

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    h0: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    lengths: List[int]
    dtype: torch.dtype
    scale: float = 1.0
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return self.q.shape[0]

    @property
    def T(self) -> int:
        return self.q.shape[1]

    @property
    def H(self) -> int:
        return self.q.shape[2]

    @property
    def DK(self) -> int:
        return self.q.shape[3]

    @property
    def DV(self) -> int:
        return self.v.shape[3]

    @property
    def N(self) -> int:
        return len(self.lengths)

    @property
    def token_heads(self) -> int:
        return int(sum(self.lengths)) * self.H

    def f64(self) -> dict:
        """float64 numpy views of the stored values (what the oracle consumes)."""
        d = {
            "q": self.q.to(torch.float64).numpy(),
            "k": self.k.to(torch.float64).numpy(),
            "v": self.v.to(torch.float64).numpy(),
            "g": self.g.to(torch.float64).numpy(),
            "beta": self.beta.to(torch.float64).numpy(),
            "h0": None if self.h0 is None else self.h0.to(torch.float64).numpy(),
            "cu_seqlens": None if self.cu_seqlens is None else self.cu_seqlens.numpy().astype(np.int64),
        }
        return d


def make_gdr(seed: int, *, lengths: Optional[Sequence[int]] = None, B: int = 1, T: int = 0,
             H: int = 1, DK: int = 128, DV: int = 128, dtype: torch.dtype = torch.bfloat16,
             varlen: bool = False, gates: str = "logsigmoid", h0_std: Optional[float] = None,
             scale: float = 1.0, name: str = "custom", rng: Optional[np.random.Generator] = None,
             ) -> GdrInputs:
    """Draw one gated-delta-rule problem.

    Dense problems give ``B`` and ``T``; packed ones give ``lengths`` (already
    drawn) and ``varlen=True``.  A dense problem can also be built from equal
    ``lengths`` with ``varlen=False``.
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        if varlen:
            B, T = 1, int(sum(lengths))
        else:
            assert len(set(lengths)) <= 1, "dense layout needs equal lengths"
            B, T = len(lengths), (lengths[0] if lengths else 0)
    else:
        lengths = [T] * B
    q = rng.standard_normal((B, T, H, DK))
    q = _to_storage(_l2_normalise(q), dtype)
    k = rng.standard_normal((B, T, H, DK))
    k = _to_storage(_l2_normalise(k), dtype)
    v = _to_storage(rng.standard_normal((B, T, H, DV)), dtype)
    if gates == "logsigmoid":
        beta = _sigmoid(rng.standard_normal((B, T, H)))
        g = _logsigmoid(rng.normal(4.0, 1.0, (B, T, H)))
    elif gates == "logsigmoid_channels":
        # per-key-channel decays: every (token, head, channel) its own logsigmoid(N(4, 1))
        beta = _sigmoid(rng.standard_normal((B, T, H)))
        g = _logsigmoid(rng.normal(4.0, 1.0, (B, T, H, DK)))
    elif gates == "channels_to_limit":
        # per-channel log decays across the whole supported range [-5, 0): U(-5, 0)
        # per (token, head, channel), every fourth channel at exactly -5
        beta = _sigmoid(rng.standard_normal((B, T, H)))
        g = -5.0 * rng.uniform(0.0, 1.0, (B, T, H, DK))
        g[..., ::4] = -5.0
    elif gates in ("logsigmoid_mid", "logsigmoid_fast"):
        beta = _sigmoid(rng.standard_normal((B, T, H)))
        mu, sd = (2.5, 0.3) if gates == "logsigmoid_mid" else (-1.0, 1.0)
        g = _logsigmoid(rng.normal(mu, sd, (B, T, H)))
    elif gates == "near_one":
        beta = rng.uniform(0.01, 0.05, (B, T, H))
        g = np.log1p(-1e-4 * rng.uniform(0.0, 1.0, (B, T, H)))
    else:
        raise ValueError(f"unknown gate recipe {gates!r}")
    beta_t = torch.from_numpy(beta.astype(np.float32))
    g_t = torch.from_numpy(g.astype(np.float32))
    N = len(lengths)
    h0 = None
    if h0_std is not None:
        h0 = torch.from_numpy((h0_std * rng.standard_normal((N, H, DK, DV))).astype(np.float32))
    cu = None
    if varlen:
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    return GdrInputs(name=name, q=q, k=k, v=v, g=g_t, beta=beta_t, h0=h0, cu_seqlens=cu,
                     lengths=list(lengths), dtype=dtype, scale=scale,
                     meta={"seed": seed, "gates": gates})


@dataclass
class AbcInputs:
    """ABC slot-recurrence inputs: k [B,T,H,K], v [B,T,H,V], s [B,T,H,M] (storage dtype)."""

    name: str
    k: torch.Tensor
    v: torch.Tensor
    s: torch.Tensor
    dtype: torch.dtype
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return self.k.shape[0]

    @property
    def T(self) -> int:
        return self.k.shape[1]

    @property
    def H(self) -> int:
        return self.k.shape[2]

    @property
    def K(self) -> int:
        return self.k.shape[3]

    @property
    def V(self) -> int:
        return self.v.shape[3]

    @property
    def M(self) -> int:
        return self.s.shape[3]

    @property
    def token_heads(self) -> int:
        return self.B * self.T * self.H

    def f64(self) -> dict:
        return {"k": self.k.to(torch.float64).numpy(), "v": self.v.to(torch.float64).numpy(),
                "s": self.s.to(torch.float64).numpy()}


def make_abc(seed: int, *, B: int, T: int, H: int, K: int, M: int, V: int,
             dtype: torch.dtype = torch.bfloat16, name: str = "custom") -> AbcInputs:
    rng = np.random.default_rng(seed)
    k = _to_storage(rng.standard_normal((B, T, H, K)), dtype)
    v = _to_storage(rng.standard_normal((B, T, H, V)), dtype)
    s = _to_storage(rng.standard_normal((B, T, H, M)), dtype)
    return AbcInputs(name=name, k=k, v=v, s=s, dtype=dtype, meta={"seed": seed})


# The seeded workloads.  Seed i belongs to workload i.
CONFIGS = {
    "tiny_fp32": dict(kind="gdr", seed=0, B=1, T=256, H=1, DK=64, DV=64, dtype="f32",
                      varlen=False, gates="logsigmoid", h0_std=None),
    "question_rows": dict(kind="gdr", seed=1, n_seqs=24, len_lo=16, len_hi=256, avoid=None,
                          H=16, DK=128, DV=128, dtype="bf16", varlen=True,
                          gates="logsigmoid", h0_std=0.1),
    "new_states": dict(kind="gdr", seed=2, n_seqs=8, len_lo=1024, len_hi=4096, avoid=64,
                       H=32, DK=128, DV=128, dtype="bf16", varlen=True,
                       gates="logsigmoid", h0_std=None),
    "long_state_h8": dict(kind="gdr", seed=3, B=1, T=65536, H=8, DK=128, DV=128, dtype="bf16",
                          varlen=False, gates="near_one", h0_std=None, n_segments=16),
    "long_state_h1": dict(kind="gdr", seed=3, B=1, T=65536, H=1, DK=128, DV=128, dtype="bf16",
                          varlen=False, gates="near_one", h0_std=None, n_segments=16),
    "abc_affine": dict(kind="abc", seed=4, B=2, T=16384, H=4, K=256, M=64, V=512, dtype="bf16"),
    # per-key-channel decay on the question-rows shape (no such workload is on the pages;
    # the shape of question_rows with a per-channel gate)
    "kda_question_rows": dict(kind="gdr", seed=5, n_seqs=24, len_lo=16, len_hi=256, avoid=None,
                              H=16, DK=128, DV=128, dtype="bf16", varlen=True,
                              gates="logsigmoid_channels", h0_std=0.1),
}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def make_config(name: str, **override):
    """Build one of the named seeded workloads (keyword overrides allowed, e.g. T=...)."""
    c = dict(CONFIGS[name])
    c.update(override)
    dtype = _DT[c["dtype"]]
    if c["kind"] == "abc":
        return make_abc(c["seed"], B=c["B"], T=c["T"], H=c["H"], K=c["K"], M=c["M"], V=c["V"],
                        dtype=dtype, name=name)
    rng = np.random.default_rng(c["seed"])
    if "n_seqs" in c:
        lengths = random_lengths(rng, c["n_seqs"], c["len_lo"], c["len_hi"], c.get("avoid"))
        inp = make_gdr(c["seed"], lengths=lengths, H=c["H"], DK=c["DK"], DV=c["DV"], dtype=dtype,
                       varlen=True, gates=c["gates"], h0_std=c["h0_std"], name=name, rng=rng)
    else:
        inp = make_gdr(c["seed"], B=c["B"], T=c["T"], H=c["H"], DK=c["DK"], DV=c["DV"], dtype=dtype,
                       varlen=False, gates=c["gates"], h0_std=c["h0_std"], name=name, rng=rng)
    if "n_segments" in c:
        inp.meta["n_segments"] = c["n_segments"]
    return inp
