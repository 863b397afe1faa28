"""GPU parity of the ABC reverse (dH) walk against the FP64 oracle
(``oracle.abc_backward_fp64``), through the C ABI: the gradients of the slot
states after every chunk, relative L2 <= 1e-2 (bfloat16 storage of the inputs
and of dhk / dhv).  The GPU side takes the normaliser z from the GPU forward
call; the oracle computes its own from the same stored logits.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
from parity import per_row_head_max, rel
from workloads import make_abc, make_config

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def pkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_chunked_amd as p

    p.lib()
    return p


def upstream(inp, seed, with_end=True):
    """Seeded reads' inputs and gradients: q [B,T,H,K], slot weights p (rows of
    a softmax), dscore, dO (bfloat16), final-state gradients (float32)."""
    r = np.random.default_rng(seed)
    B, T, H, K = inp.k.shape
    M, V = inp.s.shape[-1], inp.v.shape[-1]
    bf = torch.bfloat16
    q = torch.from_numpy(r.standard_normal((B, T, H, K)).astype(np.float32)).to(bf)
    lg = r.standard_normal((B, T, H, M))
    p = np.exp(lg - lg.max(-1, keepdims=True))
    p = torch.from_numpy((p / p.sum(-1, keepdims=True)).astype(np.float32)).to(bf)
    ds = torch.from_numpy(r.standard_normal((B, T, H, M)).astype(np.float32)).to(bf)
    do = torch.from_numpy(r.standard_normal((B, T, H, V)).astype(np.float32)).to(bf)
    ek = ev = None
    if with_end:
        ek = torch.from_numpy((0.1 * r.standard_normal((B, H, K, M))).astype(np.float32))
        ev = torch.from_numpy((0.1 * r.standard_normal((B, H, M, V))).astype(np.float32))
    return q, p, ds, do, ek, ev


def run_bwd(pkg, inp, up, scale):
    q, p, ds, do, ek, ev = up
    z, _, _, _, _ = pkg.abc_affine_scan(inp.k.cuda(), inp.v.cuda(), inp.s.cuda(), emit_z=True, emit_final=False)
    dhk, dhv = pkg.abc_affine_scan_bwd(q.cuda(), ds.cuda(), p.cuda(), do.cuda(), z,
                                       None if ek is None else ek.cuda(), None if ev is None else ev.cuda(), scale)
    torch.cuda.synchronize()
    return dhk, dhv


def check(pkg, inp, up, scale, pool=False, what=""):
    """Every (batch row, head) against the oracle (``pool``: in worker
    processes, one per (row, head)), whole tensors and per slice."""
    dhk, dhv = run_bwd(pkg, inp, up, scale)
    q, p, ds, do, ek, ev = up
    f = lambda t: None if t is None else t.to(torch.float64).numpy()
    args = (f(q), inp.s.to(torch.float64).numpy(), f(p), f(ds), f(do), f(ek), f(ev), scale)
    ref = oracle_pool.abc_backward_all(*args) if pool else oracle.abc_backward_fp64(*args)
    got = {"dhk": dhk.detach().to(torch.float64).cpu().numpy(), "dhv": dhv.detach().to(torch.float64).cpu().numpy()}
    errs = {k: rel(got[k], ref[k]) for k in got}
    worst = per_row_head_max({k: (got[k], ref[k], 2) for k in got})
    print(what, " ".join(f"{k}={v:.3e}" for k, v in errs.items()), "| per (row, head) max:",
          " ".join(f"{k}={v[0]:.3e}@{v[1:]}" for k, v in worst.items()), flush=True)
    for key, e in errs.items():
        assert e <= TOL, f"{what} {key}: rel-L2 {e:.3e}"
        assert worst.get(key, (0.0,))[0] <= TOL, f"{what} {key}: {worst[key]}"
    return dhk, dhv


@pytest.mark.parametrize("shape", [(1, 200, 2, 64, 128), (2, 65, 1, 128, 64), (1, 1, 3, 64, 64),
                                   (1, 64 * 9 + 3, 2, 192, 128)], ids=lambda s: "x".join(map(str, s)))
def test_abc_bwd_parity(pkg, shape):
    B, T, H, K, V = shape
    inp = make_abc(980 + T, B=B, T=T, H=H, K=K, M=64, V=V)
    check(pkg, inp, upstream(inp, 981 + T), 0.7, what=f"abc bwd {shape}")


@pytest.mark.parametrize("runs", [1, 3])
def test_abc_bwd_32_slots(pkg, monkeypatch, runs):
    """M = 32 slots (padded to 64 inside the walk) against the oracle."""
    inp = make_abc(989 + runs, B=2, T=1100, H=2, K=128, M=32, V=192)
    monkeypatch.setenv("GDR_ABC_SEGMENTS", str(runs))
    check(pkg, inp, upstream(inp, 990 + runs), 0.8, what=f"abc bwd M=32 runs={runs}")


def test_abc_bwd_without_final_gradient(pkg):
    inp = make_abc(985, B=1, T=300, H=2, K=64, M=64, V=64)
    check(pkg, inp, upstream(inp, 986, with_end=False), 1.0, what="abc bwd no end gradient")


@pytest.mark.parametrize("runs", [1, 2, 3])
def test_abc_bwd_runs(pkg, monkeypatch, runs):
    """Reverse walk split into runs: every tile width gives the same bits for a
    given number of runs, and each run count matches the oracle."""
    inp = make_abc(987, B=1, T=1700, H=2, K=128, M=64, V=192)
    up = upstream(inp, 988)
    monkeypatch.setenv("GDR_ABC_SEGMENTS", str(runs))
    outs = {}
    for xw in (64, 32, 16):
        monkeypatch.setenv("GDR_ABC_XW", str(xw))
        outs[xw] = run_bwd(pkg, inp, up, 0.5)
    for xw in (32, 16):
        for i in range(2):
            assert torch.equal(outs[64][i], outs[xw][i]), (runs, xw, i)
    monkeypatch.setenv("GDR_ABC_XW", "64")
    check(pkg, inp, up, 0.5, what=f"abc bwd runs={runs}")


def test_abc_bwd_benchmark_shape(pkg):
    """B=2, T=16384, H=4, K=256, M=64, V=512 (eight runs by default), against
    the oracle on every (batch row, head); deterministic run to run."""
    inp = make_config("abc_affine")
    up = upstream(inp, 989)
    a = check(pkg, inp, up, 1.0, pool=True, what="abc bwd abc_affine (all rows and heads)")
    b = run_bwd(pkg, inp, up, 1.0)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
