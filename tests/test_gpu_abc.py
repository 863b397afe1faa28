"""GPU parity of the ABC slot-state construction against the FP64 oracle.

States and finals: relative L2 <= 1e-2 (bfloat16 storage of k, v, s and of the
pre-chunk states).  The normaliser z is FP32 arithmetic on the stored logits:
relative L2 <= 1e-5.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
from parity import per_row_head_max, rel
from workloads import make_abc, make_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_chunked_amd as p

    p.lib()
    return p


def np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def run(pkg, inp, emit_z=True):
    z, hk, hv, hkf, hvf = pkg.abc_affine_scan(inp.k.cuda(), inp.v.cuda(), inp.s.cuda(), emit_z=emit_z)
    torch.cuda.synchronize()
    return {"z": z, "hk": hk, "hv": hv, "hk_final": hkf, "hv_final": hvf}


def compare(r, ref, what=""):
    """Whole tensors and every (batch row, head) slice against the oracle."""
    got = {k: np64(r[k]) for k in ("hk", "hv", "hk_final", "hv_final")}
    errs = {"z": rel(np64(r["z"]), ref["z"]) if r["z"] is not None else 0.0}
    errs.update({k: rel(got[k], ref[k]) for k in got})
    hax = {"hk": 2, "hv": 2, "hk_final": 1, "hv_final": 1}
    worst = per_row_head_max({k: (got[k], ref[k], hax[k]) for k in got})
    if r["z"] is not None:
        worst["z"] = per_row_head_max({"z": (np64(r["z"]), ref["z"], 2)})["z"]
    print(what, " ".join(f"{k}={v:.3e}" for k, v in errs.items()), "| per (row, head) max:",
          " ".join(f"{k}={v[0]:.3e}@{v[1:]}" for k, v in worst.items()), flush=True)
    assert errs["z"] <= 1e-5 and worst.get("z", (0.0,))[0] <= 1e-5
    for key in ("hk", "hv", "hk_final", "hv_final"):
        assert errs[key] <= 1e-2, f"{what} {key} {errs[key]:.3e}"
        assert worst.get(key, (0.0,))[0] <= 1e-2, f"{what} {key} {worst[key]}"


@pytest.mark.parametrize("M", [64, 32])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 127, 257])
def test_abc_small(pkg, T, M):
    """The fixture lengths and slot counts of fla#23's "Fixture-First
    Correctness Contract" (T = 63/64/65/127/257, M = 32/64) and one token."""
    inp = make_abc(900 + T + M, B=2, T=T, H=2, K=128, M=M, V=192)
    d = inp.f64()
    ref = oracle.abc_recurrent_fp64(d["k"], d["v"], d["s"])
    compare(run(pkg, inp), ref, what=f"abc T={T} M={M}")


@pytest.mark.parametrize("runs", [1, 3])
def test_abc_32_slots_tiles_and_runs(pkg, monkeypatch, runs):
    """M = 32 (the slot dimension padded to 64 inside the kernels): every tile
    width gives the same bits, split into runs or not, against the oracle."""
    inp = make_abc(975 + runs, B=2, T=1100, H=2, K=128, M=32, V=192)
    monkeypatch.setenv("GDR_ABC_SEGMENTS", str(runs))
    outs = {}
    for xw in (64, 32, 16):
        monkeypatch.setenv("GDR_ABC_XW", str(xw))
        outs[xw] = run(pkg, inp)
    for xw in (32, 16):
        for key in outs[64]:
            assert torch.equal(outs[64][key], outs[xw][key]), (runs, xw, key)
    d = inp.f64()
    compare(outs[64], oracle.abc_recurrent_fp64(d["k"], d["v"], d["s"]), what=f"abc M=32 runs={runs}")


def test_abc_affine_workload(pkg):
    """Every (batch row, head) of the benchmark shape (the oracle in a pool of
    worker processes, one per (row, head))."""
    inp = make_config("abc_affine")
    r = run(pkg, inp)
    d = inp.f64()
    compare(r, oracle_pool.abc_states_all(d["k"], d["v"], d["s"]), what="abc_affine (all rows and heads)")


def test_abc_deterministic(pkg):
    inp = make_abc(950, B=1, T=300, H=3, K=64, M=64, V=128)
    a = run(pkg, inp)
    b = run(pkg, inp)
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("T", [65, 300])
def test_abc_tile_widths_bit_identical(pkg, monkeypatch, T):
    """Every state element is the same sequence of FP32 operations whatever
    the tile width (64, 32 or 16 columns per workgroup), so the outputs agree
    bit for bit; the widest also matches the oracle."""
    inp = make_abc(960 + T, B=1, T=T, H=2, K=128, M=64, V=192)
    outs = {}
    for xw in (64, 32, 16):
        monkeypatch.setenv("GDR_ABC_XW", str(xw))
        outs[xw] = run(pkg, inp)
    for xw in (32, 16):
        for key in outs[64]:
            assert torch.equal(outs[64][key], outs[xw][key]), (xw, key)
    d = inp.f64()
    compare(outs[64], oracle.abc_recurrent_fp64(d["k"], d["v"], d["s"]), what=f"abc xw T={T}")


@pytest.mark.parametrize("runs", [1, 2, 3])
def test_abc_runs(pkg, monkeypatch, runs):
    """The state walk split into runs (end states composed per slot with the
    normaliser ratios) matches the oracle, and every tile width gives the same
    bits for a given number of runs."""
    inp = make_abc(970, B=1, T=1700, H=2, K=128, M=64, V=192)
    monkeypatch.setenv("GDR_ABC_SEGMENTS", str(runs))
    outs = {}
    for xw in (64, 32, 16):
        monkeypatch.setenv("GDR_ABC_XW", str(xw))
        outs[xw] = run(pkg, inp)
    for xw in (32, 16):
        for key in outs[64]:
            assert torch.equal(outs[64][key], outs[xw][key]), (runs, xw, key)
    d = inp.f64()
    compare(outs[64], oracle.abc_recurrent_fp64(d["k"], d["v"], d["s"]), what=f"abc runs={runs}")


def test_abc_long_carry(pkg):
    """More than 512 chunks in one row: the normaliser carry's stretches are
    longer than the part it keeps in registers (its second read of the chunk
    totals), and the state runs are longer than in the benchmark shape."""
    inp = make_abc(990, B=1, T=40000, H=1, K=64, M=64, V=64)
    d = inp.f64()
    ref = oracle.abc_recurrent_fp64(d["k"], d["v"], d["s"])
    compare(run(pkg, inp), ref, what="abc T=40000")
