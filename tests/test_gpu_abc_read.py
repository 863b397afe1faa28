"""GPU parity of the ABC chunk read (slot scores, softmax over the slots,
value read) against the FP64 token-serial oracle
(``oracle.abc_forward_fp64``), through the C ABI, on the normaliser and slot
states the GPU forward call writes.  Relative L2 <= 1e-2 for o and for the
slot weights p (bfloat16 storage of q, k, v, s, the states and the outputs).
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


def queries(inp, seed):
    r = np.random.default_rng(seed)
    return torch.from_numpy(r.standard_normal(tuple(inp.k.shape)).astype(np.float32)).to(torch.bfloat16)


def check(pkg, inp, q, scale, pool=False, what=""):
    """Every (batch row, head) against the oracle (``pool``: in worker
    processes, one per (row, head)), whole tensors and per slice."""
    o, p, _, _, _ = pkg.abc_forward(q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.s.cuda(), scale, emit_p=True)
    torch.cuda.synchronize()
    d = inp.f64()
    args = (q.to(torch.float64).numpy(), d["k"], d["v"], d["s"], scale)
    ref = oracle_pool.abc_read_all(*args) if pool else oracle.abc_forward_fp64(*args)
    got = {"o": o.detach().to(torch.float64).cpu().numpy(), "p": p.detach().to(torch.float64).cpu().numpy()}
    errs = {k: rel(got[k], ref[k]) for k in got}
    worst = per_row_head_max({k: (got[k], ref[k], 2) for k in got})
    print(what, " ".join(f"{k}={v:.3e}" for k, v in errs.items()), "| per (row, head) max:",
          " ".join(f"{k}={v[0]:.3e}@{v[1:]}" for k, v in worst.items()), flush=True)
    for key, e in errs.items():
        assert e <= TOL, f"{what} {key}: rel-L2 {e:.3e}"
        assert worst.get(key, (0.0,))[0] <= TOL, f"{what} {key}: {worst[key]}"
    return o, p


@pytest.mark.parametrize("shape", [(1, 64, 2, 64, 128), (2, 200, 1, 128, 128), (1, 1, 3, 128, 256),
                                   (1, 64 * 5 + 17, 2, 256, 256), (1, 190, 1, 256, 512)],
                         ids=lambda s: "x".join(map(str, s)))
def test_abc_read_parity(pkg, shape):
    B, T, H, K, V = shape
    inp = make_abc(990 + T, B=B, T=T, H=H, K=K, M=64, V=V)
    check(pkg, inp, queries(inp, 991 + T), K ** -0.5, what=f"abc read {shape}")


@pytest.mark.parametrize("shape", [(2, 127, 2, 128, 128), (1, 257, 1, 256, 512)], ids=lambda s: "x".join(map(str, s)))
def test_abc_read_32_slots(pkg, shape):
    """M = 32 slots (padded to 64 inside the kernel, the padding scored -inf):
    the whole forward, scan then read, against the oracle."""
    B, T, H, K, V = shape
    inp = make_abc(995 + T, B=B, T=T, H=H, K=K, M=32, V=V)
    check(pkg, inp, queries(inp, 996 + T), K ** -0.5, what=f"abc read M=32 {shape}")


def test_abc_read_benchmark_shape(pkg):
    """B=2, T=16384, H=4, K=256, M=64, V=512 against the oracle on every
    (batch row, head); deterministic run to run."""
    inp = make_config("abc_affine")
    q = queries(inp, 992)
    a = check(pkg, inp, q, 256 ** -0.5, pool=True, what="abc read abc_affine (all rows and heads)")
    o2, p2, _, _, _ = pkg.abc_forward(q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.s.cuda(), 256 ** -0.5, emit_p=True)
    assert torch.equal(a[0], o2) and torch.equal(a[1], p2)
