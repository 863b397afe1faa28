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


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def queries(inp, seed):
    r = np.random.default_rng(seed)
    return torch.from_numpy(r.standard_normal(tuple(inp.k.shape)).astype(np.float32)).to(torch.bfloat16)


def check(pkg, inp, q, scale, batches=None, heads=None, what=""):
    o, p, _, _, _ = pkg.abc_forward(q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.s.cuda(), scale, emit_p=True)
    torch.cuda.synchronize()
    d = inp.f64()
    ref = oracle.abc_forward_fp64(q.to(torch.float64).numpy(), d["k"], d["v"], d["s"], scale,
                                  batches=batches, heads=heads)

    def pick(t):
        x = t.detach().to(torch.float64).cpu().numpy()
        if batches is not None:
            x = np.take(x, batches, axis=0)
        if heads is not None:
            x = np.take(x, heads, axis=2)
        return x

    errs = {"o": rel(pick(o), ref["o"]), "p": rel(pick(p), ref["p"])}
    print(what, " ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)
    for key, e in errs.items():
        assert e <= TOL, f"{what} {key}: rel-L2 {e:.3e}"
    return o, p


@pytest.mark.parametrize("shape", [(1, 64, 2, 64, 128), (2, 200, 1, 128, 128), (1, 1, 3, 128, 256),
                                   (1, 64 * 5 + 17, 2, 256, 256), (1, 190, 1, 256, 512)],
                         ids=lambda s: "x".join(map(str, s)))
def test_abc_read_parity(pkg, shape):
    B, T, H, K, V = shape
    inp = make_abc(990 + T, B=B, T=T, H=H, K=K, M=64, V=V)
    check(pkg, inp, queries(inp, 991 + T), K ** -0.5, what=f"abc read {shape}")


def test_abc_read_benchmark_shape(pkg):
    """B=2, T=16384, H=4, K=256, M=64, V=512 against the oracle on batch row 0,
    heads 1 and 2; deterministic run to run."""
    inp = make_config("abc_affine")
    q = queries(inp, 992)
    a = check(pkg, inp, q, 256 ** -0.5, batches=[0], heads=[1, 2], what="abc read abc_affine b0 h1,2")
    o2, p2, _, _, _ = pkg.abc_forward(q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.s.cuda(), 256 ** -0.5, emit_p=True)
    assert torch.equal(a[0], o2) and torch.equal(a[1], p2)
