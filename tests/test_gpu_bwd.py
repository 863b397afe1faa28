"""GPU parity of the reverse (gradient) state recurrence against the FP64
oracle (``oracle.gdr_backward_fp64``), through the C ABI: the boundary
gradients dh, the write-vector gradient and the initial-state gradient, at
relative L2 <= 1e-2 (bfloat16 storage), plus bit-identity of packed and dense
rows and run to run.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
from parity import gate, per_sequence_max, rel
from workloads import make_config, make_gdr

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def pkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_chunked_amd as p

    p.lib()
    return p


def grads(inp, seed, with_dhT=True):
    """Seeded upstream gradients: dO in the storage dtype, dhT in float32."""
    r = np.random.default_rng(seed)
    B, T, H, DV = inp.v.shape
    dO = torch.from_numpy(r.standard_normal((B, T, H, DV))).to(torch.float32).to(inp.v.dtype)
    dhT = torch.from_numpy(0.1 * r.standard_normal((inp.N, H, inp.DK, DV))).to(torch.float32) if with_dhT else None
    return dO, dhT


def run_bwd(pkg, inp, dO, dhT, scale, state_layout="kv"):
    q, k, v, g, b = (x.cuda() for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    cu = inp.cu_seqlens
    g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, b, cu)
    dO_d = dO.cuda()
    dvl = pkg.gdr_chunk_dv_local(q, k, g_cum, dO_d, scale, cu)
    dhT_d = None
    if dhT is not None:
        dhT_d = dhT.cuda() if state_layout == "kv" else dhT.transpose(-1, -2).contiguous().cuda()
    dh, dv, dh0 = pkg.gdr_state_scan_bwd(q, k, w, g_cum, dO_d, dvl, dhT_d, scale, cu, state_layout=state_layout)
    torch.cuda.synchronize()
    if state_layout == "vk":
        dh0 = dh0.transpose(-1, -2)
    return {"dh": dh, "dv": dv, "dh0": dh0, "dvl": dvl}


def check(pkg, inp, dO, dhT, scale, state_layout="kv", what=""):
    """Every head against the oracle (a pool of worker processes over groups
    of heads for the named workloads), whole tensors and per (sequence, head)."""
    r = run_bwd(pkg, inp, dO, dhT, scale, state_layout)
    d = inp.f64()
    args = (d["q"], d["k"], d["g"], d["beta"], dO.to(torch.float64).numpy(),
            None if dhT is None else dhT.to(torch.float64).numpy(), d["cu_seqlens"], scale)
    ref = oracle.gdr_backward_fp64(*args) if inp.name == "custom" else oracle_pool.gdr_backward_all_heads(*args)

    def np64(t):
        return t.detach().to(torch.float64).cpu().numpy()

    got = {"dh": np.swapaxes(np64(r["dh"]), -1, -2), "dv_new": np64(r["dv"]), "dh0": np64(r["dh0"])}
    errs = {k: rel(got[k], ref[k]) for k in got}
    kinds = {"dh": "chunk", "dv_new": "token", "dh0": "seq"}
    worst = per_sequence_max({k: (got[k], ref[k], kinds[k]) for k in kinds}, d["cu_seqlens"], ref["chunk_offsets"])
    gate(errs, worst, TOL, what)
    return r


CASES = [
    (torch.bfloat16, 128, 128, [130, 1, 64, 200, 65], 0.5),
    (torch.bfloat16, 64, 128, [257, 3], 1.0),
    (torch.bfloat16, 128, 64, [100, 128], 0.25),
    (torch.bfloat16, 64, 64, [63, 0, 191], 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"dk{c[1]}-dv{c[2]}-L{len(c[3])}")
def test_backward_parity_shapes(pkg, case):
    dt, dk, dv, lengths, scale = case
    inp = make_gdr(840 + dk + dv + len(lengths), lengths=lengths, H=2, DK=dk, DV=dv, dtype=dt, varlen=True)
    dO, dhT = grads(inp, 841)
    check(pkg, inp, dO, dhT, scale, what=f"bwd dk{dk} dv{dv}")


def test_backward_no_final_gradient_and_vk_layout(pkg):
    inp = make_gdr(850, lengths=[150, 70], H=3, DK=128, DV=128, dtype=torch.bfloat16, varlen=True)
    dO, dhT = grads(inp, 851)
    check(pkg, inp, dO, None, 1.0, what="bwd no dhT")
    check(pkg, inp, dO, dhT, 1.0, state_layout="vk", what="bwd vk")


def test_backward_question_rows_workload(pkg):
    inp = make_config("question_rows")
    dO, dhT = grads(inp, 852)
    check(pkg, inp, dO, dhT, 1.0, what="bwd question_rows (all 16 heads)")


def test_backward_long_state_h1(pkg):
    inp = make_config("long_state_h1")
    dO, dhT = grads(inp, 853)
    check(pkg, inp, dO, dhT, 1.0, what="bwd long_state_h1")


def test_backward_packed_equals_dense_and_deterministic(pkg):
    dense = make_gdr(860, B=3, T=150, H=2, DK=128, DV=128, dtype=torch.bfloat16, varlen=False)
    packed = make_gdr(0, lengths=[150, 150, 150], H=2, DK=128, DV=128, dtype=torch.bfloat16, varlen=True)
    packed.q, packed.k, packed.v = (x.reshape(1, 450, 2, 128) for x in (dense.q, dense.k, dense.v))
    packed.g, packed.beta = (x.reshape(1, 450, 2) for x in (dense.g, dense.beta))
    dO, dhT = grads(dense, 861)
    a = run_bwd(pkg, dense, dO, dhT, 1.0)
    b = run_bwd(pkg, packed, dO.reshape(1, 450, 2, 128), dhT, 1.0)
    assert torch.equal(a["dh"], b["dh"])
    assert torch.equal(a["dv"].reshape(-1), b["dv"].reshape(-1))
    assert torch.equal(a["dh0"], b["dh0"])
    c = run_bwd(pkg, dense, dO, dhT, 1.0)
    for key in a:
        assert torch.equal(a[key], c[key]), key
