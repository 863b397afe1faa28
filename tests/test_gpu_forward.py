"""GPU tests of the whole forward step in one kernel (``gdr_chunk_forward``,
through the C ABI: chunk prepare, state scan and chunk output fused): its o,
g_cum, h, v_new and hT are the bits of ``gdr_chunk_prepare`` followed by
``gdr_state_scan_output`` on ragged packed rows (empty, one-token,
chunk-edge and multi-chunk sequences), dense rows, with and without h0,
without the optional outputs, with indexed states, at DV = 64 and 128, in a
batch of more rows than one launch holds; and the question_rows shape
against the FP64 oracle on every head (relative L2 1e-2 for bfloat16
storage, per sequence and head as well as whole)."""

import pytest
import torch

import oracle_pool
from parity import gate, per_sequence_max, rel
from workloads import make_config, make_gdr

pytestmark = pytest.mark.gpu

TOL = 1e-2
LENGTHS = [1, 63, 64, 65, 150, 0, 200, 129]


@pytest.fixture(scope="module")
def pkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_chunked_amd as p

    p.lib()
    return p


def cuda(inp):
    return [x.cuda() for x in (inp.q, inp.k, inp.v, inp.g, inp.beta)]


def two_calls(pkg, inp, scale, h0=None, **kw):
    q, k, v, g, b = cuda(inp)
    g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, b, inp.cu_seqlens)
    o, h, v_new, hT = pkg.gdr_state_scan_output(q, k, w, u, g_cum, scale, h0, inp.cu_seqlens, (64, 4, 2), **kw)
    return o, g_cum, h, v_new, hT


def fused(pkg, inp, scale, h0=None, **kw):
    q, k, v, g, b = cuda(inp)
    return pkg.gdr_chunk_forward(q, k, v, g, b, scale, h0, inp.cu_seqlens, **kw)


def assert_same(got, ref, what):
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "g_cum", "h", "v_new", "hT"), got, ref):
        if a is None or b is None:
            continue
        assert torch.equal(a, b), f"{what}: {name} differs (max |diff| {(a.float() - b.float()).abs().max().item():.3e})"


@pytest.mark.parametrize("DV", [128, 64])
@pytest.mark.parametrize("with_h0", [True, False])
def test_forward_equals_prepare_then_fused_scan(pkg, DV, with_h0):
    inp = make_gdr(700 + DV + with_h0, lengths=LENGTHS, H=3, DK=128, DV=DV, dtype=torch.bfloat16, varlen=True,
                   h0_std=0.1 if with_h0 else None)
    h0 = inp.h0.cuda() if with_h0 else None
    assert_same(fused(pkg, inp, 0.3, h0), two_calls(pkg, inp, 0.3, h0), f"DV={DV} h0={with_h0}")


def test_forward_dense_rows_and_optional_outputs(pkg):
    inp = make_gdr(741, lengths=[190, 190, 190], H=2, dtype=torch.bfloat16, varlen=False, h0_std=None)
    ref = two_calls(pkg, inp, 1.0)
    assert_same(fused(pkg, inp, 1.0), ref, "dense rows")
    o, g_cum, h, v_new, hT = fused(pkg, inp, 1.0, emit_g_cum=False, emit_h=False, emit_v_new=False, emit_final=False)
    assert g_cum is None and h is None and v_new is None and hT is None
    assert torch.equal(o, ref[0])


def test_forward_indexed_states(pkg):
    """Sequence n reads h0[idx[n]] and writes hT[idx[n]] of a pool, as the plain scan."""
    inp = make_gdr(751, lengths=[70, 0, 130, 64], H=2, dtype=torch.bfloat16, varlen=True, h0_std=0.1)
    idx = [3, 0, 5, 1]
    pool = torch.randn((6, 2, 128, 128), generator=torch.Generator().manual_seed(5)).cuda() * 0.1
    ref_pool, got_pool = pool.clone(), pool.clone()
    ref = two_calls(pkg, inp, 0.5, ref_pool, out={"hT": ref_pool}, state_indices=idx)
    got = fused(pkg, inp, 0.5, got_pool, out={"hT": got_pool}, state_indices=idx)
    assert_same(got[:4], ref[:4], "indexed states")
    assert torch.equal(got_pool, ref_pool)


def test_forward_many_rows(pkg):
    """More rows than one launch's work list (several launches in order)."""
    lengths = [(37 * i) % 200 + 1 for i in range(250)]
    inp = make_gdr(761, lengths=lengths, H=2, dtype=torch.bfloat16, varlen=True, h0_std=0.1)
    h0 = inp.h0.cuda()
    assert_same(fused(pkg, inp, 0.7, h0), two_calls(pkg, inp, 0.7, h0), "250 rows")


def test_forward_question_rows_against_oracle(pkg):
    """question_rows (24 packed sequences, 16 heads, 128 x 128): every head
    against the FP64 token recurrence; o, v_new, hT and the pre-chunk states,
    whole and per (sequence, head)."""
    inp = make_config("question_rows")
    h0 = inp.h0.cuda() if inp.h0 is not None else None
    o, g_cum, h, v_new, hT = fused(pkg, inp, inp.scale, h0)
    torch.cuda.synchronize()
    d = inp.f64()
    ref = oracle_pool.gdr_forward_all_heads(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                                            inp.scale)
    np64 = lambda t: t.detach().to(torch.float64).cpu().numpy()
    got = {"o": np64(o), "v_new": np64(v_new), "hT": np64(hT), "h": np64(h.transpose(-1, -2))}
    errs = {key: rel(got[key], ref[key]) for key in got}
    kinds = {"o": "token", "v_new": "token", "h": "chunk", "hT": "seq"}
    worst = per_sequence_max({k: (got[k], ref[k], kinds[k]) for k in kinds}, inp.cu_seqlens, ref["chunk_offsets"])
    gate(errs, worst, TOL, "question_rows forward (all 16 heads)")
