"""GPU tests of the state scan with the chunk output fused
(``gdr_state_scan_output``, through the C ABI): its o, h, v_new and hT are
the bits of ``gdr_state_scan`` followed by ``gdr_chunk_output`` on every
fused tile and width, on ragged packed rows (empty, one-token, chunk-edge
and multi-chunk sequences) and dense rows, without h / v_new, with indexed
states and in the segmented final pass; problems without a fused kernel run
the two calls; and the question_rows shape against the FP64 oracle
(relative L2 1e-2 for bfloat16 storage)."""

import numpy as np
import pytest
import torch

import oracle
from parity import gate, per_sequence_max
from workloads import make_config, make_gdr

pytestmark = pytest.mark.gpu

TOL = 1e-2
LENGTHS = [1, 63, 64, 65, 150, 0, 200]


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


def prepared(pkg, inp):
    q, k, v, g, b = (x.cuda() for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, b, inp.cu_seqlens)
    return q, k, w, u, g_cum


def two_calls(pkg, q, k, w, u, g_cum, h0, cu, scale, tile=None, **kw):
    h, v_new, hT = pkg.gdr_state_scan(k, w, u, g_cum, h0, cu, tile, **kw)
    o = pkg.gdr_chunk_output(q, k, v_new, h, g_cum, scale, cu)
    return o, h, v_new, hT


def assert_same(got, ref, what):
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "h", "v_new", "hT"), got, ref):
        if a is None:
            continue
        assert torch.equal(a, b), f"{what}: {name} differs (max |diff| {(a.float() - b.float()).abs().max().item():.3e})"


@pytest.mark.parametrize("DK,DV", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("tile", [None, (64, 4, 2), (128, 4, 2)])
def test_fused_equals_scan_then_output(pkg, DK, DV, tile):
    if tile is not None and tile[0] > DV:
        pytest.skip("the tile's columns exceed DV")
    inp = make_gdr(900 + DK + DV, lengths=LENGTHS, H=2, DK=DK, DV=DV, dtype=torch.bfloat16, varlen=True, h0_std=0.1)
    q, k, w, u, g_cum = prepared(pkg, inp)
    h0, cu = inp.h0.cuda(), inp.cu_seqlens
    ref = two_calls(pkg, q, k, w, u, g_cum, h0, cu, 0.3)
    got = pkg.gdr_state_scan_output(q, k, w, u, g_cum, 0.3, h0, cu, tile)
    assert_same(got, ref, f"{DK}x{DV} tile {tile}")


def test_fused_dense_rows_and_without_h_or_v_new(pkg):
    inp = make_gdr(931, lengths=[190, 190, 190], H=3, dtype=torch.bfloat16, varlen=False, h0_std=None)
    q, k, w, u, g_cum = prepared(pkg, inp)
    ref = two_calls(pkg, q, k, w, u, g_cum, None, None, 1.0)
    got = pkg.gdr_state_scan_output(q, k, w, u, g_cum, 1.0)
    assert_same(got, ref, "dense rows")
    o, h, v_new, hT = pkg.gdr_state_scan_output(q, k, w, u, g_cum, 1.0, emit_h=False, emit_v_new=False)
    assert h is None and v_new is None
    assert_same((o, None, None, hT), ref, "dense rows, no h / v_new")


def test_fused_indexed_states(pkg):
    inp = make_gdr(941, lengths=[70, 0, 130, 5], H=2, dtype=torch.bfloat16, varlen=True, h0_std=0.2)
    q, k, w, u, g_cum = prepared(pkg, inp)
    cu = inp.cu_seqlens
    idx = [3, 0, 5, 1]
    pool = torch.randn(7, 2, 128, 128, device="cuda") * 0.1
    for n, i in enumerate(idx):
        pool[i] = inp.h0[n].cuda()
    before = pool.clone()
    ref = two_calls(pkg, q, k, w, u, g_cum, inp.h0.cuda(), cu, 0.5)
    o, h, v_new, _ = pkg.gdr_state_scan_output(q, k, w, u, g_cum, 0.5, pool, cu, out={"hT": pool}, state_indices=idx)
    assert_same((o, h, v_new, None), ref, "indexed states")
    for n, i in enumerate(idx):
        assert torch.equal(pool[i], ref[3][n]), f"pool row {i} (sequence {n})"
    for i in (2, 4, 6):
        assert torch.equal(pool[i], before[i]), f"untouched pool row {i}"


@pytest.mark.parametrize("P", [1, 4, 7])
def test_fused_segmented_final_pass(pkg, P):
    inp = make_gdr(951, lengths=[1000, 300], H=2, dtype=torch.bfloat16, varlen=True, h0_std=0.1)
    q, k, w, u, g_cum = prepared(pkg, inp)
    cu = inp.cu_seqlens
    ss, st = pkg.gdr_segment_summaries(k, w, u, g_cum, P, cu)
    si, _ = pkg.gdr_segment_compose(k, 128, ss, st, P, inp.h0.cuda(), cu)
    ref = two_calls(pkg, q, k, w, u, g_cum, None, cu, 0.25, None, n_segments=P, seg_init=si)
    got = pkg.gdr_state_scan_output(q, k, w, u, g_cum, 0.25, None, cu, None, n_segments=P, seg_init=si)
    assert_same(got, ref, f"segmented P={P}")


def test_unfused_problems_run_the_two_calls(pkg):
    # an explicit tile without a fused form, float32 storage, and DK = 256
    for dtype, DK, tile in ((torch.bfloat16, 128, (32, 2, 2)), (torch.float32, 128, None), (torch.bfloat16, 256, None)):
        inp = make_gdr(961, lengths=[70, 130], H=2, DK=DK, DV=128, dtype=dtype, varlen=True, h0_std=0.1)
        q, k, w, u, g_cum = prepared(pkg, inp)
        h0, cu = inp.h0.cuda(), inp.cu_seqlens
        ref = two_calls(pkg, q, k, w, u, g_cum, h0, cu, 0.7, tile)
        got = pkg.gdr_state_scan_output(q, k, w, u, g_cum, 0.7, h0, cu, tile)
        assert_same(got, ref, f"{dtype} DK={DK} tile {tile}")
        with pytest.raises(pkg.GdrError):
            pkg.gdr_state_scan_output(q, k, w, u, g_cum, 0.7, h0, cu, tile, emit_h=False)


def test_fused_question_rows_against_oracle(pkg):
    inp = make_config("question_rows")
    q, k, w, u, g_cum = prepared(pkg, inp)
    h0 = None if inp.h0 is None else inp.h0.cuda()
    ref2 = two_calls(pkg, q, k, w, u, g_cum, h0, inp.cu_seqlens, inp.scale)
    got = pkg.gdr_state_scan_output(q, k, w, u, g_cum, inp.scale, h0, inp.cu_seqlens)
    assert_same(got, ref2, "question_rows")
    again = pkg.gdr_state_scan_output(q, k, w, u, g_cum, inp.scale, h0, inp.cu_seqlens)
    assert_same(again, got, "question_rows run to run")
    d = inp.f64()
    ref = oracle.gdr_recurrent_fp64(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], inp.scale)
    o, h, v_new, hT = (t.detach().to(torch.float64).cpu().numpy() for t in got)
    got = {"o": o, "v_new": v_new, "hT": hT, "h": h.transpose(0, 1, 3, 2)}
    errs = {k: rel(got[k], ref[k]) for k in got}
    kinds = {"o": "token", "v_new": "token", "h": "chunk", "hT": "seq"}
    worst = per_sequence_max({k: (got[k], ref[k], kinds[k]) for k in kinds}, d["cu_seqlens"], ref["chunk_offsets"])
    gate(errs, worst, TOL, "fused question_rows")


@pytest.mark.parametrize("name", ["question_rows", "kda_question_rows"])
def test_dense_and_full_forms_bit_identical(pkg, monkeypatch, name):
    """The scan's dense form (three workgroups per CU: operands read step by
    step, staging in the chunk tiles' place) and its full form give the same
    bits: plain scan and fused scan + output on question rows, and the
    per-channel-decay scan."""
    inp = make_config(name)
    q, k, v, g, b = (x.cuda() for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    h0 = inp.h0.cuda()
    cu = inp.cu_seqlens
    outs = {}
    for form in ("0", "1"):
        monkeypatch.setenv("GDR_SCAN_DENSE", form)
        if name == "question_rows":
            g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, b, cu)
            scan = pkg.gdr_state_scan(k, w, u, g_cum, h0, cu)
            fused = pkg.gdr_state_scan_output(q, k, w, u, g_cum, inp.scale, h0, cu)
            outs[form] = list(scan) + list(fused)
        else:
            g_cum, w, u, kg, decay = pkg.kda_chunk_prepare(k, v, g, b, cu)
            outs[form] = list(pkg.kda_state_scan(kg, w, u, decay, h0, cu))
        torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip(outs["0"], outs["1"])):
        assert torch.equal(x, y), f"{name}: output {i} differs between the dense and the full form"
