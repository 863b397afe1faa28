"""GPU tests that the kernels write nothing past their output tensors.

The token-row outputs (o, v_new, w, u, dv_local, the gradient of v_new, the
per-channel-decay kg, the ABC read's o and p) of the last sequence end
inside a 64-token chunk; the kernels issue the
whole chunk's stores and rely on the buffer range check to drop the rows
past the tensor's last token.  Each output here is a view at the start of a
larger buffer whose tail holds a sentinel pattern: after the call the tail
must be untouched and the view must equal the output of the ordinary call
(exact-size tensors from the binding), bit for bit.  The same for the
per-chunk states h and dh, whose last chunk is also the buffer's last."""

import ctypes

import pytest
import torch

from workloads import make_gdr

pytestmark = pytest.mark.gpu

LENGTHS = [70, 33, 100]  # the last sequence ends 36 rows into its second chunk
SENTINEL = 0x7FC1        # a bfloat16 NaN payload no kernel writes
GUARD = 1 << 16          # elements of sentinel after each view


@pytest.fixture(scope="module")
def pkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_chunked_amd as p

    p.lib()
    return p


def guarded(like):
    """A view shaped like `like` at the start of a buffer with a sentinel tail."""
    n = like.numel()
    buf = torch.empty(n + GUARD, dtype=like.dtype, device=like.device)
    buf.view(torch.int16).fill_(SENTINEL)
    return buf, buf[:n].view(like.shape)


def tail_intact(buf, n):
    torch.cuda.synchronize()
    t = buf[n:].view(torch.int16)
    return bool((t == SENTINEL).all().item())


@pytest.fixture(scope="module")
def problem(pkg):
    inp = make_gdr(41, lengths=LENGTHS, H=2, DK=128, DV=128, varlen=True, h0_std=0.1)
    d = {n: getattr(inp, n).cuda() for n in ("q", "k", "v", "g", "beta", "h0")}
    d["cu"] = inp.cu_seqlens
    d["scale"] = inp.scale
    return d


def test_prepare_stays_in_bounds(pkg, problem):
    d = problem
    B, L = pkg.binding, pkg.lib()
    g_ref, w_ref, u_ref = pkg.gdr_chunk_prepare(d["k"], d["v"], d["g"], d["beta"], d["cu"])
    wb, w = guarded(w_ref)
    ub, u = guarded(u_ref)
    g_cum = torch.empty_like(g_ref)
    P = B.Problem(d["k"], d["v"].shape[-1], d["cu"])
    B._check(L.gdr_chunk_prepare(P.ref, B._ptr(d["k"]), B._ptr(d["v"]), B._ptr(d["g"]), B._ptr(d["beta"]),
                                 B._ptr(g_cum), B._ptr(w), B._ptr(u), None), "prepare")
    assert tail_intact(wb, w.numel()) and tail_intact(ub, u.numel())
    assert torch.equal(w, w_ref) and torch.equal(u, u_ref) and torch.equal(g_cum, g_ref)


def test_fused_scan_output_stays_in_bounds(pkg, problem):
    d = problem
    B, L = pkg.binding, pkg.lib()
    g_cum, w, u = pkg.gdr_chunk_prepare(d["k"], d["v"], d["g"], d["beta"], d["cu"])
    o_ref, h_ref, vn_ref, hT_ref = pkg.gdr_state_scan_output(d["q"], d["k"], w, u, g_cum, d["scale"], d["h0"], d["cu"])
    ob, o = guarded(o_ref)
    hb, h = guarded(h_ref)
    vb, vn = guarded(vn_ref)
    hT = torch.empty_like(hT_ref)
    P = B.Problem(d["k"], d["v"].shape[-1], d["cu"])
    B._check(L.gdr_state_scan_output(P.ref, None, None, B._ptr(d["q"]), B._ptr(d["k"]), B._ptr(w), B._ptr(u),
                                     B._ptr(g_cum), B._ptr(d["h0"]), ctypes.c_float(d["scale"]), B._ptr(h),
                                     B._ptr(vn), B._ptr(hT), B._ptr(o), None), "scan + output")
    assert tail_intact(ob, o.numel()), "o: rows past the last token were written"
    assert tail_intact(hb, h.numel()), "h: past the last chunk was written"
    assert tail_intact(vb, vn.numel()), "v_new: rows past the last token were written"
    for a, b in ((o, o_ref), (h, h_ref), (vn, vn_ref), (hT, hT_ref)):
        assert torch.equal(a, b)


def test_chunk_output_stays_in_bounds(pkg, problem):
    d = problem
    B, L = pkg.binding, pkg.lib()
    g_cum, w, u = pkg.gdr_chunk_prepare(d["k"], d["v"], d["g"], d["beta"], d["cu"])
    h, v_new, _ = pkg.gdr_state_scan(d["k"], w, u, g_cum, d["h0"], d["cu"])
    o_ref = pkg.gdr_chunk_output(d["q"], d["k"], v_new, h, g_cum, d["scale"], d["cu"])
    ob, o = guarded(o_ref)
    P = B.Problem(d["k"], d["v"].shape[-1], d["cu"])
    B._check(L.gdr_chunk_output(P.ref, B._ptr(d["q"]), B._ptr(d["k"]), B._ptr(v_new), B._ptr(h), B._ptr(g_cum),
                                ctypes.c_float(d["scale"]), B._ptr(o), None), "output")
    assert tail_intact(ob, o.numel()), "o: rows past the last token were written"
    assert torch.equal(o, o_ref)


def test_reverse_pass_stays_in_bounds(pkg, problem):
    d = problem
    B, L = pkg.binding, pkg.lib()
    g_cum, w, u = pkg.gdr_chunk_prepare(d["k"], d["v"], d["g"], d["beta"], d["cu"])
    gen = torch.Generator(device="cuda").manual_seed(5)
    dO = torch.randn(d["v"].shape, generator=gen, device="cuda").to(d["v"].dtype)
    P = B.Problem(d["k"], d["v"].shape[-1], d["cu"])
    dvl_ref = torch.empty_like(dO)
    B._check(L.gdr_chunk_dv_local(P.ref, B._ptr(d["q"]), B._ptr(d["k"]), B._ptr(g_cum), B._ptr(dO),
                                  ctypes.c_float(d["scale"]), B._ptr(dvl_ref), None), "dv_local")
    lb, dvl = guarded(dvl_ref)
    B._check(L.gdr_chunk_dv_local(P.ref, B._ptr(d["q"]), B._ptr(d["k"]), B._ptr(g_cum), B._ptr(dO),
                                  ctypes.c_float(d["scale"]), B._ptr(dvl), None), "dv_local")
    assert tail_intact(lb, dvl.numel()), "dv_local: rows past the last token were written"
    assert torch.equal(dvl, dvl_ref)
    nt = pkg.gdr_num_chunks(d["k"], d["v"].shape[-1], d["cu"])
    H, DK, DV = d["k"].shape[2], d["k"].shape[3], d["v"].shape[3]
    dh_ref = torch.empty((nt, H, DV, DK), dtype=d["k"].dtype, device="cuda")
    dv_ref = torch.empty_like(dO)

    def bwd(dh, dv):
        B._check(L.gdr_state_scan_bwd(P.ref, B._ptr(d["q"]), B._ptr(d["k"]), B._ptr(w), B._ptr(g_cum), B._ptr(dO),
                                      B._ptr(dvl_ref), None, ctypes.c_float(d["scale"]), B._ptr(dh), B._ptr(dv),
                                      None, None), "reverse scan")

    bwd(dh_ref, dv_ref)
    hb, dh = guarded(dh_ref)
    vb, dv = guarded(dv_ref)
    bwd(dh, dv)
    assert tail_intact(hb, dh.numel()), "dh: past the last chunk was written"
    assert tail_intact(vb, dv.numel()), "dv_new gradient: rows past the last token were written"
    assert torch.equal(dh, dh_ref) and torch.equal(dv, dv_ref)


def test_per_channel_decay_stays_in_bounds(pkg):
    """kda_chunk_prepare's w, u, kg and kda_chunk_output's o on the same
    ragged batch, per-channel log decays."""
    inp = make_gdr(43, lengths=LENGTHS, H=2, DK=128, DV=128, varlen=True, gates="logsigmoid_channels", h0_std=0.1)
    q, k, v, g, beta, h0 = (getattr(inp, n).cuda() for n in ("q", "k", "v", "g", "beta", "h0"))
    cu = inp.cu_seqlens
    B, L = pkg.binding, pkg.lib()
    P = B.Problem(k, v.shape[-1], cu)
    g_ref, w_ref, u_ref, kg_ref, dec_ref = pkg.kda_chunk_prepare(k, v, g, beta, cu)
    (wb, w), (ub, u), (kb, kg) = guarded(w_ref), guarded(u_ref), guarded(kg_ref)
    g_cum, dec = torch.empty_like(g_ref), torch.empty_like(dec_ref)
    B._check(L.kda_chunk_prepare(P.ref, B._ptr(k), B._ptr(v), B._ptr(g), B._ptr(beta), B._ptr(g_cum), B._ptr(w),
                                 B._ptr(u), B._ptr(kg), B._ptr(dec), None), "kda prepare")
    assert tail_intact(wb, w.numel()) and tail_intact(ub, u.numel()) and tail_intact(kb, kg.numel())
    assert torch.equal(w, w_ref) and torch.equal(u, u_ref) and torch.equal(kg, kg_ref)
    h, v_new, _ = pkg.kda_state_scan(kg_ref, w_ref, u_ref, dec_ref, h0, cu)
    o_ref = pkg.kda_chunk_output(q, k, v_new, h, g_ref, inp.scale, cu)
    ob, o = guarded(o_ref)
    B._check(L.kda_chunk_output(P.ref, B._ptr(q), B._ptr(k), B._ptr(v_new), B._ptr(h), B._ptr(g_ref),
                                ctypes.c_float(inp.scale), B._ptr(o), None), "kda output")
    assert tail_intact(ob, o.numel()), "o: rows past the last token were written"
    assert torch.equal(o, o_ref)


def test_abc_read_stays_in_bounds(pkg):
    """The ABC read's o (and slot weights p) of a sequence that ends 17 rows
    into its last chunk."""
    from workloads import make_abc

    inp = make_abc(47, B=1, T=64 * 2 + 17, H=2, K=128, M=64, V=128)
    k, v, s = inp.k.cuda(), inp.v.cuda(), inp.s.cuda()
    gen = torch.Generator(device="cuda").manual_seed(9)
    q = torch.randn(k.shape, generator=gen, device="cuda").to(k.dtype)
    z, hk, hv, _, _ = pkg.abc_affine_scan(k, v, s, emit_z=True, emit_final=False)
    o_ref, p_ref = pkg.abc_chunk_output(q, k, v, s, z, hk, hv, 1.0, emit_p=True)
    ob, o = guarded(o_ref)
    pb, p = guarded(p_ref)
    B, L = pkg.binding, pkg.lib()
    pr = B.abc_problem(1, k.shape[1], 2, 128, 64, 128, B.GDR_BF16)
    B._check(L.abc_chunk_output(ctypes.byref(pr), B._ptr(q), B._ptr(k), B._ptr(v), B._ptr(s), B._ptr(z), B._ptr(hk),
                                B._ptr(hv), ctypes.c_float(1.0), B._ptr(o), B._ptr(p), None), "abc read")
    assert tail_intact(ob, o.numel()), "o: rows past the last token were written"
    assert tail_intact(pb, p.numel()), "p: rows past the last token were written"
    assert torch.equal(o, o_ref) and torch.equal(p, p_ref)
