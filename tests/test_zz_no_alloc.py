"""The allocation-free segment summaries (gdr_segment_summaries_noalloc: the
half-segment workspace is the library's static scratch) against the entry
point with a caller workspace (gdr_segment_summaries_ws), through the C ABI:
the same kernels on the same data, so the outputs must be identical bit for
bit.  Two calls in a row, the second on a smaller problem, so the second
reuses the scratch the first left behind."""

import ctypes

import pytest
import torch

from workloads import make_gdr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_chunked_amd as p

    p.lib()
    return p


def prepared(pkg, seed, lengths, H, dtype=torch.bfloat16):
    inp = make_gdr(seed, lengths=lengths, H=H, DK=128, DV=128, dtype=dtype, varlen=True)
    k, v, g, b = (x.cuda() for x in (inp.k, inp.v, inp.g, inp.beta))
    g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, b, inp.cu_seqlens)
    return inp, k, w, u, g_cum


def with_workspace(pkg, inp, k, w, u, g_cum, P):
    """gdr_segment_summaries_ws with a caller workspace of the asked size."""
    B, L = pkg.binding, pkg.lib()
    p = B.Problem(k, 128, inp.cu_seqlens)
    n = p.N * P
    ss = torch.empty((n, p.H, 128, 128), dtype=torch.float32, device=k.device)
    st = torch.empty((n, p.H, 128, 128), dtype=torch.float32, device=k.device)
    ws_bytes = int(L.gdr_segment_summaries_workspace_size(p.ref, P))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=k.device)
    B._check(L.gdr_segment_summaries_ws(p.ref, None, P, B._ptr(k), B._ptr(w), B._ptr(u), B._ptr(g_cum), B._ptr(ss),
                                        B._ptr(st), B._ptr(ws), ws_bytes, B._stream()), "gdr_segment_summaries_ws")
    return ss, st, ws_bytes


def without_allocation(pkg, inp, k, w, u, g_cum, P):
    """gdr_segment_summaries_noalloc into preallocated outputs."""
    B, L = pkg.binding, pkg.lib()
    p = B.Problem(k, 128, inp.cu_seqlens)
    n = p.N * P
    ss = torch.full((n, p.H, 128, 128), float("nan"), dtype=torch.float32, device=k.device)
    st = torch.full((n, p.H, 128, 128), float("nan"), dtype=torch.float32, device=k.device)
    B._check(L.gdr_segment_summaries_noalloc(p.ref, None, P, B._ptr(k), B._ptr(w), B._ptr(u), B._ptr(g_cum),
                                             B._ptr(ss), B._ptr(st), B._stream()), "gdr_segment_summaries_noalloc")
    return ss, st


def test_noalloc_summaries_match_caller_workspace_twice(pkg):
    cases = [(881, [3000, 1000], 4, 8), (882, [700], 2, 4)]  # the second call is the smaller one
    for seed, lengths, H, P in cases:
        inp, k, w, u, g_cum = prepared(pkg, seed, lengths, H)
        ref_ss, ref_st, ws_bytes = with_workspace(pkg, inp, k, w, u, g_cum, P)
        assert ws_bytes > 0, "the half-segment form (with workspace) applies to this problem"
        ss, st = without_allocation(pkg, inp, k, w, u, g_cum, P)
        torch.cuda.synchronize()
        print(f"lengths {lengths} H={H} P={P}: workspace {ws_bytes} bytes", flush=True)
        assert torch.equal(ss, ref_ss), f"seg_state differs ({lengths}, P={P})"
        assert torch.equal(st, ref_st), f"seg_trans differs ({lengths}, P={P})"


def test_noalloc_direct_form_and_binding(pkg):
    """A problem the direct form serves (float32 storage: no workspace) and
    the Python binding's wrapper of the same call."""
    inp, k, w, u, g_cum = prepared(pkg, 883, [500, 64, 1], 2, dtype=torch.float32)
    ref = pkg.gdr_segment_summaries(k, w, u, g_cum, 3, inp.cu_seqlens)
    got = pkg.binding.gdr_segment_summaries_noalloc(k, w, u, g_cum, 3, inp.cu_seqlens)
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
