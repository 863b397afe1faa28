"""Indexed state pools and graph capture, through the C ABI.

* Pools (kev pull request #259, "Not covered": question rows whose cached
  states are addressed by index): sequence n reads h0[idx[n]] and writes
  hT[idx[n]]; the results must be bit-identical to the same scan run on the
  gathered states, and every other pool entry must stay untouched, also when
  the update is in place (h0 and hT the same buffer).
* Graphs (the same page's "Test plan": graphs match eager): the whole forward
  step (prepare, scan with an in-place pool, output; also with the scan and
  output fused) captured once in a HIP graph and replayed several times, with
  eager work and synchronisation in between, must give bit for bit what the
  eager steps give.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import make_gdr

pytestmark = pytest.mark.gpu


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


IDX = [7, 2, 4, 0, 8]
POOL = 9


def _inputs(layout="kv"):
    inp = make_gdr(820, lengths=[130, 17, 64, 200, 1], H=4, DK=128, DV=128, dtype=torch.bfloat16, varlen=True,
                   h0_std=0.1)
    rng = np.random.default_rng(821)
    pool = torch.from_numpy(rng.standard_normal((POOL, 4, 128, 128)).astype(np.float32))
    for n, i in enumerate(IDX):
        pool[i] = inp.h0[n]
    if layout == "vk":
        pool = pool.transpose(-1, -2).contiguous()
    return inp, pool


def _prepared(pkg, inp):
    k, v, g, b = (x.cuda() for x in (inp.k, inp.v, inp.g, inp.beta))
    g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, b, inp.cu_seqlens)
    return k, w, u, g_cum


@pytest.mark.parametrize("layout", ["kv", "vk"])
def test_pool_gather_scatter(pkg, layout):
    inp, pool = _inputs(layout)
    k, w, u, g_cum = _prepared(pkg, inp)
    h0 = inp.h0 if layout == "kv" else inp.h0.transpose(-1, -2).contiguous()
    h_r, v_r, hT_r = pkg.gdr_state_scan(k, w, u, g_cum, h0.cuda(), inp.cu_seqlens, state_layout=layout)
    sentinel = torch.full_like(pool, 123.0).cuda()
    h, v_new, hT = pkg.gdr_state_scan(k, w, u, g_cum, pool.cuda(), inp.cu_seqlens, state_layout=layout,
                                      out={"hT": sentinel}, state_indices=IDX)
    torch.cuda.synchronize()
    assert torch.equal(h, h_r) and torch.equal(v_new, v_r)
    for n, i in enumerate(IDX):
        assert torch.equal(hT[i], hT_r[n]), (n, i)
    untouched = [i for i in range(POOL) if i not in IDX]
    assert torch.equal(hT[untouched].cpu(), torch.full_like(pool[untouched], 123.0))
    # and the scattered states are the oracle's final states
    d = inp.f64()
    ref = oracle.gdr_recurrent_fp64(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], inp.scale)
    got = hT[IDX].cpu().to(torch.float64)
    if layout == "vk":
        got = got.transpose(-1, -2)
    e = rel(got.numpy(), ref["hT"])
    print(f"pool {layout} hT rel-L2 {e:.3e}", flush=True)
    assert e <= 1e-2


def test_pool_in_place(pkg):
    inp, pool = _inputs()
    k, w, u, g_cum = _prepared(pkg, inp)
    _, _, hT_r = pkg.gdr_state_scan(k, w, u, g_cum, inp.h0.cuda(), inp.cu_seqlens)
    p = pool.cuda()
    pkg.gdr_state_scan(k, w, u, g_cum, p, inp.cu_seqlens, out={"hT": p}, state_indices=IDX)
    torch.cuda.synchronize()
    for n, i in enumerate(IDX):
        assert torch.equal(p[i], hT_r[n]), (n, i)
    untouched = [i for i in range(POOL) if i not in IDX]
    assert torch.equal(p[untouched].cpu(), pool[untouched])


@pytest.mark.parametrize("fused", [False, True])
def test_graph_capture_matches_eager(pkg, fused):
    inp, pool = _inputs()
    q, k, v, g, b = (x.cuda() for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    cu = inp.cu_seqlens
    nt = pkg.gdr_num_chunks(k, 128, cu)

    def buffers():
        return {"g_cum": torch.empty(g.shape, dtype=torch.float32, device="cuda"), "w": torch.empty_like(k),
                "u": torch.empty_like(v), "h": torch.empty((nt, 4, 128, 128), dtype=k.dtype, device="cuda"),
                "v_new": torch.empty_like(v), "o": torch.empty_like(v), "pool": pool.clone().cuda()}

    def step(bf):
        # through the C ABI with preallocated outputs, so a captured step allocates nothing
        B, L = pkg.binding, pkg.lib()
        P = B.Problem(k, 128, cu)
        s = B._stream(torch.cuda.current_stream())
        B._check(L.gdr_chunk_prepare(P.ref, B._ptr(k), B._ptr(v), B._ptr(g), B._ptr(b), B._ptr(bf["g_cum"]),
                                     B._ptr(bf["w"]), B._ptr(bf["u"]), s), "prepare")
        Pp = B.Problem(k, 128, cu, "kv", IDX, POOL)
        if fused:  # the state scan with the chunk output fused
            B._check(L.gdr_state_scan_output(Pp.ref, None, None, B._ptr(q), B._ptr(k), B._ptr(bf["w"]),
                                             B._ptr(bf["u"]), B._ptr(bf["g_cum"]), B._ptr(bf["pool"]),
                                             float(inp.scale), B._ptr(bf["h"]), B._ptr(bf["v_new"]),
                                             B._ptr(bf["pool"]), B._ptr(bf["o"]), s), "scan + output")
            return
        B._check(L.gdr_state_scan(Pp.ref, None, None, B._ptr(k), B._ptr(bf["w"]), B._ptr(bf["u"]),
                                  B._ptr(bf["g_cum"]), B._ptr(bf["pool"]), B._ptr(bf["h"]), B._ptr(bf["v_new"]),
                                  B._ptr(bf["pool"]), s), "scan")
        B._check(L.gdr_chunk_output(P.ref, B._ptr(q), B._ptr(k), B._ptr(bf["v_new"]), B._ptr(bf["h"]),
                                    B._ptr(bf["g_cum"]), float(inp.scale), B._ptr(bf["o"]), s), "output")

    eager = buffers()
    snaps = []
    for _ in range(3):  # the pool advances by one step per call
        step(eager)
        torch.cuda.synchronize()
        snaps.append({key: t.clone() for key, t in eager.items()})

    gb = buffers()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(gb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(gb["pool"].cpu(), pool), "capture must not execute"
    other = buffers()
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for key in ("o", "h", "v_new", "w", "u", "g_cum", "pool"):
            assert torch.equal(gb[key], snaps[i][key]), (i, key)
        step(other)  # eager work between replays
        torch.cuda.synchronize()
