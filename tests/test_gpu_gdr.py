"""GPU parity of the gated-delta path against the FP64 oracle, plus the
bit-identity contracts (tiles, dense vs packed, resume at a chunk boundary,
run-to-run).  Every call goes through the C ABI (ctypes binding).

Tolerances (relative L2, oracle as reference): 1e-5 for float32 storage and
1e-2 for bfloat16 storage, over each whole tensor and, separately, over every
(sequence, head) slice of it (the largest of those is gated too, so an error
confined to one short sequence cannot hide in the whole-tensor figure).  The
named workloads are compared on every head.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
from parity import gate, per_sequence_max, rel
from workloads import make_config, make_gdr

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}


@pytest.fixture(scope="module")
def pkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_chunked_amd as p

    p.lib()
    return p


def to_np(t):
    return t.detach().to(torch.float64).cpu().numpy()


def dev(t):
    return None if t is None else t.cuda()


def run_path(pkg, inp, n_segments=None, tile=None, scale=None, state_layout="kv"):
    h0 = dev(inp.h0)
    if h0 is not None and state_layout == "vk":
        h0 = h0.transpose(-1, -2).contiguous()
    q, k, v, g, b = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, b, inp.cu_seqlens)
    if n_segments is None:
        h, v_new, hT = pkg.gdr_state_scan(k, w, u, g_cum, h0, inp.cu_seqlens, tile, state_layout=state_layout)
        extra = {}
    else:
        ss, st = pkg.gdr_segment_summaries(k, w, u, g_cum, n_segments, inp.cu_seqlens, tile)
        si, hTc = pkg.gdr_segment_compose(k, v.shape[-1], ss, st, n_segments, h0, inp.cu_seqlens,
                                          state_layout=state_layout, emit_final=True)
        h, v_new, hT = pkg.gdr_state_scan(k, w, u, g_cum, None, inp.cu_seqlens, tile, n_segments, si,
                                          state_layout=state_layout)
        extra = {"seg_state": ss, "seg_trans": st, "seg_init": si, "hT_compose": hTc}
    o = pkg.gdr_chunk_output(q, k, v_new, h, g_cum, inp.scale if scale is None else scale, inp.cu_seqlens)
    torch.cuda.synchronize()
    if state_layout == "vk":
        hT = hT.transpose(-1, -2)
    return dict(o=o, h=h, v_new=v_new, hT=hT, g_cum=g_cum, w=w, u=u, **extra)


_CACHE = {}


def config(name):
    if name not in _CACHE:
        _CACHE[name] = make_config(name)
    return _CACHE[name]


def ref_of(inp, scale=None):
    """The FP64 oracle over every head (a pool of worker processes for the
    named workloads, one per group of heads)."""
    key = (inp.name, scale)
    if inp.name != "custom" and key in _CACHE:
        return _CACHE[key]
    d = inp.f64()
    sc = inp.scale if scale is None else scale
    if inp.name == "custom":
        r = oracle.gdr_recurrent_fp64(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], sc)
    else:
        r = oracle_pool.gdr_forward_all_heads(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], sc)
        _CACHE[key] = r
    return r


def check(r, ref, tol, cu=None, what=""):
    got = {"o": to_np(r["o"]), "v_new": to_np(r["v_new"]), "hT": to_np(r["hT"]),
           "h": to_np(r["h"].transpose(-1, -2))}
    errs = {key: rel(got[key], ref[key]) for key in ("o", "v_new", "hT", "h")}
    kinds = {"o": "token", "v_new": "token", "h": "chunk", "hT": "seq"}
    worst = per_sequence_max({k: (got[k], ref[k], kinds[k]) for k in kinds}, cu, ref["chunk_offsets"])
    gate(errs, worst, tol, what)
    return errs


# --------------------------------------------------------------------------- named workloads
def test_tiny_fp32_workload(pkg):
    inp = config("tiny_fp32")
    r = run_path(pkg, inp)
    ref = ref_of(inp)
    check(r, ref, TOL[torch.float32], what="tiny_fp32")
    d = inp.f64()
    c = oracle.gdr_chunked_fp64(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"])
    for key in ("g_cum", "w", "u"):
        e = rel(to_np(r[key]), c[key])
        assert e <= 1e-5, f"prepare {key}: {e:.3e}"


def test_question_rows_workload(pkg):
    inp = config("question_rows")
    r = run_path(pkg, inp)
    check(r, ref_of(inp), TOL[torch.bfloat16], inp.cu_seqlens, what="question_rows")


def test_new_states_workload(pkg):
    inp = config("new_states")
    r = run_path(pkg, inp)
    check(r, ref_of(inp), TOL[torch.bfloat16], inp.cu_seqlens, what="new_states (all 32 heads)")


@pytest.mark.parametrize("segmented", [False, True])
def test_long_state_h1(pkg, segmented):
    inp = config("long_state_h1")
    r = run_path(pkg, inp, n_segments=16 if segmented else None)
    check(r, ref_of(inp), TOL[torch.bfloat16], inp.cu_seqlens, what=f"long_state_h1 segmented={segmented}")


@pytest.mark.parametrize("segmented", [False, True])
def test_long_state_h8(pkg, segmented):
    inp = config("long_state_h8")
    r = run_path(pkg, inp, n_segments=16 if segmented else None)
    check(r, ref_of(inp), TOL[torch.bfloat16], inp.cu_seqlens, what=f"long_state_h8 (all 8 heads) seg={segmented}")


def test_long_state_h1_cp_vs_serial_report(pkg):
    """The segmented path against the serial scan on the 64K one-head state
    at 2, 4, 8 and 16 segments, reported as relative L2 of the outputs, the
    final state and the outputs of the last 8K tokens, the table cuLA#127
    ("Accuracy") gives (a report, not a gate: every path is gated against the
    FP64 oracle elsewhere)."""
    inp = config("long_state_h1")
    a = run_path(pkg, inp)
    for P in (2, 4, 8, 16):
        b = run_path(pkg, inp, n_segments=P)
        out = rel(to_np(b["o"]), to_np(a["o"]))
        fin = rel(to_np(b["hT"]), to_np(a["hT"]))
        last = rel(to_np(b["o"][:, -8192:]), to_np(a["o"][:, -8192:]))
        print(f"CP vs serial (long_state_h1, {P} segments): out {out:.4e} final {fin:.4e} last-8K {last:.4e}",
              flush=True)
        assert np.isfinite([out, fin, last]).all()


# --------------------------------------------------------------------------- shapes and edges
CASES = [
    # dtype, DK, DV, lengths, h0, scale
    (torch.float32, 64, 64, [1, 63, 64, 65, 127, 257, 0], True, 1.0),
    (torch.float32, 128, 128, [200, 70], False, 128 ** -0.5),
    (torch.float32, 64, 128, [130, 5], True, 1.0),
    (torch.float32, 128, 64, [64, 191], True, 1.0),
    (torch.bfloat16, 64, 64, [1, 63, 64, 65, 127, 257, 0], True, 1.0),
    (torch.bfloat16, 128, 128, [200, 70, 1], True, 128 ** -0.5),
    (torch.bfloat16, 64, 128, [130, 5], False, 1.0),
    (torch.bfloat16, 128, 64, [64, 191], True, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{str(c[0])[6:]}-dk{c[1]}-dv{c[2]}-L{len(c[3])}")
def test_parity_shapes(pkg, case):
    dt, DK, DV, lengths, h0, scale = case
    inp = make_gdr(101 + DK + DV, lengths=lengths, H=3, DK=DK, DV=DV, dtype=dt, varlen=True,
                   h0_std=0.1 if h0 else None, scale=scale)
    r = run_path(pkg, inp)
    check(r, ref_of(inp), TOL[dt], inp.cu_seqlens, what=f"shape {case[:3]}")


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_segment_summaries_and_compose(pkg, dt):
    lengths = [700, 130]
    P = 4
    inp = make_gdr(303, lengths=lengths, H=2, DK=128, DV=128, dtype=dt, varlen=True, h0_std=0.1)
    r = run_path(pkg, inp, n_segments=P)
    d = inp.f64()
    cu = d["cu_seqlens"]
    tol = TOL[dt]
    for n in range(len(lengths)):
        s, e = cu[n], cu[n + 1]
        bounds = oracle.segment_bounds(e - s, P)
        S_loc, M = oracle.gdr_segment_summaries_fp64(d["k"][0, s:e], d["v"][0, s:e], d["g"][0, s:e],
                                                     d["beta"][0, s:e], bounds)
        inits, fin = oracle.gdr_segment_compose_fp64(S_loc, M, d["h0"][n])
        gs = to_np(r["seg_state"][n * P:(n + 1) * P]).transpose(0, 1, 3, 2)
        gm = to_np(r["seg_trans"][n * P:(n + 1) * P])
        gi = to_np(r["seg_init"][n * P:(n + 1) * P]).transpose(0, 1, 3, 2)
        es, em, ei = rel(gs, S_loc), rel(gm, M), rel(gi, inits)
        ef = rel(to_np(r["hT_compose"][n]), fin)
        print(f"seq {n}: S_loc {es:.3e} M {em:.3e} S_init {ei:.3e} composed final {ef:.3e}")
        assert max(es, em, ei, ef) <= tol
    check(r, ref_of(inp), tol, inp.cu_seqlens, what="segmented path")


@pytest.mark.parametrize("gates", ["logsigmoid_mid", "logsigmoid_fast"])
def test_segment_summaries_strong_decay(pkg, gates):
    """Segments long enough for the summaries' state scale to leave its range:
    with about -0.08 per token a 500-token segment decays by e^-40 (one
    renormalising chunk per segment); with about -1.4 per token every chunk's
    decay underflows float32 and every chunk renormalises."""
    lengths = [1500, 300]
    P = 3
    inp = make_gdr(311, lengths=lengths, H=2, DK=128, DV=128, dtype=torch.bfloat16, varlen=True, h0_std=0.1,
                   gates=gates)
    r = run_path(pkg, inp, n_segments=P)
    if gates == "logsigmoid_mid":
        d = inp.f64()
        cu = d["cu_seqlens"]
        for n in range(len(lengths)):
            s, e = cu[n], cu[n + 1]
            S_loc, M = oracle.gdr_segment_summaries_fp64(d["k"][0, s:e], d["v"][0, s:e], d["g"][0, s:e],
                                                         d["beta"][0, s:e], oracle.segment_bounds(e - s, P))
            gs = to_np(r["seg_state"][n * P:(n + 1) * P]).transpose(0, 1, 3, 2)
            gm = to_np(r["seg_trans"][n * P:(n + 1) * P])
            for j in range(P):  # per segment: the transitions differ by orders of magnitude
                es, em = rel(gs[j], S_loc[j]), rel(gm[j], M[j])
                print(f"{gates} seq {n} segment {j}: S_loc {es:.3e} M {em:.3e} (|M| {np.abs(M[j]).max():.2e})")
                assert es <= 1e-2 and em <= 1e-2
    check(r, ref_of(inp), 1e-2, inp.cu_seqlens, what=f"segmented path, {gates}")


def test_half_segment_summaries_match_direct_and_oracle(pkg):
    """The summaries formed from two half segments (with the workspace) and the
    direct ones both match the FP64 oracle's; 11 and 3 chunks over 4 segments
    give odd halves, one-chunk segments (an empty second half) and an empty
    segment."""
    lengths = [700, 130]
    P = 4
    inp = make_gdr(309, lengths=lengths, H=2, DK=128, DV=128, dtype=torch.bfloat16, varlen=True)
    k, v, g, b = (dev(x) for x in (inp.k, inp.v, inp.g, inp.beta))
    cu = inp.cu_seqlens
    assert pkg.gdr_segment_summaries_workspace_size(k, 128, P, cu) == 2 * 2 * P * 2 * 128 * 256 * 4
    g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, b, cu)
    split = pkg.gdr_segment_summaries(k, w, u, g_cum, P, cu)
    direct = pkg.gdr_segment_summaries(k, w, u, g_cum, P, cu, workspace=False)
    torch.cuda.synchronize()
    d = inp.f64()
    cuh = d["cu_seqlens"]
    for n in range(len(lengths)):
        s, e = cuh[n], cuh[n + 1]
        S_loc, M = oracle.gdr_segment_summaries_fp64(d["k"][0, s:e], d["v"][0, s:e], d["g"][0, s:e],
                                                     d["beta"][0, s:e], oracle.segment_bounds(e - s, P))
        for name, (ss, st) in (("split", split), ("direct", direct)):
            es = rel(to_np(ss[n * P:(n + 1) * P]).transpose(0, 1, 3, 2), S_loc)
            em = rel(to_np(st[n * P:(n + 1) * P]), M)
            print(f"seq {n} {name}: S_loc {es:.3e} M {em:.3e}", flush=True)
            assert es <= 1e-2 and em <= 1e-2
    # the two forms agree closely (FP32 composition of the halves)
    assert rel(to_np(split[1]), to_np(direct[1])) <= 1e-2


def test_many_sequences_span_several_launches(pkg):
    """More packed sequences than one launch's work list holds (112 rows): the
    scan, prepare and output split the batch over launches; empty and
    one-token sequences are mixed in."""
    rng = np.random.default_rng(5)
    lengths = [int(x) for x in rng.integers(0, 71, 250)]
    lengths[:4] = [0, 1, 64, 65]
    inp = make_gdr(313, lengths=lengths, H=2, DK=64, DV=64, dtype=torch.bfloat16, varlen=True, h0_std=0.1)
    r = run_path(pkg, inp)
    check(r, ref_of(inp), TOL[torch.bfloat16], inp.cu_seqlens, what=f"{len(lengths)} sequences")


def test_segmented_many_sequences_span_several_launches(pkg):
    """40 sequences x 3 segments: 120 summary rows (240 half rows with the
    workspace) and 120 final-pass rows, each over several launches."""
    rng = np.random.default_rng(6)
    lengths = [int(x) for x in rng.integers(1, 400, 40)]
    inp = make_gdr(314, lengths=lengths, H=2, DK=128, DV=128, dtype=torch.bfloat16, varlen=True, h0_std=0.1)
    assert pkg.gdr_segment_summaries_workspace_size(inp.k.cuda(), 128, 3, inp.cu_seqlens) > 0
    r = run_path(pkg, inp, n_segments=3)
    check(r, ref_of(inp), TOL[torch.bfloat16], inp.cu_seqlens, what="40 sequences, 3 segments")


@pytest.mark.parametrize("DK,DV", [(256, 256), (256, 128), (128, 256)])
def test_parity_dims_256(pkg, DK, DV):
    """Key or value width 256 (bfloat16): prepare, scan and output against the
    oracle on ragged packed sequences with initial states."""
    inp = make_gdr(321 + DK + DV, lengths=[1, 63, 65, 200, 0], H=2, DK=DK, DV=DV, dtype=torch.bfloat16,
                   varlen=True, h0_std=0.1, scale=DK ** -0.5)
    r = run_path(pkg, inp)
    check(r, ref_of(inp), TOL[torch.bfloat16], inp.cu_seqlens, what=f"dims {DK}x{DV}")


def test_bit_identical_across_tiles_dims_256(pkg):
    inp = make_gdr(333, lengths=[1, 64, 65, 300, 129], H=2, DK=256, DV=256, dtype=torch.bfloat16, varlen=True,
                   h0_std=0.1)
    tiles = [(32, 2, 1), (32, 2, 2), (64, 4, 1), (64, 4, 2)]
    base = run_path(pkg, inp, tile=tiles[0])
    for t in tiles[1:]:
        r = run_path(pkg, inp, tile=t)
        for key in ("h", "v_new", "hT", "o"):
            assert torch.equal(r[key], base[key]), f"tile {t} changed {key}"


def test_empty_and_single_token_sequences(pkg):
    inp = make_gdr(404, lengths=[0, 1, 0, 2, 0], H=2, DK=64, DV=64, dtype=torch.float32, varlen=True, h0_std=0.3)
    r = run_path(pkg, inp)
    hT = to_np(r["hT"])
    h0 = inp.h0.double().numpy()
    for n in (0, 2, 4):
        assert np.array_equal(hT[n], h0[n]), "an empty sequence keeps its initial state"
    check(r, ref_of(inp), 1e-5, inp.cu_seqlens, what="empty/single")


def test_state_layout_vk(pkg):
    inp = make_gdr(505, lengths=[150, 77], H=2, DK=128, DV=64, dtype=torch.bfloat16, varlen=True, h0_std=0.1)
    a = run_path(pkg, inp, state_layout="kv")
    b = run_path(pkg, inp, state_layout="vk")
    assert torch.equal(a["hT"], b["hT"])
    assert torch.equal(a["o"], b["o"])


# --------------------------------------------------------------------------- bit identity
TILES = {torch.bfloat16: [(32, 2, 2), (32, 2, 3), (64, 2, 3), (64, 4, 2), (64, 4, 3), (128, 4, 2), (128, 4, 3)],
         torch.float32: [(32, 2, 1), (32, 2, 2), (64, 4, 1), (64, 4, 2)]}


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_bit_identical_across_tiles(pkg, dt):
    inp = make_gdr(606, lengths=[1, 64, 65, 300, 129], H=3, DK=128, DV=128, dtype=dt, varlen=True, h0_std=0.1)
    base = run_path(pkg, inp, tile=TILES[dt][0])
    for t in TILES[dt][1:]:
        r = run_path(pkg, inp, tile=t)
        for key in ("h", "v_new", "hT", "o"):
            assert torch.equal(r[key], base[key]), f"tile {t} changed {key}"


BIT_MATRIX = [(dk, dv, H) for dk in (64, 128) for dv in (64, 128) for H in (16, 32, 48)]


@pytest.mark.parametrize("dk,dv,H", BIT_MATRIX, ids=lambda x: str(x))
def test_bit_identical_across_tiles_shape_matrix(pkg, dk, dv, H):
    """Every built tile gives the same bits over a shape matrix: key / value
    widths 64 and 128, 16, 32 and 48 heads, a packed batch of ragged
    sequences (4 to 32 of them, 1 to 700 tokens) and one long row (a
    separate 3000-token batch for the widest shapes); h, v_new, hT and the
    chunk output.  The tile table's choice is one of the tiles compared."""
    rng = np.random.default_rng(dk + 3 * dv + H)
    n = int(rng.integers(4, 33))
    lengths = [int(x) for x in rng.integers(1, 701, n)]
    lengths[0] = 64
    batches = [lengths]
    if dk == dv == 128:
        batches.append([3000])
    for lens in batches:
        inp = make_gdr(640 + H + dk + dv, lengths=lens, H=H, DK=dk, DV=dv, dtype=torch.bfloat16, varlen=True,
                       h0_std=0.1)
        base = run_path(pkg, inp, tile=TILES[torch.bfloat16][0])
        default = run_path(pkg, inp)
        for key in ("h", "v_new", "hT", "o"):
            assert torch.equal(default[key], base[key]), f"planner tile changed {key}"
        for t in TILES[torch.bfloat16][1:]:
            if dv % t[0] != 0 and t[0] > dv:
                continue
            r = run_path(pkg, inp, tile=t)
            for key in ("h", "v_new", "hT", "o"):
                assert torch.equal(r[key], base[key]), f"tile {t} changed {key} ({len(lens)} sequences, H={H})"


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_bit_identical_segment_summaries_across_tiles(pkg, dt):
    inp = make_gdr(607, lengths=[900], H=2, DK=128, DV=128, dtype=dt, varlen=True)
    base = run_path(pkg, inp, n_segments=3, tile=TILES[dt][0])
    if dt == torch.bfloat16:  # the summary-only tile (all 256 columns of a segment-head in one block)
        k, w, u, g_cum = (base[x] if x in base else dev(getattr(inp, x)) for x in ("k", "w", "u", "g_cum"))
        ss, st = pkg.gdr_segment_summaries(k, w, u, g_cum, 3, inp.cu_seqlens, (256, 8, 2))
        assert torch.equal(ss, base["seg_state"]) and torch.equal(st, base["seg_trans"]), "tile (256, 8, 2)"
    for t in TILES[dt][1:]:
        r = run_path(pkg, inp, n_segments=3, tile=t)
        for key in ("seg_state", "seg_trans", "seg_init", "h", "hT", "o"):
            assert torch.equal(r[key], base[key]), f"tile {t} changed {key}"


def test_packed_equals_dense(pkg):
    lengths = [190, 190, 190]
    dense = make_gdr(707, lengths=lengths, H=2, DK=128, DV=128, dtype=torch.bfloat16, varlen=False, h0_std=0.1)
    packed = make_gdr(707, lengths=lengths, H=2, DK=128, DV=128, dtype=torch.bfloat16, varlen=True, h0_std=0.1)
    for name in ("q", "k", "v", "g", "beta"):
        assert torch.equal(getattr(dense, name).reshape(-1), getattr(packed, name).reshape(-1))
    a = run_path(pkg, dense)
    b = run_path(pkg, packed)
    assert torch.equal(a["o"].reshape(-1), b["o"].reshape(-1))
    assert torch.equal(a["h"], b["h"])
    assert torch.equal(a["hT"], b["hT"])


def test_each_packed_sequence_equals_itself_alone(pkg):
    inp = make_gdr(708, lengths=[100, 257, 3], H=2, DK=64, DV=128, dtype=torch.bfloat16, varlen=True, h0_std=0.1)
    full = run_path(pkg, inp)
    cu = inp.cu_seqlens.tolist()
    offs = np.concatenate([[0], np.cumsum([(L + 63) // 64 for L in inp.lengths])])
    for n in range(inp.N):
        s, e = cu[n], cu[n + 1]
        one = make_gdr(0, lengths=[e - s], H=2, DK=64, DV=128, dtype=torch.bfloat16, varlen=False)
        one.q, one.k, one.v = inp.q[:, s:e], inp.k[:, s:e], inp.v[:, s:e]
        one.g, one.beta, one.h0 = inp.g[:, s:e], inp.beta[:, s:e], inp.h0[n:n + 1]
        r = run_path(pkg, one)
        assert torch.equal(r["o"][0], full["o"][0, s:e])
        assert torch.equal(r["hT"][0], full["hT"][n])
        assert torch.equal(r["h"], full["h"][offs[n]:offs[n + 1]])


def test_resume_at_chunk_boundary(pkg):
    inp = make_gdr(709, lengths=[320], H=2, DK=128, DV=128, dtype=torch.bfloat16, varlen=False, h0_std=0.1)
    full = run_path(pkg, inp)
    first = make_gdr(0, lengths=[192], H=2, DK=128, DV=128, dtype=torch.bfloat16, varlen=False)
    first.q, first.k, first.v, first.g, first.beta = (x[:, :192] for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    first.h0 = inp.h0
    a = run_path(pkg, first)
    second = make_gdr(0, lengths=[128], H=2, DK=128, DV=128, dtype=torch.bfloat16, varlen=False)
    second.q, second.k, second.v, second.g, second.beta = (x[:, 192:] for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    second.h0 = a["hT"].cpu()
    b = run_path(pkg, second)
    assert torch.equal(b["hT"], full["hT"])
    assert torch.equal(torch.cat([a["o"], b["o"]], 1), full["o"])
    assert torch.equal(torch.cat([a["h"], b["h"]], 0), full["h"])


def test_run_to_run_determinism(pkg):
    inp = make_gdr(710, lengths=[500, 33, 1000], H=4, DK=128, DV=128, dtype=torch.bfloat16, varlen=True, h0_std=0.1)
    a = run_path(pkg, inp)
    b = run_path(pkg, inp)
    for key in ("o", "h", "v_new", "hT", "w", "u", "g_cum"):
        assert torch.equal(a[key], b[key]), key


def test_poisoned_outputs_fully_written(pkg):
    inp = make_gdr(711, lengths=[65, 1, 128], H=2, DK=128, DV=128, dtype=torch.bfloat16, varlen=True, h0_std=0.1)
    k, v, g, b = (dev(x) for x in (inp.k, inp.v, inp.g, inp.beta))
    g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, b, inp.cu_seqlens)
    nt = pkg.gdr_num_chunks(k, 128, inp.cu_seqlens)
    out = {"h": torch.full((nt, 2, 128, 128), float("nan"), dtype=k.dtype, device=k.device),
           "v_new": torch.full_like(u, float("nan")),
           "hT": torch.full((3, 2, 128, 128), float("nan"), device=k.device)}
    h, v_new, hT = pkg.gdr_state_scan(k, w, u, g_cum, dev(inp.h0), inp.cu_seqlens, out=out)
    torch.cuda.synchronize()
    for name, t in (("h", h), ("v_new", v_new), ("hT", hT)):
        assert not torch.isnan(t).any(), f"{name} has unwritten elements"


# --------------------------------------------------------------------------- scheduler-chosen segmentation
@pytest.mark.parametrize("name,want", [("long_state_h8", 16), ("long_state_h1", 32), ("question_rows", 0)])
def test_auto_segmentation(pkg, name, want):
    """The forward with the scheduler's segmentation (gdr_state_scan_auto
    behind chunk_gated_delta_rule with no n_segments) picks the expected
    split, gives the explicit call's bits (n_segments = P, or the serial
    scan for P = 0) and matches the FP64 oracle."""
    inp = config(name)
    q, k, v, g, b = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    P = pkg.gdr_plan_segments(k, v.shape[-1], inp.cu_seqlens)
    assert P == want
    h0 = dev(inp.h0)
    auto = pkg.chunk_gated_delta_rule(q, k, v, g, b, h0, inp.cu_seqlens, inp.scale)
    expl = pkg.chunk_gated_delta_rule(q, k, v, g, b, h0, inp.cu_seqlens, inp.scale, n_segments=P)
    torch.cuda.synchronize()
    for key in ("o", "h", "v_new", "hT"):
        assert torch.equal(auto[key], expl[key]), f"{name}: auto and explicit split differ in {key}"
    check(auto, ref_of(inp), TOL[torch.bfloat16], inp.cu_seqlens, what=f"{name} auto ({P} segments)")


def test_auto_segmentation_with_h0_and_graph_capture(pkg):
    """The scheduler's split with an initial state gives the explicit split's
    bits; captured in a HIP graph, replays give the eager bits, with eager
    work and synchronisation between them."""
    inp = make_gdr(1201, lengths=[9000, 700, 5000], H=2, dtype=torch.bfloat16, varlen=True, h0_std=0.1)
    q, k, v, g, b = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    h0 = dev(inp.h0)
    P = pkg.gdr_plan_segments(k, v.shape[-1], inp.cu_seqlens)
    assert P >= 2
    g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, b, inp.cu_seqlens)
    eager = pkg.gdr_state_scan_auto(q, k, w, u, g_cum, inp.scale, h0, inp.cu_seqlens)
    expl = pkg.chunk_gated_delta_rule(q, k, v, g, b, h0, inp.cu_seqlens, inp.scale, n_segments=P)
    torch.cuda.synchronize()
    for i, key in enumerate(("o", "h", "v_new", "hT")):
        assert torch.equal(eager[i], expl[key]), f"auto with h0 and explicit split differ in {key}"
    outs = [torch.empty_like(x) for x in eager]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        cap = pkg.gdr_state_scan_auto(q, k, w, u, g_cum, inp.scale, h0, inp.cu_seqlens, stream=s)  # warm-up
        s.synchronize()
        with torch.cuda.graph(graph, stream=s):
            cap = pkg.gdr_state_scan_auto(q, k, w, u, g_cum, inp.scale, h0, inp.cu_seqlens, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in cap:
            x.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, key in enumerate(("o", "h", "v_new", "hT")):
            assert torch.equal(cap[i], eager[i]), f"graph replay {rep}: {key} differs"
