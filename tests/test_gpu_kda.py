"""GPU parity of the per-key-channel decay path (prepare, state scan, output,
and the segmented pass) against the FP64 oracle, through the C ABI, plus the
bit-identity contracts it shares with the gated-delta scan (every tile, dense
vs packed).

Tolerances (relative L2 over a whole tensor, oracle as reference): 1e-2 for
bfloat16 storage of the outputs, states and prepared factors; 1e-5 for the
FP32 cumulative decays and chunk decays.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import kda_ref
from parity import gate, per_sequence_max
from workloads import make_config, make_gdr

pytestmark = pytest.mark.gpu

TOL = 1e-2
TILES = [(32, 2, 2), (32, 2, 3), (64, 2, 3), (64, 4, 2), (64, 4, 3), (128, 4, 2), (128, 4, 3)]


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


def to_np(t):
    return t.detach().to(torch.float64).cpu().numpy()


def dev(t):
    return None if t is None else t.cuda()


def problem(seed, lengths, H=2, DK=128, DV=128, h0_std=0.1, varlen=True):
    return make_gdr(seed, lengths=lengths, H=H, DK=DK, DV=DV, dtype=torch.bfloat16, varlen=varlen,
                    gates="logsigmoid_channels", h0_std=h0_std)


def gpu_forward(pkg, inp, scale, tile=None, n_segments=None):
    q, k, v, g, b = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    h0 = dev(inp.h0)
    g_cum, w, u, kg, decay = pkg.kda_chunk_prepare(k, v, g, b, inp.cu_seqlens)
    if n_segments is None:
        h, v_new, hT = pkg.kda_state_scan(kg, w, u, decay, h0, inp.cu_seqlens, tile)
    else:
        ss, st = pkg.kda_segment_summaries(kg, w, u, decay, n_segments, inp.cu_seqlens, tile)
        si, _ = pkg.gdr_segment_compose(k, v.shape[-1], ss, st, n_segments, h0, inp.cu_seqlens)
        h, v_new, hT = pkg.kda_state_scan(kg, w, u, decay, None, inp.cu_seqlens, tile, n_segments, si)
    o = pkg.kda_chunk_output(q, k, v_new, h, g_cum, scale, inp.cu_seqlens)
    torch.cuda.synchronize()
    return dict(o=o, h=h, v_new=v_new, hT=hT, g_cum=g_cum, w=w, u=u, kg=kg, decay=decay)


def check_against_oracle(out, inp, scale, what, factors=True):
    d = inp.f64()
    ref = kda_ref.kda_recurrent_fp64(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], scale)
    h_gpu = to_np(out["h"]).transpose(0, 1, 3, 2)  # value-major -> [NT, H, DK, DV]
    errs = {"o": rel(to_np(out["o"]), ref["o"]), "v_new": rel(to_np(out["v_new"]), ref["v_new"]),
            "h": rel(h_gpu, ref["h"]), "hT": rel(to_np(out["hT"]), ref["hT"])}
    if factors:
        fr = kda_ref.kda_chunked_fp64(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], scale)
        errs.update(w=rel(to_np(out["w"]), fr["w"]), u=rel(to_np(out["u"]), fr["u"]),
                    kg=rel(to_np(out["kg"]), fr["kg"]))
        e_g = rel(to_np(out["g_cum"]), fr["g_cum"])
        e_d = rel(to_np(out["decay"]), fr["decay"])
        print(what, f"g_cum={e_g:.2e} decay={e_d:.2e}", flush=True)
        assert e_g <= 1e-5 and e_d <= 1e-5, (what, e_g, e_d)
    got = {"o": to_np(out["o"]), "v_new": to_np(out["v_new"]), "h": h_gpu, "hT": to_np(out["hT"])}
    kinds = {"o": "token", "v_new": "token", "h": "chunk", "hT": "seq"}
    worst = per_sequence_max({k: (got[k], ref[k], kinds[k]) for k in kinds}, d["cu_seqlens"], ref["chunk_offsets"])
    gate(errs, worst, TOL, what)


@pytest.mark.parametrize("DK,DV", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_kda_parity_ragged(pkg, DK, DV):
    inp = problem(500 + DK + DV, [1, 63, 64, 65, 150], DK=DK, DV=DV)
    out = gpu_forward(pkg, inp, DK ** -0.5)
    check_against_oracle(out, inp, DK ** -0.5, f"kda ragged {DK}x{DV}")


def test_kda_dense_rows_and_no_initial_state(pkg):
    inp = problem(611, [200, 200], H=3, h0_std=None, varlen=False)
    out = gpu_forward(pkg, inp, 1.0)
    check_against_oracle(out, inp, 1.0, "kda dense B=2")


def test_kda_bit_identical_across_tiles_and_layouts(pkg):
    lengths = [130, 64, 200]
    packed = problem(623, lengths)
    ref = gpu_forward(pkg, packed, 0.5)
    for t in TILES:
        out = gpu_forward(pkg, packed, 0.5, tile=t)
        for key in ("h", "v_new", "hT", "o"):
            assert torch.equal(out[key], ref[key]), f"tile {t}: {key} differs"
    # every packed sequence equals itself run alone as a dense row
    cu = packed.cu_seqlens.tolist()
    for n, L in enumerate(lengths):
        s, e = cu[n], cu[n + 1]
        one = problem(623, [L])
        one.q, one.k, one.v = packed.q[:, s:e], packed.k[:, s:e], packed.v[:, s:e]
        one.g, one.beta, one.h0 = packed.g[:, s:e], packed.beta[:, s:e], packed.h0[n:n + 1]
        one.cu_seqlens = None
        out = gpu_forward(pkg, one, 0.5)
        c0 = sum((x + 63) // 64 for x in lengths[:n])
        assert torch.equal(out["hT"][0], ref["hT"][n]), f"sequence {n}: hT"
        assert torch.equal(out["h"], ref["h"][c0:c0 + (L + 63) // 64]), f"sequence {n}: h"
        assert torch.equal(out["o"][0], ref["o"][0, s:e]), f"sequence {n}: o"


def test_kda_uniform_channels_match_scalar_decay(pkg):
    """Every channel decaying alike: the per-channel path and the scalar
    gated-delta path agree (each within tolerance of its own oracle)."""
    inp = make_gdr(641, lengths=[100, 190], H=2, dtype=torch.bfloat16, varlen=True, h0_std=0.1)
    kd = problem(641, [100, 190])
    kd.q, kd.k, kd.v, kd.beta, kd.h0 = inp.q, inp.k, inp.v, inp.beta, inp.h0
    kd.g = inp.g[..., None].expand(*inp.g.shape, 128).contiguous()
    out = gpu_forward(pkg, kd, 1.0)
    d = inp.f64()
    ref = oracle.gdr_recurrent_fp64(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], 1.0)
    e_o, e_hT = rel(to_np(out["o"]), ref["o"]), rel(to_np(out["hT"]), ref["hT"])
    print(f"kda uniform channels vs scalar oracle: o={e_o:.3e} hT={e_hT:.3e}", flush=True)
    assert e_o <= TOL and e_hT <= TOL


def test_kda_segmented_pass(pkg):
    inp = problem(653, [1000], H=2, h0_std=0.1)
    for P in (1, 4, 7):
        out = gpu_forward(pkg, inp, 0.25, n_segments=P)
        check_against_oracle(out, inp, 0.25, f"kda segmented P={P}", factors=False)


def test_kda_decays_at_the_input_limit(pkg):
    """Per-channel log decays drawn over the whole supported range, U(-5, 0),
    with every fourth channel at exactly -5 in every token (the largest
    within-block growth factor the kernels' block referencing allows, e^75):
    prepare, scan and output stay finite and match the oracle, serial and
    segmented."""
    inp = make_gdr(655, lengths=[1, 64, 65, 200, 17], H=2, DK=128, DV=128, dtype=torch.bfloat16, varlen=True,
                   gates="channels_to_limit", h0_std=0.1)
    assert float(inp.g.min()) == -5.0
    out = gpu_forward(pkg, inp, 0.5)
    for key in ("o", "h", "hT", "v_new", "w", "u", "kg"):
        assert torch.isfinite(out[key].float()).all(), key
    check_against_oracle(out, inp, 0.5, "kda decays at the limit")
    seg = gpu_forward(pkg, inp, 0.5, n_segments=2)
    check_against_oracle(seg, inp, 0.5, "kda decays at the limit, 2 segments", factors=False)


def test_kda_question_rows_workload(pkg):
    """The question-rows shape (24 packed sequences, 3400 tokens, 16 heads)
    with per-channel decays, against the oracle on every head."""
    inp = make_config("kda_question_rows")
    out = gpu_forward(pkg, inp, 128 ** -0.5)
    check_against_oracle(out, inp, 128 ** -0.5, "kda question rows", factors=False)
    again = gpu_forward(pkg, inp, 128 ** -0.5)
    for key in ("o", "h", "hT", "v_new"):
        assert torch.equal(out[key], again[key]), f"run to run: {key}"


def test_kda_many_sequences_span_several_launches(pkg):
    """More packed sequences than one launch's work list holds (112 rows):
    prepare, scan and output split the batch over launches."""
    rng = np.random.default_rng(7)
    lengths = [int(x) for x in rng.integers(0, 71, 200)]
    lengths[:3] = [0, 1, 65]
    inp = problem(671, lengths, H=2, DK=64, DV=64)
    out = gpu_forward(pkg, inp, 0.5)
    check_against_oracle(out, inp, 0.5, f"kda {len(lengths)} sequences", factors=False)


def test_kda_empty_single_token_and_pool(pkg):
    """Empty and one-token sequences (an empty sequence keeps its initial
    state and writes nothing else), and indexed states: sequence n reads and
    writes pool row idx[n] in place, other rows untouched."""
    inp = problem(667, [0, 1, 0, 2, 70, 0], H=2, DK=64, DV=64, h0_std=0.3)
    out = gpu_forward(pkg, inp, 1.0)
    check_against_oracle(out, inp, 1.0, "kda empty/single", factors=False)
    h0 = inp.h0.numpy()
    for n, L in enumerate(inp.lengths):
        if L == 0:
            assert np.array_equal(out["hT"][n].cpu().numpy(), h0[n]), "an empty sequence keeps its initial state"
    # pooled states, updated in place
    q, k, v, g, b = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    g_cum, w, u, kg, decay = pkg.kda_chunk_prepare(k, v, g, b, inp.cu_seqlens)
    idx = [5, 0, 3, 7, 2, 6]
    pool = torch.randn(9, 2, 64, 64, device="cuda") * 0.1
    for n, i in enumerate(idx):
        pool[i] = inp.h0[n].cuda()
    before = pool.clone()
    B = pkg.binding
    p = B.Problem(kg, 64, inp.cu_seqlens, "kv", idx, pool.shape[0])
    nt = pkg.gdr_num_chunks(kg, 64, inp.cu_seqlens)
    h = torch.empty((nt, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    vn = torch.empty_like(u)
    B._check(B.lib().kda_state_scan(p.ref, None, None, B._ptr(kg), B._ptr(w), B._ptr(u), B._ptr(decay),
                                    B._ptr(pool), B._ptr(h), B._ptr(vn), B._ptr(pool), None), "kda_state_scan")
    torch.cuda.synchronize()
    for n, i in enumerate(idx):
        assert torch.equal(pool[i], out["hT"][n]), f"pool row {i} (sequence {n})"
    for i in (1, 4, 8):
        assert torch.equal(pool[i], before[i]), f"untouched pool row {i}"
    assert torch.equal(h, out["h"]) and torch.equal(vn, out["v_new"])
