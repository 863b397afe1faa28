"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, validates arguments before any launch, and the scheduler's
plans are what the design says."""

import ctypes
import os
import re

import numpy as np

import pytest

from linear_attention_chunked_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "gdr.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("gdr_", "abc_", "kda_"))))


def test_every_declared_symbol_is_exported():
    L = B.lib()
    names = _declared()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(L, n), f"missing export {n}"


def _prob(B_=1, T=128, H=2, DK=128, DV=128, N=None, cu=None, dtype=B.GDR_BF16, layout=0):
    arr = None
    if cu is not None:
        arr = (ctypes.c_int32 * len(cu))(*cu)
        N = len(cu) - 1
    elif N is None:
        N = B_
    p = B.gdr_problem(B_, T, H, DK, DV, N, arr, dtype, layout)
    return p, arr


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first


def _scan(p, k=FAKE, w=FAKE, u=FAKE, g=FAKE, h0=None, tile=None):
    t = None if tile is None else ctypes.byref(B.gdr_tile(*tile))
    return B.lib().gdr_state_scan(ctypes.byref(p), t, None, k, w, u, g, h0, None, None, None, None)


@pytest.mark.parametrize("cu,T", [([1, 5, 9], 9), ([0, 5, 3], 5), ([0, 5, 9], 10)])
def test_bad_cu_seqlens_rejected(cu, T):
    p, keep = _prob(T=T, cu=cu)
    assert _scan(p) == B.GDR_ERR_INVALID_ARG
    assert B.lib().gdr_last_error().decode()


def test_packed_needs_single_row():
    p, keep = _prob(B_=2, T=9, cu=[0, 4, 9])
    assert _scan(p) == B.GDR_ERR_INVALID_ARG


@pytest.mark.parametrize("dk,dv", [(32, 128), (128, 96), (512, 128)])
def test_unsupported_dims(dk, dv):
    p, _ = _prob(DK=dk, DV=dv)
    assert _scan(p) == B.GDR_ERR_INVALID_ARG


def test_dims_256():
    """DK or DV = 256: bfloat16 only; the plain pass takes the generic kernel's
    tiles; the segment summaries, the reverse pass and the per-channel decay
    entry points report GDR_ERR_UNSUPPORTED (before any launch)."""
    L = B.lib()
    p, _ = _prob(DK=256, DV=64, dtype=B.GDR_F32)
    assert _scan(p) == B.GDR_ERR_INVALID_ARG
    assert b"bfloat16" in L.gdr_last_error()
    q, _ = _prob(B_=1, DK=256, DV=256, T=4096, H=8)
    assert _query(q)[:3] == (32, 2, 2)  # few units: the narrower tile
    p, _ = _prob(B_=8, DK=256, DV=256, T=4096, H=8)
    assert _query(p)[:3] == (64, 4, 2)
    assert _scan(p, tile=(128, 4, 3)) == B.GDR_ERR_UNSUPPORTED  # a scan2 tile: not built at DK = 256
    assert L.gdr_segment_summaries(ctypes.byref(p), None, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == B.GDR_ERR_UNSUPPORTED
    assert L.gdr_segment_compose(ctypes.byref(p), 2, FAKE, FAKE, None, FAKE, None, None) == B.GDR_ERR_UNSUPPORTED
    assert L.gdr_chunk_dv_local(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, ctypes.c_float(1.0), FAKE,
                                None) == B.GDR_ERR_UNSUPPORTED
    assert L.kda_chunk_output(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(1.0), FAKE,
                              None) == B.GDR_ERR_UNSUPPORTED


def test_null_and_misaligned_pointers():
    p, _ = _prob()
    assert _scan(p, k=None) == B.GDR_ERR_INVALID_ARG
    assert b"k must not be NULL" in B.lib().gdr_last_error()
    assert _scan(p, u=ctypes.c_void_p(0x10004)) == B.GDR_ERR_INVALID_ARG
    assert b"aligned" in B.lib().gdr_last_error()
    assert _scan(p, h0=ctypes.c_void_p(0x10008)) == B.GDR_ERR_INVALID_ARG


def test_unbuilt_tile_rejected():
    p, _ = _prob()
    assert _scan(p, tile=(48, 3, 1)) == B.GDR_ERR_UNSUPPORTED
    p, _ = _prob(DV=64)
    assert _scan(p, tile=(128, 4, 3)) == B.GDR_ERR_UNSUPPORTED  # bv must divide DV


def test_num_chunks():
    p, keep = _prob(T=3400, cu=[0, 130, 130, 269, 3400])
    # ceil(130/64)=3, 0, ceil(139/64)=3, ceil(3131/64)=49
    assert B.lib().gdr_num_chunks(ctypes.byref(p)) == 3 + 0 + 3 + 49
    p, _ = _prob(B_=3, T=65)
    assert B.lib().gdr_num_chunks(ctypes.byref(p)) == 6


def _query(p, tile=None, nseg=0):
    out = (ctypes.c_int64 * 6)()
    t = None if tile is None else ctypes.byref(B.gdr_tile(*tile))
    st = B.lib().gdr_plan_query(ctypes.byref(p), t, nseg, out)
    assert st == B.GDR_OK, B.lib().gdr_last_error()
    return tuple(out)


def test_plan_grid_and_launch_split():
    # 300 sequences -> 3 launches of <= 112 rows; grid padded to whole XCD groups of 8 pairs
    cu = [0]
    for i in range(300):
        cu.append(cu[-1] + 1 + (i % 70))
    p, keep = _prob(T=cu[-1], cu=cu, H=3)
    bv, waves, stages, wgs, launches, maxrows = _query(p, tile=(64, 4, 3))
    assert (bv, waves, stages) == (64, 4, 3)
    assert launches == 3 and maxrows == 112
    pairs = [112 * 3, 112 * 3, 76 * 3]
    assert wgs == sum(8 * 2 * ((x + 7) // 8) for x in pairs)


def test_plan_segments_and_table():
    # 16 segments x 8 heads: 256 direct 128-column blocks would give one wave per
    # SIMD, so every segment's summary comes from its two halves (32 rows), one
    # 8-wave block of all DV + DK columns per (half, head)
    p, _ = _prob(B_=1, T=65536, H=8)
    bv, waves, stages, wgs, launches, maxrows = _query(p, nseg=16)
    assert maxrows == 32 and launches == 1
    assert (bv, waves, stages) == (256, 8, 2)
    assert wgs == 8 * ((128 + 128) // bv) * ((32 * 8 + 7) // 8)
    # 64 segments: direct (512 blocks of 128 columns already fill the CUs twice)
    bv, waves, stages, wgs, launches, maxrows = _query(p, nseg=64)
    assert maxrows == 64 and (bv, waves, stages) == (256, 8, 2)


def test_summary_workspace_size():
    L = B.lib()
    p, _ = _prob(B_=1, T=65536, H=8)
    # the half summaries: 2 N P (S_loc, M) pairs in FP32
    assert L.gdr_segment_summaries_workspace_size(ctypes.byref(p), 16) == 2 * 16 * 8 * 128 * 256 * 4
    assert L.gdr_segment_summaries_workspace_size(ctypes.byref(p), 32) == 0  # 512 blocks: direct
    for kw in (dict(dtype=B.GDR_F32), dict(DK=64, DV=64), dict(DK=128, DV=64)):
        q, _ = _prob(B_=1, T=4096, H=2, **kw)
        assert L.gdr_segment_summaries_workspace_size(ctypes.byref(q), 4) == 0, kw
    assert L.gdr_segment_summaries_workspace_size(ctypes.byref(p), 0) == 0
    assert b"n_segments" in L.gdr_last_error()
    assert L.gdr_segment_summaries_workspace_size(ctypes.byref(p), 32) == 0 and L.gdr_last_error() == b""
    # a workspace smaller than asked for is an argument error (before any launch)
    small = 2 * 16 * 8 * 128 * 256 * 4 - 16
    assert L.gdr_segment_summaries_ws(ctypes.byref(p), None, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, small,
                                      None) == B.GDR_ERR_INVALID_ARG
    assert "workspace_bytes" in L.gdr_last_error().decode()
    assert L.gdr_segment_summaries_ws(ctypes.byref(p), None, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      ctypes.c_void_p(0x10008), 1 << 30, None) == B.GDR_ERR_INVALID_ARG


def test_force_tile_env(monkeypatch):
    p, _ = _prob(B_=4, T=256, H=32)
    monkeypatch.setenv("GDR_FORCE_TILE", "128,4,3")
    assert _query(p)[:3] == (128, 4, 3)
    monkeypatch.setenv("GDR_FORCE_TILE", "bogus")
    out = (ctypes.c_int64 * 6)()
    assert B.lib().gdr_plan_query(ctypes.byref(p), None, 0, out) == B.GDR_ERR_UNSUPPORTED


def test_cpu_tensors_rejected():
    import torch

    k = torch.zeros(1, 64, 1, 64)
    with pytest.raises(ValueError):
        B.gdr_chunk_prepare(k, k, torch.zeros(1, 64, 1), torch.zeros(1, 64, 1))


def test_status_strings():
    L = B.lib()
    assert L.gdr_status_string(0) == b"GDR_OK"
    assert L.gdr_status_string(3) == b"GDR_ERR_HIP"


def _pool_prob(idx, pool_size):
    cu = [0, 3, 10, 20]
    arr = (ctypes.c_int32 * len(cu))(*cu)
    ia = (ctypes.c_int32 * len(idx))(*idx)
    p = B.gdr_problem(1, 20, 2, 128, 128, 3, arr, B.GDR_BF16, 0, ia, pool_size)
    return p, (arr, ia)


@pytest.mark.parametrize("idx,pool", [([0, 1, 1], 4), ([0, 4, 1], 4), ([0, -1, 2], 4), ([0, 1, 2], 0)])
def test_bad_state_indices_rejected(idx, pool):
    p, keep = _pool_prob(idx, pool)
    assert _scan(p) == B.GDR_ERR_INVALID_ARG
    assert "index" in B.lib().gdr_last_error().decode() or "pool" in B.lib().gdr_last_error().decode()


def test_state_pool_serial_only():
    p, keep = _pool_prob([3, 0, 2], 4)
    L = B.lib()
    assert L.gdr_segment_summaries(ctypes.byref(p), None, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == B.GDR_ERR_UNSUPPORTED
    assert L.gdr_segment_compose(ctypes.byref(p), 2, FAKE, FAKE, None, FAKE, None, None) == B.GDR_ERR_UNSUPPORTED
    seg = B.gdr_segments(2, FAKE.value)
    assert L.gdr_state_scan(ctypes.byref(p), None, ctypes.byref(seg), FAKE, FAKE, FAKE, FAKE, None, None, None, None,
                            None) == B.GDR_ERR_UNSUPPORTED
    # a valid pool passes validation up to the pointer checks
    assert _scan(p, k=None) == B.GDR_ERR_INVALID_ARG
    assert "k" in L.gdr_last_error().decode()


def test_reverse_pass_validation():
    L = B.lib()
    p, keep = _prob(dtype=B.GDR_F32)
    assert L.gdr_chunk_dv_local(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, ctypes.c_float(1.0), FAKE,
                                None) == B.GDR_ERR_UNSUPPORTED
    assert L.gdr_state_scan_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, ctypes.c_float(1.0),
                                FAKE, FAKE, FAKE, None) == B.GDR_ERR_UNSUPPORTED
    p, keep = _prob()
    assert L.gdr_state_scan_bwd(ctypes.byref(p), FAKE, None, FAKE, FAKE, FAKE, FAKE, None, ctypes.c_float(1.0),
                                FAKE, FAKE, FAKE, None) == B.GDR_ERR_INVALID_ARG
    pp, keep2 = _pool_prob([3, 0, 2], 4)
    assert L.gdr_state_scan_bwd(ctypes.byref(pp), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, ctypes.c_float(1.0),
                                FAKE, FAKE, FAKE, None) == B.GDR_ERR_UNSUPPORTED


def test_abc_reverse_validation():
    L = B.lib()
    p = B.abc_problem(1, 128, 2, 64, 64, 64, B.GDR_BF16)
    ws = L.abc_bwd_workspace_size(ctypes.byref(p))
    assert ws >= 128 * 2 * 64 * 2 * 2
    args = [FAKE] * 5 + [None, None, ctypes.c_float(1.0), FAKE, FAKE, FAKE, ws, None]
    bad = list(args)
    bad[4] = None  # z is required
    assert L.abc_affine_scan_bwd(ctypes.byref(p), *bad) == B.GDR_ERR_INVALID_ARG
    assert "z" in L.gdr_last_error().decode()
    small = list(args)
    small[11] = ws - 1
    assert L.abc_affine_scan_bwd(ctypes.byref(p), *small) == B.GDR_ERR_INVALID_ARG
    p32 = B.abc_problem(1, 128, 2, 64, 64, 64, B.GDR_F32)
    assert L.abc_affine_scan_bwd(ctypes.byref(p32), *args) == B.GDR_ERR_INVALID_ARG


def test_abc_slot_counts():
    """M = 32 and 64 slots are accepted by the scan (its run end states keep 64
    padded slots whatever M is, which the workspace size covers); other counts
    are argument errors before any launch, for the scan and the read."""
    L = B.lib()
    B_, T, H, K, V = 2, 16384, 4, 256, 512
    for m in (32, 64):
        p = B.abc_problem(B_, T, H, K, m, V, B.GDR_BF16)
        ws = L.abc_workspace_size(ctypes.byref(p))
        nc = T // 64
        runs = 8  # the run split of this shape (64-column tiles: 768 units)
        assert ws >= 2 * B_ * nc * H * m * 4 + B_ * T * H * m * 2 + B_ * H * (runs - 1) * (K + V) * 64 * 4, m
        assert L.abc_bwd_workspace_size(ctypes.byref(p)) >= B_ * H * (runs - 1) * (K + V) * 64 * 4
    for m in (16, 48, 128):
        p = B.abc_problem(1, 128, 2, 64, m, 64, B.GDR_BF16)
        assert L.abc_workspace_size(ctypes.byref(p)) == 0, m
        args = [FAKE] * 3 + [None, FAKE, FAKE, None, None, FAKE, 1 << 20, None]
        assert L.abc_affine_scan(ctypes.byref(p), *args) == B.GDR_ERR_INVALID_ARG
        assert "M" in L.gdr_last_error().decode()
        rargs = [FAKE] * 7 + [ctypes.c_float(1.0), FAKE, None, None]
        assert L.abc_chunk_output(ctypes.byref(p), *rargs) == B.GDR_ERR_INVALID_ARG


def test_abc_read_validation():
    L = B.lib()
    p = B.abc_problem(1, 128, 2, 64, 64, 64, B.GDR_BF16)  # V = 64 is not built
    args = [FAKE] * 7 + [ctypes.c_float(1.0), FAKE, None, None]
    assert L.abc_chunk_output(ctypes.byref(p), *args) == B.GDR_ERR_UNSUPPORTED
    p = B.abc_problem(1, 128, 2, 256, 64, 512, B.GDR_BF16)
    bad = list(args)
    bad[4] = None  # z
    assert L.abc_chunk_output(ctypes.byref(p), *bad) == B.GDR_ERR_INVALID_ARG
    assert "z" in L.gdr_last_error().decode()


def test_kda_validation():
    """The per-channel decay entry points validate before any launch."""
    L = B.lib()
    p, keep = _prob(T=128, dtype=B.GDR_F32)
    args = [FAKE] * 9
    assert L.kda_chunk_prepare(ctypes.byref(p), *args, None) == B.GDR_ERR_UNSUPPORTED  # bfloat16 only
    p, keep = _prob(T=128)
    bad = [FAKE] * 9
    bad[2] = None  # g
    assert L.kda_chunk_prepare(ctypes.byref(p), *bad, None) == B.GDR_ERR_INVALID_ARG
    assert "g" in L.gdr_last_error().decode()
    assert L.kda_state_scan(ctypes.byref(p), None, None, FAKE, FAKE, FAKE, None, None, None, None, None,
                            None) == B.GDR_ERR_INVALID_ARG  # decay missing
    assert L.kda_chunk_output(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, ctypes.c_float(1.0), FAKE,
                              None) == B.GDR_ERR_INVALID_ARG  # g_cum missing
    assert L.kda_segment_summaries(ctypes.byref(p), None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == B.GDR_ERR_INVALID_ARG  # n_segments


def _scan_out(p, q=FAKE, k=FAKE, o=FAKE, h=None, v_new=None, seg=None, tile=None):
    t = None if tile is None else ctypes.byref(B.gdr_tile(*tile))
    s = None if seg is None else ctypes.byref(seg)
    return B.lib().gdr_state_scan_output(ctypes.byref(p), t, s, q, k, FAKE, FAKE, FAKE, None, ctypes.c_float(1.0),
                                         h, v_new, None, o, None)


def test_fused_scan_output_validation():
    L = B.lib()
    p, keep = _prob()
    assert _scan_out(p, q=None) == B.GDR_ERR_INVALID_ARG and "q" in L.gdr_last_error().decode()
    assert _scan_out(p, o=None) == B.GDR_ERR_INVALID_ARG and "o" in L.gdr_last_error().decode()
    assert _scan_out(p, q=ctypes.c_void_p(0x10004)) == B.GDR_ERR_INVALID_ARG
    assert _scan_out(p, seg=B.gdr_segments(0, FAKE.value)) == B.GDR_ERR_INVALID_ARG
    # without a fused kernel (float32 storage, or a tile that has none) h and v_new must be given
    p32, keep32 = _prob(dtype=B.GDR_F32)
    assert _scan_out(p32) == B.GDR_ERR_UNSUPPORTED and "h and v_new" in L.gdr_last_error().decode()
    assert _scan_out(p, tile=(32, 2, 2), h=FAKE) == B.GDR_ERR_UNSUPPORTED
    pool, keepp = _pool_prob([3, 0, 2], 4)
    assert _scan_out(pool, seg=B.gdr_segments(2, FAKE.value)) == B.GDR_ERR_UNSUPPORTED


def test_binding_rejects_mismatched_state_pools():
    """The Python binding checks the state pools before any call: the index
    list must have one entry per sequence, each pool must be float32 with the
    state's shape, and with two pools the smaller bounds the indices."""
    import torch

    k = torch.zeros((1, 20, 2, 128), dtype=torch.bfloat16)
    w, u = torch.zeros_like(k), torch.zeros((1, 20, 2, 128), dtype=torch.bfloat16)
    g = torch.zeros((1, 20, 2))
    cu = [0, 5, 12, 20]
    pool = torch.zeros((4, 2, 128, 128))
    with pytest.raises(ValueError, match="entries for 3 sequences"):
        B.gdr_state_scan(k, w, u, g, pool, cu, out={"hT": pool}, state_indices=[0, 1])
    with pytest.raises(ValueError, match="float32"):
        B.gdr_state_scan(k, w, u, g, pool, cu, out={"hT": pool.to(torch.bfloat16)}, state_indices=[0, 1, 2])
    with pytest.raises(ValueError, match="float32"):
        B.gdr_state_scan_output(k, k, w, u, g, 1.0, pool[:, :1], cu, out={"hT": pool}, state_indices=[0, 1, 2])
    small = torch.zeros((2, 2, 128, 128))
    assert B._pool_size(pool, small, k, 128, "kv") == 2
    assert B._pool_size(None, pool, k, 128, "kv") == 4
    with pytest.raises(ValueError):
        B._pool_size(torch.zeros((4, 2, 64, 128)), None, k, 128, "kv")


def test_noalloc_summaries_reject_oversized_problems():
    """gdr_segment_summaries_noalloc refuses, before any device call, a
    problem whose half-segment workspace exceeds the static scratch."""
    L = B.lib()
    cu = (ctypes.c_int32 * 2)(0, 65536)
    # 64K tokens x 13 heads x 16 segments: 2 * 16 * 13 * 128 * 256 * 4 bytes = 52 MiB > 48 MiB
    p = B.gdr_problem(1, 65536, 13, 128, 128, 1, cu, B.GDR_BF16, 0, None, 0)
    assert L.gdr_segment_summaries_workspace_size(ctypes.byref(p), 16) == 52 << 20
    s = L.gdr_segment_summaries_noalloc(ctypes.byref(p), None, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert s == B.GDR_ERR_INVALID_ARG
    assert "static scratch" in L.gdr_last_error().decode()
    bad = B.gdr_problem(1, 65536, 17, 128, 128, 1, cu, B.GDR_BF16, 0, None, 0)
    assert L.gdr_segment_summaries_noalloc(ctypes.byref(bad), None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           None) == B.GDR_ERR_INVALID_ARG


def _lens_problem(lengths, H, dtype=None, DK=128, DV=128, pool=None):
    cu = (ctypes.c_int32 * (len(lengths) + 1))(*([0] + list(np.cumsum(lengths))))
    ia = None if pool is None else (ctypes.c_int32 * len(pool))(*pool)
    p = B.gdr_problem(1, int(sum(lengths)), H, DK, DV, len(lengths), cu, B.GDR_BF16 if dtype is None else dtype, 0,
                      ia, 0 if pool is None else len(pool))
    return p, (cu, ia)


@pytest.mark.parametrize("lengths,H,want", [
    ([65536], 8, 16), ([65536], 1, 32), ([65536], 2, 32), ([65536], 4, 32), ([16384], 8, 16), ([16384], 2, 16),
    ([8192], 4, 16), ([4096], 16, 16), ([600], 2, 2), ([300], 1, 0),
    ([130, 139, 197, 245, 24, 50, 214, 244, 76, 91, 225, 118, 81, 215, 77, 114, 171, 148, 36, 22, 224, 197, 217, 145],
     16, 0),
    ([3597, 1827, 1359, 1941, 2295, 3526, 2410, 1306], 32, 0),
])
def test_plan_segments_rule(lengths, H, want):
    """The scheduler's segment count: the serial scan when the (sequence,
    head, 64-column) units fill half the GPU or the sequences are short, else
    16 (32 for up to four chains of 64K tokens), fewer when segments would
    drop below 4 chunks."""
    p, keep = _lens_problem(lengths, H)
    assert B.lib().gdr_plan_segments(ctypes.byref(p)) == want
    ws = B.lib().gdr_state_scan_auto_workspace_size(ctypes.byref(p))
    assert (ws == 0) == (want == 0)
    if want:
        n = want * H
        assert ws >= 3 * n * 128 * 128 * 4


def test_plan_segments_pools_and_wide_states_are_serial():
    p, keep = _lens_problem([65536], 2, pool=[0])
    assert B.lib().gdr_plan_segments(ctypes.byref(p)) == 0
    p, keep = _lens_problem([65536], 2, DK=256, DV=256)
    assert B.lib().gdr_plan_segments(ctypes.byref(p)) == 0
    bad = B.gdr_problem(1, 10, 2, 100, 128, 1, None, B.GDR_BF16, 0, None, 0)
    assert B.lib().gdr_plan_segments(ctypes.byref(bad)) == -1


def test_state_scan_auto_validates_before_launch():
    """Arguments are checked before any launch: q without o, a missing or
    small workspace."""
    L = B.lib()
    p, keep = _lens_problem([65536], 8)
    ws = L.gdr_state_scan_auto_workspace_size(ctypes.byref(p))
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, None, ctypes.c_float(1.0), FAKE, FAKE, FAKE]
    assert L.gdr_state_scan_auto(ctypes.byref(p), *args, None, FAKE, ws, None) == B.GDR_ERR_INVALID_ARG  # q, no o
    assert L.gdr_state_scan_auto(ctypes.byref(p), *args, FAKE, None, ws, None) == B.GDR_ERR_INVALID_ARG
    assert L.gdr_state_scan_auto(ctypes.byref(p), *args, FAKE, FAKE, ws - 16, None) == B.GDR_ERR_INVALID_ARG
    assert "workspace" in L.gdr_last_error().decode()


def _fwd(p, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE):
    return B.lib().gdr_chunk_forward(ctypes.byref(p), q, k, v, g, beta, None, ctypes.c_float(1.0), None, None, None,
                                     None, o, None)


def test_chunk_forward_validation():
    """The fused forward step checks its arguments before any launch: missing
    inputs are invalid, and problems outside its build (float32 storage,
    DK = 64, DV not a multiple of 64) are unsupported."""
    p, keep = _prob()
    for kw in ("q", "k", "v", "g", "beta", "o"):
        assert _fwd(p, **{kw: None}) == B.GDR_ERR_INVALID_ARG, kw
    q, keep3 = _prob(dtype=B.GDR_F32)
    assert _fwd(q) == B.GDR_ERR_UNSUPPORTED
    q, keep4 = _prob(DK=64)
    assert _fwd(q) == B.GDR_ERR_UNSUPPORTED


def test_plan_table_long_rows():
    """The plain pass takes 128-column blocks when 64-column blocks would exceed
    two per CU on long rows (16+ chunks per row on average), else 64-column
    blocks of four waves (the measured sweep behind the table)."""
    def packed(lengths, H, DK=128, DV=128):
        cu = [0]
        for n in lengths:
            cu.append(cu[-1] + n)
        return _prob(T=cu[-1], cu=cu, H=H, DK=DK, DV=DV)

    long8 = [1306, 1359, 1827, 1941, 2295, 2410, 3526, 3597]
    p, keep = packed(long8, 48)
    assert _query(p)[:3] == (128, 4, 2)
    p, keep = packed(long8, 32)  # 512 blocks of 64 columns: two per CU
    assert _query(p)[:3] == (64, 4, 2)
    p, keep = packed(long8, 48, DK=64, DV=64)  # one 64-column block per (row, head)
    assert _query(p)[:3] == (64, 4, 2)
    short = [16 + (37 * i) % 240 for i in range(24)]
    p, keep = packed(short, 48)
    assert _query(p)[:3] == (64, 4, 2)
