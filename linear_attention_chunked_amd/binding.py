"""ctypes binding of libgdr.so (include/gdr.h), same names as the C entry points.

This layer only marshals arguments: it reads shapes, allocates outputs with
torch on the inputs' device, passes raw device pointers and the current HIP
stream, and raises on any non-OK status.  Every arithmetic step runs in the
HIP kernels; there is no CPU fallback, and calling without the built library
or with CPU tensors raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdr.so")

GDR_OK, GDR_ERR_INVALID_ARG, GDR_ERR_UNSUPPORTED, GDR_ERR_HIP = 0, 1, 2, 3
GDR_F32, GDR_BF16 = 0, 1
GDR_STATE_KV, GDR_STATE_VK = 0, 1


class GdrError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class gdr_problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("T", ctypes.c_int64),
        ("H", ctypes.c_int32),
        ("DK", ctypes.c_int32),
        ("DV", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
        ("dtype", ctypes.c_int),
        ("state_layout", ctypes.c_int),
        ("state_indices_host", ctypes.POINTER(ctypes.c_int32)),
        ("pool_size", ctypes.c_int32),
    ]


class gdr_tile(ctypes.Structure):
    _fields_ = [("bv", ctypes.c_int32), ("waves", ctypes.c_int32), ("stages", ctypes.c_int32)]


class gdr_segments(ctypes.Structure):
    _fields_ = [("n_segments", ctypes.c_int32), ("seg_init", ctypes.c_void_p)]


class abc_problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("T", ctypes.c_int64),
        ("H", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("M", ctypes.c_int32),
        ("V", ctypes.c_int32),
        ("dtype", ctypes.c_int),
    ]


_P = ctypes.c_void_p
_SIGS = {
    "gdr_num_chunks": (ctypes.c_int64, [ctypes.POINTER(gdr_problem)]),
    "gdr_chunk_prepare": (ctypes.c_int, [ctypes.POINTER(gdr_problem), _P, _P, _P, _P, _P, _P, _P, _P]),
    "gdr_state_scan": (ctypes.c_int, [ctypes.POINTER(gdr_problem), ctypes.POINTER(gdr_tile),
                                      ctypes.POINTER(gdr_segments), _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "gdr_chunk_output": (ctypes.c_int, [ctypes.POINTER(gdr_problem), _P, _P, _P, _P, _P, ctypes.c_float, _P, _P]),
    "gdr_state_scan_output": (ctypes.c_int, [ctypes.POINTER(gdr_problem), ctypes.POINTER(gdr_tile),
                                             ctypes.POINTER(gdr_segments), _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                             _P, _P, _P, _P, _P]),
    "gdr_chunk_forward": (ctypes.c_int, [ctypes.POINTER(gdr_problem), _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                         _P, _P, _P, _P, _P, _P]),
    "gdr_segment_summaries": (ctypes.c_int, [ctypes.POINTER(gdr_problem), ctypes.POINTER(gdr_tile), ctypes.c_int32,
                                             _P, _P, _P, _P, _P, _P, _P]),
    "gdr_segment_summaries_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(gdr_problem), ctypes.c_int32]),
    "gdr_segment_summaries_ws": (ctypes.c_int, [ctypes.POINTER(gdr_problem), ctypes.POINTER(gdr_tile),
                                                ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "gdr_segment_summaries_noalloc": (ctypes.c_int, [ctypes.POINTER(gdr_problem), ctypes.POINTER(gdr_tile),
                                                     ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P]),
    "gdr_segment_compose": (ctypes.c_int, [ctypes.POINTER(gdr_problem), ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
    "kda_chunk_prepare": (ctypes.c_int, [ctypes.POINTER(gdr_problem), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "kda_state_scan": (ctypes.c_int, [ctypes.POINTER(gdr_problem), ctypes.POINTER(gdr_tile),
                                      ctypes.POINTER(gdr_segments), _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "kda_segment_summaries": (ctypes.c_int, [ctypes.POINTER(gdr_problem), ctypes.POINTER(gdr_tile), ctypes.c_int32,
                                             _P, _P, _P, _P, _P, _P, _P]),
    "kda_chunk_output": (ctypes.c_int, [ctypes.POINTER(gdr_problem), _P, _P, _P, _P, _P, ctypes.c_float, _P, _P]),
    "gdr_chunk_dv_local": (ctypes.c_int, [ctypes.POINTER(gdr_problem), _P, _P, _P, _P, ctypes.c_float, _P, _P]),
    "gdr_state_scan_bwd": (ctypes.c_int, [ctypes.POINTER(gdr_problem), _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                          _P, _P, _P, _P]),
    "abc_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(abc_problem)]),
    "abc_affine_scan": (ctypes.c_int, [ctypes.POINTER(abc_problem), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]),
    "abc_bwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(abc_problem)]),
    "abc_chunk_output": (ctypes.c_int, [ctypes.POINTER(abc_problem), _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P,
                                        _P, _P]),
    "abc_affine_scan_bwd": (ctypes.c_int, [ctypes.POINTER(abc_problem), _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                           _P, _P, _P, ctypes.c_size_t, _P]),
    "gdr_plan_segments": (ctypes.c_int32, [ctypes.POINTER(gdr_problem)]),
    "gdr_state_scan_auto_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(gdr_problem)]),
    "gdr_state_scan_auto": (ctypes.c_int, [ctypes.POINTER(gdr_problem), _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                           _P, _P, _P, ctypes.c_size_t, _P]),
    "gdr_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gdr_last_error": (ctypes.c_char_p, []),
    "gdr_plan_query": (ctypes.c_int, [ctypes.POINTER(gdr_problem), ctypes.POINTER(gdr_tile), ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int64)]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libgdr.so (raises ImportError if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first (python -c "
                              "'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != GDR_OK:
        L = lib()
        raise GdrError(status, f"{what}: {L.gdr_status_string(status).decode()}: {L.gdr_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("all tensors must be on the GPU (there is no CPU path)")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return GDR_F32
    if dt == torch.bfloat16:
        return GDR_BF16
    raise ValueError(f"unsupported storage dtype {dt}")


class Problem:
    """A gdr_problem plus the host cu_seqlens it points to (kept alive)."""

    def __init__(self, k: torch.Tensor, DV: int, cu_seqlens=None, state_layout: str = "kv", state_indices=None,
                 pool_size: int = 0):
        B, T, H, DK = k.shape
        self._cu = None
        self._idx = None
        if cu_seqlens is not None:
            cu = [int(x) for x in (cu_seqlens.tolist() if torch.is_tensor(cu_seqlens) else cu_seqlens)]
            N = len(cu) - 1
            self._cu = (ctypes.c_int32 * len(cu))(*cu)
            cu_ptr = self._cu
        else:
            N = B
            cu_ptr = None
        idx_ptr = None
        if state_indices is not None:
            idx = [int(x) for x in (state_indices.tolist() if torch.is_tensor(state_indices) else state_indices)]
            if len(idx) != N:
                raise ValueError(f"state_indices has {len(idx)} entries for {N} sequences")
            self._idx = (ctypes.c_int32 * max(1, len(idx)))(*idx)
            idx_ptr = self._idx
        self.s = gdr_problem(B, T, H, DK, DV, N, cu_ptr, _dtype_code(k.dtype),
                             GDR_STATE_VK if state_layout == "vk" else GDR_STATE_KV, idx_ptr, int(pool_size))
        self.B, self.T, self.H, self.DK, self.DV, self.N = B, T, H, DK, DV, N

    @property
    def ref(self):
        return ctypes.byref(self.s)


def _pool_size(h0, hT, k, DV, state_layout) -> int:
    """Entries of the state pools h0 / hT addressed by state_indices: each
    given pool must be a float32 [pool_size, H, DK, DV] (or [.., DV, DK] for
    the "vk" layout) tensor; with two pools of different sizes the smaller
    bounds the indices, so no index can reach past either pool."""
    H, DK = k.shape[2], k.shape[3]
    state = (H, DV, DK) if state_layout == "vk" else (H, DK, DV)
    sizes = []
    for name, t in (("h0", h0), ("hT", hT)):
        if t is None:
            continue
        if t.dtype != torch.float32 or t.dim() != 4 or tuple(t.shape[1:]) != state:
            raise ValueError(f"state pool {name} must be float32 [pool_size, {state[0]}, {state[1]}, {state[2]}], "
                             f"got {t.dtype} {tuple(t.shape)}")
        sizes.append(int(t.shape[0]))
    if not sizes:
        raise ValueError("indexed states need a pool (h0 or hT)")
    return min(sizes)


def _tile(tile) -> Optional[gdr_tile]:
    if tile is None:
        return None
    bv, waves, stages = tile
    return gdr_tile(bv, waves, stages)


def gdr_num_chunks(k: torch.Tensor, DV: int, cu_seqlens=None) -> int:
    n = lib().gdr_num_chunks(Problem(k, DV, cu_seqlens).ref)
    if n < 0:
        _check(GDR_ERR_INVALID_ARG, "gdr_num_chunks")
    return int(n)


def gdr_plan_query(k: torch.Tensor, DV: int, cu_seqlens=None, tile=None, n_segments: int = 0):
    """(bv, waves, stages, workgroups, launches, max rows per launch) the scheduler picks."""
    out = (ctypes.c_int64 * 6)()
    p = Problem(k, DV, cu_seqlens)
    t = _tile(tile)
    _check(lib().gdr_plan_query(p.ref, ctypes.byref(t) if t is not None else None, n_segments, out),
           "gdr_plan_query")
    return tuple(int(x) for x in out)


def gdr_chunk_prepare(k, v, g, beta, cu_seqlens=None, stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """WY factors: returns (g_cum float32 [B,T,H], w [B,T,H,DK], u [B,T,H,DV])."""
    p = Problem(k, v.shape[-1], cu_seqlens)
    g_cum = torch.empty(g.shape, dtype=torch.float32, device=k.device)
    w = torch.empty_like(k)
    u = torch.empty_like(v)
    _check(lib().gdr_chunk_prepare(p.ref, _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(g_cum), _ptr(w), _ptr(u),
                                   _stream(stream)), "gdr_chunk_prepare")
    return g_cum, w, u


def gdr_state_scan(k, w, u, g_cum, h0=None, cu_seqlens=None, tile=None, n_segments: Optional[int] = None,
                   seg_init=None, state_layout: str = "kv", emit_h: bool = True, emit_v_new: bool = True,
                   emit_final: bool = True, out=None, state_indices=None, stream=None):
    """Returns (h [NT,H,DV,DK] | None, v_new | None, hT [N,H,DK,DV] fp32 | None).

    ``out`` may hold preallocated "h", "v_new" and "hT" tensors to write into.
    With ``state_indices`` (N ints), h0 and out["hT"] are state pools
    [pool_size, H, ...]: sequence n reads h0[idx[n]] and writes hT[idx[n]]
    (the same tensor for an in-place update)."""
    DV = u.shape[-1]
    out = out or {}
    pool_size = 0
    if state_indices is not None:
        if emit_final and out.get("hT") is None:
            raise ValueError("indexed states write into a pool: pass out={'hT': pool}")
        pool_size = _pool_size(h0, out.get("hT") if emit_final else None, k, DV, state_layout)
    p = Problem(k, DV, cu_seqlens, state_layout, state_indices, pool_size)
    L = lib()
    nt = gdr_num_chunks(k, DV, cu_seqlens)
    h = v_new = hT = None
    if emit_h:
        h = out.get("h")
        if h is None:
            h = torch.empty((nt, p.H, DV, p.DK), dtype=k.dtype, device=k.device)
    if emit_v_new:
        v_new = out.get("v_new")
        if v_new is None:
            v_new = torch.empty_like(u)
    if emit_final:
        hT = out.get("hT")
        if hT is None:
            shape = (p.N, p.H, DV, p.DK) if state_layout == "vk" else (p.N, p.H, p.DK, DV)
            hT = torch.empty(shape, dtype=torch.float32, device=k.device)
    t = _tile(tile)
    seg = None
    if n_segments is not None:
        if seg_init is None or not seg_init.is_cuda:
            raise ValueError("the segmented pass needs seg_init on the GPU")
        seg = gdr_segments(n_segments, seg_init.data_ptr())
    _check(L.gdr_state_scan(p.ref, ctypes.byref(t) if t is not None else None,
                            ctypes.byref(seg) if seg is not None else None,
                            _ptr(k), _ptr(w), _ptr(u), _ptr(g_cum), _ptr(h0), _ptr(h), _ptr(v_new), _ptr(hT),
                            _stream(stream)), "gdr_state_scan")
    return h, v_new, hT


def gdr_state_scan_output(q, k, w, u, g_cum, scale: float = 1.0, h0=None, cu_seqlens=None, tile=None,
                          n_segments: Optional[int] = None, seg_init=None, state_layout: str = "kv",
                          emit_h: bool = True, emit_v_new: bool = True, emit_final: bool = True, out=None,
                          state_indices=None, stream=None):
    """The state scan with the chunk output fused: returns (o, h | None, v_new | None, hT | None), the
    same tensors as ``gdr_state_scan`` followed by ``gdr_chunk_output``.  ``out`` may hold preallocated
    "o", "h", "v_new" and "hT"; other arguments as in ``gdr_state_scan``."""
    DV = u.shape[-1]
    out = out or {}
    pool_size = 0
    if state_indices is not None:
        if emit_final and out.get("hT") is None:
            raise ValueError("indexed states write into a pool: pass out={'hT': pool}")
        pool_size = _pool_size(h0, out.get("hT") if emit_final else None, k, DV, state_layout)
    p = Problem(k, DV, cu_seqlens, state_layout, state_indices, pool_size)
    nt = gdr_num_chunks(k, DV, cu_seqlens)
    o = out.get("o")
    if o is None:
        o = torch.empty_like(u)
    h = v_new = hT = None
    if emit_h:
        h = out.get("h")
        if h is None:
            h = torch.empty((nt, p.H, DV, p.DK), dtype=k.dtype, device=k.device)
    if emit_v_new:
        v_new = out.get("v_new")
        if v_new is None:
            v_new = torch.empty_like(u)
    if emit_final:
        hT = out.get("hT")
        if hT is None:
            shape = (p.N, p.H, DV, p.DK) if state_layout == "vk" else (p.N, p.H, p.DK, DV)
            hT = torch.empty(shape, dtype=torch.float32, device=k.device)
    t = _tile(tile)
    seg = None
    if n_segments is not None:
        if seg_init is None or not seg_init.is_cuda:
            raise ValueError("the segmented pass needs seg_init on the GPU")
        seg = gdr_segments(n_segments, seg_init.data_ptr())
    _check(lib().gdr_state_scan_output(p.ref, ctypes.byref(t) if t is not None else None,
                                       ctypes.byref(seg) if seg is not None else None,
                                       _ptr(q), _ptr(k), _ptr(w), _ptr(u), _ptr(g_cum), _ptr(h0), float(scale),
                                       _ptr(h), _ptr(v_new), _ptr(hT), _ptr(o), _stream(stream)),
           "gdr_state_scan_output")
    return o, h, v_new, hT


def gdr_chunk_forward(q, k, v, g, beta, scale: float = 1.0, h0=None, cu_seqlens=None, state_layout: str = "kv",
                      emit_g_cum: bool = True, emit_h: bool = True, emit_v_new: bool = True, emit_final: bool = True,
                      out=None, state_indices=None, stream=None):
    """The forward step in one kernel (chunk prepare, state scan and chunk
    output fused): returns (o, g_cum | None, h | None, v_new | None, hT | None),
    the same bits as ``gdr_chunk_prepare`` followed by
    ``gdr_state_scan_output``.  bfloat16, DK = 128, DV a multiple of 64 (else
    GdrError GDR_ERR_UNSUPPORTED).  ``out`` may hold preallocated "o",
    "g_cum", "h", "v_new" and "hT"; other arguments as in ``gdr_state_scan``."""
    DV = v.shape[-1]
    out = out or {}
    pool_size = 0
    if state_indices is not None:
        if emit_final and out.get("hT") is None:
            raise ValueError("indexed states write into a pool: pass out={'hT': pool}")
        pool_size = _pool_size(h0, out.get("hT") if emit_final else None, k, DV, state_layout)
    p = Problem(k, DV, cu_seqlens, state_layout, state_indices, pool_size)
    nt = gdr_num_chunks(k, DV, cu_seqlens)
    o = out.get("o")
    if o is None:
        o = torch.empty_like(v)
    g_cum = h = v_new = hT = None
    if emit_g_cum:
        g_cum = out.get("g_cum")
        if g_cum is None:
            g_cum = torch.empty(g.shape, dtype=torch.float32, device=k.device)
    if emit_h:
        h = out.get("h")
        if h is None:
            h = torch.empty((nt, p.H, DV, p.DK), dtype=k.dtype, device=k.device)
    if emit_v_new:
        v_new = out.get("v_new")
        if v_new is None:
            v_new = torch.empty_like(v)
    if emit_final:
        hT = out.get("hT")
        if hT is None:
            shape = (p.N, p.H, DV, p.DK) if state_layout == "vk" else (p.N, p.H, p.DK, DV)
            hT = torch.empty(shape, dtype=torch.float32, device=k.device)
    _check(lib().gdr_chunk_forward(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), float(scale),
                                   _ptr(g_cum), _ptr(h), _ptr(v_new), _ptr(hT), _ptr(o), _stream(stream)),
           "gdr_chunk_forward")
    return o, g_cum, h, v_new, hT


def gdr_chunk_output(q, k, v_new, h, g_cum, scale: float = 1.0, cu_seqlens=None, stream=None) -> torch.Tensor:
    p = Problem(k, v_new.shape[-1], cu_seqlens)
    o = torch.empty_like(v_new)
    _check(lib().gdr_chunk_output(p.ref, _ptr(q), _ptr(k), _ptr(v_new), _ptr(h), _ptr(g_cum), float(scale), _ptr(o),
                                  _stream(stream)), "gdr_chunk_output")
    return o


def gdr_segment_summaries(k, w, u, g_cum, n_segments: int, cu_seqlens=None, tile=None, stream=None,
                          workspace: bool = True):
    """Returns (seg_state [N*P,H,DV,DK], seg_trans [N*P,H,DK,DK]) float32.

    With ``workspace`` (the default) the call passes the device workspace
    ``gdr_segment_summaries_workspace_size`` asks for (the half-segment form
    when it is nonzero); ``workspace=False`` calls the direct form."""
    DV = u.shape[-1]
    p = Problem(k, DV, cu_seqlens)
    seg_state = torch.empty((p.N * n_segments, p.H, DV, p.DK), dtype=torch.float32, device=k.device)
    seg_trans = torch.empty((p.N * n_segments, p.H, p.DK, p.DK), dtype=torch.float32, device=k.device)
    t = _tile(tile)
    L = lib()
    tp = ctypes.byref(t) if t is not None else None
    ws_bytes = int(L.gdr_segment_summaries_workspace_size(p.ref, n_segments)) if workspace else 0
    if ws_bytes > 0:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=k.device)
        _check(L.gdr_segment_summaries_ws(p.ref, tp, n_segments, _ptr(k), _ptr(w), _ptr(u), _ptr(g_cum),
                                          _ptr(seg_state), _ptr(seg_trans), _ptr(ws), ws_bytes, _stream(stream)),
               "gdr_segment_summaries_ws")
    else:
        _check(L.gdr_segment_summaries(p.ref, tp, n_segments, _ptr(k), _ptr(w), _ptr(u), _ptr(g_cum),
                                       _ptr(seg_state), _ptr(seg_trans), _stream(stream)), "gdr_segment_summaries")
    return seg_state, seg_trans


def gdr_segment_summaries_noalloc(k, w, u, g_cum, n_segments: int, cu_seqlens=None, tile=None, out=None,
                                  stream=None):
    """gdr_segment_summaries with the library's static scratch as the
    half-segment workspace (the C call allocates nothing).  ``out`` may hold
    preallocated "seg_state" and "seg_trans".  Returns (seg_state, seg_trans)."""
    DV = u.shape[-1]
    p = Problem(k, DV, cu_seqlens)
    out = out or {}
    seg_state = out.get("seg_state")
    if seg_state is None:
        seg_state = torch.empty((p.N * n_segments, p.H, DV, p.DK), dtype=torch.float32, device=k.device)
    seg_trans = out.get("seg_trans")
    if seg_trans is None:
        seg_trans = torch.empty((p.N * n_segments, p.H, p.DK, p.DK), dtype=torch.float32, device=k.device)
    t = _tile(tile)
    _check(lib().gdr_segment_summaries_noalloc(p.ref, ctypes.byref(t) if t is not None else None, n_segments,
                                               _ptr(k), _ptr(w), _ptr(u), _ptr(g_cum), _ptr(seg_state),
                                               _ptr(seg_trans), _stream(stream)), "gdr_segment_summaries_noalloc")
    return seg_state, seg_trans


def gdr_segment_summaries_workspace_size(k, DV: int, n_segments: int, cu_seqlens=None) -> int:
    """Bytes of device workspace the half-segment summaries need (0: direct form)."""
    p = Problem(k, DV, cu_seqlens)
    return int(lib().gdr_segment_summaries_workspace_size(p.ref, n_segments))


def gdr_segment_compose(k, DV: int, seg_state, seg_trans, n_segments: int, h0=None, cu_seqlens=None,
                        state_layout: str = "kv", emit_final: bool = False, stream=None):
    """Returns (seg_init [N*P,H,DV,DK] fp32, hT | None)."""
    p = Problem(k, DV, cu_seqlens, state_layout)
    seg_init = torch.empty_like(seg_state)
    hT = None
    if emit_final:
        shape = (p.N, p.H, DV, p.DK) if state_layout == "vk" else (p.N, p.H, p.DK, DV)
        hT = torch.empty(shape, dtype=torch.float32, device=k.device)
    _check(lib().gdr_segment_compose(p.ref, n_segments, _ptr(seg_state), _ptr(seg_trans), _ptr(h0), _ptr(seg_init),
                                     _ptr(hT), _stream(stream)), "gdr_segment_compose")
    return seg_init, hT


def kda_chunk_prepare(k, v, g, beta, cu_seqlens=None, stream=None):
    """Per-channel-decay WY factors: returns (g_cum [B,T,H,DK] fp32, w, u, kg, decay [NT,H,DK] fp32)."""
    DV = v.shape[-1]
    p = Problem(k, DV, cu_seqlens)
    nt = gdr_num_chunks(k, DV, cu_seqlens)
    g_cum = torch.empty(g.shape, dtype=torch.float32, device=k.device)
    w = torch.empty_like(k)
    u = torch.empty_like(v)
    kg = torch.empty_like(k)
    decay = torch.empty((nt, p.H, p.DK), dtype=torch.float32, device=k.device)
    _check(lib().kda_chunk_prepare(p.ref, _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(g_cum), _ptr(w), _ptr(u),
                                   _ptr(kg), _ptr(decay), _stream(stream)), "kda_chunk_prepare")
    return g_cum, w, u, kg, decay


def kda_state_scan(kg, w, u, decay, h0=None, cu_seqlens=None, tile=None, n_segments: Optional[int] = None,
                   seg_init=None, state_layout: str = "kv", emit_h: bool = True, emit_v_new: bool = True,
                   emit_final: bool = True, stream=None):
    """Per-channel-decay state scan.  Returns (h [NT,H,DV,DK] | None, v_new | None, hT | None)."""
    DV = u.shape[-1]
    p = Problem(kg, DV, cu_seqlens, state_layout)
    nt = gdr_num_chunks(kg, DV, cu_seqlens)
    h = torch.empty((nt, p.H, DV, p.DK), dtype=kg.dtype, device=kg.device) if emit_h else None
    v_new = torch.empty_like(u) if emit_v_new else None
    hT = None
    if emit_final:
        shape = (p.N, p.H, DV, p.DK) if state_layout == "vk" else (p.N, p.H, p.DK, DV)
        hT = torch.empty(shape, dtype=torch.float32, device=kg.device)
    t = _tile(tile)
    seg = None
    if n_segments is not None:
        if seg_init is None or not seg_init.is_cuda:
            raise ValueError("the segmented pass needs seg_init on the GPU")
        seg = gdr_segments(n_segments, seg_init.data_ptr())
    _check(lib().kda_state_scan(p.ref, ctypes.byref(t) if t is not None else None,
                                ctypes.byref(seg) if seg is not None else None, _ptr(kg), _ptr(w), _ptr(u),
                                _ptr(decay), _ptr(h0), _ptr(h), _ptr(v_new), _ptr(hT), _stream(stream)),
           "kda_state_scan")
    return h, v_new, hT


def kda_segment_summaries(kg, w, u, decay, n_segments: int, cu_seqlens=None, tile=None, stream=None):
    """Returns (seg_state [N*P,H,DV,DK], seg_trans [N*P,H,DK,DK]) float32."""
    DV = u.shape[-1]
    p = Problem(kg, DV, cu_seqlens)
    seg_state = torch.empty((p.N * n_segments, p.H, DV, p.DK), dtype=torch.float32, device=kg.device)
    seg_trans = torch.empty((p.N * n_segments, p.H, p.DK, p.DK), dtype=torch.float32, device=kg.device)
    t = _tile(tile)
    _check(lib().kda_segment_summaries(p.ref, ctypes.byref(t) if t is not None else None, n_segments, _ptr(kg),
                                       _ptr(w), _ptr(u), _ptr(decay), _ptr(seg_state), _ptr(seg_trans),
                                       _stream(stream)), "kda_segment_summaries")
    return seg_state, seg_trans


def kda_chunk_output(q, k, v_new, h, g_cum, scale: float = 1.0, cu_seqlens=None, stream=None) -> torch.Tensor:
    p = Problem(k, v_new.shape[-1], cu_seqlens)
    o = torch.empty_like(v_new)
    _check(lib().kda_chunk_output(p.ref, _ptr(q), _ptr(k), _ptr(v_new), _ptr(h), _ptr(g_cum), float(scale), _ptr(o),
                                  _stream(stream)), "kda_chunk_output")
    return o


def chunk_kda(q, k, v, g, beta, scale: float = 1.0, h0=None, cu_seqlens=None, tile=None, stream=None):
    """The whole per-channel-decay forward: prepare, state scan, output.
    Returns (o, hT, h, v_new)."""
    g_cum, w, u, kg, decay = kda_chunk_prepare(k, v, g, beta, cu_seqlens, stream)
    h, v_new, hT = kda_state_scan(kg, w, u, decay, h0, cu_seqlens, tile, stream=stream)
    o = kda_chunk_output(q, k, v_new, h, g_cum, scale, cu_seqlens, stream)
    return o, hT, h, v_new


def abc_workspace_size(B: int, T: int, H: int, K: int, M: int, V: int, dtype=torch.bfloat16) -> int:
    p = abc_problem(B, T, H, K, M, V, _dtype_code(dtype))
    return int(lib().abc_workspace_size(ctypes.byref(p)))


def abc_affine_scan(k, v, s, emit_z: bool = False, emit_final: bool = True, stream=None):
    """Returns (z | None, hk [B,NC,H,K,M], hv [B,NC,H,M,V], hk_final | None, hv_final | None)."""
    B, T, H, K = k.shape
    V = v.shape[-1]
    M = s.shape[-1]
    NC = (T + 63) // 64
    p = abc_problem(B, T, H, K, M, V, _dtype_code(k.dtype))
    L = lib()
    ws_bytes = int(L.abc_workspace_size(ctypes.byref(p)))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=k.device)
    z = torch.empty((B, T, H, M), dtype=torch.float32, device=k.device) if emit_z else None
    hk = torch.empty((B, NC, H, K, M), dtype=k.dtype, device=k.device)
    hv = torch.empty((B, NC, H, M, V), dtype=k.dtype, device=k.device)
    hkf = torch.empty((B, H, K, M), dtype=torch.float32, device=k.device) if emit_final else None
    hvf = torch.empty((B, H, M, V), dtype=torch.float32, device=k.device) if emit_final else None
    _check(L.abc_affine_scan(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(s), _ptr(z), _ptr(hk), _ptr(hv), _ptr(hkf),
                             _ptr(hvf), _ptr(ws), ws_bytes, _stream(stream)), "abc_affine_scan")
    return z, hk, hv, hkf, hvf


def abc_chunk_output(q, k, v, s, z, hk, hv, scale: float = 1.0, emit_p: bool = False, stream=None):
    """ABC read per chunk.  Returns (o [B,T,H,V], p [B,T,H,M] | None)."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    M = s.shape[-1]
    pr = abc_problem(B, T, H, K, M, V, _dtype_code(q.dtype))
    o = torch.empty((B, T, H, V), dtype=q.dtype, device=q.device)
    p = torch.empty((B, T, H, M), dtype=q.dtype, device=q.device) if emit_p else None
    _check(lib().abc_chunk_output(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(z), _ptr(hk), _ptr(hv),
                                  float(scale), _ptr(o), _ptr(p), _stream(stream)), "abc_chunk_output")
    return o, p


def abc_forward(q, k, v, s, scale: float = 1.0, emit_p: bool = False, stream=None):
    """The whole ABC forward: normaliser and slot states (abc_affine_scan),
    then the chunk read.  Returns (o, p | None, z, hk, hv)."""
    z, hk, hv, _, _ = abc_affine_scan(k, v, s, emit_z=True, emit_final=False, stream=stream)
    o, p = abc_chunk_output(q, k, v, s, z, hk, hv, scale, emit_p, stream)
    return o, p, z, hk, hv


def abc_affine_scan_bwd(q, dscore, p, dO, z, dhk_final=None, dhv_final=None, scale: float = 1.0, stream=None):
    """Reverse (dH) walk of the ABC slot states.  Returns (dhk [B,NC,H,K,M],
    dhv [B,NC,H,M,V]) in the storage dtype: the gradients of the states after
    every chunk."""
    B, T, H, K = q.shape
    V = dO.shape[-1]
    M = dscore.shape[-1]
    NC = (T + 63) // 64
    pr = abc_problem(B, T, H, K, M, V, _dtype_code(q.dtype))
    L = lib()
    ws_bytes = int(L.abc_bwd_workspace_size(ctypes.byref(pr)))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    dhk = torch.empty((B, NC, H, K, M), dtype=q.dtype, device=q.device)
    dhv = torch.empty((B, NC, H, M, V), dtype=q.dtype, device=q.device)
    _check(L.abc_affine_scan_bwd(ctypes.byref(pr), _ptr(q), _ptr(dscore), _ptr(p), _ptr(dO), _ptr(z),
                                 _ptr(dhk_final), _ptr(dhv_final), float(scale), _ptr(dhk), _ptr(dhv), _ptr(ws),
                                 ws_bytes, _stream(stream)), "abc_affine_scan_bwd")
    return dhk, dhv


def gdr_chunk_dv_local(q, k, g_cum, dO, scale: float = 1.0, cu_seqlens=None, stream=None) -> torch.Tensor:
    """Chunk-local part of the write-vector gradient, scale P^T dO, per chunk."""
    p = Problem(k, dO.shape[-1], cu_seqlens)
    dvl = torch.empty_like(dO)
    _check(lib().gdr_chunk_dv_local(p.ref, _ptr(q), _ptr(k), _ptr(g_cum), _ptr(dO), float(scale), _ptr(dvl),
                                    _stream(stream)), "gdr_chunk_dv_local")
    return dvl


def gdr_state_scan_bwd(q, k, w, g_cum, dO, dv_local, dhT=None, scale: float = 1.0, cu_seqlens=None,
                       state_layout: str = "kv", emit_dh: bool = True, emit_dv: bool = True, emit_dh0: bool = True,
                       stream=None):
    """Reverse state scan.  Returns (dh [NT,H,DV,DK] | None, dv_new_grad [B,T,H,DV] | None,
    dh0 [N,H,DK,DV] fp32 (or [N,H,DV,DK] for "vk") | None)."""
    DV = dO.shape[-1]
    p = Problem(k, DV, cu_seqlens, state_layout)
    nt = gdr_num_chunks(k, DV, cu_seqlens)
    dh = torch.empty((nt, p.H, DV, p.DK), dtype=k.dtype, device=k.device) if emit_dh else None
    dv = torch.empty_like(dO) if emit_dv else None
    shape = (p.N, p.H, DV, p.DK) if state_layout == "vk" else (p.N, p.H, p.DK, DV)
    dh0 = torch.empty(shape, dtype=torch.float32, device=k.device) if emit_dh0 else None
    _check(lib().gdr_state_scan_bwd(p.ref, _ptr(q), _ptr(k), _ptr(w), _ptr(g_cum), _ptr(dO), _ptr(dv_local),
                                    _ptr(dhT), float(scale), _ptr(dh), _ptr(dv), _ptr(dh0), _stream(stream)),
           "gdr_state_scan_bwd")
    return dh, dv, dh0


def gdr_plan_segments(k, DV: int, cu_seqlens=None) -> int:
    """Segments per sequence the scheduler picks for this problem (0 = the serial scan)."""
    n = int(lib().gdr_plan_segments(Problem(k, DV, cu_seqlens).ref))
    if n < 0:
        _check(GDR_ERR_INVALID_ARG, "gdr_plan_segments")
    return n


def gdr_state_scan_auto(q, k, w, u, g_cum, scale: float = 1.0, h0=None, cu_seqlens=None, out=None, stream=None):
    """The state scan (with the chunk output fused when q is given) with the
    scheduler's segmentation: returns (o | None, h, v_new, hT).  ``out`` may
    hold preallocated "o", "h", "v_new", "hT" and "workspace" tensors."""
    DV = u.shape[-1]
    out = out or {}
    p = Problem(k, DV, cu_seqlens)
    L = lib()
    nt = gdr_num_chunks(k, DV, cu_seqlens)
    h = out.get("h")
    if h is None:
        h = torch.empty((nt, p.H, DV, p.DK), dtype=k.dtype, device=k.device)
    v_new = out.get("v_new")
    if v_new is None:
        v_new = torch.empty_like(u)
    hT = out.get("hT")
    if hT is None:
        hT = torch.empty((p.N, p.H, p.DK, DV), dtype=torch.float32, device=k.device)
    o = None
    if q is not None:
        o = out.get("o")
        if o is None:
            o = torch.empty_like(u)
    ws_bytes = int(L.gdr_state_scan_auto_workspace_size(p.ref))
    ws = out.get("workspace")
    if ws_bytes > 0 and (ws is None or ws.numel() * ws.element_size() < ws_bytes):
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=k.device)
    _check(L.gdr_state_scan_auto(p.ref, _ptr(q), _ptr(k), _ptr(w), _ptr(u), _ptr(g_cum), _ptr(h0), float(scale),
                                 _ptr(h), _ptr(v_new), _ptr(hT), _ptr(o), _ptr(ws) if ws_bytes > 0 else None,
                                 ws_bytes, _stream(stream)), "gdr_state_scan_auto")
    return o, h, v_new, hT


def chunk_gated_delta_rule(q, k, v, g, beta, h0=None, cu_seqlens=None, scale: float = 1.0,
                           n_segments: Optional[int] = None, tile=None, stream=None) -> dict:
    """The whole forward path: prepare -> scan with the chunk output fused
    into the scan where a fused kernel exists (else scan, then output).  The
    scan is split into segments (summaries + compose + segmented pass) as the
    scheduler chooses when n_segments is None (gdr_state_scan_auto), serial
    with n_segments = 0, and split into n_segments when that is >= 1.  Returns
    a dict with o, h, v_new, hT, g_cum, w, u (and seg_state, seg_trans,
    seg_init for an explicit split)."""
    g_cum, w, u = gdr_chunk_prepare(k, v, g, beta, cu_seqlens, stream)
    out = {"g_cum": g_cum, "w": w, "u": u}
    if n_segments is None and tile is None:
        o, h, v_new, hT = gdr_state_scan_auto(q, k, w, u, g_cum, scale, h0, cu_seqlens, stream=stream)
    elif not n_segments:
        o, h, v_new, hT = gdr_state_scan_output(q, k, w, u, g_cum, scale, h0, cu_seqlens, tile, stream=stream)
    else:
        seg_state, seg_trans = gdr_segment_summaries(k, w, u, g_cum, n_segments, cu_seqlens, tile, stream)
        seg_init, _ = gdr_segment_compose(k, v.shape[-1], seg_state, seg_trans, n_segments, h0, cu_seqlens,
                                          stream=stream)
        o, h, v_new, hT = gdr_state_scan_output(q, k, w, u, g_cum, scale, None, cu_seqlens, tile, n_segments,
                                                seg_init, stream=stream)
        out.update(seg_state=seg_state, seg_trans=seg_trans, seg_init=seg_init)
    out.update(o=o, h=h, v_new=v_new, hT=hT)
    return out
