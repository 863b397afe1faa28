"""Throughput of the gated-delta state-scan path on one MI355X.

One step = one pass of the whole forward path over one batch of the
synthetic "question rows" workload (24 packed sequences of 16..256 tokens,
16 heads, dk = dv = 128, bfloat16 q/k/v, FP32 initial and final states):
chunk preparation -> inter-chunk state scan -> chunk output.  Inputs are
resident in HBM before the timed region; W untimed warm-up steps, then K
timed steps between two device synchronisations.

Printed (one JSON line): token-heads per second of the whole step (in
Mtok-head/s), plus
  roofline      the state scan (the dominant kernel): algorithmic bytes per
                launch / its mean duration from HIP events recorded around
                each scan launch inside the timed region, against 8 TB/s;
  cpu_baseline  the FP64 numpy oracle timed on the host on the same batch;
  long_state    the 64K-token single-sequence workload (8 heads), serial
                and 16-segment (whole path and each phase), measured after
                the timed region.
The roofline fractions are also given against the measured rate of a plain
512 MiB device copy ("copy_gbs", "frac_of_copy").
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ROOF_REPS = 30
SETTLE_MS = 50.0  # untimed back-to-back work before each timed measurement (see settle())
BF16_PEAK_TFLOPS = 2500.0


def scan_alg_bytes(lengths, H, DK, DV, in_bytes, h_bytes, has_h0, has_hT):
    """Bytes the state scan must move: read k, w (DK each), u (DV), g_cum (4 B)
    per token-head and h0 per sequence-head; write v_new (DV) per token-head,
    h (DK x DV) per chunk-head and hT per sequence-head."""
    toks = sum(lengths)
    chunks = sum((L + 63) // 64 for L in lengths)
    n = len(lengths)
    per_tok = (2 * DK + DV) * in_bytes + 4 + DV * in_bytes
    b = toks * H * per_tok + chunks * H * DK * DV * h_bytes
    b += n * H * DK * DV * 4 * (int(has_h0) + int(has_hT))
    return b


def scan_flops(lengths, H, DK, DV):
    """4 DK DV per token-head: W S (2 DK DV) and K^T D' (2 DK DV)."""
    return 4 * DK * DV * sum(lengths) * H


def fused_alg_bytes(lengths, H, DK, DV, in_bytes, h_bytes, has_h0, has_hT):
    """The scan's bytes plus the chunk output's own: read q (DK) and write o
    (DV) per token-head (h, v_new, k and g_cum it takes on chip)."""
    return (scan_alg_bytes(lengths, H, DK, DV, in_bytes, h_bytes, has_h0, has_hT)
            + sum(lengths) * H * (DK + DV) * in_bytes)


def fused_flops(lengths, H, DK, DV):
    """The scan's flops plus the output's: Q S (2 DK DV per token-head) and,
    for token j of a chunk, its j + 1 causal terms of Q K^T (2 DK each) and of
    P v_new (2 DV each)."""
    causal = 0
    for L in lengths:
        full, tail = divmod(L, 64)
        causal += full * (64 * 65 // 2) + tail * (tail + 1) // 2
    return scan_flops(lengths, H, DK, DV) + H * (2 * DK * DV * sum(lengths) + 2 * (DK + DV) * causal)


def source_sha():
    h = hashlib.sha256()
    for f in ("scan2.hip", "gfx950.hpp", "common.hpp", "kernels.hpp", "plan.cpp", "api.cpp", "wy_core.hpp"):
        with open(os.path.join(ROOT, "linear_attention_chunked_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per scan launch from the committed rocprofv3 counter summary,
    or None when the scan sources changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"scan_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        t = json.load(fh)
    if t.get("source_sha") != source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


class HipEvent:
    """A timing event on the HIP runtime directly, created without the
    system-scope release fence (hipEventDisableSystemFence): torch's events
    flush the caches to system scope at every record, which costs the stream
    several microseconds per record and lands inside whatever they bracket."""

    _hip = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes

        if HipEvent._hip is None:
            HipEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        rc = HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), ctypes.c_uint(self.FLAGS))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = HipEvent._hip.hipEventRecord(self.ev, self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, end):
        ms = self._ct.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        hip = getattr(HipEvent, "_hip", None) if HipEvent is not None else None
        if hip is not None and self.ev:  # (at interpreter exit the module's globals may already be gone)
            hip.hipEventDestroy(self.ev)


class Evictor:
    """Evicts L2 and the 256 MB Infinity Cache between timed launches: a fill
    of a 1 GiB scratch buffer, then a read of another 1 GiB buffer, so that
    the caches hold only unrelated, clean lines when the timed kernel starts
    (the lines the fill leaves behind would otherwise be written back to HBM
    while the timed kernel runs)."""

    what = "a 1 GiB fill, then a 1 GiB read of another buffer"

    def __init__(self, torch, dev):
        self.torch = torch
        self.a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        self.b = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        self.s = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self):
        self.a.fill_(1.0)
        self.torch.sum(self.b, dim=0, out=self.s)


CPU_BASELINE_S = 10.0  # wall time the oracle is given (whole passes over the batch, at most 30)


def cpu_baseline(inp):
    """The FP64 oracle on the same batch, on the host cores: whole passes
    over the batch until CPU_BASELINE_S seconds have gone by (at most 30)."""
    import oracle

    d = inp.f64()
    t0, c0 = time.perf_counter(), time.process_time()
    passes = 0
    while passes < 30:
        oracle.gdr_recurrent_fp64(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], inp.scale)
        passes += 1
        if time.perf_counter() - t0 >= CPU_BASELINE_S:
            break
    wall = time.perf_counter() - t0
    cpu = time.process_time() - c0
    return {
        "value": passes * inp.token_heads / wall / 1e6,
        "unit": "Mtok-head/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"{passes} whole passes over the {inp.name} batch ({inp.N} sequences, {sum(inp.lengths)} tokens "
                  f"x {inp.H} heads), token-serial FP64 numpy; {wall:.2f} s wall, {cpu:.2f} s CPU",
        "host": host_info(),
    }


def host_info():
    """The host the CPU baseline ran on: logical cores (os.cpu_count()), the
    cores this process may use, the CPU model and the BLAS thread pools numpy
    would use (the oracle's token loop itself is serial numpy)."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info

        blas = [{"api": d.get("internal_api"), "threads": d.get("num_threads")} for d in threadpool_info()]
    except Exception:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_count": os.cpu_count(), "usable_cores": usable, "cpu_model": model, "blas_threads": blas,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="question_rows", choices=["question_rows", "new_states"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-state", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line: time every built tile on the workloads the scheduler's table "
                         "covers (one JSON line per workload and tile)")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="also run a plain 'copy' of this many MiB (counter reference for rocprofv3 --pmc)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_attention_chunked_amd as pkg
    from workloads import make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pkg.lib()
    dev = torch.device("cuda:0")
    if args.sweep:
        sweep(pkg, torch, dev)
        return
    inp = make_config(args.workload)
    q, k, v, g, beta = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    h0 = inp.h0.to(dev) if inp.h0 is not None else None
    cu = inp.cu_seqlens
    DV = v.shape[-1]
    nt = pkg.gdr_num_chunks(k, DV, cu)
    # outputs allocated once; the step writes into them
    g_cum = torch.empty(g.shape, dtype=torch.float32, device=dev)
    w = torch.empty_like(k)
    u = torch.empty_like(v)
    h = torch.empty((nt, inp.H, DV, inp.DK), dtype=k.dtype, device=dev)
    v_new = torch.empty_like(v)
    hT = torch.empty((inp.N, inp.H, inp.DK, DV), dtype=torch.float32, device=dev)
    o = torch.empty_like(v)
    B = pkg.binding
    L = pkg.lib()
    P = B.Problem(k, DV, cu)
    stream = torch.cuda.current_stream()
    s_ptr = B._stream(stream)
    ptr = B._ptr

    def step(ev=None):
        B._check(L.gdr_chunk_prepare(P.ref, ptr(k), ptr(v), ptr(g), ptr(beta), ptr(g_cum), ptr(w), ptr(u), s_ptr),
                 "prepare")
        if ev is not None:
            ev[0].record(stream)
        B._check(L.gdr_state_scan_output(P.ref, None, None, ptr(q), ptr(k), ptr(w), ptr(u), ptr(g_cum), ptr(h0),
                                         float(inp.scale), ptr(h), ptr(v_new), ptr(hT), ptr(o), s_ptr),
                 "scan + output")
        if ev is not None:
            ev[1].record(stream)

    settle(torch, step)  # the clocks reach their level under this load (untimed)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: K steps back to back, no events inside
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = inp.token_heads / (elapsed / args.steps) / 1e6

    in_bytes = 2 if inp.dtype == torch.bfloat16 else 4
    alg = fused_alg_bytes(inp.lengths, inp.H, inp.DK, DV, in_bytes, in_bytes, h0 is not None, True)
    flops = fused_flops(inp.lengths, inp.H, inp.DK, DV)
    tile = pkg.gdr_plan_query(k, DV, cu)

    # The roofline kernel (the fused scan) after the timed region, over
    # ROOF_REPS dedicated steps each, with a pair of HIP events on the launch
    # stream around the kernel alone:
    #   cold: before every step the caches are evicted (evict_caches(), outside
    #         the events), so the step's inputs come from HBM, as when the
    #         question rows arrive from elsewhere; this is the headline figure;
    #   warm: steps back to back (inputs and part of the outputs still in the
    #         256 MB Infinity Cache from the previous step).
    flush = Evictor(torch, dev)
    cold_k, cold_s, warm_k = [], [], []
    for i in range(ROOF_REPS + 3):
        flush()
        e, s0, s1 = (HipEvent(), HipEvent()), HipEvent(), HipEvent()
        s0.record(stream)
        step(e)
        s1.record(stream)
        torch.cuda.synchronize()
        if i >= 3:
            cold_k.append(e[0].elapsed_ms(e[1]))
            cold_s.append(s0.elapsed_ms(s1))
    evs = [(HipEvent(), HipEvent()) for _ in range(ROOF_REPS)]
    for _ in range(3):
        step()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    warm_k = [a.elapsed_ms(b) for a, b in evs]
    cold_k.sort()
    warm_k.sort()
    cold_mean = sum(cold_k) / len(cold_k)
    warm_mean = sum(warm_k) / len(warm_k)
    achieved = alg / (cold_mean * 1e-3) / 1e9
    warm_achieved = alg / (warm_mean * 1e-3) / 1e9
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": load_traffic(args.workload),
        "kernel": f"gdr state scan with the chunk output fused (bv={tile[0]}, waves={tile[1]}, stages={tile[2]}, "
                  f"{tile[3]} workgroups" + (", dense form: three workgroups per CU" if tile[3] > 512 else "") + ")",
        "alg_bytes_per_launch": alg,
        "cache": f"cold: {flush.what} before each of {ROOF_REPS} dedicated steps, outside the events",
        "launch_us_mean": round(cold_mean * 1e3, 2),
        "launch_us_median": round(cold_k[len(cold_k) // 2] * 1e3, 2),
        "launch_us_stats": _stats_us(cold_k),
        "step_us_median": round(sorted(cold_s)[len(cold_s) // 2] * 1e3, 2),
        "mfma_frac": round(flops / (cold_mean * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "warm": {"launch_us_mean": round(warm_mean * 1e3, 2), "launch_us_stats": _stats_us(warm_k),
                 "achieved": round(warm_achieved, 1), "frac": round(warm_achieved / HBM_PEAK_GBS, 4),
                 "cache": f"{ROOF_REPS} steps back to back after 3 more (part of the working set stays in the "
                          "256 MB Infinity Cache)"},
    }

    # The state scan alone (gdr_state_scan, the unfused kernel, same outputs
    # but o): cold (caches evicted before each launch) and warm (back to
    # back), ROOF_REPS launches each between a pair of HIP events.
    def scan_alone(ev):
        ev[0].record(stream)
        B._check(L.gdr_state_scan(P.ref, None, None, ptr(k), ptr(w), ptr(u), ptr(g_cum), ptr(h0), ptr(h),
                                  ptr(v_new), ptr(hT), s_ptr), "scan")
        ev[1].record(stream)

    sa_alg = scan_alg_bytes(inp.lengths, inp.H, inp.DK, DV, in_bytes, in_bytes, h0 is not None, True)
    cold_sa = []
    for i in range(ROOF_REPS + 3):
        flush()
        B._check(L.gdr_chunk_prepare(P.ref, ptr(k), ptr(v), ptr(g), ptr(beta), ptr(g_cum), ptr(w), ptr(u), s_ptr),
                 "prepare")
        e = (HipEvent(), HipEvent())
        scan_alone(e)
        torch.cuda.synchronize()
        if i >= 3:
            cold_sa.append(e[0].elapsed_ms(e[1]) * 1e3)
    for _ in range(5):
        scan_alone((HipEvent(), HipEvent()))
    sa = [(HipEvent(), HipEvent()) for _ in range(ROOF_REPS)]
    for ev in sa:
        scan_alone(ev)
    torch.cuda.synchronize()
    sa_us = sorted(a.elapsed_ms(b) * 1e3 for a, b in sa)
    cold_sa.sort()
    cmed, wmed = cold_sa[len(cold_sa) // 2], sa_us[len(sa_us) // 2]
    roofline["state_scan_alone"] = {
        "alg_bytes_per_launch": sa_alg,
        "cold": {"launch_us_median": round(cmed, 2), "frac": round(sa_alg / (cmed * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                 "cache": f"{flush.what} and the chunk prepare before each launch"},
        "warm": {"launch_us_median": round(wmed, 2), "frac": round(sa_alg / (wmed * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    del flush

    out = {
        "metric": "gated-delta state-scan Mtok-head/s + % roofline (varlen batch, 64K seq)",
        "value": round(value, 2),
        "unit": "Mtok-head/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": SETTLE_MS,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "sequences": inp.N,
            "tokens": sum(inp.lengths),
            "heads": inp.H,
            "dk": inp.DK,
            "dv": DV,
            "step": "chunk prepare + state scan with the chunk output fused",
        },
        "roofline": roofline,
    }

    if args.copy_ref_mib:
        n = args.copy_ref_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        out["copy_ref"] = {"bytes_read": n * 4, "bytes_written": n * 4, "launches": 3}

    copy_gbs = copy_bandwidth(torch, dev)
    roofline["copy_gbs"] = round(copy_gbs, 1)
    roofline["frac_of_copy"] = round(achieved / copy_gbs, 4)
    roofline["warm"]["frac_of_copy"] = round(warm_achieved / copy_gbs, 4)
    for leg in roofline["state_scan_alone"]["cold"], roofline["state_scan_alone"]["warm"]:
        leg["frac_of_copy"] = round(sa_alg / (leg["launch_us_median"] * 1e-6) / 1e9 / copy_gbs, 4)

    if not args.no_long_state:
        out["long_state"] = long_state(pkg, torch, dev, copy_gbs=copy_gbs)
        out["long_state_h1"] = long_state(pkg, torch, dev, name="long_state_h1", copy_gbs=copy_gbs)
        out["new_states"] = new_states(pkg, torch, dev)
        out["abc_affine"] = abc_affine(pkg, torch, dev)
        out["reverse"] = reverse(pkg, torch, dev, args.workload)
        out["per_channel_decay"] = per_channel_decay(pkg, torch, dev)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp)

    print(json.dumps(out), flush=True)


def _stats_us(ms_sorted):
    """n, mean, std, min and the 10/20/50/80/90th percentiles (us) of sorted
    durations in ms."""
    import statistics

    us = [x * 1e3 for x in ms_sorted]
    pct = lambda p: us[min(len(us) - 1, int(round(p / 100 * (len(us) - 1))))]
    return {"n": len(us), "mean": round(statistics.fmean(us), 2), "std": round(statistics.pstdev(us), 2),
            "min": round(us[0], 2), "p10": round(pct(10), 2), "p20": round(pct(20), 2), "p50": round(pct(50), 2),
            "p80": round(pct(80), 2), "p90": round(pct(90), 2)}


def sweep(pkg, torch, dev):
    """Every built bfloat16 tile on the workloads the scheduler's table covers:
    the state scan on question_rows and new_states, and the 64K x 8-head
    segmented pass (summaries per tile, with and without the half-segment
    split, and the final pass per tile).  One JSON line per measurement, each
    the median of 5 x the mean of 4 back-to-back calls between HIP events."""
    from workloads import make_config

    tiles = [(32, 2, 2), (32, 2, 3), (64, 2, 3), (64, 4, 2), (64, 4, 3), (128, 4, 2), (128, 4, 3)]
    # the named packed workloads, the same lengths at 48 heads and at
    # dk = dv = 64, and two long rows at 8 heads
    cases = [("question_rows", {}), ("question_rows", {"H": 48}), ("question_rows", {"DK": 64, "DV": 64}),
             ("new_states", {}), ("new_states", {"H": 48}), ("new_states", {"DK": 64, "DV": 64}),
             ("long_state_h8", {"B": 2, "T": 16384})]
    for name, over in cases:
        inp = make_config(name, **over)
        label = name + "".join(f" {k}={v}" for k, v in over.items())
        k, v, g, b = (x.to(dev) for x in (inp.k, inp.v, inp.g, inp.beta))
        h0 = inp.h0.to(dev) if inp.h0 is not None else None
        cu = inp.cu_seqlens
        g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, b, cu)
        h, v_new, hT = pkg.gdr_state_scan(k, w, u, g_cum, h0, cu)
        out = {"h": h, "v_new": v_new, "hT": hT}
        default = pkg.gdr_plan_query(k, v.shape[-1], cu)[:3]
        for t in tiles:
            if t[0] > v.shape[-1]:
                continue
            us = _event_median_us(torch, lambda: pkg.gdr_state_scan(k, w, u, g_cum, h0, cu, t, out=out))
            print(json.dumps({"sweep": "state scan", "workload": label, "tile": t, "default": tuple(default) == t,
                              "us": round(us, 1)}), flush=True)
        del k, v, g, b, g_cum, w, u, h, v_new, hT, out
    inp = make_config("long_state_h8")
    k, v, g, b = (x.to(dev) for x in (inp.k, inp.v, inp.g, inp.beta))
    g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, b)
    P = 16
    for t in tiles + [(256, 8, 2)]:
        for ws in (False, True):
            us = _event_median_us(torch, lambda: pkg.gdr_segment_summaries(k, w, u, g_cum, P, None, t, workspace=ws))
            print(json.dumps({"sweep": "segment summaries", "workload": "long_state_h8, 16 segments", "tile": t,
                              "half_segments": ws, "us": round(us, 1)}), flush=True)
    ss, st = pkg.gdr_segment_summaries(k, w, u, g_cum, P)
    si, _ = pkg.gdr_segment_compose(k, v.shape[-1], ss, st, P)
    for t in tiles:
        us = _event_median_us(torch, lambda: pkg.gdr_state_scan(k, w, u, g_cum, None, None, t, P, si))
        print(json.dumps({"sweep": "segmented final pass", "workload": "long_state_h8, 16 segments", "tile": t,
                          "us": round(us, 1)}), flush=True)


def long_state(pkg, torch, dev, name="long_state_h8", reps=5, copy_gbs=None, cp_splits=(2, 4, 8, 16)):
    """One 64K-token sequence (8 heads, or 1 with name="long_state_h1"):
    serial scan and the 16-segment path (summaries + compose + segmented
    final pass, whole and each phase), timed with HIP events; then the
    CP-vs-serial accuracy table at each split count in ``cp_splits``."""
    from workloads import make_config

    inp = make_config(name)
    k, v, g, beta = (x.to(dev) for x in (inp.k, inp.v, inp.g, inp.beta))
    g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, beta)
    DV = v.shape[-1]
    P = 16

    # every buffer allocated once; the timed calls go straight through the C ABI
    B = pkg.binding
    L = pkg.lib()
    pr = B.Problem(k, DV)
    nt = pkg.gdr_num_chunks(k, DV)
    H, DK = inp.H, inp.DK
    h = torch.empty((nt, H, DV, DK), dtype=k.dtype, device=dev)
    v_new = torch.empty_like(u)
    hT = torch.empty((1, H, DK, DV), dtype=torch.float32, device=dev)
    sp = B._stream(torch.cuda.current_stream())
    ptr = B._ptr

    def seg_buffers(P):
        ss = torch.empty((P, H, DV, DK), dtype=torch.float32, device=dev)
        st = torch.empty((P, H, DK, DK), dtype=torch.float32, device=dev)
        si = torch.empty((P, H, DV, DK), dtype=torch.float32, device=dev)
        ws_bytes = int(L.gdr_segment_summaries_workspace_size(pr.ref, P))
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        return ss, st, si, ws, ws_bytes, B.gdr_segments(P, si.data_ptr())

    def serial():
        B._check(L.gdr_state_scan(pr.ref, None, None, ptr(k), ptr(w), ptr(u), ptr(g_cum), None, ptr(h), ptr(v_new),
                                  ptr(hT), sp), "scan")

    def path(P, bufs):
        ss, st, si, ws, ws_bytes, seg = bufs

        def summaries():
            B._check(L.gdr_segment_summaries_ws(pr.ref, None, P, ptr(k), ptr(w), ptr(u), ptr(g_cum), ptr(ss),
                                                ptr(st), ptr(ws), ws_bytes, sp), "summaries")

        def compose():
            B._check(L.gdr_segment_compose(pr.ref, P, ptr(ss), ptr(st), None, ptr(si), None, sp), "compose")

        def final_pass():
            B._check(L.gdr_state_scan(pr.ref, None, ctypes.byref(seg), ptr(k), ptr(w), ptr(u), ptr(g_cum), None,
                                      ptr(h), ptr(v_new), ptr(hT), sp), "final pass")

        def segmented():
            summaries()
            compose()
            final_pass()

        return {"summaries": summaries, "compose": compose, "final_pass": final_pass, "segmented": segmented}

    bufs16 = seg_buffers(P)
    fns = path(P, bufs16)
    res = {}
    serial_alg = scan_alg_bytes(inp.lengths, inp.H, inp.DK, DV, 2, 2, False, True)
    # segmented path: summaries read k, w, u, g_cum and write (S_loc, M) in
    # FP32; compose reads them and writes S_init; the final pass is the serial
    # scan's traffic plus reading S_init
    summ = P * inp.H * inp.DK * (DV + inp.DK) * 4
    init = P * inp.H * inp.DK * DV * 4
    alg_phase = {"summaries": inp.token_heads * ((2 * inp.DK + DV) * 2 + 4) + summ,
                 "compose": summ + init,
                 "final_pass": serial_alg + init}
    seg_alg = sum(alg_phase.values())
    for leg, fn in (("serial", serial), ("segmented", fns["segmented"])):
        t = _event_median_us(torch, fn, reps=reps) * 1e-6
        res[leg] = {"us": round(t * 1e6, 1), "Mtok_head_per_s": round(inp.token_heads / t / 1e6, 1),
                    "serial_alg_bytes": serial_alg, "frac_of_hbm_at_serial_bytes": round(serial_alg / t / 8e12, 4)}
    t = res["segmented"]["us"] * 1e-6
    res["segmented"].update(alg_bytes=seg_alg, frac_of_hbm=round(seg_alg / t / 8e12, 4), segments=P)
    # the same pass through the scheduler's entry point (gdr_state_scan_auto:
    # it picks the segment count), workspace allocated once
    ap = L.gdr_plan_segments(pr.ref)
    aws_bytes = int(L.gdr_state_scan_auto_workspace_size(pr.ref))
    aws = torch.empty(max(aws_bytes, 16), dtype=torch.uint8, device=dev)

    def auto():
        B._check(L.gdr_state_scan_auto(pr.ref, None, ptr(k), ptr(w), ptr(u), ptr(g_cum), None, 1.0, ptr(h),
                                       ptr(v_new), ptr(hT), None, ptr(aws), aws_bytes, sp), "auto")

    ta = _event_median_us(torch, auto, reps=reps) * 1e-6
    res["segmented_auto"] = {"us": round(ta * 1e6, 1), "segments": int(ap),
                             "Mtok_head_per_s": round(inp.token_heads / ta / 1e6, 1),
                             "alg_bytes": seg_alg, "frac_of_hbm": round(seg_alg / ta / 8e12, 4)}
    if copy_gbs:
        res["segmented"]["frac_of_copy"] = round(seg_alg / t / 1e9 / copy_gbs, 4)
    # each phase alone (the buffers hold the previous phases' outputs)
    res["segmented"]["phases"] = {}
    for ph in ("summaries", "compose", "final_pass"):
        tp = _event_median_us(torch, fns[ph], reps=reps) * 1e-6
        res["segmented"]["phases"][ph] = {"us": round(tp * 1e6, 1), "alg_bytes": alg_phase[ph],
                                          "frac_of_hbm": round(alg_phase[ph] / tp / 8e12, 4)}
    # CP vs serial, reported as the pages' accuracy table does (not a gate:
    # each path is checked against the FP64 oracle in the tests): relative L2
    # between the segmented and the serial path's outputs o, final states and
    # o over the last 8K tokens, at each split count (with the time of the
    # whole segmented path at that split)
    q = inp.q.to(dev)

    def output():
        o = torch.empty_like(v)
        B._check(L.gdr_chunk_output(pr.ref, ptr(q), ptr(k), ptr(v_new), ptr(h), ptr(g_cum), float(inp.scale),
                                    ptr(o), sp), "output")
        torch.cuda.synchronize()
        return o.double(), hT.double().clone()

    def rl(x, y):
        return float(torch.linalg.vector_norm(x - y) / torch.linalg.vector_norm(y))

    serial()
    os_, hs = output()
    table = {}
    for Pc in cp_splits:
        bf = bufs16 if Pc == P else seg_buffers(Pc)
        f = path(Pc, bf)["segmented"]
        us = _event_median_us(torch, f, reps=3)
        f()
        oc, hc = output()
        table[str(Pc)] = {"out": rl(oc, os_), "final": rl(hc, hs), "last_8k": rl(oc[:, -8192:], os_[:, -8192:]),
                          "segmented_us": round(us, 1)}
        del bf
    res["cp_vs_serial_rel_l2"] = table
    res["workload"] = f"{name} (T=65536, H={H}, dk=dv=128, bf16, 16 segments)"
    return res


def copy_bandwidth(torch, dev, mib=512, reps=5):
    """Achievable HBM rate of a plain device copy (torch copy_ of `mib` MiB:
    the bytes read plus the bytes written, over the median of `reps`)."""
    n = mib * (1 << 20) // 4
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    us = _event_median_us(torch, lambda: b.copy_(a), reps=reps, per=2)
    del a, b
    return 2 * n * 4 / (us * 1e-6) / 1e9


def settle(torch, fn, ms=SETTLE_MS):
    """Runs fn back to back for at least `ms` milliseconds of wall time (then
    synchronizes): the GPU's clocks take tens of milliseconds to reach their
    level under a new load (the 64K x 8-head segmented pass measured 350 us
    on its first calls and 300 us after 30 ms), so every timed leg starts
    from that level."""
    t0 = time.perf_counter()
    while True:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            return


def _event_median_us(torch, fn, reps=5, per=4):
    """Median over `reps` of the mean time of `per` back-to-back calls,
    between two HIP events on the current stream (so a call's host-side
    argument marshalling overlaps the previous call's kernels), after
    settle()."""
    settle(torch, fn)
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        a, b = HipEvent(), HipEvent()
        a.record(stream)
        for _ in range(per):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_ms(b) * 1e3 / per)
    return sorted(times)[len(times) // 2]


def new_states(pkg, torch, dev):
    """8 packed sequences of 1306..3597 tokens, 32 heads: the state scan alone
    (pre-chunk states emitted in bf16)."""
    from workloads import make_config

    inp = make_config("new_states")
    k, v, g, beta = (x.to(dev) for x in (inp.k, inp.v, inp.g, inp.beta))
    cu = inp.cu_seqlens
    g_cum, w, u = pkg.gdr_chunk_prepare(k, v, g, beta, cu)
    h, v_new, hT = pkg.gdr_state_scan(k, w, u, g_cum, None, cu)
    bufs = {"h": h, "v_new": v_new, "hT": hT}
    us = _event_median_us(torch, lambda: pkg.gdr_state_scan(k, w, u, g_cum, None, cu, out=bufs))
    alg = scan_alg_bytes(inp.lengths, inp.H, inp.DK, inp.DV, 2, 2, False, True)
    return {"workload": "new_states (8 seqs, 18261 tokens, H=32, dk=dv=128, bf16)", "scan_us": round(us, 1),
            "Mtok_head_per_s": round(inp.token_heads / us, 1), "alg_bytes": alg,
            "frac_of_hbm": round(alg / (us * 1e-6) / 8e12, 4)}


def kda_alg_bytes(lengths, H, DK, DV):
    """Per-channel decay, bf16 storage, FP32 h0/hT: minimum bytes of each call.
    prepare: read k, v (bf16), g (FP32 per channel), beta; write g_cum (FP32 per
    channel), w, u, kg (bf16) and the chunk decays (FP32, DK per chunk-head).
    scan: read kg, w, u, the chunk decays and h0; write v_new, h (bf16) and hT.
    output: read q, k, v_new (bf16), g_cum (FP32 per channel) and h; write o."""
    toks = sum(lengths) * H
    chunks = sum((L + 63) // 64 for L in lengths) * H
    seqs = len(lengths) * H
    prep = toks * ((DK + DV) * 2 + DK * 4 + 4 + DK * 4 + (2 * DK + DV) * 2) + chunks * DK * 4
    scan = toks * ((2 * DK + DV) * 2 + DV * 2) + chunks * (DK * 4 + DK * DV * 2) + seqs * DK * DV * 4 * 2
    outp = toks * ((2 * DK + DV) * 2 + DK * 4 + DV * 2) + chunks * DK * DV * 2
    return prep, scan, outp


def per_channel_decay(pkg, torch, dev):
    """The per-key-channel decay forward on the question-rows shape (24 packed
    sequences, 3400 tokens, 16 heads, per-channel gates): prepare, state scan
    and output, each timed alone."""
    from workloads import make_config

    inp = make_config("kda_question_rows")
    q, k, v, g, beta, h0 = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0))
    cu = inp.cu_seqlens
    g_cum, w, u, kg, decay = pkg.kda_chunk_prepare(k, v, g, beta, cu)
    h, v_new, hT = pkg.kda_state_scan(kg, w, u, decay, h0, cu)
    scale = inp.DK ** -0.5
    t_p = _event_median_us(torch, lambda: pkg.kda_chunk_prepare(k, v, g, beta, cu))
    t_s = _event_median_us(torch, lambda: pkg.kda_state_scan(kg, w, u, decay, h0, cu))
    t_o = _event_median_us(torch, lambda: pkg.kda_chunk_output(q, k, v_new, h, g_cum, scale, cu))
    bp, bs, bo = kda_alg_bytes(inp.lengths, inp.H, inp.DK, inp.DV)

    def leg(us, b):
        return {"us": round(us, 1), "alg_bytes": b, "frac_of_hbm": round(b / (us * 1e-6) / 8e12, 4)}

    return {"workload": "kda_question_rows (24 seqs, 3400 tokens, H=16, dk=dv=128, bf16, per-channel decay)",
            "prepare": leg(t_p, bp), "scan": leg(t_s, bs), "output": leg(t_o, bo),
            "step_us": round(t_p + t_s + t_o, 1),
            "Mtok_head_per_s": round(inp.token_heads / (t_p + t_s + t_o), 1)}


def abc_alg_bytes(B, T, H, K, M, V):
    """Read k, v, s once; write the bf16 pre-chunk states and the FP32 finals
    (the normaliser and weight workspaces are this implementation's choice and
    not counted)."""
    nc = (T + 63) // 64
    return B * T * H * (K + V + M) * 2 + B * nc * H * (K * M + M * V) * 2 + B * H * (K * M + M * V) * 4


def abc_affine(pkg, torch, dev):
    """ABC slot-state construction at B=2, T=16384, H=4, K=256, M=64, V=512."""
    from workloads import make_config

    inp = make_config("abc_affine")
    k, v, s = (x.to(dev) for x in (inp.k, inp.v, inp.s))
    us = _event_median_us(torch, lambda: pkg.abc_affine_scan(k, v, s))
    alg = abc_alg_bytes(inp.B, inp.T, inp.H, inp.K, inp.M, inp.V)
    # the reverse (dH) walk on the same shape: seeded q, slot weights, score
    # and output gradients (bf16), final-state gradients (fp32)
    import numpy as np

    r = np.random.default_rng(11)
    B, T, H, K, M, V = inp.B, inp.T, inp.H, inp.K, inp.M, inp.V
    bf = torch.bfloat16

    def draw(*shape, dt=bf, sc=1.0):
        return torch.from_numpy((sc * r.standard_normal(shape)).astype(np.float32)).to(dt).to(dev)

    q, ds, dO = draw(B, T, H, K), draw(B, T, H, M), draw(B, T, H, V)
    p = torch.softmax(draw(B, T, H, M, dt=torch.float32), dim=-1).to(bf)
    ek, ev = draw(B, H, K, M, dt=torch.float32, sc=0.1), draw(B, H, M, V, dt=torch.float32, sc=0.1)
    z = pkg.abc_affine_scan(k, v, s, emit_z=True)[0]
    rus = _event_median_us(torch, lambda: pkg.abc_affine_scan_bwd(q, ds, p, dO, z, ek, ev, 1.0))
    ralg = abc_bwd_alg_bytes(B, T, H, K, M, V)
    return {"workload": "abc_affine (B=2, T=16384, H=4, K=256, M=64, V=512, bf16)", "us": round(us, 1),
            "Mtok_head_per_s": round(inp.token_heads / us, 1), "alg_bytes": alg,
            "frac_of_hbm": round(alg / (us * 1e-6) / 8e12, 4),
            "reverse": {"us": round(rus, 1), "alg_bytes": ralg, "frac_of_hbm": round(ralg / (rus * 1e-6) / 8e12, 4)}}


def abc_bwd_alg_bytes(B, T, H, K, M, V):
    """Reverse walk: read q, dscore, p, dO (bf16) and z (fp32) once, the final
    states' gradients (fp32); write dhk, dhv after every chunk (bf16)."""
    nc = (T + 63) // 64
    return (B * T * H * ((K + 2 * M + V) * 2 + M * 4) + B * nc * H * (K * M + M * V) * 2
            + B * H * (K * M + M * V) * 4)


def reverse_alg_bytes(lengths, H, DK, DV, nt, has_dhT):
    """Reverse pass, minimum traffic of each kernel (bf16 storage, float32
    gates and state gradients).  dv_local: read q, k, dO, g_cum, write
    dv_local.  Reverse scan: read q, k, w, dO, dv_local, g_cum (and dhT),
    write dh at every chunk (bf16), the write-vector gradient and dh0 (fp32)."""
    tok = int(sum(lengths)) * H
    n = len(lengths)
    dvl = tok * (2 * DK * 2 + DV * 2 + 4 + DV * 2)
    scan = tok * (3 * DK * 2 + 2 * DV * 2 + 4 + DV * 2) + nt * H * DK * DV * 2 + n * H * DK * DV * 4
    if has_dhT:
        scan += n * H * DK * DV * 4
    return dvl, scan


def reverse(pkg, torch, dev, workload):
    """The reverse pass of the same workload: chunk-local write-vector
    gradient, then the serial reverse state walk (dh per chunk, dv_new
    gradient, dh0), seeded dO (bf16) and dhT (fp32)."""
    import numpy as np
    from workloads import make_config

    inp = make_config(workload)
    q, k, v, g, beta = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    cu = inp.cu_seqlens
    DV = v.shape[-1]
    r = np.random.default_rng(7)
    dO = torch.from_numpy(r.standard_normal(tuple(v.shape)).astype(np.float32)).to(v.dtype).to(dev)
    dhT = torch.from_numpy(0.1 * r.standard_normal((inp.N, inp.H, inp.DK, DV)).astype(np.float32)).to(dev)
    g_cum, w, _ = pkg.gdr_chunk_prepare(k, v, g, beta, cu)
    nt = pkg.gdr_num_chunks(k, DV, cu)
    dvl = torch.empty_like(dO)
    dh = torch.empty((nt, inp.H, DV, inp.DK), dtype=k.dtype, device=dev)
    dv = torch.empty_like(dO)
    dh0 = torch.empty((inp.N, inp.H, inp.DK, DV), dtype=torch.float32, device=dev)
    B = pkg.binding
    L = pkg.lib()
    P = B.Problem(k, DV, cu)
    ptr = B._ptr
    s_ptr = B._stream(torch.cuda.current_stream())
    scale = float(inp.scale)

    def dv_local():
        B._check(L.gdr_chunk_dv_local(P.ref, ptr(q), ptr(k), ptr(g_cum), ptr(dO), scale, ptr(dvl), s_ptr),
                 "dv_local")

    def scan_bwd():
        B._check(L.gdr_state_scan_bwd(P.ref, ptr(q), ptr(k), ptr(w), ptr(g_cum), ptr(dO), ptr(dvl), ptr(dhT),
                                      scale, ptr(dh), ptr(dv), ptr(dh0), s_ptr), "scan_bwd")

    def both():
        dv_local()
        scan_bwd()

    a_us = _event_median_us(torch, dv_local, reps=7, per=8)
    b_us = _event_median_us(torch, scan_bwd, reps=7, per=8)
    t_us = _event_median_us(torch, both, reps=7, per=8)
    a_alg, b_alg = reverse_alg_bytes(inp.lengths, inp.H, inp.DK, DV, nt, True)
    return {"workload": f"{workload} reverse pass (dO bf16, dhT fp32)", "us": round(t_us, 1),
            "Mtok_head_per_s": round(inp.token_heads / t_us, 1),
            "dv_local": {"us": round(a_us, 1), "alg_bytes": a_alg,
                         "frac_of_hbm": round(a_alg / (a_us * 1e-6) / 8e12, 4)},
            "scan_bwd": {"us": round(b_us, 1), "alg_bytes": b_alg,
                         "frac_of_hbm": round(b_alg / (b_us * 1e-6) / 8e12, 4)}}


if __name__ == "__main__":
    main()
