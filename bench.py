"""Decode-attention benchmark of the R-SWA / SR-SWA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--mode fused|separate]

A step is one pass of the decode hot path over one batch: ring append, then
(SR-SWA) block scores, 1.5-entmax top-k and sparse decode, or (R-SWA) dense
decode.  The block index is built once per layer before timing (it depends
only on the static prefix).  Steps rotate over --layers independent per-layer
decode states, as a decoder does while generating one token, so that a
step's working set has left the 256 MB Infinity Cache before the same layer
is visited again: bandwidth figures are HBM figures, not cache hits.

The K timed steps are replayed from HIP graphs (as a serving loop runs decode
steps); eager host-launched
throughput is reported beside it.  Prints one JSON line: throughput in
attention unit-steps per second (units = batch x heads), the roofline of the
dominant kernel (algorithmic bytes over its average duration, from HIP events
around the timed region) and the CPU oracle's throughput on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, AMD published

# HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of
# this script (summaries under profiles/), scaled by what the counters read for
# a plain device copy of known size: FETCH_SIZE x 2.0, WRITE_SIZE x 1.0.  Valid
# only for the kernel source they were taken on (sha256 prefix of
# uocr_kernels.hip); otherwise the traffic is reported as null.
COUNTER_TRAFFIC = {
    # (kernel, workload): (kernel source sha256[:16], fetch bytes, write bytes)
    ('uocr_srswa_step', 'srswa-40p-b32'): ('d95115f5fa62f511', 45176646, 307712),
    ('uocr_srswa_step', 'srswa-125p-b8'): ('d95115f5fa62f511', 18890109, 76928),
    ('uocr_srswa_step', 'srswa-40p-b32-wide'): ('d95115f5fa62f511', 118613853, 307712),
    ('uocr_srswa_step', 'srswa-125p-b8-wide'): ('d95115f5fa62f511', 37049953, 76928),
    ('uocr_rswa_step', 'dense-10p-b64'): ('d95115f5fa62f511', 892108762, 1024667),
    ('uocr_rswa_step', 'dense-1p-b512'): ('d95115f5fa62f511', 1092732502, 3940448),
    ('uocr_rswa_step', 'dense-40p-b32'): ('d95115f5fa62f511', 1699100325, 686845),
    ('uocr_rswa_step', 'dense-125p-b8'): ('d95115f5fa62f511', 1316147184, 302165),
    ('uocr_rope_page2d', 'srswa-40p-b32-rope-chunk2048'): ('d95115f5fa62f511', 169090846, 167781105),
}
METRIC = "decode attn steps/s (batch×heads) + achieved HBM GB/s vs peak at 40 pages"
UNIT = "steps/s (batch×heads)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2400)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="srswa-40p-b32")
    ap.add_argument("--layers", type=int, default=0,
                    help="independent per-layer states cycled by the steps (0: enough that their working set is "
                         "twice the 256 MB Infinity Cache, at least 12)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--t0", type=int, default=None,
                    help="generated tokens before the first step (default: the workload's; for flatness runs)")
    ap.add_argument("--pages", type=int, default=None,
                    help="prefix pages of 256 tokens instead of the workload's (document-length sweeps)")
    ap.add_argument("--batch", type=int, default=None,
                    help="sequences instead of the workload's (document-length sweeps)")
    ap.add_argument("--mode", choices=["fused", "separate"], default="fused",
                    help="fused: one uocr_*_step launch per step; separate: one launch per row")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ngram-ban", type=int, default=0, metavar="B",
                    help="instead of the decode step, time uocr_ngram_ban on B sequences (n = 35, window 1024, "
                         "vocabulary 129280, float32 logits)")
    ap.add_argument("--prefill-route", type=int, default=0, metavar="TQ",
                    help="instead of the decode step, time uocr_prefill_route on a chunk of TQ queries per "
                         "(sequence, head) (the sparse workload's last TQ prefix positions)")
    ap.add_argument("--rope-page2d", type=int, default=0, metavar="TQ",
                    help="instead of the decode step, time uocr_rope_page2d over the keys of a prefill chunk of TQ "
                         "tokens per (sequence, head) of the workload (page_mod 2, base 10000)")
    ap.add_argument("--rope", action="store_true",
                    help="fuse the page2d rotary embedding of q and k_new into the step kernels")
    ap.add_argument("--calibrate", action="store_true",
                    help="instead of the decode step, measure the denominators: plain and nontemporal read "
                         "streams over 2 GiB, empty launches and per-workgroup pulls")
    ap.add_argument("--phases", action="store_true",
                    help="instead of the throughput line, where the time of one fused SR-SWA step goes: the "
                         "phase stamps of every workgroup, from libuocr_stamps.so")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device-to-device copy (known bytes) so that a "
                         "counter profile of this run can scale FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


# ----------------------------------------------------------------------------
# algorithmic bytes per launch: what each kernel must read and write
# ----------------------------------------------------------------------------
def algorithmic_bytes(w, live_blocks_per_unit=None):
    """Bytes each kernel must read + write per launch for the workload."""
    units, D, es, n = w.units, w.head_dim, w.elem_bytes, w.window
    row = D * es
    wnd = min(n, w.t0 + 1)   # window size during the steps (ring full in every benchmark workload)
    b = {"uocr_ring_append": units * (2 * row + 2 * row) + w.batch * 8}
    if w.sparse:
        nb, k = w.n_blocks, w.topk
        b["uocr_block_score"] = units * (row + nb * w.idx_dim * 4 + nb * 4) + D * w.idx_dim * 4 + w.batch * 4
        b["uocr_entmax15_topk"] = units * (nb * 4 + k * 12) + w.batch * 4
        live = units * min(k, nb) if live_blocks_per_unit is None else int(live_blocks_per_unit)
        b["uocr_srswa_decode"] = (units * (row + k * 8 + 2 * wnd * row + row) + live * 2 * w.block * row
                                  + w.batch * 8)
    else:
        b["uocr_rswa_decode"] = units * (row + 2 * (w.prefix_len + wnd) * row + row) + w.batch * 8
    return b


def kernel_source_hash() -> str:
    import hashlib
    path = os.path.join(ROOT, "long_context_decode_attn_amd", "csrc", "uocr_kernels.hip")
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def counter_traffic(kernel: str, workload: str):
    rec = COUNTER_TRAFFIC.get((kernel, workload))
    if rec is None or rec[0] != kernel_source_hash():
        return None
    return rec[1] + rec[2]


def index_bytes(w):
    return w.units * (w.prefix_len * w.head_dim * w.elem_bytes + w.n_blocks * w.idx_dim * 4)


# ----------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample
# ----------------------------------------------------------------------------
def host_cores() -> int:
    """Host threads this process may use (its CPU affinity), at most 16: the
    host share of one GPU on the boxes this runs on."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_unit_steps(w, b, h, budget_s):
    """One (sequence, head) unit's decode steps with the oracle (append,
    scores from the prebuilt block index, entmax top-k, sparse or dense
    attention), one thread, until the budget is spent; returns (steps, s)."""
    from threadpoolctl import threadpool_limits

    from long_context_decode_attn_amd import synth as S
    from oracle import uocr_oracle as O

    P = S.projection(w).astype(np.float64) if w.sparse else None
    Kp, Vp = S.prefix_kv_seq(w, b)
    Kp, Vp = S.widen(Kp[h], w.dtype), S.widen(Vp[h], w.dtype)
    Kr, Vr, t_gen = S.initial_ring(w)
    Kr, Vr = S.widen(Kr[b:b + 1, h:h + 1], w.dtype), S.widen(Vr[b:b + 1, h:h + 1], w.dtype)
    t = t_gen[b:b + 1].astype(np.int64).copy()
    kbar = O.block_index(Kp, w.prefix_len, P) if w.sparse else None   # one-time, not timed
    pool = []   # this unit's inputs of 16 steps, cycled (drawn before timing)
    for i in range(16):
        q, k, v = S.step_inputs(w, i)
        pool.append((S.widen(q[b, h], w.dtype), S.widen(k[b:b + 1, h:h + 1], w.dtype),
                     S.widen(v[b:b + 1, h:h + 1], w.dtype)))
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            qd, k, v = pool[done % len(pool)]
            O.ring_append(Kr, Vr, t, k, v)
            wk, wv = O.ring_window(Kr[0, 0], int(t[0])), O.ring_window(Vr[0, 0], int(t[0]))
            if w.sparse:
                s32 = O.as_f32(O.block_scores(qd, P, kbar))
                idx, _, bias = O.route_unit(s32, w.topk)
                O.srswa_unit(qd, Kp, Vp, w.prefix_len, idx, bias, wk, wv, w.scale)
            else:
                O.rswa_unit(qd, Kp, Vp, w.prefix_len, wk, wv, w.scale)
            done += 1
        return done, time.perf_counter() - t0


def _oracle_worker(arg):
    w, b, h, budget_s = arg
    return _oracle_unit_steps(w, b, h, budget_s)


def cpu_baseline(w, budget_s: float):
    """The oracle timed on the host: one thread on one unit, then every
    usable host core at once, one unit per core (processes forked before the
    GPU is touched).  value = the all-cores rate in unit-steps per second."""
    import multiprocessing as mp

    rng = np.random.default_rng(0)
    cores = host_cores()
    units = [(int(rng.integers(w.batch)), int(rng.integers(w.heads))) for _ in range(cores)]
    n1, dt1 = _oracle_unit_steps(w, units[0][0], units[0][1], budget_s / 3)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as pool:
        res = pool.map(_oracle_worker, [(w, b, h, 2 * budget_s / 3) for b, h in units])
    wall = time.perf_counter() - t0
    done = sum(r[0] for r in res)
    rate = done / max(r[1] for r in res)
    return {"value": rate, "unit": UNIT, "cores": cores, "kind": "oracle",
            "single_thread_value": n1 / dt1, "cpu_model": cpu_model(),
            "sample": f"{w.name}: {done} unit-steps on {cores} processes of one thread each, one (sequence, head) "
                      f"unit per process ({wall:.1f} s wall, {2 * budget_s / 3:.1f} s of steps each); one thread "
                      f"alone: {n1} unit-steps in {dt1:.1f} s; float64 numpy; block index built before timing"}


# ----------------------------------------------------------------------------
# prefill-side routing (a separate measurement; the decode step is the default)
# ----------------------------------------------------------------------------
FP64_PEAK_TFLOPS = 78.6


def prefill_cpu_baseline(w, tq, q_pos, budget_s):
    """The oracle's prefill_route_unit on whole units of the same chunk, one
    at a time, until the budget is spent; returns queries/s."""
    from threadpoolctl import threadpool_limits

    from long_context_decode_attn_amd import synth as S
    from oracle import uocr_oracle as O
    P = S.projection(w).astype(np.float64)
    qd = S.widen(S.prefill_queries(w, tq), w.dtype)[:, :, :tq]
    Kp, _ = S.prefix_kv_seq(w, 0)
    done, units, spent = 0, 0, 0.0
    with threadpool_limits(limits=1):
        while spent < budget_s:
            h = units % w.heads
            kb = O.block_index(S.widen(Kp[h], w.dtype), w.prefix_len, P)   # one-time per unit, not timed
            t1 = time.perf_counter()
            O.prefill_route_unit(qd[0, h], q_pos, P, kb, w.prefix_len, w.topk)
            spent += time.perf_counter() - t1
            done += len(qd[0, h])
            units += 1
    dt = spent
    return {"value": done / dt, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} queries ({units} units x {tq}) of {w.name}, float64 numpy, 1 thread"}


def prefill_main(args):
    import torch

    from long_context_decode_attn_amd import synth as S
    from long_context_decode_attn_amd import uocr as U
    from long_context_decode_attn_amd.session import DecodeSession, to_device

    U.load_library()
    w = S.WORKLOADS[args.workload]
    assert w.sparse, "prefill routing needs a sparse workload"
    tq = args.prefill_route
    q_pos = max(w.prefix_len - tq, 0)
    sessions = [DecodeSession(w)]
    sessions += [sessions[0].clone() for _ in range(3)]
    for s in sessions:
        s.build_index()
    q = to_device(S.prefill_queries(w, tq), w.dtype)
    pos = torch.full((w.batch,), q_pos, dtype=torch.int32, device="cuda")
    outs = [tuple(torch.empty((w.batch, w.heads, tq, w.topk), dtype=dt, device="cuda")
                  for dt in (torch.int32, torch.float32, torch.float32)) for _ in sessions]

    def run(i):
        s, (idx, prob, bias) = sessions[i % len(sessions)], outs[i % len(sessions)]
        U.uocr_prefill_route(s.shape, s.route, q, pos, s.proj, s.kbar, s.prefix_len, idx, prob, bias)

    for i in range(max(args.warmup // 20, 3)):
        run(i)
    torch.cuda.synchronize()
    K = max(args.steps // 100, 10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    queries = w.units * tq
    nb = w.n_blocks
    visible = sum(min(nb, (q_pos + i) // w.block) if q_pos + i < w.prefix_len else nb for i in range(tq))
    flops = w.units * (2.0 * w.idx_dim * visible + 2.0 * w.head_dim * w.idx_dim * tq)
    achieved = flops / (ms * 1e-3) / 1e12
    hbm = w.units * (tq * w.head_dim * w.elem_bytes + nb * w.idx_dim * 4 + tq * w.topk * 12)
    # the chunk's block-key update: blocks from the one holding the chunk's first
    # token to the end of the prefix (uocr_block_index_range), against a full build
    first, last = q_pos // w.block, nb
    iu = []
    for fn in ("range", "full"):
        for i in range(3):
            s = sessions[i % len(sessions)]
            (U.uocr_block_index_range(s.shape, s.route, s.k_prefix, s.prefix_len, s.proj, s.kbar, first, last)
             if fn == "range" else s.build_index())
        torch.cuda.synchronize()
        e0.record()
        for i in range(K):
            s = sessions[i % len(sessions)]
            (U.uocr_block_index_range(s.shape, s.route, s.k_prefix, s.prefix_len, s.proj, s.kbar, first, last)
             if fn == "range" else s.build_index())
        e1.record()
        torch.cuda.synchronize()
        iu.append(round(e0.elapsed_time(e1) / K * 1e3, 2))
    result = {
        "metric": "prefill routing queries/s (batch x heads x chunk tokens)", "value": round(queries / (ms * 1e-3), 1),
        "unit": "queries/s", "n_gpus": 1, "steps": K, "warmup": max(args.warmup // 20, 3),
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64", "data": "synthetic",
        "config": {"workload": w.name + f"-prefill-chunk{tq}", "batch": w.batch, "heads": w.heads,
                   "prefix_tokens": w.prefix_len, "blocks": nb, "chunk_queries": tq, "chunk_start": q_pos,
                   "topk": w.topk, "sessions_cycled": len(sessions)},
        "roofline": {"kernel": "uocr_prefill_route", "bound": "alu", "achieved": round(achieved, 2),
                     "peak": FP64_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / FP64_PEAK_TFLOPS, 4),
                     "traffic": None},
        "flops_per_launch": flops, "hbm_bytes_per_launch": hbm,
        "hbm_gbs": round(hbm / (ms * 1e-3) / 1e9, 1),
        "index_update": {"blocks": [first, last], "range_us": iu[0], "full_build_us": iu[1]},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = prefill_cpu_baseline(w, min(tq, 256), q_pos, args.cpu_seconds)
    print(json.dumps(result), flush=True)


# ----------------------------------------------------------------------------
# no-repeat n-gram ban (a separate measurement)
# ----------------------------------------------------------------------------
def ngram_main(args):
    import torch

    from long_context_decode_attn_amd import synth as S
    from long_context_decode_attn_amd import uocr as U

    U.load_library()
    B, n, W, V, T = args.ngram_ban, 35, 1024, 129280, 6144
    hist = S.token_history(B, T, V, 11, phrase=105, repeat_p=0.5, lookback=W - 105)
    ring = torch.from_numpy(np.ascontiguousarray(hist[:, T - W:])).cuda()   # position pos at pos % W
    ring = torch.roll(ring, shifts=(T - W) % W, dims=1).contiguous()
    n_gen = torch.full((B,), T, dtype=torch.int32, device="cuda")
    page = torch.zeros((B,), dtype=torch.int32, device="cuda")
    logits = [torch.randn((B, V), device="cuda") for _ in range(8)]

    def run(i):
        U.uocr_ngram_ban(ring, n_gen, page, logits[i % len(logits)], n, W, page_token=128827, eos_token=1,
                         max_page_tokens=20000)

    for i in range(20):
        run(i)
    torch.cuda.synchronize()
    G, reps = 64, 40    # a HIP graph of G launches replayed: the launch rate of the host is not timed
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(G):
            run(i)
    graph.replay()
    torch.cuda.synchronize()
    K = G * reps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    probe = torch.zeros((B, V), device="cuda")
    U.uocr_ngram_ban(ring, n_gen, page, probe, n, W, page_token=128827, eos_token=1, max_page_tokens=20000)
    banned = int(torch.isneginf(probe).sum().item())
    hbm = B * (W * 4 + 8) + banned * 4
    result = {
        "metric": "n-gram ban sequences/s", "value": round(B / (ms * 1e-3), 1), "unit": "sequences/s",
        "n_gpus": 1, "steps": K, "warmup": 20, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": f"ngram-ban-b{B}-n{n}-w{W}", "batch": B, "ngram": n, "window": W, "vocab": V,
                   "generated": T, "timing": "HIP graph of 64 launches replayed 40 times between HIP events"},
        "roofline": {"kernel": "uocr_ngram_ban", "bound": "hbm", "achieved": round(hbm / (ms * 1e-3) / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(hbm / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 6),
                     "traffic": None},
        "note": "latency-bound: one workgroup per sequence; the bytes are the last window of tokens",
        "banned_logits_per_step": banned,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = ngram_cpu_baseline(hist, n, W, V, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def ngram_cpu_baseline(hist, n, W, V, budget_s):
    """The oracle's ngram_process, one sequence at a time, until the budget
    is spent; returns sequences/s."""
    from oracle import uocr_oracle as O
    logits = np.zeros(V)
    done, spent = 0, 0.0
    while spent < budget_s:
        b = done % len(hist)
        t1 = time.perf_counter()
        O.ngram_process(logits, hist[b].tolist(), n, W, 0, 20000, 128827, 1)
        spent += time.perf_counter() - t1
        done += 1
    return {"value": done / spent, "unit": "sequences/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} sequences of {len(hist[0])} generated tokens, window {W}, n {n}, python, 1 thread"}


def calibration_copy():
    """One plain 256 MiB device-to-device copy of known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters of the same run."""
    import torch
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def rope_main(args):
    import torch

    from long_context_decode_attn_amd import synth as S
    from long_context_decode_attn_amd import uocr as U
    from long_context_decode_attn_amd.session import to_device

    U.load_library()
    if args.copy_calibration:
        calibration_copy()
    w = S.WORKLOADS[args.workload]
    B, H, D, T = w.batch, w.heads, w.head_dim, args.rope_page2d
    tag = f"{w.name}-rope-chunk{T}"
    shape = U.Shape.of(w)
    page, offset = S.page_positions(5, B, T, page_tokens=400, first_page=3, start_offset=100)
    tp, to = torch.from_numpy(page).cuda(), torch.from_numpy(offset).cuda()
    x0 = to_device(S.rope_rows(5, B, H, T, D, w.dtype), w.dtype)
    row_bytes = B * H * T * D * w.elem_bytes
    # enough copies that the ones in rotation exceed the 256 MB Infinity Cache
    nbuf = max(2, -(-3 * 256 * 2 ** 20 // row_bytes))
    xs = [x0.clone() for _ in range(nbuf)]
    for i in range(args.warmup):
        U.uocr_rope_page2d(shape, xs[i % nbuf], tp, to)
    torch.cuda.synchronize()
    # a HIP graph of launches over the buffers in turn, replayed: the host's
    # launch rate is not timed
    G = nbuf * max(1, 48 // nbuf)
    chunk_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(chunk_graph):
        for i in range(G):
            U.uocr_rope_page2d(shape, xs[i % nbuf], tp, to)
    chunk_graph.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-args.steps // G))
    K = G * reps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        chunk_graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    # one decode step's queries and keys (T = 1, one launch for both) in a HIP
    # graph: the latency of a launch
    q1 = torch.zeros((B, H, 1, D), dtype=x0.dtype, device="cuda")
    k1 = torch.zeros_like(q1)
    p1, o1 = tp[:, :1].contiguous(), to[:, :1].contiguous()
    for _ in range(3):
        U.uocr_rope_page2d(shape, q1, p1, o1, y=k1)
    G1, reps1 = 64, 20
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(G1):
            U.uocr_rope_page2d(shape, q1, p1, o1, y=k1)
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps1):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) / (G1 * reps1) * 1e3
    hbm = 2 * row_bytes + B * T * 8
    gbs = hbm / (ms * 1e-3) / 1e9
    result = {
        "metric": "page2d RoPE tokens/s (batch x heads x chunk tokens)", "value": round(B * H * T / (ms * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": tag, "batch": B, "heads": H, "head_dim": D, "tokens": T,
                   "page_mod": 2, "base": 10000.0, "buffers_cycled": nbuf,
                   "timing": f"HIP graph of {G} launches replayed {reps} times between HIP events"},
        "roofline": {"kernel": "uocr_rope_page2d", "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic("uocr_rope_page2d", tag)},
        "hbm_bytes_per_launch": hbm,
        "decode_step_us": round(step_us, 3),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = rope_cpu_baseline(w, page, offset, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def rope_cpu_baseline(w, page, offset, budget_s):
    """The oracle's rope_page2d over every head of one token at a time, until
    the budget is spent; returns tokens/s (token = one (sequence, head, position))."""
    from long_context_decode_attn_amd import synth as S
    from oracle import uocr_oracle as O
    T = page.shape[1]
    x = S.widen(S.rope_rows(5, 1, w.heads, min(T, 256), w.head_dim, w.dtype), w.dtype)[0]
    done, spent, t = 0, 0.0, 0
    while spent < budget_s:
        tt = t % x.shape[1]
        t1 = time.perf_counter()
        O.rope_page2d(x[:, tt], int(page[0, tt]), int(offset[0, tt]), 2)
        spent += time.perf_counter() - t1
        done += w.heads
        t += 1
    return {"value": done / spent, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{t} positions x {w.heads} heads of {w.name}, float64 numpy, 1 thread"}


# ----------------------------------------------------------------------------
# calibration: attainable read bandwidth, launch floor, per-workgroup pull
# ----------------------------------------------------------------------------
def _graph_time_us(fn, per_graph=32, reps=20):
    """Average time of fn() replayed from a HIP graph of per_graph calls."""
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (per_graph * reps)


def calibrate_main(args):
    """Denominators measured on this machine: a plain and a nontemporal read
    stream over 2 GiB, an empty launch at the decode steps' grids, the time
    workgroups take to pull their own bytes when only some compute units are
    busy, when the workgroups of a launch start on each XCD, and what merging
    workgroups' partials inside one kernel costs (uocr_calib_* in
    include/uocr_calib.h)."""
    import torch

    from long_context_decode_attn_amd import uocr as U
    U.load_library()
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(3)
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    out = {"metric": "calibration", "peak_gbs": HBM_PEAK_GBS, "stream_bytes": nbytes}
    for nt in (False, True):
        us = _graph_time_us(lambda: U.uocr_calib_read(src, nt, sink), per_graph=4, reps=10)
        out[f"read_{'nontemporal' if nt else 'plain'}_gbs"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        print(json.dumps({"step": "read", "nontemporal": nt, "us": round(us, 2)}), flush=True)
    out["empty_launch_us"] = {}
    for groups, threads in [(1, 64), (80, 512), (320, 512), (2560, 256), (10240, 256)]:
        out["empty_launch_us"][f"{groups}x{threads}"] = round(
            _graph_time_us(lambda: U.uocr_calib_empty(groups, threads)), 3)
    print(json.dumps({"step": "empty", **out["empty_launch_us"]}), flush=True)
    pull = {}
    for groups in (80, 256, 320, 640):
        sk = torch.zeros(groups, dtype=torch.int32, device="cuda")
        for kb in (16, 64, 128, 256):
            per = kb * 1024
            # rotate over disjoint regions of the 2 GiB buffer, at least twice the
            # 256 MB Infinity Cache in all, so that the reads come from HBM
            regions = max(1, nbytes // (groups * per))
            want = max(8, -(-(512 << 20) // (groups * per)))
            views = [src[r * groups * per:(r + 1) * groups * per] for r in range(min(regions, want))]
            state = {"i": 0}

            def call():
                v = views[state["i"] % len(views)]
                state["i"] += 1
                U.uocr_calib_pull(v, per, groups, 512, True, sk)
            us = _graph_time_us(call, per_graph=len(views), reps=10)
            pull[f"{groups}x{kb}KiB"] = {"us": round(us, 3), "gbs": round(groups * per / (us * 1e-6) / 1e9, 1),
                                         "per_group_gbs": round(per / (us * 1e-6) / 1e9, 2)}
        print(json.dumps({"step": "pull", "groups": groups}), flush=True)
    out["pull_512_threads_nontemporal"] = pull
    # start of the workgroups of one launch, by XCD (workgroup g runs on XCD
    # g mod 8): the real-time counter runs at 100 MHz
    starts = {}
    for groups in (80, 320):
        st = torch.zeros(groups, dtype=torch.int64, device="cuda")
        _graph_time_us(lambda: U.uocr_calib_start(groups, 512, st), per_graph=8, reps=4)
        t = st.cpu().numpy().astype(np.int64)
        t0 = int(t.min())
        starts[f"{groups}x512"] = {f"xcd{x}": round(float((t[x::8] - t0).min()) / 100.0, 3) for x in range(8)}
        starts[f"{groups}x512"]["last_start_us"] = round(float(t.max() - t0) / 100.0, 3)
    out["workgroup_start_us_by_xcd"] = starts
    print(json.dumps({"step": "starts", **starts}), flush=True)
    # merging workgroups' partials inside one kernel (no workgroup waits; the
    # last to arrive merges) against an empty launch of the same grid
    ex = {}
    for units, split in ((80, 4), (320, 2), (320, 4)):
        part = torch.zeros(units * split * 130, dtype=torch.float32, device="cuda")
        cnt = torch.zeros(units, dtype=torch.int32, device="cuda")
        res = torch.zeros(units * 130, dtype=torch.float32, device="cuda")
        row = {"empty": round(_graph_time_us(lambda: U.uocr_calib_empty(units * split, 256)), 3)}
        for mode, name in ((2, "count_only"), (1, "agent_atomics"), (0, "threadfence")):
            res.zero_()
            row[name] = round(_graph_time_us(lambda: U.uocr_calib_exchange(mode, units, split, part, cnt, res),
                                             per_graph=16, reps=5), 3)
            if mode != 2:
                want = split * (split + 1) / 2 + split * torch.arange(130, device="cuda", dtype=torch.float32)
                row[name + "_merged_right"] = bool(torch.equal(res.view(units, 130), want.expand(units, 130)))
        ex[f"{units}x{split}"] = row
    out["merge_inside_one_kernel_us"] = ex
    print(json.dumps(out), flush=True)


# ----------------------------------------------------------------------------
def _quantiles(x):
    x = np.asarray(x, dtype=np.float64).ravel()
    return {"p10": round(float(np.percentile(x, 10)), 3), "p50": round(float(np.median(x)), 3),
            "p90": round(float(np.percentile(x, 90)), 3), "max": round(float(x.max()), 3)}


def phases_main(args):
    """--phases: the phase stamps of the fused SR-SWA step (include/uocr_calib.h,
    uocr_phase_stamps) in the bench's own setup (cloned layers, a HIP graph of
    two steps per layer), read after each of `reps` replays: they are those
    of the graph's last launch, which follows the others back to back.  Times
    are microseconds after the first workgroup of that launch started."""
    from long_context_decode_attn_amd import synth as S
    w = S.WORKLOADS[args.workload]
    if not w.sparse:
        print("--phases times the fused SR-SWA step: pick a sparse workload", file=sys.stderr)
        sys.exit(2)
    import torch

    from long_context_decode_attn_amd import uocr as U
    from long_context_decode_attn_amd.runner import LayeredDecoder
    from long_context_decode_attn_amd.session import DecodeSession

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    U.use_phase_stamps()
    U.load_library()
    torch.cuda.set_device(0)
    base = DecodeSession(w, num_splits=args.num_splits, fused=True)
    base.build_index()
    n_layers = args.layers if args.layers > 0 else _layers_needed(w, base)
    dec = LayeredDecoder(w, n_layers, num_splits=args.num_splits, fused=True, base=base, rope=args.rope)
    dec.build_index()
    dec.fill_pool(64)
    dec.run_eager(args.warmup)
    graph = dec.capture()
    graph.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(20):
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    us_step = start.elapsed_time(stop) * 1e3 / (20 * dec.G)

    units, W, reps = w.units, (args.num_splits or 8), 40
    rows = []
    for _ in range(reps):
        graph.replay()
        rows.append(U.uocr_phase_stamps(units).astype(np.int64))
    A = np.stack(rows)                                   # [reps, units, 64]
    t = (A - A[:, :, 0].min(axis=1)[:, None, None]) * 0.01   # us after the launch's first start
    t0 = t[:, :, 0]
    win = t[:, :, 17:16 + W].max(axis=2)                 # waves 1 .. W-1
    live = t[:, :, 48:48 + W].max(axis=2)
    end = t[:, :, 4]
    span = end.max(axis=1)
    xcc = A[0, :, 3] & 0xF
    hw = A[0, :, 8]
    cu = (xcc << 8) | ((hw >> 8) & 0xFF)                  # XCD, engine, array, CU
    _, inv, cnt = np.unique(cu, return_inverse=True, return_counts=True)
    shared = cnt[inv] > 1                                # units whose CU ran two or more of them
    life = end - t0
    res = {
        "workload": w.name, "units": units, "waves": W, "layers_cycled": dec.L, "replays": reps,
        "stamping_build_us_per_step": round(us_step, 3),
        "launch_span_us": _quantiles(span),
        "gap_between_launches_us": round(us_step - float(np.median(span)), 3),
        "start_us": _quantiles(t0),
        "q_idx_us": _quantiles(t[:, :, 5] - t0),
        "first_keys_scored_us": _quantiles(t[:, :, 6] - t0),
        "scores_in_lds_us": _quantiles(t[:, :, 1] - t0),
        "routed_us": _quantiles(t[:, :, 2] - t0),
        "window_done_us": _quantiles(win - t0),
        "live_done_us": _quantiles(live - t0),
        "merge_groups_done_us": _quantiles(t[:, :, 56:56 + W].max(axis=2) - t0),
        "merge_barrier_us": _quantiles(t[:, :, 7] - t0),
        "end_us": _quantiles(life),
        "routing_us": _quantiles(t[:, :, 2] - t[:, :, 1]),
        # inside the routing (one-wave path): max, threshold, compaction, ranks, entmax, outputs
        "routing_parts_us": [round(float(np.median(b - a)), 3) for a, b in
                             ((t[:, :, 1], t[:, :, 9]), (t[:, :, 9], t[:, :, 10]), (t[:, :, 10], t[:, :, 11]),
                              (t[:, :, 11], t[:, :, 12]), (t[:, :, 12], t[:, :, 13]), (t[:, :, 13], t[:, :, 2]))],
        "window_after_scores_us": _quantiles(win - t[:, :, 1]),
        "live_after_routing_us": _quantiles(live - np.maximum(t[:, :, 2], win)),
        "finish_us": _quantiles(end - live),
        "cus_used": int(len(cnt)), "units_on_shared_cus": int(shared.sum()),
        "end_us_alone": _quantiles(life[:, ~shared]) if (~shared).any() else None,
        "end_us_shared": _quantiles(life[:, shared]) if shared.any() else None,
        "shared_vs_alone_p50_us": {
            k: [round(float(np.median(v[:, ~shared])), 3) if (~shared).any() else None,
                round(float(np.median(v[:, shared])), 3) if shared.any() else None]
            for k, v in (("q_idx", t[:, :, 5] - t0), ("scores_in_lds", t[:, :, 1] - t0),
                         ("routed", t[:, :, 2] - t0), ("window_done", win - t0), ("live_done", live - t0),
                         ("end", life))},
        "units_per_xcd": np.bincount(xcc.astype(np.int64), minlength=8).tolist(),
        "start_us_p50_by_xcd": [round(float(np.median(t0[:, xcc == k])), 3) if (xcc == k).any() else None
                                for k in range(8)],
        "kernel_source": kernel_source_hash(),
    }
    print(json.dumps({"phases": res}), flush=True)


def _layers_needed(w, base):
    """Layers to cycle: enough that the steps' working set is twice the
    Infinity Cache; the sparse step's bytes depend on the live blocks,
    measured on one step of a scratch copy."""
    from long_context_decode_attn_amd import synth as S
    from long_context_decode_attn_amd.runner import layers_for
    from long_context_decode_attn_amd.session import to_device
    live_est = None
    if w.sparse:
        probe = base.clone()
        q, k, v = S.step_inputs(w, 0)
        probe.step(to_device(q, w.dtype), to_device(k, w.dtype), to_device(v, w.dtype))
        live_est = int(np.sum((probe.sel_idx.cpu().numpy() >= 0) & np.isfinite(probe.sel_bias.cpu().numpy())))
        del probe
    return layers_for(sum(algorithmic_bytes(w, live_est).values()))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the decode path has no "
              f"cross-GPU step: sequences (and heads) split across GPUs with no communication.",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate:
        return calibrate_main(args)
    if args.prefill_route:
        return prefill_main(args)
    if args.rope_page2d:
        return rope_main(args)
    if args.ngram_ban:
        return ngram_main(args)
    if args.phases:
        return phases_main(args)

    from long_context_decode_attn_amd import synth as S
    w = S.WORKLOADS[args.workload]
    if args.t0 is not None:
        w = w.replace(t0=args.t0)
    if args.pages is not None or args.batch is not None:
        pages = w.pages if args.pages is None else args.pages
        batch = w.batch if args.batch is None else args.batch
        if pages < 1 or batch < 1 or (w.sparse and pages * S.TOKENS_PER_PAGE // w.block < w.planted):
            sys.exit(f"--pages {pages} --batch {batch}: out of range for {w.name}")
        w = w.replace(name=f"{w.name}@{pages}p-b{batch}", pages=pages, batch=batch)
    # the CPU baseline forks its worker processes before anything touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds)

    import torch

    from long_context_decode_attn_amd import uocr as U
    from long_context_decode_attn_amd.runner import LayeredDecoder
    from long_context_decode_attn_amd.session import DecodeSession

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    U.load_library()
    torch.cuda.set_device(0)
    t_setup = time.perf_counter()
    fused = args.mode == "fused"
    base = DecodeSession(w, num_splits=args.num_splits, fused=fused)
    if w.sparse:
        base.build_index()   # the first launch also loads the kernel; the build is timed below

    n_layers = args.layers if args.layers > 0 else _layers_needed(w, base)
    dec = LayeredDecoder(w, n_layers, num_splits=args.num_splits, fused=fused, base=base, rope=args.rope)
    torch.cuda.synchronize()

    # one-time block index per layer (timed on its own, reported separately)
    idx_ms = None
    if w.sparse:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dec.build_index()
        e1.record()
        torch.cuda.synchronize()
        idx_ms = e0.elapsed_time(e1) / dec.L

    if args.copy_calibration:
        calibration_copy()
    dec.fill_pool(64)
    setup_s = time.perf_counter() - t_setup

    dec.run_eager(args.warmup)
    torch.cuda.synchronize()

    # ---- eager (host-launched) throughput, for reference ----
    n_eager = min(args.steps, 500)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    dec.run_eager(n_eager)
    e1.record()
    torch.cuda.synchronize()
    eager_ms_per_step = e0.elapsed_time(e1) / n_eager

    # ---- HIP graphs: G = 2 L steps (two per layer), and a tail for K mod G ----
    G = dec.G
    graph = dec.capture()
    graph.replay()
    torch.cuda.synchronize()
    reps, rest = divmod(args.steps, G)
    tail = None
    if rest:
        tail = dec.capture(rest)
        tail.replay()
        torch.cuda.synchronize()
        dec.fix_tail_counts(rest)
    steps = reps * G + rest

    # ---- timed region: exactly K steps ----
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        graph.replay()
    if tail is not None:
        tail.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop)
    ms_per_step = ms / steps
    value = w.units * steps / (ms / 1e3)

    # ---- per-kernel durations ----
    if fused:
        # one kernel per step: its average duration in the timed region
        names = ["uocr_srswa_step" if w.sparse else "uocr_rswa_step"]
        kern_ms = {names[0]: ms_per_step}
    else:
        # separate launches: HIP events around each launch (eager; adds the
        # event overhead to every kernel)
        names = ["uocr_ring_append"] + (["uocr_block_score", "uocr_entmax15_topk", "uocr_srswa_decode"]
                                        if w.sparse else ["uocr_rswa_decode"])
        nk = min(args.steps, 500)
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
              for _ in range(nk)]
        torch.cuda.synchronize()
        for i in range(nk):
            s = dec.layers[i % dec.L]
            q, k, v = dec.q[i % G], dec.k[i % G], dec.v[i % G]
            calls = [lambda: s.append(k, v)]
            if w.sparse:
                calls += [lambda: s.score(q), s.select, lambda: s.attend(q)]
            else:
                calls += [lambda: s.attend(q)]
            for (a, b), c in zip(ev[i], calls):
                a.record()
                c()
                b.record()
        torch.cuda.synchronize()
        kern_ms = {n: float(np.mean([ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(nk)]))
                   for j, n in enumerate(names)}

    live = None
    if w.sparse:
        if fused:   # the selections of the last replay's steps
            slots = range(min(steps, G))
            live = sum(dec.live_blocks(g) for g in slots) / len(slots)
        else:
            sb, si = dec.layers[0].sel_bias.cpu().numpy(), dec.layers[0].sel_idx.cpu().numpy()
            live = int(np.sum((si >= 0) & np.isfinite(sb)))
    abytes = algorithmic_bytes(w, live)
    if fused:   # the step kernel moves what the rows it fuses move (scores stay on chip)
        total = sum(abytes.values())
        if w.sparse:
            total -= 2 * w.units * w.n_blocks * 4
        abytes = {names[0]: int(total)}
    kernels = {n: {"avg_us": round(kern_ms[n] * 1e3, 3), "algorithmic_bytes": abytes[n],
                   "gbs": round(abytes[n] / (kern_ms[n] * 1e-3) / 1e9, 1)} for n in names}
    dom = max(names, key=lambda n: kern_ms[n])
    achieved = abytes[dom] / (kern_ms[dom] * 1e-3) / 1e9
    step_bytes = sum(abytes.values())

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": UNIT, "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "prefix_tokens": w.prefix_len, "pages": w.pages, "window": w.window, "t0": w.t0,
                   "sparse": w.sparse, "topk": w.topk if w.sparse else None,
                   "block": w.block if w.sparse else None, "layers_cycled": dec.L,
                   "splits": ((args.num_splits or 8) if w.sparse and fused
                              else U.uocr_srswa_splits(base.shape, base.route, args.num_splits) if w.sparse
                              else U.uocr_rswa_splits(base.shape, args.num_splits)),
                   "mode": args.mode, "rope": "page2d fused" if args.rope else None,
                   "accumulate": "f32 attention, f64 routing",
                   "parallelism": "single-gpu"},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic(dom, w.name)},
        "step_gbs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "timing": (f"HIP graph of {G} steps replayed {reps} times" + (f" + a {rest}-step graph" if rest else "")
                   + f" between HIP events; eager launches: {eager_ms_per_step * 1e3:.2f} us/step"),
        "eager_ms_per_step": round(eager_ms_per_step, 5),
        "kernels": kernels,
        "kernel_source": kernel_source_hash(),
    }
    if w.sparse:
        result["routing"] = {"live_blocks_per_unit": round(live / w.units, 3),
                             "index_build_ms_per_layer": round(idx_ms, 4),
                             "index_build_gbs": round(index_bytes(w) / (idx_ms * 1e-3) / 1e9, 1)}
    result["setup_s"] = round(setup_s, 1)
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
