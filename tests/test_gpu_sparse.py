"""GPU parity of the SR-SWA path (block index, block scores, 1.5-entmax top-k,
sparse decode) against the oracle, called through the C ABI."""
import math

import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import synth as S
from long_context_decode_attn_amd import uocr as U
from long_context_decode_attn_amd.session import DecodeSession, to_device, to_host
from oracle import uocr_oracle as O
from tests._gpu_common import HostMirror, assert_close, need_gpu, say

pytestmark = pytest.mark.gpu

PROB_TOL = 1e-6      # |p_gpu - p_oracle|: fp64 threshold on both sides
BIAS_TOL = 1e-4      # |ln p_gpu - ln p_oracle| where p_oracle > 1e-3


def _small_sparse(**kw):
    base = dict(name="sparse-small", batch=2, heads=3, head_dim=128, dtype="bf16", pages=6, prompt=0,
                t0=128, steps=4, seed=91, sparse=True, planted=5, fixed_query=True)
    base.update(kw)
    return S.Workload(**base)


def _check_selection(got_idx, got_prob, got_bias, s32, k, s64=None, eps=None, what=""):
    """Selected set bit-exact against the oracle's routing of the same scores.
    When the GPU computed the scores itself (s64 and eps given) and its set
    differs, the set must be one that scores within the certified bounds can
    select: every surely selected block in it, no surely dropped one."""
    idx, prob, bias = O.route_unit(s32, k)
    if not np.array_equal(got_idx, idx):
        assert s64 is not None and O.selection_within_bounds(got_idx, s64, eps, k), f"{what}: {got_idx} != {idx}"
        return False
    # Weights: same fp32 scores -> PROB_TOL.  When the GPU computed the scores
    # itself they may differ from the oracle's by the certified bound eps;
    # p = (s/2 - tau)^2 moves by at most 2 * max|ds| (|s/2 - tau| <= 1 and tau
    # moves by at most max|ds|/2).
    ptol = PROB_TOL if eps is None else PROB_TOL + 2.0 * float(np.max(eps, initial=0.0))
    np.testing.assert_allclose(got_prob, prob, atol=ptol, err_msg=what)
    big = prob > 1e-3
    np.testing.assert_allclose(got_bias[big], bias[big], atol=BIAS_TOL + ptol / 1e-3, err_msg=what)
    dead = (prob == 0) & (idx >= 0)
    assert (got_prob[dead] <= ptol).all(), what
    assert (np.isneginf(got_bias[dead]) | (got_bias[dead] <= math.log(ptol))).all(), what
    assert np.isneginf(got_bias[idx < 0]).all() and (got_idx[idx < 0] == -1).all()
    return True


# ----------------------------------------------------------------------------
# routing pieces
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,head_dim", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_block_index_and_scores_match_oracle(dtype, head_dim):
    need_gpu()
    for pages, prompt, plens in [(6, 0, None), (2, 17, [529, 31, 1]), (9, 5, [1000, 0, 70, 33])]:
        w = _small_sparse(batch=len(plens) if plens else 2, pages=pages, prompt=prompt, dtype=dtype,
                          head_dim=head_dim)
        say("block index/score", dtype, head_dim, pages, prompt, plens)
        sess = DecodeSession(w)
        host = HostMirror(w)
        if plens:
            sess.prefix_len.copy_(torch.tensor(plens, dtype=torch.int32))
            host.prefix_len = np.asarray(plens)
        sess.build_index()
        q, _, _ = S.step_inputs(w, 0)
        sess.score(to_device(q, w.dtype))
        torch.cuda.synchronize()
        kbar = sess.kbar.cpu().numpy().astype(np.float64)
        scores = sess.scores.cpu().numpy().astype(np.float64)
        P = S.projection(w).astype(np.float64)
        qd = S.widen(q, w.dtype)
        for b in range(w.batch):
            m = int(host.prefix_len[b])
            nb = -(-m // 32)
            for h in range(w.heads):
                kb = O.block_index(host.Kp[b, h], m, P)
                np.testing.assert_allclose(kbar[b, h, :nb], kb, rtol=1e-6, atol=1e-7)
                assert (kbar[b, h, nb:] == 0).all()
                s64 = O.block_scores(qd[b, h], P, kb)
                eps = O.score_error_bound(qd[b, h], P, kb)
                assert (np.abs(scores[b, h, :nb] - s64) <= eps).all()
                assert np.isneginf(scores[b, h, nb:]).all()


@pytest.mark.parametrize("nb,spread,k", [(1, 1.0, 16), (5, 1.0, 16), (16, 1.0, 16), (17, 1.0, 16),
                                         (320, 4.0, 16), (1000, 4.0, 16), (1000, 0.05, 16),
                                         (4096, 0.01, 16), (4096, 4.0, 64), (300, 0.3, 1)])
def test_entmax_topk_bit_exact_selection(nb, spread, k):
    """Selection and weights from the same fp32 scores: bit-exact indices.
    Small spreads give hundreds or thousands of entmax candidates (the sorted
    path), large spreads a handful."""
    need_gpu()
    B, H = 3, 2
    shape = U.Shape(B, H, 128, nb * 32)
    route = U.Route(topk=k)
    sc = S.random_scores(nb * 7 + k, B * H, nb, spread).reshape(B, H, nb)
    plen = np.array([nb * 32, max(1, nb * 32 - 45), 31])   # full, ragged, one block
    scores = torch.from_numpy(sc).cuda()
    pl = torch.from_numpy(plen.astype(np.int32)).cuda()
    idx = torch.empty((B, H, k), dtype=torch.int32, device="cuda")
    prob = torch.empty((B, H, k), dtype=torch.float32, device="cuda")
    bias = torch.empty((B, H, k), dtype=torch.float32, device="cuda")
    U.uocr_entmax15_topk(shape, route, scores, pl, idx, prob, bias)
    torch.cuda.synchronize()
    gi, gp, gb = idx.cpu().numpy(), prob.cpu().numpy().astype(np.float64), bias.cpu().numpy().astype(np.float64)
    for b in range(B):
        nbb = -(-int(plen[b]) // 32)
        for h in range(H):
            assert _check_selection(gi[b, h], gp[b, h], gb[b, h], sc[b, h, :nbb].astype(np.float64), k,
                                    what=f"nb={nb} b={b} h={h}")


def test_entmax_topk_ties_resolved_by_index():
    need_gpu()
    B, H, nb, k = 2, 2, 200, 16
    rng = np.random.default_rng(4)
    sc = rng.integers(-2, 3, size=(B, H, nb)).astype(np.float32)   # many exact ties
    sc[1, 1] = 0.0                                                  # all equal: uniform entmax
    shape, route = U.Shape(B, H, 128, nb * 32), U.Route(topk=k)
    idx = torch.empty((B, H, k), dtype=torch.int32, device="cuda")
    prob = torch.empty((B, H, k), dtype=torch.float32, device="cuda")
    bias = torch.empty((B, H, k), dtype=torch.float32, device="cuda")
    U.uocr_entmax15_topk(shape, route, torch.from_numpy(sc).cuda(),
                         torch.full((B,), nb * 32, dtype=torch.int32, device="cuda"), idx, prob, bias)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            assert _check_selection(idx.cpu().numpy()[b, h], prob.cpu().numpy()[b, h].astype(float),
                                    bias.cpu().numpy()[b, h].astype(float), sc[b, h].astype(float), k)
    np.testing.assert_allclose(prob.cpu().numpy()[1, 1], 1.0 / nb, rtol=1e-6)


@pytest.mark.parametrize("dtype,head_dim", [("bf16", 128), ("f32", 64)])
def test_block_index_range_grows_with_the_prefix(dtype, head_dim):
    """Chunked prefill: after each chunk, rebuilding only the blocks from the
    one holding the old end gives, bit for bit, what a full build at the new
    lengths gives (per-sequence lengths differ; blocks past a sequence's
    prefix are zero in both)."""
    need_gpu()
    w = _small_sparse(batch=3, heads=2, pages=6, prompt=0, dtype=dtype, head_dim=head_dim)
    say("index range", dtype, head_dim)
    kv = S.prefix_kv(w)
    sess = DecodeSession(w, prefix_kv=kv)
    full = DecodeSession(w, prefix_kv=kv)
    sess.kbar.zero_()
    old = np.zeros(w.batch, dtype=np.int64)
    for step, base in enumerate([70, 700, 701, 1100, w.prefix_len]):
        new = np.minimum(base + 37 * np.arange(w.batch), w.prefix_len)
        first = int(old.min()) // 32
        last = -(-int(new.max()) // 32)
        pl = torch.from_numpy(new.astype(np.int32)).cuda()
        sess.prefix_len.copy_(pl)
        U.uocr_block_index_range(sess.shape, sess.route, sess.k_prefix, sess.prefix_len, sess.proj, sess.kbar,
                                 first, last)
        full.prefix_len.copy_(pl)
        full.build_index()
        torch.cuda.synchronize()
        assert torch.equal(sess.kbar, full.kbar), f"chunk {step}: range [{first}, {last})"
        old = new


@pytest.mark.parametrize("nb", [50, 100, 200, 400, 1000])
def test_entmax_topk_one_wave_ties_and_signed_zeros(nb):
    """The one-wave path (a small candidate set) with exact ties across the
    rank-k boundary, and with +0 and -0 scores, which the float order takes as
    equal: the selection must follow (score desc, index asc) bit for bit."""
    need_gpu()
    say("one-wave ties", nb)
    B, H, k = 2, 2, 16
    rng = np.random.default_rng(nb)
    sc = (rng.standard_normal((B, H, nb)) - 30.0).astype(np.float32)
    for h in range(H):
        top = rng.permutation(nb)[:22]
        sc[0, h, top[:10]] = 3.0          # ranks 0-9
        sc[0, h, top[10:]] = 2.75         # 12 equal scores across rank 16
        zeros = rng.permutation(nb)[:20]
        sc[1, h, zeros[:10]] = 0.0
        sc[1, h, zeros[10:]] = -0.0       # 20 zeros of both signs: the top 16 by index
        sc[1, h, rng.permutation(np.setdiff1d(np.arange(nb), zeros))[:5]] = -0.5
    shape, route = U.Shape(B, H, 128, nb * 32), U.Route(topk=k)
    idx = torch.empty((B, H, k), dtype=torch.int32, device="cuda")
    prob = torch.empty((B, H, k), dtype=torch.float32, device="cuda")
    bias = torch.empty((B, H, k), dtype=torch.float32, device="cuda")
    U.uocr_entmax15_topk(shape, route, torch.from_numpy(sc).cuda(),
                         torch.full((B,), nb * 32, dtype=torch.int32, device="cuda"), idx, prob, bias)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            assert _check_selection(idx.cpu().numpy()[b, h], prob.cpu().numpy()[b, h].astype(float),
                                    bias.cpu().numpy()[b, h].astype(float), sc[b, h].astype(float), k,
                                    what=f"nb={nb} b={b} h={h}")


@pytest.mark.parametrize("live,with_bias,num_splits", [(0, True, 0), (1, True, 0), (5, True, 0), (16, True, 0),
                                                        (16, False, 0), (16, True, 1), (5, True, 3), (16, True, 64)])
def test_srswa_decode_given_selection(live, with_bias, num_splits):
    """Sparse decode on its own, for a given routing result: every live
    block, dead blocks (bias -inf, never read: their rows are NaN), -1 padding;
    one workgroup per unit or several (merged through the workspace; 64 leaves
    most workgroups without rows)."""
    need_gpu()
    w = _small_sparse(batch=3, heads=2, pages=3, prompt=20, t0=0)
    say("srswa given selection", live, with_bias, num_splits)
    t0 = [0, 7, 300]
    Kr, Vr, tg = S.initial_ring(w, t0)
    kv = S.prefix_kv(w)
    sess = DecodeSession(w, prefix_kv=kv, ring=(Kr, Vr, tg), num_splits=num_splits)
    host = HostMirror(w, prefix_kv=kv, ring=(Kr, Vr, tg))
    nb = w.n_blocks
    idx, bias = S.random_selection(5 + live, w.units, nb, 16, live)
    idx = idx.reshape(w.batch, w.heads, 16)
    bias = bias.reshape(w.batch, w.heads, 16)
    idx[0, 0, -1] = -1                    # padding entry
    bias = bias if with_bias else None
    Kp = kv[0].copy()
    Vp = kv[1].copy()
    if with_bias:                          # poison dead blocks: they must not be read
        for b in range(w.batch):
            for h in range(w.heads):
                for i in range(16):
                    if idx[b, h, i] >= 0 and np.isneginf(bias[b, h, i]):
                        j = idx[b, h, i]
                        Kp[b, h, 32 * j:32 * j + 32] = S.NAN_BITS["bf16"]
                        Vp[b, h, 32 * j:32 * j + 32] = S.NAN_BITS["bf16"]
        sess.k_prefix.copy_(to_device(Kp, "bf16"))
        sess.v_prefix.copy_(to_device(Vp, "bf16"))
    q, _, _ = S.step_inputs(w, 0)
    sess.sel_idx.copy_(torch.from_numpy(idx))
    sb = None if bias is None else torch.from_numpy(bias).cuda()
    U.uocr_srswa_decode(sess.shape, sess.route, to_device(q, "bf16"), sess.k_prefix, sess.v_prefix,
                        sess.prefix_len, sess.sel_idx, sb, sess.k_ring, sess.v_ring, sess.t_gen, sess.out,
                        sess.workspace, num_splits)
    torch.cuda.synchronize()
    qd = S.widen(q, "bf16")
    got = to_host(sess.out)
    ref = np.zeros_like(got)
    for b in range(w.batch):
        for h in range(w.heads):
            ref[b, h] = O.srswa_unit(qd[b, h], host.Kp[b, h], host.Vp[b, h], w.prefix_len, idx[b, h],
                                     None if bias is None else bias[b, h], *host.window(b, h), w.scale)
    assert_close(got, ref, "bf16", f"live={live}")


@pytest.mark.parametrize("num_splits,fused", [(0, False), (1, False), (3, False), (8, False),
                                              (0, True), (4, True), (8, True), (16, True)])
def test_srswa_pipeline_small(num_splits, fused):
    """append -> score -> entmax top-k -> sparse decode for several steps,
    selections and outputs against the oracle's own routing."""
    need_gpu()
    w = _small_sparse(pages=7, prompt=11, planted=6)
    say("srswa pipeline, splits", num_splits, "fused" if fused else "")
    _run_sparse(w, steps=5, num_splits=num_splits, fused=fused)


@pytest.mark.parametrize("fused", [False, True])
def test_srswa_wide_support_and_ragged(fused):
    """Flat routing (most blocks inside the entmax support, all 16 selected
    blocks live), a ragged last block and per-sequence generated counts."""
    need_gpu()
    w = _small_sparse(batch=3, pages=5, prompt=23, planted=0, t0=0, fixed_query=False)
    _run_sparse(w, steps=4, fused=fused, t_gen=[0, 9, 500], flat=True)


@pytest.mark.parametrize("fused", [False, True])
def test_srswa_per_sequence_prefix_lengths(fused):
    """One batch whose sequences have their own prefix lengths: none, one
    token, one token into the second block, a prefix ending inside a block and
    the full prefix.  Rows past each prefix hold NaN, so a read of one would
    show in the output."""
    need_gpu()
    w = _small_sparse(batch=5, pages=4, prompt=9, planted=3, t0=0)
    plens = [0, 1, 33, 500, w.prefix_len]
    say("srswa per-sequence prefixes", plens, "fused" if fused else "")
    _run_sparse(w, steps=3, fused=fused, t_gen=[0, 5, 127, 128, 400], plens=plens)


@pytest.mark.parametrize("fused", [False, True])
def test_srswa_over_1024_blocks(fused):
    """130 pages (1040 blocks): past the one-wave routing, so the whole
    workgroup routes before the live blocks are read."""
    need_gpu()
    w = _small_sparse(batch=2, heads=2, pages=130, planted=4, t0=0)
    say("srswa 1040 blocks", "fused" if fused else "")
    _run_sparse(w, steps=2, fused=fused, t_gen=[3, 300])


@pytest.mark.parametrize("fused", [False, True])
def test_srswa_all_blocks_tied(fused):
    """Every block scores the same, so more than 64 blocks tie at the k-th
    score and the one-wave routing hands over to the workgroup path.  Entmax is
    uniform (p = 1/nb on every block) and the first 16 blocks by index are
    selected, all of them live."""
    need_gpu()
    w = _small_sparse(batch=2, heads=2, pages=13, planted=0, t0=0)
    say("srswa tied blocks", "fused" if fused else "")
    _run_sparse(w, steps=2, fused=fused, t_gen=[0, 200], tied=True)


# unusual shapes: head dims, dtypes, windows from 1 to 1024 slots, top-k from
# 1 to 64, prefixes that end inside a block, counts before / across a wrap
_SWEEP = [
    dict(dtype="bf16", head_dim=64, window=8, topk=4, pages=2, prompt=5, t_gen=[0, 3, 20]),
    dict(dtype="bf16", head_dim=128, window=200, topk=40, pages=3, prompt=31, t_gen=[0, 150, 1000]),
    dict(dtype="f32", head_dim=128, window=64, topk=1, pages=1, prompt=0, t_gen=[64]),
    dict(dtype="bf16", head_dim=128, window=128, topk=64, pages=9, prompt=7, t_gen=[127, 128, 129]),
    dict(dtype="f32", head_dim=64, window=1, topk=16, pages=2, prompt=1, t_gen=[0, 1]),
    dict(dtype="bf16", head_dim=64, window=1024, topk=16, pages=4, prompt=17, t_gen=[0, 700, 3000]),
]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("cfg", range(len(_SWEEP)))
def test_srswa_shape_sweep(cfg, fused):
    need_gpu()
    c = dict(_SWEEP[cfg])
    t_gen = c.pop("t_gen")
    w = _small_sparse(batch=len(t_gen), heads=2, planted=3, t0=0, seed=200 + cfg, **c)
    say("srswa sweep", cfg, c, t_gen, "fused" if fused else "")
    _run_sparse(w, steps=3, fused=fused, t_gen=t_gen)


def _run_sparse(w, steps, units=None, num_splits=0, k=None, fused=False, t_gen=None, flat=False, plens=None,
                tied=False):
    kv = S.prefix_kv(w)
    if flat:   # shrink the keys so that block scores are close together (wide support)
        Kf = S.widen(kv[0], w.dtype) * 0.05
        kv = (S.store(Kf.astype(np.float32), w.dtype), kv[1])
    if tied:   # every block's keys are block 0's: all block scores tie exactly
        nbk = w.prefix_len // w.block
        kv = (np.ascontiguousarray(np.tile(kv[0][:, :, :w.block], (1, 1, nbk, 1))), kv[1])
    if plens is not None:   # rows past each sequence's own prefix hold NaN: never read
        for b, m in enumerate(plens):
            kv[0][b, :, m:] = S.NAN_BITS[w.dtype]
            kv[1][b, :, m:] = S.NAN_BITS[w.dtype]
    ring = S.initial_ring(w, t_gen)
    sess = DecodeSession(w, prefix_kv=kv, ring=ring, num_splits=num_splits, fused=fused)
    host = HostMirror(w, prefix_kv=kv, ring=ring)
    if plens is not None:
        sess.prefix_len.copy_(torch.tensor(plens, dtype=torch.int32))
        host.prefix_len = np.asarray(plens)
    del kv
    sess.build_index()
    P = S.projection(w).astype(np.float64)
    units = [(b, h) for b in range(w.batch) for h in range(w.heads)] if units is None else units
    k = w.topk
    routing = {}
    amb = 0
    for step in range(steps):
        q, kn, vn = S.step_inputs(w, step)
        out = sess.step(to_device(q, w.dtype), to_device(kn, w.dtype), to_device(vn, w.dtype))
        host.append(kn, vn)
        got = to_host(out)
        assert np.isfinite(got).all()
        assert np.array_equal(sess.t_gen.cpu().numpy(), host.t_gen.astype(np.int32))
        gi = sess.sel_idx.cpu().numpy()
        gp = sess.sel_prob.cpu().numpy().astype(np.float64)
        gb = sess.sel_bias.cpu().numpy().astype(np.float64)
        qd = S.widen(q, w.dtype)
        ref, sel = [], []
        for b, h in units:
            key = (b, h, None if w.fixed_query else step)
            if key not in routing:
                m = int(host.prefix_len[b])
                kb = O.block_index(host.Kp[b, h], m, P)
                s64 = O.block_scores(qd[b, h], P, kb)
                routing[key] = (s64, O.as_f32(s64), O.score_error_bound(qd[b, h], P, kb))
            s64, s32, eps = routing[key]
            exact = _check_selection(gi[b, h], gp[b, h], gb[b, h], s32, k, s64, eps, f"step {step} unit {(b, h)}")
            amb += 0 if exact else 1
            ridx, _, rbias = O.route_unit(s32, k)
            ref.append(O.srswa_unit(qd[b, h], host.Kp[b, h], host.Vp[b, h], int(host.prefix_len[b]), ridx, rbias,
                                    *host.window(b, h), w.scale))
            sel.append(got[b, h])
        assert_close(np.stack(sel), np.stack(ref), w.dtype, f"{w.name} step {step}")
        if flat:
            assert (np.isfinite(gb) & (gi >= 0)).sum(axis=-1).min() == min(k, w.n_blocks)
    say("ambiguous boundaries:", amb)
    return amb


@pytest.mark.parametrize("name,fused", [("srswa-40p-b32", False), ("srswa-125p-b8", False),
                                        ("srswa-40p-b32", True), ("srswa-125p-b8", True)])
def test_srswa_full_size(name, fused):
    """Full-size SR-SWA workloads (40 pages x 32 sequences; 125 pages x 8
    sequences) in the benchmark's launch configuration: every unit's routing
    and output checked for two steps."""
    need_gpu()
    w = S.WORKLOADS[name]
    say("full-size sparse", name, "fused" if fused else "")
    _run_sparse(w, steps=2, fused=fused)


def test_srswa_reduces_to_dense_when_every_block_is_kept():
    """topk >= number of blocks and zero bias: sparse decode == dense R-SWA."""
    need_gpu()
    w = _small_sparse(pages=1, prompt=64, planted=0, topk=16)      # 320 tokens = 10 blocks
    kv = S.prefix_kv(w)
    ring = S.initial_ring(w)
    sess = DecodeSession(w, prefix_kv=kv, ring=ring)
    dense = DecodeSession(w.replace(sparse=False), prefix_kv=kv, ring=ring)
    host = HostMirror(w, prefix_kv=kv, ring=ring)
    nb = w.n_blocks
    idx = np.full((w.batch, w.heads, 16), -1, np.int32)
    idx[:, :, :nb] = np.arange(nb)
    sess.sel_idx.copy_(torch.from_numpy(idx))
    q, _, _ = S.step_inputs(w, 0)
    qt = to_device(q, "bf16")
    U.uocr_srswa_decode(sess.shape, sess.route, qt, sess.k_prefix, sess.v_prefix, sess.prefix_len, sess.sel_idx,
                        None, sess.k_ring, sess.v_ring, sess.t_gen, sess.out, sess.workspace)
    dense.attend(qt)
    torch.cuda.synchronize()
    qd = S.widen(q, "bf16")
    ref = np.stack([[O.rswa_unit(qd[b, h], host.Kp[b, h], host.Vp[b, h], w.prefix_len, *host.window(b, h), w.scale)
                     for h in range(w.heads)] for b in range(w.batch)])
    assert_close(to_host(sess.out), ref, "bf16", "sparse(all blocks)")
    assert_close(to_host(dense.out), ref, "bf16", "dense")
    assert np.abs(to_host(sess.out) - to_host(dense.out)).max() <= 2 ** -7


@pytest.mark.parametrize("fused", [False, True])
def test_page_window_advance_keeps_the_ring(fused):
    """Page-window scheduling's KV-tail carry-over: after some steps the
    prefix is replaced by the next window of pages (new K/V, a shorter
    prefix, the block index rebuilt) while the ring and the generated count
    carry over; every step matches the oracle run over the same sequence of
    prefixes and one continuous ring."""
    need_gpu()
    wA = _small_sparse(pages=6, prompt=0, planted=4)
    wB = wA.replace(seed=wA.seed + 1)
    say("page-window advance", "fused" if fused else "separate")
    kvA, kvB = S.prefix_kv(wA), S.prefix_kv(wB)
    ring = S.initial_ring(wA)
    sess = DecodeSession(wA, prefix_kv=kvA, ring=ring, fused=fused)
    host = HostMirror(wA, prefix_kv=kvA, ring=ring)
    sess.build_index()
    P = S.projection(wA).astype(np.float64)
    mB = wA.prefix_len - 100
    for step in range(6):
        if step == 3:   # next window of pages
            KB, VB = to_device(kvB[0], wA.dtype), to_device(kvB[1], wA.dtype)
            sess.k_prefix.copy_(KB)
            sess.v_prefix.copy_(VB)
            sess.prefix_len.fill_(mB)
            sess.build_index()
            host.Kp, host.Vp = S.widen(kvB[0], wA.dtype), S.widen(kvB[1], wA.dtype)
            host.prefix_len = np.full(wA.batch, mB)
        q, kn, vn = S.step_inputs(wA, step)
        out = to_host(sess.step(to_device(q, wA.dtype), to_device(kn, wA.dtype), to_device(vn, wA.dtype)))
        host.append(kn, vn)
        assert np.array_equal(sess.t_gen.cpu().numpy(), host.t_gen.astype(np.int32))
        qd = S.widen(q, wA.dtype)
        gi = sess.sel_idx.cpu().numpy()
        ref, got = [], []
        for b in range(wA.batch):
            for h in range(wA.heads):
                m = int(host.prefix_len[b])
                kb = O.block_index(host.Kp[b, h], m, P)
                s64 = O.block_scores(qd[b, h], P, kb)
                s32 = O.as_f32(s64)
                eps = O.score_error_bound(qd[b, h], P, kb)
                _check_selection(gi[b, h], sess.sel_prob[b, h].cpu().numpy().astype(np.float64),
                                 sess.sel_bias[b, h].cpu().numpy().astype(np.float64), s32, wA.topk, s64, eps,
                                 f"step {step} unit {(b, h)}")
                ridx, _, rbias = O.route_unit(s32, wA.topk)
                ref.append(O.srswa_unit(qd[b, h], host.Kp[b, h], host.Vp[b, h], m, ridx, rbias,
                                        *host.window(b, h), wA.scale))
                got.append(out[b, h])
        assert_close(np.stack(got), np.stack(ref), wA.dtype, f"step {step}")
