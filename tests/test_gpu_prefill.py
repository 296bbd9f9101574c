"""GPU parity of prefill-side routing (uocr_prefill_route) against the
oracle's prefill_route_unit, called through the C ABI: every query of the
chunk routed over the blocks wholly before it."""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import synth as S
from long_context_decode_attn_amd.session import DecodeSession, to_device
from oracle import uocr_oracle as O
from tests._gpu_common import need_gpu, say
from tests.test_gpu_sparse import _check_selection

pytestmark = pytest.mark.gpu


def _run(w, tq, q_pos, plens=None, units=None, chunk=0):
    sess = DecodeSession(w)
    kv = None
    if plens is not None:
        sess.prefix_len.copy_(torch.tensor(plens, dtype=torch.int32))
    sess.build_index()
    qs = S.prefill_queries(w, tq, chunk)
    idx, prob, bias = sess.prefill_route(to_device(qs, w.dtype),
                                         torch.tensor(q_pos, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    idx, prob, bias = idx.cpu().numpy(), prob.cpu().numpy().astype(np.float64), bias.cpu().numpy().astype(np.float64)
    P = S.projection(w).astype(np.float64)
    qd = S.widen(qs, w.dtype)
    units = [(b, h) for b in range(w.batch) for h in range(w.heads)] if units is None else units
    exact = ties = 0
    for b in sorted({u[0] for u in units}):
        Kp, _ = S.prefix_kv_seq(w, b)
        m = w.prefix_len if plens is None else int(plens[b])
        for h in [u[1] for u in units if u[0] == b]:
            kb = O.block_index(S.widen(Kp[h], w.dtype), m, P)
            for i in range(tq):
                nbv = O.visible_blocks(int(q_pos[b]) + i, m)
                if nbv == 0:   # nothing visible: every entry empty
                    assert (idx[b, h, i] == -1).all() and (prob[b, h, i] == 0).all()
                    assert np.isneginf(bias[b, h, i]).all()
                    exact += 1
                    continue
                s64 = O.block_scores(qd[b, h, i], P, kb[:nbv])
                eps = O.score_error_bound(qd[b, h, i], P, kb[:nbv])
                ok = _check_selection(idx[b, h, i], prob[b, h, i], bias[b, h, i], O.as_f32(s64), w.topk,
                                      s64, eps, f"{w.name} b={b} h={h} i={i} t={int(q_pos[b]) + i}")
                exact += ok
                ties += not ok
                sel = idx[b, h, i][idx[b, h, i] >= 0]
                assert (np.minimum(32 * (sel + 1), m) <= int(q_pos[b]) + i).all()   # causal
    say(w.name, "queries checked", exact + ties, "certified near-tie swaps", ties)
    assert exact > 0


def _small(**kw):
    base = dict(name="prefill-small", batch=2, heads=3, head_dim=128, dtype="bf16", pages=6, prompt=0,
                t0=0, steps=1, seed=77, sparse=True, planted=5, fixed_query=True)
    base.update(kw)
    return S.Workload(**base)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
def test_prefill_route_small_chunks_cross_the_prefix_end(dtype, D):
    """Chunks that start inside the prefix (causal: few blocks visible) and
    run past its end (every block visible), ragged prefix lengths."""
    need_gpu()
    w = _small(dtype=dtype, head_dim=D)
    say("prefill route", dtype, D)
    _run(w, 200, [1400, 20], plens=[1536, 1201])


def test_prefill_route_tile_edges_and_empty():
    """tq not a multiple of the per-workgroup tile, a chunk entirely before
    the first whole block (nothing visible) and an empty prefix."""
    need_gpu()
    w = _small(batch=3, pages=3)
    say("prefill route edges")
    _run(w, 37, [0, 700, 5], plens=[768, 768, 0])


def test_prefill_route_over_1024_blocks_takes_the_workgroup_path():
    """More than 1024 visible blocks: every query is routed by the fallback
    kernel (whole workgroup, block-wide selection)."""
    need_gpu()
    w = _small(batch=1, heads=2, pages=130, planted=8)
    say("prefill route > 1024 blocks")
    _run(w, 20, [w.prefix_len - 10])


def test_prefill_route_full_size_125_pages_sampled():
    """The 125-page shape (8 x 10 units, 1000 blocks), a 64-query chunk at
    the end of the prefix, in the launch configuration the bench times; six
    units checked against the oracle."""
    need_gpu()
    w = S.WORKLOADS["srswa-125p-b8"]
    say("prefill route full size")
    _run(w, 64, [w.prefix_len - 48] * w.batch, units=[(0, 0), (1, 3), (3, 9), (5, 5), (7, 1), (7, 8)])


def test_prefill_route_wide_entmax_support():
    """200 blocks and near-flat scores for a quarter of the queries: the
    entmax support holds far more than 64 blocks, so those queries take the
    wide path (Newton on the threshold, closed form on the support found)."""
    need_gpu()
    w = _small(pages=25, planted=10)
    say("prefill route wide support")
    _run(w, 64, [w.prefix_len - 16, w.prefix_len - 40])


def test_prefill_route_builds_agree_at_512_blocks():
    """The kernel is built twice, by the most blocks a query can see: 8 routing
    slots per lane up to 512 blocks, 16 above.  The same 512-block prefix
    routed once with a capacity of 512 blocks and once with room for 520 (so
    the 16-slot build runs) gives the same selections, weights and biases bit
    for bit; a sample of queries is also checked against the oracle."""
    need_gpu()
    w = _small(batch=2, heads=2, pages=64, planted=12)
    assert w.n_blocks == 512
    tq = 48
    q_pos = torch.tensor([w.prefix_len - 32, w.prefix_len - 400], dtype=torch.int32, device="cuda")
    qs = to_device(S.prefill_queries(w, tq), w.dtype)
    outs = []
    for cap in (w.prefix_len, w.prefix_len + 8 * w.block):
        sess = DecodeSession(w, prefix_cap=cap)
        say("prefill builds: capacity", cap, "blocks", sess.shape.nb_cap)
        sess.build_index()
        outs.append([x.cpu().numpy() for x in sess.prefill_route(qs, q_pos)])
        del sess
    torch.cuda.synchronize()
    for a, b, name in zip(outs[0], outs[1], ("idx", "prob", "bias")):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{name} differs between the builds"
    idx, prob, bias = outs[0][0], outs[0][1].astype(np.float64), outs[0][2].astype(np.float64)
    P = S.projection(w).astype(np.float64)
    qd = S.widen(S.prefill_queries(w, tq), w.dtype)
    pos = q_pos.cpu().numpy()
    for b in range(w.batch):
        Kp, _ = S.prefix_kv_seq(w, b)
        for h in range(w.heads):
            kb = O.block_index(S.widen(Kp[h], w.dtype), w.prefix_len, P)
            for i in (0, 1, 2, 3, tq - 1):
                nbv = O.visible_blocks(int(pos[b]) + i, w.prefix_len)
                s64 = O.block_scores(qd[b, h, i], P, kb[:nbv])
                eps = O.score_error_bound(qd[b, h, i], P, kb[:nbv])
                _check_selection(idx[b, h, i], prob[b, h, i], bias[b, h, i], O.as_f32(s64), w.topk, s64, eps,
                                 f"builds b={b} h={h} i={i}")
