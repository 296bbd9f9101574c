"""Decode steps captured in a HIP graph: every replay matches the same steps
run eagerly, with eager work and synchronisations between the replays."""
import pytest
import torch

from long_context_decode_attn_amd import synth as S
from long_context_decode_attn_amd.session import DecodeSession, to_device
from tests._gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("sparse,fused,splits", [(True, True, 0), (True, False, 0), (False, True, 0),
                                                 (False, True, 5), (False, False, 3)])
def test_graph_replays_match_eager(sparse, fused, splits):
    need_gpu()
    if sparse:
        w = S.Workload("graph-sparse", batch=2, heads=3, head_dim=128, dtype="bf16", pages=5, prompt=0, t0=126,
                       steps=2, seed=13, sparse=True, planted=3, fixed_query=False)
    else:
        w = S.Workload("graph-dense", batch=2, heads=3, head_dim=128, dtype="bf16", pages=2, prompt=7, t0=126,
                       steps=2, seed=14)
    say("graph", w.name, "fused" if fused else "separate", splits)
    kv = S.prefix_kv(w)
    ring = S.initial_ring(w)
    g_sess = DecodeSession(w, prefix_kv=kv, ring=ring, fused=fused, num_splits=splits)
    e_sess = DecodeSession(w, prefix_kv=kv, ring=ring, fused=fused, num_splits=splits)
    if sparse:
        g_sess.build_index()
        e_sess.build_index()
    inputs = [tuple(to_device(x, w.dtype) for x in S.step_inputs(w, s)) for s in range(2)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for q, k, v in inputs:
            g_sess.step(q, k, v)
    torch.cuda.synchronize()
    # capture enqueues nothing: the state must still be the initial one
    assert torch.equal(g_sess.t_gen.cpu(), torch.from_numpy(ring[2]))
    for rep in range(4):
        graph.replay()
        for q, k, v in inputs:
            e_sess.step(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(_bits(g_sess.out), _bits(e_sess.out)), rep
        assert torch.equal(g_sess.t_gen, e_sess.t_gen), rep
        assert torch.equal(_bits(g_sess.k_ring), _bits(e_sess.k_ring)), rep
        if sparse:
            assert torch.equal(g_sess.sel_idx, e_sess.sel_idx), rep
        # eager work of the program between replays
        _ = (e_sess.out.float() * 2).sum().item()


def test_prefill_route_and_ngram_ban_in_a_graph():
    """Prefill routing (two kernels per call) and the n-gram ban captured in a
    graph: every replay gives the eager results."""
    need_gpu()
    from long_context_decode_attn_amd import uocr as U
    w = S.Workload("graph-prefill", batch=2, heads=3, head_dim=128, dtype="bf16", pages=40, prompt=0, t0=0,
                   steps=1, seed=21, sparse=True, planted=4, fixed_query=True)
    say("graph prefill route + ngram ban")
    sess = DecodeSession(w)
    sess.build_index()
    q = to_device(S.prefill_queries(w, 40), w.dtype)
    pos = torch.tensor([w.prefix_len - 20, 3000], dtype=torch.int32, device="cuda")
    eager = [t.clone() for t in sess.prefill_route(q, pos)]
    hist = torch.from_numpy(S.token_history(4, 700, 500, 5, phrase=20, repeat_p=0.5, lookback=100)).cuda()
    n_gen = torch.tensor([700, 650, 30, 699], dtype=torch.int32, device="cuda")
    page = torch.tensor([0, 25, 3, 40], dtype=torch.int32, device="cuda")
    base = torch.randn((4, 500), device="cuda")
    ref = base.clone()
    U.uocr_ngram_ban(hist, n_gen, page, ref, 5, 128, page_token=7, eos_token=1, max_page_tokens=25)
    outs = [torch.empty_like(t) for t in eager]
    lg = base.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        U.uocr_prefill_route(sess.shape, sess.route, q, pos, sess.proj, sess.kbar, sess.prefix_len, *outs)
        U.uocr_ngram_ban(hist, n_gen, page, lg, 5, 128, page_token=7, eos_token=1, max_page_tokens=25)
    for rep in range(4):
        for t in outs:
            t.fill_(-7)
        lg.copy_(base)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), rep
        assert torch.equal(lg, ref), rep
        _ = (lg.float() * 2).sum().item()   # eager work between replays
