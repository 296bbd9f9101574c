"""Decode steps captured in a HIP graph: every replay matches the same steps
run eagerly, with eager work and synchronisations between the replays."""
import numpy as np
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
