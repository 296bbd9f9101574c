"""The dense decode with the library's static workspace
(uocr_rswa_decode_static), called through the C ABI: its output equals that of
uocr_rswa_decode (caller's workspace, same split count, the same kernels) and
lies within the bf16 tolerances of the oracle, on two calls in a row, the
second with a smaller input, so that the second call runs on the partials
the first one left in the shared array.  (The refusal of a split count whose
partials exceed the array is checked on the CPU, in test_abi.py.)"""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import synth as S
from long_context_decode_attn_amd import uocr as U
from long_context_decode_attn_amd.session import DecodeSession, to_device, to_host
from oracle import uocr_oracle as O
from tests._gpu_common import HostMirror, assert_close, need_gpu, say

pytestmark = pytest.mark.gpu


def _check(w, num_splits):
    sess = DecodeSession(w, num_splits=num_splits)
    host = HostMirror(w)
    q, _, _ = S.step_inputs(w, 3)
    qt = to_device(q, w.dtype)
    ref = torch.empty_like(sess.out)
    U.uocr_rswa_decode(sess.shape, qt, sess.k_prefix, sess.v_prefix, sess.prefix_len, sess.k_ring, sess.v_ring,
                       sess.t_gen, ref, sess.workspace, num_splits)
    got = torch.full_like(sess.out, float("nan"))
    U.uocr_rswa_decode_static(sess.shape, qt, sess.k_prefix, sess.v_prefix, sess.prefix_len, sess.k_ring,
                              sess.v_ring, sess.t_gen, got, num_splits)
    torch.cuda.synchronize()
    splits = U.uocr_rswa_splits(sess.shape, num_splits)
    say(f"static workspace: {w.name} units {w.units} splits {splits}")
    assert splits > 1, "the case must use the workspace"
    assert torch.equal(got, ref), "static workspace differs from the caller's workspace"
    qd = S.widen(q, w.dtype)
    units = [(0, 0), (w.batch - 1, w.heads - 1), (w.batch // 2, 1)]
    want = np.stack([O.rswa_unit(qd[b, h], host.Kp[b, h], host.Vp[b, h], w.prefix_len, *host.window(b, h), w.scale)
                     for b, h in units])
    g = to_host(got)
    assert_close(np.stack([g[b, h] for b, h in units]), want, w.dtype, f"{w.name} static")


def test_static_workspace_two_calls_second_smaller():
    need_gpu()
    big = S.Workload("static-big", batch=16, heads=10, head_dim=128, dtype="bf16", pages=12, prompt=7, t0=300,
                     steps=1, seed=515)
    small = S.Workload("static-small", batch=2, heads=3, head_dim=128, dtype="bf16", pages=3, prompt=1, t0=50,
                       steps=1, seed=516)
    _check(big, 0)
    _check(small, 5)
