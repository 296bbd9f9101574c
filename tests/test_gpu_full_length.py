"""Full-length parity of the timed configuration: the benchmark's own setup
(per-layer states cloned from one seeded state, HIP graphs of two steps per
layer replayed, double-buffered generated-token counts, fused step kernels)
runs every workload for its whole step count on every layer, and is checked
against the oracle:

* every 64 steps of a layer (and at its first and last step), a sample of
  (sequence, head) units: the selection bit for bit (or, where the scores
  fall within their certified bounds of each other, a selection those bounds
  allow; the count of such cases is reported and must be 0 where the oracle
  flags no near-tie), the sparse weights, and the attention output within the
  bf16 tolerances;
* at the end, every layer's generated-token counts and both rings of every
  unit, bit for bit.

Step i of the run goes to layer i mod L with the inputs synth.step_inputs(w,
i); layer l's local token tau (counted from t0) therefore holds generated
token t0 + (tau - t0) * L + l, so the oracle rebuilds any layer's window
directly from the seeded inputs.  The 125-page workload's 2048 steps wrap the
ring 16 times on every layer.
"""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import synth as S
from long_context_decode_attn_amd.runner import LayeredDecoder
from long_context_decode_attn_amd.session import to_host
from oracle import uocr_oracle as O
from tests._gpu_common import assert_close, need_gpu, say
from tests.test_gpu_sparse import _check_selection

pytestmark = pytest.mark.gpu

LAYERS = 12
CHECK_EVERY = 64
UNITS_PER_CHECK = 6


def _token(w, L, layer, tau):
    """(k, v) storage arrays [B][H][D] of layer `layer`'s local token tau."""
    g = tau if tau < w.t0 else w.t0 + (tau - w.t0) * L + layer
    return S.history_token(w, g)


def _windows(w, L, layer, T):
    """The layer's visible window after T local tokens, every unit, in token
    order: float64 K, V [B][H][w][D]."""
    taus = O.window_positions(T, w.window)
    ks, vs = [], []
    for tau in taus:
        k, v = _token(w, L, layer, tau)
        ks.append(S.widen(k, w.dtype))
        vs.append(S.widen(v, w.dtype))
    return np.stack(ks, axis=2), np.stack(vs, axis=2)


def _run(name, steps=None, layers=LAYERS):
    need_gpu()
    w = S.WORKLOADS[name]
    steps = w.steps if steps is None else steps
    assert steps % 2 == 0
    L = layers
    say(f"full-length {name}: {L} layers x {steps} steps, graphs of {2 * L} steps")
    dec = LayeredDecoder(w, L, fused=True)
    dec.build_index()
    graph = dec.capture()
    G = dec.G
    rng = np.random.default_rng(5)
    P = S.projection(w).astype(np.float64) if w.sparse else None
    prefix = {}        # b -> (K, V) float64 [H][m][D]
    kbars = {}         # (b, h) -> kbar
    flags = swaps = checked = 0

    def prefix_of(b):
        if b not in prefix:
            Kp, Vp = S.prefix_kv_seq(w, b)
            prefix[b] = (S.widen(Kp, w.dtype), S.widen(Vp, w.dtype))
            if len(prefix) > 4:
                prefix.pop(next(iter(prefix)))
        return prefix[b]

    for r in range(steps // 2):
        dec.fill_inputs([S.step_inputs(w, r * G + g) for g in range(G)])
        graph.replay()
        local = (2 * r, 2 * r + 1)
        due = [s for s in local if s % CHECK_EVERY == CHECK_EVERY - 1 or s == 0 or s == steps - 1]
        if not due:
            continue
        torch.cuda.synchronize()
        for s in due:
            layer = (s // CHECK_EVERY) % L
            g = layer + (s % 2) * L            # graph slot of that layer's step
            i = r * G + g                      # global step
            q = S.widen(S.step_query(w, i), w.dtype)
            T = w.t0 + s + 1
            units = sorted({(int(rng.integers(w.batch)), int(rng.integers(w.heads))) for _ in range(UNITS_PER_CHECK)})
            got = to_host(dec.out[g])
            if w.sparse:
                gi = dec.sel_idx[g].cpu().numpy()
                gp = dec.sel_prob[g].cpu().numpy().astype(np.float64)
                gb = dec.sel_bias[g].cpu().numpy().astype(np.float64)
            ref, out = [], []
            WK, WV = _windows(w, L, layer, T)
            for b, h in units:
                Kp, Vp = prefix_of(b)
                wk, wv = WK[b, h], WV[b, h]
                if w.sparse:
                    if (b, h) not in kbars:
                        kbars[(b, h)] = O.block_index(Kp[h], w.prefix_len, P)
                    kb = kbars[(b, h)]
                    s64 = O.block_scores(q[b, h], P, kb)
                    eps = O.score_error_bound(q[b, h], P, kb)
                    amb = O.ambiguous_boundary(s64, eps, w.topk)
                    exact = _check_selection(gi[b, h], gp[b, h], gb[b, h], O.as_f32(s64), w.topk, s64, eps,
                                             f"{name} layer {layer} step {s} unit {(b, h)}")
                    flags += amb
                    swaps += not exact
                    assert exact or amb
                    ridx, _, rbias = O.route_unit(O.as_f32(s64), w.topk)
                    ref.append(O.srswa_unit(q[b, h], Kp[h], Vp[h], w.prefix_len, ridx, rbias, wk, wv, w.scale))
                else:
                    ref.append(O.rswa_unit(q[b, h], Kp[h], Vp[h], w.prefix_len, wk, wv, w.scale))
                out.append(got[b, h])
                checked += 1
            assert_close(np.stack(out), np.stack(ref), w.dtype, f"{name} layer {layer} local step {s}")
        if r % 128 == 0:
            say(f"  replay {r} of {steps // 2}: {checked} unit-steps checked")
    torch.cuda.synchronize()

    # every layer's counts and rings, bit for bit
    n = w.window
    T = w.t0 + steps
    for layer in range(L):
        st = dec.layers[layer]
        assert (st.t_gen.cpu().numpy() == T).all(), f"layer {layer} t_gen"
        kr = st.k_ring.view(torch.int16).cpu().numpy().view(np.uint16) if w.dtype == "bf16" else st.k_ring.cpu().numpy()
        vr = st.v_ring.view(torch.int16).cpu().numpy().view(np.uint16) if w.dtype == "bf16" else st.v_ring.cpu().numpy()
        want_k, want_v = np.empty_like(kr), np.empty_like(vr)
        for tau in range(T - n, T):
            k, v = _token(w, L, layer, tau)
            want_k[:, :, tau % n] = k
            want_v[:, :, tau % n] = v
        assert np.array_equal(kr, want_k) and np.array_equal(vr, want_v), f"layer {layer} ring"
    say(f"{name}: {checked} unit-steps checked, {flags} flagged near-ties, {swaps} selections within the bounds "
        f"but not the oracle's; t_gen = {T} and both rings bit-exact on all {L} layers "
        f"({(T - w.t0) // n} wraps)")
    return flags, swaps


@pytest.mark.parametrize("name", ["srswa-125p-b8", "srswa-125p-b8-qnoise", "srswa-125p-b8-wide",
                                  "srswa-40p-b32", "srswa-40p-b32-qnoise", "srswa-40p-b32-wide",
                                  "dense-10p-b64"])
def test_full_length_timed_configuration(name):
    flags, swaps = _run(name)
    assert swaps <= flags


def test_full_length_high_concurrency_dense():
    """512 sequences x 10 heads (one page + prompt) for 1000 steps on 4
    layers (the same graphs, fewer layers, so that drawing the per-step
    inputs of 512 sequences stays within a minute)."""
    _run("dense-1p-b512", layers=4)
