"""GPU parity of the page2d two-axis rotary embedding (uocr_rope_page2d)
against the oracle, through the C ABI.  fp32 results must agree to 1e-5
(the kernel takes cos and sin in fp32 of an fp64-reduced angle); bf16 results
must be the oracle's value rounded to bf16, or its neighbour when the exact
value lies within fp32 rounding of a tie."""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import synth as S
from long_context_decode_attn_amd import uocr as U
from long_context_decode_attn_amd.session import to_device, to_host
from oracle import uocr_oracle as O
from tests._gpu_common import assert_close, need_gpu, say

pytestmark = pytest.mark.gpu


def _oracle(x64, page, offset, page_mod, base, tokens_sample=None):
    """Oracle rotation of x64 [B][H][T][D] (float64) token by token."""
    B, H, T, D = x64.shape
    out = np.empty_like(x64)
    sample = [(b, t) for b in range(B) for t in range(T)] if tokens_sample is None else tokens_sample
    for b, t in sample:
        out[b, :, t] = O.rope_page2d(x64[b, :, t], int(page[b, t]), int(offset[b, t]), page_mod, base)
    return out


def _check(got, want, dtype, what):
    if dtype == "f32":
        err = np.abs(got - want).max() if got.size else 0.0
        assert err <= 1e-5, f"{what}: max-abs {err:.3e}"
    else:
        # within half a bf16 ulp of the exact value, plus what fp32 rounding
        # before the bf16 rounding can move it
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 2.0 ** -126))) - 7)
        bad = np.abs(got - want) > 0.5 * ulp + 1e-6 * (1 + np.abs(want))
        assert not bad.any(), f"{what}: {int(bad.sum())} elements off by more than half a bf16 ulp"
    assert_close(got, want, dtype, what)


def _run(B, H, T, D, dtype, page_mod=2, base=10000.0, page_tokens=256, first_page=0, start_offset=0,
         seed=1, sample=None, page=None, offset=None):
    say("rope", B, H, T, D, dtype, page_mod, base, first_page, start_offset)
    x = S.rope_rows(seed, B, H, T, D, dtype)
    if page is None:
        page, offset = S.page_positions(seed, B, T, page_tokens, first_page, start_offset)
    shape = U.Shape(B, H, D, 0, dtype=U.UOCR_F32 if dtype == "f32" else U.UOCR_BF16)
    tx = to_device(x, dtype)
    U.uocr_rope_page2d(shape, tx, torch.from_numpy(page).cuda(), torch.from_numpy(offset).cuda(), page_mod, base)
    torch.cuda.synchronize()
    got = to_host(tx)
    x64 = S.widen(x, dtype)
    clamp = lambda a: np.maximum(a, 0)
    want = _oracle(x64, clamp(page), clamp(offset), page_mod, base, sample)
    if sample is not None:
        idx = tuple(np.array(sample).T)
        got, want = got[idx[0], :, idx[1]], want[idx[0], :, idx[1]]
    return got, want


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_rope_matches_oracle(dtype, D):
    need_gpu()
    got, want = _run(3, 4, 37, D, dtype)            # 16-token tiles with a ragged last tile
    _check(got, want, dtype, f"rope {dtype} D={D}")


@pytest.mark.parametrize("page_mod", [0, 2, 3])
def test_rope_page_mod(page_mod):
    need_gpu()
    got, want = _run(2, 3, 50, 128, "f32", page_mod=page_mod, page_tokens=8, first_page=5)
    _check(got, want, "f32", f"page_mod={page_mod}")


def test_rope_large_positions_keep_the_angle():
    """Offsets near 2^20 and page numbers near 10^6 (page_mod 0): angles of
    up to ~10^6 rad still come out exact to fp32."""
    need_gpu()
    got, want = _run(2, 2, 40, 128, "f32", page_mod=0, page_tokens=1 << 21, first_page=999_000,
                     start_offset=(1 << 20) - 60)
    _check(got, want, "f32", "large positions")


def test_rope_other_base_and_decode_shape():
    need_gpu()
    got, want = _run(32, 10, 1, 128, "bf16", base=500000.0, first_page=3, start_offset=17)   # one decode step
    _check(got, want, "bf16", "decode step, base 5e5")


@pytest.mark.parametrize("T", [1, 37])
def test_rope_queries_and_keys_in_one_launch(T):
    """x = queries, y = keys: both turned by the same positions, each exactly
    as a call of its own would turn it."""
    need_gpu()
    B, H, D = 4, 3, 128
    say("rope q+k", B, H, T, D)
    q = S.rope_rows(21, B, H, T, D, "bf16")
    k = S.rope_rows(22, B, H, T, D, "bf16")
    page, offset = S.page_positions(4, B, T, 64, first_page=1, start_offset=30)
    shape = U.Shape(B, H, D, 0, dtype=U.UOCR_BF16)
    tq, tk = to_device(q, "bf16"), to_device(k, "bf16")
    tp, to = torch.from_numpy(page).cuda(), torch.from_numpy(offset).cuda()
    U.uocr_rope_page2d(shape, tq, tp, to, y=tk)
    tk2 = to_device(k, "bf16")
    U.uocr_rope_page2d(shape, tk2, tp, to)
    torch.cuda.synchronize()
    assert torch.equal(tk, tk2)
    for name, src, t in [("q", q, tq), ("k", k, tk)]:
        want = _oracle(S.widen(src, "bf16"), page, offset, 2, 10000.0)
        _check(to_host(t), want, "bf16", f"{name} T={T}")


def test_rope_negative_positions_count_as_zero_and_empty_is_a_no_op():
    need_gpu()
    B, H, T, D = 2, 2, 20, 64
    page = np.full((B, T), -3, np.int32)
    offset = np.tile(np.arange(-10, 10, dtype=np.int32), (B, 1))
    got, want = _run(B, H, T, D, "f32", page=page, offset=offset)
    _check(got, want, "f32", "negative positions")
    shape = U.Shape(B, H, D, 0, dtype=U.UOCR_F32)
    x = torch.ones((B, H, 0, D), device="cuda")
    z = torch.zeros((B, 0), dtype=torch.int32, device="cuda")
    U.uocr_rope_page2d(shape, x, z, z)
    torch.cuda.synchronize()


def test_rope_prefill_chunk_shape_sampled():
    """The bench's launch: 32 sequences x 10 heads x 2048 tokens, D = 128,
    bf16; 300 sampled tokens, every head, against the oracle."""
    need_gpu()
    B, T = 32, 2048
    rng = np.random.default_rng(9)
    sample = sorted({(int(b), int(t)) for b, t in zip(rng.integers(0, B, 300), rng.integers(0, T, 300))})
    sample += [(0, 0), (B - 1, T - 1)]
    got, want = _run(B, 10, T, 128, "bf16", page_tokens=400, first_page=2, start_offset=100, sample=sample)
    _check(got, want, "bf16", "prefill chunk")


# ----------------------------------------------------------------------------
# page2d RoPE fused into the decode steps
# ----------------------------------------------------------------------------
def _stored(t, dtype):
    """Device tensor -> storage bits (bf16 as uint16, f32 as uint32)."""
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("sparse,dtype,D,num_splits", [(True, "bf16", 128, 0), (True, "f32", 64, 0),
                                                        (True, "bf16", 64, 4), (False, "bf16", 128, 0),
                                                        (False, "bf16", 128, 3), (False, "f32", 128, 8)])
def test_fused_step_with_rope(sparse, dtype, D, num_splits):
    """uocr_srswa_step / uocr_rswa_step with page2d RoPE equal, bit for bit,
    uocr_rope_page2d on (q, k_new) followed by the step without it (output,
    selection, rings, counts), over several steps with per-sequence counts
    before and across a wrap; and the output agrees with the oracle run on
    the oracle's own rotation (queries and the ring's keys turned in fp64)."""
    from long_context_decode_attn_amd.session import DecodeSession
    from tests._gpu_common import HostMirror
    need_gpu()
    w = S.Workload("rope-step", batch=3, heads=2, head_dim=D, dtype=dtype, pages=5, prompt=7, t0=0, steps=4,
                   seed=77, sparse=sparse, planted=6 if sparse else 0, fixed_query=sparse, topk=4)
    say("fused rope", sparse, dtype, D, num_splits)
    t0 = [0, 50, 126]
    ring = S.initial_ring(w, t0)
    kv = S.prefix_kv(w)
    fused = DecodeSession(w, prefix_kv=kv, ring=ring, fused=True, num_splits=num_splits)
    plain = DecodeSession(w, prefix_kv=kv, ring=ring, fused=True, num_splits=num_splits)
    host = HostMirror(w, prefix_kv=kv, ring=ring)
    if sparse:
        fused.build_index()
        plain.build_index()
    page, offset = S.page_positions(9, w.batch, w.steps, page_tokens=300, first_page=2, start_offset=40)
    page_mod, base = 2, 10000.0
    P = S.projection(w).astype(np.float64) if sparse else None
    for step in range(w.steps):
        q, k, v = S.step_inputs(w, step)
        tq, tk, tv = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
        pg = torch.from_numpy(np.ascontiguousarray(page[:, step])).cuda()
        of = torch.from_numpy(np.ascontiguousarray(offset[:, step])).cuda()
        fused.fused_step(tq, tk, tv, rope=(pg, of, page_mod, base))
        # the separate path: rotate copies of q and k_new, then the plain step
        q2, k2 = tq.clone(), tk.clone()
        U.uocr_rope_page2d(plain.shape, q2.view(w.batch, w.heads, 1, D), pg.view(w.batch, 1), of.view(w.batch, 1),
                           page_mod, base, y=k2.view(w.batch, w.heads, 1, D))
        plain.fused_step(q2, k2, tv)
        torch.cuda.synchronize()
        assert torch.equal(tq, to_device(q, dtype)) and torch.equal(tk, to_device(k, dtype)), "inputs modified"
        assert torch.equal(fused.out, plain.out), f"step {step}: output differs from rope + step"
        assert torch.equal(fused.t_gen, plain.t_gen)
        assert np.array_equal(_stored(fused.k_ring, dtype), _stored(plain.k_ring, dtype)), f"step {step}: k ring"
        assert np.array_equal(_stored(fused.v_ring, dtype), _stored(plain.v_ring, dtype)), f"step {step}: v ring"
        if sparse:
            assert torch.equal(fused.sel_idx, plain.sel_idx) and torch.equal(fused.sel_bias, plain.sel_bias)
            assert torch.equal(fused.sel_prob, plain.sel_prob)
        # oracle: q and k_new turned in fp64; the ring keeps the turned keys
        qd, kd = S.widen(q, dtype), S.widen(k, dtype)
        for b in range(w.batch):
            qd[b] = O.rope_page2d(qd[b], int(page[b, step]), int(offset[b, step]), page_mod, base)
            kd[b] = O.rope_page2d(kd[b], int(page[b, step]), int(offset[b, step]), page_mod, base)
        O.ring_append(host.Kr, host.Vr, host.t_gen, kd, S.widen(v, dtype))
        ref = np.zeros((w.batch, w.heads, D))
        for b in range(w.batch):
            for h in range(w.heads):
                wk, wv = host.window(b, h)
                if sparse:
                    kb = O.block_index(host.Kp[b, h], w.prefix_len, P)
                    idx, _, bias = O.route_unit(O.as_f32(O.block_scores(qd[b, h], P, kb)), w.topk)
                    assert np.array_equal(fused.sel_idx[b, h].cpu().numpy(), idx), (step, b, h)
                    ref[b, h] = O.srswa_unit(qd[b, h], host.Kp[b, h], host.Vp[b, h], w.prefix_len, idx, bias, wk, wv,
                                             w.scale)
                else:
                    ref[b, h] = O.rswa_unit(qd[b, h], host.Kp[b, h], host.Vp[b, h], w.prefix_len, wk, wv, w.scale)
        assert_close(to_host(fused.out), ref, dtype, f"fused rope step {step}")
