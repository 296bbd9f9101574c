"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each check is written as a function that takes the oracle routine it checks,
so that test_oracle_mutations.py can hand it a deliberately broken copy and
show that the check catches the mistake.  No GPU is used here.
"""
import heapq
import math
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import uocr_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name), encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if line:
            rows.append(line.split())
    return rows


def _sdpa(q, K, V, scale, bias=None):
    """torch's scaled_dot_product_attention in float64 on the CPU for one query."""
    qt = torch.tensor(np.asarray(q, np.float64))[None, None, None, :]
    Kt = torch.tensor(np.asarray(K, np.float64))[None, None]
    Vt = torch.tensor(np.asarray(V, np.float64))[None, None]
    mask = None if bias is None else torch.tensor(np.asarray(bias, np.float64))[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask, scale=scale)
    return o[0, 0, 0].numpy()


# ----------------------------------------------------------------------------
# cache law and ring
# ----------------------------------------------------------------------------
def check_cache_law(cache_len=O.cache_len, full_len=O.full_attention_cache_len):
    g = {r[0]: r[1:] for r in _golden("kv_cache_table.txt")}
    per_tok = int(g["bytes_per_token"][0])
    m = int(g["reference_tokens"][0])
    mib = 1 << 20
    assert m * per_tok == int(g["prefix_mib"][0]) * mib
    for key, val in g.items():
        if key.isdigit():
            T = int(key)
            assert full_len(m, T) * per_tok == int(val[0]) * mib, T
            # a window at least as long as the output is plain causal attention
            assert cache_len(m, T, T) == full_len(m, T)
            assert cache_len(m, 10 ** 9, T) == full_len(m, T)
    for T in [0, 1, 5, 127, 128, 129, 1000, 32768]:
        assert cache_len(m, 128, T) == m + min(128, T)
        assert cache_len(m, 128, T) <= m + 128
    assert cache_len(m, 128, 32768) * per_tok == (m + 128) * per_tok   # constant in T


def test_cache_law_matches_printed_table():
    check_cache_law()


def check_ring(ring_append=O.ring_append, ring_window=O.ring_window,
               window_positions=O.window_positions, ring_slot=O.ring_slot, cache_len=O.cache_len):
    rng = np.random.default_rng(7)
    for n, steps, t0 in [(4, 13, 0), (8, 30, 5), (128, 400, 0), (16, 40, 1000)]:
        B, H, D = 2, 3, 4
        ring_k = np.full((B, H, n, D), np.nan)
        ring_v = np.full((B, H, n, D), np.nan)
        t_gen = np.full((B,), t0, dtype=np.int64)
        hist_k = [np.full((B, H, D), np.nan)] * t0  # tokens before t0 never visible here
        hist_v = list(hist_k)
        # pre-fill the ring with the window at t0 as a ring holding it would
        for tau in range(max(0, t0 - n), t0):
            hk, hv = rng.standard_normal((B, H, D)), rng.standard_normal((B, H, D))
            hist_k[tau], hist_v[tau] = hk, hv
            ring_k[:, :, tau % n], ring_v[:, :, tau % n] = hk, hv
        for step in range(steps):
            k_new, v_new = rng.standard_normal((B, H, D)), rng.standard_normal((B, H, D))
            t_before = int(t_gen[0])
            ring_append(ring_k, ring_v, t_gen, k_new, v_new)
            hist_k.append(k_new)
            hist_v.append(v_new)
            t = t_before + 1
            assert int(t_gen[0]) == t == len(hist_k)
            # the slot just written is t_before mod n (bit-exact index)
            assert ring_slot(t_before, n) == t_before % n
            assert np.array_equal(ring_k[0, 0, t_before % n], k_new[0, 0])
            # window = the last min(n, t) tokens of the full history
            pos = window_positions(t, n)
            assert pos == list(range(max(0, t - n), t))
            assert len(pos) + 7 == cache_len(7, n, t)
            for b in range(B):
                for h in range(H):
                    w = ring_window(ring_k[b, h], t)
                    brute = np.stack([hist_k[tau][b, h] for tau in range(max(0, t - n), t)])
                    assert np.array_equal(w, brute)
                    dq = O.deque_window([hist_k[tau][b, h] for tau in range(max(0, t - n - 3), t)], n)
                    assert np.array_equal(w, np.stack(dq))
                    assert not np.isnan(w).any()   # never reads an unwritten slot


def test_ring_equals_history_window():
    check_ring()


def test_deque_semantics_drop_oldest():
    d = O.deque_window(list(range(10)), 4)
    assert d == [6, 7, 8, 9]
    assert O.deque_window([1, 2], 4) == [1, 2]


# ----------------------------------------------------------------------------
# dense attention
# ----------------------------------------------------------------------------
def check_attention(attention=O.attention, rswa_unit=O.rswa_unit):
    rng = np.random.default_rng(11)
    for L, D in [(1, 8), (5, 16), (300, 64), (700, 128)]:
        q, K, V = rng.standard_normal(D), rng.standard_normal((L, D)), rng.standard_normal((L, D))
        s = 1 / math.sqrt(D)
        np.testing.assert_allclose(attention(q, K, V, s), _sdpa(q, K, V, s), rtol=1e-12, atol=1e-13)
        bias = rng.uniform(-5, 0, size=L)
        np.testing.assert_allclose(attention(q, K, V, s, bias), _sdpa(q, K, V, s, bias),
                                   rtol=1e-12, atol=1e-13)
        # permutation of the key set leaves the output unchanged
        perm = rng.permutation(L)
        np.testing.assert_allclose(attention(q, K[perm], V[perm], s, bias[perm]),
                                   attention(q, K, V, s, bias), rtol=1e-12, atol=1e-13)
        # all keys equal -> mean of V
        Ke = np.repeat(K[:1], L, axis=0)
        np.testing.assert_allclose(attention(q, Ke, V, s), V.mean(axis=0), rtol=1e-12, atol=1e-13)
        # one key far ahead of the rest -> its value
        K2 = K.copy()
        j = L // 2
        K2[j] = q * 1e3
        np.testing.assert_allclose(attention(q, K2, V, s), V[j], atol=1e-12)
        # a -inf bias removes a key
        if L > 1:
            b2 = np.zeros(L)
            b2[0] = -np.inf
            np.testing.assert_allclose(attention(q, K, V, s, b2), attention(q, K[1:], V[1:], s),
                                       rtol=1e-12, atol=1e-13)
    # empty key set -> zeros (reading where the pages are silent)
    assert np.array_equal(attention(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 0.5), np.zeros(4))


def test_attention_definition():
    check_attention()


def check_rswa_reductions(rswa_decode=O.rswa_decode, ring_append=O.ring_append):
    """n >= T: R-SWA is full causal attention over prefix + every generated
    token; m = 0: it is plain sliding-window attention over the last n."""
    rng = np.random.default_rng(5)
    B, H, D, m_cap = 2, 2, 32, 70
    prefix_len = np.array([70, 33])
    Kp, Vp = rng.standard_normal((B, H, m_cap, D)), rng.standard_normal((B, H, m_cap, D))
    for n, m_zero in [(64, False), (64, True), (8, False), (8, True)]:
        pl = np.zeros(B, dtype=np.int64) if m_zero else prefix_len
        ring_k = np.full((B, H, n, D), np.nan)
        ring_v = np.full((B, H, n, D), np.nan)
        t_gen = np.zeros(B, dtype=np.int64)
        hk, hv = [], []
        for step in range(40):
            kn, vn = rng.standard_normal((B, H, D)), rng.standard_normal((B, H, D))
            ring_append(ring_k, ring_v, t_gen, kn, vn)
            hk.append(kn)
            hv.append(vn)
            q = rng.standard_normal((B, H, D))
            out = rswa_decode(q, Kp, Vp, pl, ring_k, ring_v, t_gen, 0.2)
            T = step + 1
            for b in range(B):
                for h in range(H):
                    lo = max(0, T - n)
                    K = np.concatenate([Kp[b, h, :pl[b]], np.stack([x[b, h] for x in hk[lo:T]])])
                    V = np.concatenate([Vp[b, h, :pl[b]], np.stack([x[b, h] for x in hv[lo:T]])])
                    np.testing.assert_allclose(out[b, h], _sdpa(q[b, h], K, V, 0.2),
                                               rtol=1e-11, atol=1e-12)


def test_rswa_reduces_to_full_and_sliding_attention():
    check_rswa_reductions()


# ----------------------------------------------------------------------------
# block index and scores
# ----------------------------------------------------------------------------
def check_block_index(block_index=O.block_index, block_scores=O.block_scores, block_ranges=O.block_ranges):
    rng = np.random.default_rng(3)
    D, d = 16, 8
    P = rng.standard_normal((D, d))
    for m in [1, 31, 32, 33, 64, 100]:
        K = rng.standard_normal((m + 5, D))
        kb = block_index(K, m, P, 32)
        assert kb.shape == (-(-m // 32), d)
        assert block_ranges(m, 32)[-1][1] == m
        # linearity: project-then-mean equals mean-then-project
        for j, (lo, hi) in enumerate([(lo, min(lo + 32, m)) for lo in range(0, m, 32)]):
            np.testing.assert_allclose(kb[j], P.T @ K[lo:hi].mean(axis=0), rtol=1e-12, atol=1e-13)
    # exact rationals on small integer inputs
    Pi = rng.integers(-3, 4, size=(D, d))
    for m in [5, 32, 45]:
        Ki = rng.integers(-4, 5, size=(m, D))
        qi = rng.integers(-4, 5, size=D)
        kb = block_index(Ki.astype(float), m, Pi.astype(float), 32)
        s = block_scores(qi.astype(float), Pi.astype(float), kb)
        for j, lo in enumerate(range(0, m, 32)):
            hi = min(lo + 32, m)
            qidx = [sum(int(Pi[t, i]) * int(qi[t]) for t in range(D)) for i in range(d)]
            kbar = [Fraction(sum(int(Pi[t, i]) * int(Ki[r, t]) for r in range(lo, hi) for t in range(D)), hi - lo)
                    for i in range(d)]
            exact = sum(Fraction(qidx[i]) * kbar[i] for i in range(d))
            assert abs(s[j] - float(exact)) <= 1e-9 * max(1.0, abs(float(exact)))


def test_block_index_and_scores():
    check_block_index()


# ----------------------------------------------------------------------------
# 1.5-entmax
# ----------------------------------------------------------------------------
def check_entmax(entmax=O.entmax15):
    # the pair case from the problem statement
    np.testing.assert_allclose(entmax(np.array([0.0, 0.0])), [0.5, 0.5], atol=1e-15)
    # uniform input -> uniform output
    for N in [1, 3, 17, 1000]:
        np.testing.assert_allclose(entmax(np.full(N, 2.5)), np.full(N, 1.0 / N), rtol=1e-12)
    # two-element closed form: a = (z1 - z2)/2; p1 = (a + sqrt(2 - a^2))^2 / 4 for a < 1
    for a in [0.0, 0.1, 0.37, 0.5, 0.9, 0.999, 1.0, 1.5, 7.0]:
        p = entmax(np.array([2 * a + 0.3, 0.3]))
        p1 = (a + math.sqrt(2 - a * a)) ** 2 / 4 if a < 1 else 1.0
        np.testing.assert_allclose(p, [p1, 1 - p1], atol=1e-12)
    rng = np.random.default_rng(13)
    for trial in range(200):
        N = int(rng.integers(1, 40))
        z = rng.standard_normal(N) * float(rng.choice([0.1, 1.0, 3.0, 20.0]))
        p = entmax(z)
        assert abs(p.sum() - 1.0) < 1e-12
        assert (p >= 0).all()
        # shift invariance
        np.testing.assert_allclose(entmax(z + 12.5), p, atol=1e-12)
        # monotone in z: larger score never gets less weight
        o = np.argsort(-z, kind="stable")
        assert (np.diff(p[o]) <= 1e-15).all()
        # KKT: p_j = (z_j/2 - tau)^2 on the support, tau >= z_j/2 off it, tau in [u_max - 1, u_max)
        u = z / 2
        sup = p > 0
        tau = u[sup][0] - math.sqrt(p[sup][0])
        np.testing.assert_allclose(np.sqrt(p[sup]), u[sup] - tau, atol=1e-10)
        assert (u[~sup] <= tau + 1e-12).all()
        assert u.max() - 1 - 1e-12 <= tau < u.max()
        # exactly one-hot iff the top gap is at least 2 (= 1/(alpha-1))
        if N >= 2:
            zs = np.sort(z)[::-1]
            gap = zs[0] - zs[1]
            if gap >= 2 + 1e-9:
                assert abs(p.max() - 1.0) < 1e-12 and np.count_nonzero(p) == 1
            elif gap < 2 - 1e-9:
                assert np.count_nonzero(p) >= 2


def test_entmax_closed_forms_and_invariants():
    check_entmax()


def test_entmax_three_routes_agree():
    rng = np.random.default_rng(17)
    for trial in range(150):
        N = int(rng.integers(1, 11))
        z = rng.standard_normal(N) * float(rng.choice([0.3, 1.0, 4.0]))
        p = O.entmax15(z)
        np.testing.assert_allclose(O.entmax15_bisect(z), p, atol=1e-12)
        np.testing.assert_allclose(O.entmax15_bruteforce(z), p, atol=1e-12)
    for trial in range(20):
        z = rng.standard_normal(1000) * 3
        np.testing.assert_allclose(O.entmax15_bisect(z), O.entmax15(z), atol=1e-12)


# ----------------------------------------------------------------------------
# top-k selection and routing
# ----------------------------------------------------------------------------
def check_topk(topk_blocks=O.topk_blocks):
    rng = np.random.default_rng(19)
    for trial in range(300):
        N = int(rng.integers(1, 60))
        k = int(rng.integers(1, 20))
        # few distinct values so that ties are frequent
        s = rng.integers(-3, 4, size=N).astype(float) if trial % 2 else rng.standard_normal(N)
        expect = sorted(j for _, j in heapq.nsmallest(min(k, N), [(-s[j], j) for j in range(N)]))
        assert topk_blocks(s, k) == expect


def test_topk_matches_heap_selection():
    check_topk()


def test_route_unit_bias_is_log_prob_without_renormalisation():
    rng = np.random.default_rng(23)
    for N, k in [(1, 16), (5, 16), (16, 16), (40, 16), (320, 16), (1000, 16), (50, 4)]:
        s = rng.standard_normal(N) * 0.2          # flat scores: wide support
        idx, prob, bias = O.route_unit(s, k)
        p = O.entmax15(s)
        kk = min(k, N)
        assert list(idx[:kk]) == O.topk_blocks(s, k) and (idx[kk:] == -1).all()
        assert list(idx[:kk]) == sorted(idx[:kk])
        np.testing.assert_allclose(prob[:kk], p[idx[:kk]], atol=0)
        live = prob[:kk] > 0
        np.testing.assert_allclose(bias[:kk][live], np.log(prob[:kk][live]), atol=0)
        assert np.isneginf(bias[:kk][~live]).all() and np.isneginf(bias[kk:]).all()
        # no renormalisation: the kept weights sum to at most 1, to 1 iff all of the support is kept
        assert prob.sum() <= 1 + 1e-12
        if np.count_nonzero(p) <= kk:
            assert abs(prob.sum() - 1) < 1e-12


def test_working_set_constants():
    g = {r[0]: int(r[1]) for r in _golden("routing_constants.txt")}
    assert g["block_size"] * g["topk_blocks"] == g["working_reference_tokens"]
    # sparse key set with every selected block live and full = 512 + min(n, T)
    rng = np.random.default_rng(2)
    D, m, n = 8, 40 * g["tokens_per_page"], g["window"]
    q, K, V = rng.standard_normal(D), rng.standard_normal((m, D)), rng.standard_normal((m, D))
    sel = np.arange(0, 2 * g["topk_blocks"], 2)
    bias = np.zeros(g["topk_blocks"])
    wk, wv = rng.standard_normal((n, D)), rng.standard_normal((n, D))
    keys = np.concatenate([K[j * 32:(j + 1) * 32] for j in sel] + [wk])
    assert keys.shape[0] == g["working_reference_tokens"] + n
    vals = np.concatenate([V[j * 32:(j + 1) * 32] for j in sel] + [wv])
    np.testing.assert_allclose(O.srswa_unit(q, K, V, m, sel, bias, wk, wv, 0.3),
                               _sdpa(q, keys, vals, 0.3), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# sparse decode
# ----------------------------------------------------------------------------
def check_srswa(srswa_unit=O.srswa_unit, rswa_unit=O.rswa_unit):
    rng = np.random.default_rng(29)
    D = 16
    for m in [32, 100, 320]:
        K, V = rng.standard_normal((m, D)), rng.standard_normal((m, D))
        wk, wv = rng.standard_normal((9, D)), rng.standard_normal((9, D))
        q = rng.standard_normal(D)
        nb = -(-m // 32)
        # every block selected with zero bias == dense R-SWA (identical key set)
        dense = rswa_unit(q, K, V, m, wk, wv, 0.25)
        np.testing.assert_allclose(srswa_unit(q, K, V, m, np.arange(nb), np.zeros(nb), wk, wv, 0.25),
                                   dense, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(srswa_unit(q, K, V, m, np.arange(nb), None, wk, wv, 0.25),
                                   dense, rtol=1e-13, atol=1e-14)
        # one block with p = 1, the others p = 0 -> dense attention over that block + window
        j = nb - 1
        sel = np.arange(min(nb, 16))
        sel[-1] = j
        sel = np.unique(sel)
        b = np.full(len(sel), -np.inf)
        b[list(sel).index(j)] = 0.0
        lo, hi = 32 * j, min(32 * j + 32, m)
        np.testing.assert_allclose(srswa_unit(q, K, V, m, sel, b, wk, wv, 0.25),
                                   _sdpa(q, np.concatenate([K[lo:hi], wk]), np.concatenate([V[lo:hi], wv]), 0.25),
                                   rtol=1e-12, atol=1e-13)
        # weighted softmax with finite biases on every selected block
        sel = np.sort(rng.choice(nb, size=min(nb, 16), replace=False))
        bb = np.log(rng.uniform(0.01, 1, size=len(sel)))
        keys = np.concatenate([K[32 * s:min(32 * s + 32, m)] for s in sel] + [wk])
        vals = np.concatenate([V[32 * s:min(32 * s + 32, m)] for s in sel] + [wv])
        tb = np.concatenate([np.full(min(32 * s + 32, m) - 32 * s, bv) for s, bv in zip(sel, bb)] + [np.zeros(9)])
        np.testing.assert_allclose(srswa_unit(q, K, V, m, sel, bb, wk, wv, 0.25),
                                   _sdpa(q, keys, vals, 0.25, tb), rtol=1e-12, atol=1e-13)
        # -1 entries are ignored
        sel2 = np.concatenate([sel, [-1, -1]])
        np.testing.assert_allclose(srswa_unit(q, K, V, m, sel2, np.concatenate([bb, [0, 0]]), wk, wv, 0.25),
                                   srswa_unit(q, K, V, m, sel, bb, wk, wv, 0.25), rtol=1e-14)


def test_srswa_reductions_and_weighted_softmax():
    check_srswa()


def test_route_end_to_end_planted_support():
    """Planted keys (+0.5 q*) dominate the routing: the top-k are planted
    blocks and the entmax support is a subset of them."""
    from long_context_decode_attn_amd import synth as S
    w = S.WORKLOADS["srswa-40p-b32"].replace(batch=2, heads=2, pages=12, planted=6)
    P = S.projection(w)
    Kp, _ = S.prefix_kv(w)
    q = S.widen(S.step_query(w, 0), w.dtype)
    res = O.route(q, S.widen(Kp, w.dtype), np.full(w.batch, w.prefix_len), P.astype(float), 4)
    for b in range(w.batch):
        planted = set(S.planted_blocks(w, b).tolist())
        for h in range(w.heads):
            idx = res["idx"][b, h]
            assert set(idx.tolist()) <= planted
            p = O.entmax15(res["s32"][b, h])
            assert set(np.nonzero(p)[0].tolist()) <= planted
            assert abs(p.sum() - 1) < 1e-12


def check_route(route=O.route):
    """The batched routing against explicit loops and enumeration, on
    small-integer inputs where every block key and score is exact: block
    keys as per-token sums of P^T k averaged over the block (partial last
    blocks included), scores as plain sums, the top-k by a full sort of
    (-score, index) and 1.5-entmax by enumerating support sets."""
    rng = np.random.default_rng(41)
    B, H, D, d, k = 2, 2, 6, 4, 3
    P = rng.integers(-2, 3, size=(D, d)).astype(float)
    m_cap = 7 * 32
    K = rng.integers(-3, 4, size=(B, H, m_cap, D)).astype(float)
    q = rng.integers(-2, 3, size=(B, H, D)).astype(float) / 8.0
    for plens in ([m_cap, 40], [0, 97]):
        res = route(q, K, np.array(plens), P, k)
        for b in range(B):
            m = plens[b]
            nb = -(-m // 32)
            for h in range(H):
                kbar = []
                for j in range(nb):
                    toks = range(32 * j, min(32 * j + 32, m))
                    kbar.append([sum(sum(P[t, i] * K[b, h, r, t] for t in range(D)) for r in toks) / len(toks)
                                 for i in range(d)])
                qi = [sum(P[t, i] * q[b, h, t] for t in range(D)) for i in range(d)]
                sc = np.array([sum(qi[i] * kbar[j][i] for i in range(d)) for j in range(nb)])
                assert np.array_equal(res["s32"][b, h], sc), (b, h)
                sel, p = _route_by_enumeration(sc, k)
                want = np.full(k, -1)
                want[:len(sel)] = sel
                assert np.array_equal(res["idx"][b, h], want), (b, h, res["idx"][b, h], want)
                for a, j in enumerate(sel):
                    assert abs(res["prob"][b, h, a] - p[j]) < 1e-12
                    lp = res["bias"][b, h, a]
                    assert (lp == -math.inf) if p[j] == 0 else abs(lp - math.log(p[j])) < 1e-12
                assert (res["prob"][b, h, len(sel):] == 0).all() and np.isneginf(res["bias"][b, h, len(sel):]).all()


def test_route_against_enumeration():
    check_route()


def test_ambiguity_rule_flags_only_near_ties():
    s = np.array([5.0, 3.0, 3.0 + 1e-9, 1.0])
    eps = np.full(4, 1e-7)
    assert O.ambiguous_boundary(s, eps, 2)        # rank 2 vs 3 within bounds
    assert not O.ambiguous_boundary(s, eps, 1)
    assert not O.ambiguous_boundary(s, eps, 3)
    assert not O.ambiguous_boundary(s, eps, 4)    # fewer than k+1 blocks


# ----------------------------------------------------------------------------
# prefill-side routing: causal visibility and per-query routing
# ----------------------------------------------------------------------------
def _visible_by_tokens(t, m, block=32):
    """Count the blocks none of whose prefix tokens is at a position >= t,
    token by token."""
    late = set()
    for p in range(m):
        if p >= t:
            late.add(p // block)
    n_blocks = (m + block - 1) // block
    return sum(1 for b in range(n_blocks) if b not in late)


def _route_by_enumeration(s, k):
    """Top-k by a full sort of (-score, index) and 1.5-entmax by enumerating
    every support set."""
    if len(s) == 0:
        return [], np.zeros(0)
    order = sorted(range(len(s)), key=lambda j: (-float(s[j]), j))
    return sorted(order[:min(k, len(s))]), O.entmax15_bruteforce(s)


def check_prefill_route(visible_blocks=O.visible_blocks, prefill_route_unit=O.prefill_route_unit):
    for m in [0, 1, 31, 32, 33, 100, 128, 130]:
        for t in range(-2, m + 70):
            assert visible_blocks(t, m) == _visible_by_tokens(t, m), (t, m)
    rng = np.random.default_rng(17)
    D, d, k = 8, 4, 3
    P = rng.normal(size=(D, d))
    for m, q_pos, Tq in [(300, 0, 40), (300, 250, 70), (40, 30, 12), (64, 64, 3)]:
        nb = (m + 31) // 32
        kbar = O.as_f32(rng.normal(size=(nb, d)))
        q = rng.normal(size=(Tq, D)) * 3.0
        idx, prob, bias = prefill_route_unit(q, q_pos, P, kbar, m, k)
        for i in range(Tq):
            t = q_pos + i
            nbv = _visible_by_tokens(t, m)
            s = np.array([float(np.float32(sum(float(q[i] @ P[:, c]) * kbar[j, c] for c in range(d))))
                          for j in range(nbv)])
            sel, p = _route_by_enumeration(s, k)
            want = np.full(k, -1)
            want[:len(sel)] = sel
            assert np.array_equal(idx[i], want), (m, q_pos, i)
            for a, j in enumerate(sel):
                assert abs(prob[i, a] - p[j]) < 1e-12
                assert (bias[i, a] == -math.inf) if p[j] == 0 else abs(bias[i, a] - math.log(p[j])) < 1e-12
                assert min(32 * (j + 1), m) <= t          # no token at or after the query
            assert (prob[i, len(sel):] == 0).all() and np.isneginf(bias[i, len(sel):]).all()
            if t >= m:   # after the prefix: the routing of a decode query
                d_idx, d_prob, _ = O.route_unit(O.as_f32(O.block_scores(q[i], P, kbar)), k)
                assert np.array_equal(idx[i], d_idx) and np.allclose(prob[i], d_prob, atol=1e-12)


def test_prefill_route_causal_and_enumerated():
    check_prefill_route()


# ----------------------------------------------------------------------------
# windowed no-repeat n-gram ban
# ----------------------------------------------------------------------------
def _ngram_by_dictionary(gen, n, window):
    """Every n-gram inside the window goes into a dictionary from its first
    n-1 tokens to the tokens that followed them; the ban is the entry of the
    last n-1 tokens."""
    w = list(gen)[-window:] if window > 0 else []
    table = {}
    for p in range(len(w) - n + 1):
        table.setdefault(tuple(w[p:p + n - 1]), set()).add(w[p + n - 1])
    if len(w) < n:
        return []
    return sorted(table.get(tuple(w[len(w) - n + 1:]), set()))


def check_ngram(ngram_banned=O.ngram_banned, ngram_process=O.ngram_process):
    # worked cases
    assert ngram_banned([5, 6, 7, 5, 6], 3, 128) == [7]          # "5 6 7 ... 5 6" bans 7
    assert ngram_banned([5, 6, 7, 5, 6, 9, 5, 6], 3, 128) == [7, 9]
    assert ngram_banned([5, 6, 7, 5, 6], 3, 4) == []              # 5 6 7 starts outside the window
    assert ngram_banned([5, 6, 7, 5, 6], 3, 5) == [7]             # ... and just inside it
    assert ngram_banned([1, 2], 3, 128) == []                     # shorter than n
    assert ngram_banned([4, 4, 4, 4], 1, 128) == [4]              # n = 1: every token in the window
    assert ngram_banned([3, 3, 3], 2, 128) == [3]
    # brute force against a dictionary of n-grams, random small vocabularies
    rng = np.random.default_rng(5)
    for trial in range(300):
        T = int(rng.integers(0, 60))
        gen = rng.integers(0, int(rng.integers(1, 5)), size=T).tolist()
        n, window = int(rng.integers(1, 7)), int(rng.integers(1, 70))
        assert ngram_banned(gen, n, window) == _ngram_by_dictionary(gen, n, window), (gen, n, window)
    # page guard: only the page marker and end-of-sequence stay open
    lg = np.arange(10, dtype=np.float64)
    out = ngram_process(lg, [1, 2, 1], 2, 128, page_tokens=20, max_page_tokens=20, page_token=7, eos_token=1)
    assert np.isneginf(out[[0, 2, 3, 4, 5, 6, 8, 9]]).all() and out[7] == 7 and out[1] == 1
    out = ngram_process(lg, [1, 2, 1], 2, 128, page_tokens=19, max_page_tokens=20, page_token=7, eos_token=1)
    assert np.isneginf(out[2]) and np.isfinite(np.delete(out, 2)).all()
    out = ngram_process(lg, [1, 2, 1], 2, 128, page_tokens=99, max_page_tokens=0, page_token=7, eos_token=1)
    assert np.isneginf(out[2]) and np.isfinite(np.delete(out, 2)).all()   # cap <= 0 disables the guard


def test_ngram_ban_worked_cases_and_brute_force():
    check_ngram()


# ----------------------------------------------------------------------------
# page2d rotary embedding: values worked out by hand from the rotation and the
# stated axis split, and the invariants of every rotary embedding
# ----------------------------------------------------------------------------
def check_rope(rope_page2d=O.rope_page2d):
    c, s = math.cos, math.sin
    z4 = np.zeros(4)
    # D = 4: pair 0 = dims (0, 2) on the token axis, pair 1 = dims (1, 3) on the
    # page axis, theta = 1 for both
    np.testing.assert_allclose(rope_page2d(np.array([1., 0, 0, 0]), 5, 2, 0), [c(2), 0, s(2), 0], atol=1e-15)
    np.testing.assert_allclose(rope_page2d(np.array([0., 0, 1, 0]), 5, 2, 0), [-s(2), 0, c(2), 0], atol=1e-15)
    np.testing.assert_allclose(rope_page2d(np.array([0., 1, 0, 0]), 3, 7, 0), [0, c(3), 0, s(3)], atol=1e-15)
    np.testing.assert_allclose(rope_page2d(np.array([0., 1, 0, 0]), 3, 7, 2), [0, c(1), 0, s(1)], atol=1e-15)
    np.testing.assert_allclose(rope_page2d(np.array([0., 0, 0, 1]), 3, 7, 2), [0, -s(1), 0, c(1)], atol=1e-15)
    assert np.array_equal(rope_page2d(z4, 9, 9, 0), z4)
    # D = 8: pairs 0, 1 on the token axis with theta 1 and 10000^(-1/2) = 0.01,
    # pairs 2, 3 on the page axis with the same two frequencies
    e = np.eye(8)
    np.testing.assert_allclose(rope_page2d(e[1], 0, 100, 0), c(1) * e[1] + s(1) * e[5], atol=1e-14)
    np.testing.assert_allclose(rope_page2d(e[0], 0, 100, 0), c(100) * e[0] + s(100) * e[4], atol=1e-13)
    np.testing.assert_allclose(rope_page2d(e[3], 100, 0, 0), c(1) * e[3] + s(1) * e[7], atol=1e-14)
    np.testing.assert_allclose(rope_page2d(e[2], 100, 0, 0), c(100) * e[2] + s(100) * e[6], atol=1e-13)
    np.testing.assert_allclose(rope_page2d(e[3], 100, 0, 3), c(0.01) * e[3] + s(0.01) * e[7], atol=1e-15)
    np.testing.assert_allclose(rope_page2d(e[1], 0, 100, 0, base=100.0), c(10) * e[1] + s(10) * e[5], atol=1e-13)
    rng = np.random.default_rng(11)
    for D in (8, 64, 128):
        x = rng.standard_normal((3, D))
        # position (0, 0) and a page that page_mod maps to 0 leave x as it is
        assert np.array_equal(rope_page2d(x, 0, 0, 2), x)
        assert np.array_equal(rope_page2d(x, 4, 37, 2), rope_page2d(x, 0, 37, 2))
        assert np.array_equal(rope_page2d(x, 5, 37, 2), rope_page2d(x, 1, 37, 2))
        # every pair keeps its length, so does the vector
        y = rope_page2d(x, 7, 1234, 0)
        h = D // 2
        np.testing.assert_allclose(y[:, :h] ** 2 + y[:, h:] ** 2, x[:, :h] ** 2 + x[:, h:] ** 2, rtol=1e-12)
        # the rows (heads) are turned independently, by the same rotation
        for r in range(3):
            np.testing.assert_allclose(rope_page2d(x[r], 7, 1234, 0), y[r], rtol=0, atol=0)
        # a dot product depends only on the differences of the positions
        q, k = rng.standard_normal(D), rng.standard_normal(D)
        for (p1, o1, p2, o2) in [(3, 40, 1, 7), (0, 5, 9, 5), (12, 0, 12, 300)]:
            lhs = rope_page2d(q, p1, o1, 0) @ rope_page2d(k, p2, o2, 0)
            rhs = rope_page2d(q, p1 - p2, o1 - o2, 0) @ k
            assert abs(lhs - rhs) <= 1e-11 * (1 + abs(lhs)), (D, p1, o1, p2, o2)
        # rotations compose by adding positions, and position (-p, -o) undoes (p, o)
        np.testing.assert_allclose(rope_page2d(rope_page2d(x, 2, 30, 0), 5, 11, 0), rope_page2d(x, 7, 41, 0),
                                   atol=1e-12)
        np.testing.assert_allclose(rope_page2d(rope_page2d(x, 6, 900, 0), -6, -900, 0), x, atol=1e-12)
        # the token axis alone moves the first half of the pairs, the page axis the second
        a = rope_page2d(x, 0, 55, 0) - x
        b = rope_page2d(x, 55, 0, 0) - x
        q4 = D // 4
        tok = np.r_[0:q4, h:h + q4]
        pag = np.r_[q4:h, h + q4:D]
        assert np.array_equal(a[:, pag], np.zeros_like(a[:, pag])) and np.abs(a[:, tok]).max() > 1e-3
        assert np.array_equal(b[:, tok], np.zeros_like(b[:, tok])) and np.abs(b[:, pag]).max() > 1e-3


def test_rope_page2d_worked_cases_and_invariants():
    check_rope()
