"""Plain float64 CPU oracle for R-SWA / SR-SWA single-step decode attention.

TEST INFRASTRUCTURE ONLY.  This module is the checker, not the product: only
tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may import
or call it.  It shares no code with the HIP path (long_context_decode_attn_amd/)
and imports nothing from it; both sides only read the same seeded inputs.

Every function writes the definition out directly, in float64, with numpy
primitives (matrix-vector products, sorts) as steps and no blocking, splitting
or fusion.  Sources (web pages, cited by title and section):

* [R-SWA summary]  "百度Unlimited OCR" paper summary (lshu.cn/news/33052),
  section 二 "核心创新 R-SWA": 1. core design (permanent reference prefix of m
  tokens, always visible, never evicted; causal window of the last n = 128
  generated tokens), 2. KV-cache law C(T) = L_m + min(n, T).
* [R-SWA blog]  "百度 Unlimited OCR 深度实战" (chenxutan.com/d/4055.html),
  section 2.2.1 (the window holds y_{t-n} .. y_{t-1} when producing y_t),
  section 3.3.1 (mask: every reference token visible, only the last n outputs
  visible), section 3.3.2 (deque(maxlen=n) ring), section 5.1 (KV table).
* [SR-SWA explainer]  Unlimited-OCR-2 article (nxmr.cn/news/162408), sections
  "稀疏路由" (32-token blocks, low-dimensional index projection scores,
  1.5-entmax top-k selection, log-bias fusion, 16 blocks = 512 tokens) and
  "环形缓冲" (ring buffer: the new token overwrites the oldest slot in place,
  the write pointer advances circularly).
* 1.5-entmax: Peters, Niculae & Martins (2019), "Sparse Sequence-to-Sequence
  Models", the exact sort-based algorithm; bisection on the threshold follows
  Blondel, Martins & Niculae (2020).  The pages name the distribution only.

Readings where the pages are silent (each listed in the design notes):
append-then-attend; ring slot of token tau is tau mod n; only the prefix is
blocked; a partial last block averages its valid tokens; score = (P^T q) .
mean_t(P^T k_t) with no scale; entmax over all blocks, then the top-k by (score
desc, index asc), emitted in ascending index order, with bias ln p (-inf where
p = 0) and no renormalisation; the routing decision is taken on scores rounded
to float32, the precision the scores are stored in; an empty key set gives a
zero output.
"""
from __future__ import annotations

import itertools
import math
from collections import deque
from typing import List, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64
NEG_INF = -math.inf


# ============================================================================
# Ring buffer and cache law   ([R-SWA summary] section 2; [SR-SWA explainer]
# "环形缓冲"; [R-SWA blog] section 3.3.2)
# ============================================================================
def cache_len(m: int, n: int, t: int) -> int:
    """Cached tokens visible after t generated tokens: the m-token prefix plus
    the min(n, t) most recent generated tokens ([R-SWA summary] section 2)."""
    return m + min(n, t)


def full_attention_cache_len(m: int, t: int) -> int:
    """Plain causal attention keeps every generated token: m + t."""
    return m + t


def window_positions(t: int, n: int) -> List[int]:
    """Generated-token positions visible after t appends: t-n .. t-1 (clipped at 0)."""
    return list(range(max(0, t - n), t))


def ring_slot(tau: int, n: int) -> int:
    """Slot of generated token tau: the write pointer starts at 0 and advances
    by one per token, wrapping at n, so token tau lands in tau mod n."""
    return tau % n


def ring_append(ring_k: np.ndarray, ring_v: np.ndarray, t_gen: np.ndarray,
                k_new: np.ndarray, v_new: np.ndarray) -> None:
    """One decode step's append for every sequence, in place.

    ring_k, ring_v: [B][H][n][D]; t_gen: [B] tokens generated so far;
    k_new, v_new: [B][H][D].  The new token overwrites slot t_gen mod n (the
    oldest entry once the ring is full), then t_gen advances by one.
    """
    n = ring_k.shape[2]
    for b in range(ring_k.shape[0]):
        slot = ring_slot(int(t_gen[b]), n)
        ring_k[b, :, slot, :] = k_new[b]
        ring_v[b, :, slot, :] = v_new[b]
        t_gen[b] += 1


def ring_window(ring: np.ndarray, t: int) -> np.ndarray:
    """Read the visible window of one unit's ring [n][D] after t appends, in
    generation order: token tau of the window sits in slot tau mod n."""
    n = ring.shape[0]
    return np.stack([ring[ring_slot(tau, n)] for tau in window_positions(t, n)]) \
        if t > 0 else ring[:0]


def deque_window(history: Sequence[np.ndarray], n: int) -> List[np.ndarray]:
    """The same window kept the way [R-SWA blog] 3.3.2 keeps it: a deque with
    maxlen n that drops its oldest entry on overflow."""
    d: deque = deque(maxlen=n)
    for x in history:
        d.append(x)
    return list(d)


# ============================================================================
# Dense attention over a key set   ([R-SWA blog] 2.2.1, 3.3.1)
# ============================================================================
def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
              bias: Optional[np.ndarray] = None) -> np.ndarray:
    """o = sum_j softmax_j(scale * q.k_j + bias_j) v_j, in float64.

    q [D], K [L][D], V [L][D], bias [L] or None.  Keys with bias -inf carry
    zero weight.  An empty key set (or one whose logits are all -inf) returns
    zeros: the reading taken where the pages do not define it.
    """
    q = np.asarray(q, dtype=F64)
    K = np.asarray(K, dtype=F64)
    V = np.asarray(V, dtype=F64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1] if V.ndim == 2 else q.shape[0], dtype=F64)
    logits = scale * (K @ q)
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=F64)
    if not np.any(np.isfinite(logits)):
        return np.zeros(V.shape[1], dtype=F64)
    keep = np.isfinite(logits)
    lg = logits[keep]
    e = np.exp(lg - lg.max())
    return (e @ V[keep]) / e.sum()


def rswa_unit(q: np.ndarray, k_prefix: np.ndarray, v_prefix: np.ndarray, m: int,
              k_window: np.ndarray, v_window: np.ndarray, scale: float) -> np.ndarray:
    """Dense R-SWA decode of one (sequence, head): the key set is the whole
    reference prefix [0, m) plus the visible window ([R-SWA summary] 2.1,
    [R-SWA blog] 3.3.1)."""
    K = np.concatenate([np.asarray(k_prefix[:m], dtype=F64), np.asarray(k_window, dtype=F64)])
    V = np.concatenate([np.asarray(v_prefix[:m], dtype=F64), np.asarray(v_window, dtype=F64)])
    return attention(q, K, V, scale)


def rswa_decode(q, k_prefix, v_prefix, prefix_len, ring_k, ring_v, t_gen, scale) -> np.ndarray:
    """Batched dense R-SWA decode reading the ring: q [B][H][D] (float64),
    prefix K/V [B][H][m_cap][D], prefix_len [B], ring K/V [B][H][n][D],
    t_gen [B].  Returns out [B][H][D] float64."""
    B, H = q.shape[0], q.shape[1]
    out = np.zeros(q.shape, dtype=F64)
    for b in range(B):
        m, t = int(prefix_len[b]), int(t_gen[b])
        for h in range(H):
            out[b, h] = rswa_unit(q[b, h], k_prefix[b, h], v_prefix[b, h], m,
                                  ring_window(ring_k[b, h], t), ring_window(ring_v[b, h], t), scale)
    return out


# ============================================================================
# Block index and block scores   ([SR-SWA explainer] "稀疏路由" steps 1-2)
# ============================================================================
def block_ranges(m: int, block: int = 32) -> List[Tuple[int, int]]:
    """The prefix cut into consecutive blocks of `block` tokens; the last one
    may be shorter when block does not divide m."""
    return [(lo, min(lo + block, m)) for lo in range(0, m, block)]


def block_index(k_prefix: np.ndarray, m: int, proj: np.ndarray, block: int = 32) -> np.ndarray:
    """Block keys of one unit: for block j, the mean over its tokens of the
    projected key P^T k_t.  k_prefix [m_cap][D], proj [D][d].  Returns [nb][d]."""
    P = np.asarray(proj, dtype=F64)
    K = np.asarray(k_prefix, dtype=F64)
    rows = []
    for lo, hi in block_ranges(m, block):
        projected = K[lo:hi] @ P           # each token's P^T k_t
        rows.append(projected.mean(axis=0))
    return np.array(rows, dtype=F64).reshape(len(rows), P.shape[1])


def block_scores(q: np.ndarray, proj: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """Relevance of every block to the query: s_j = (P^T q) . kbar_j, no scale."""
    q_idx = np.asarray(proj, dtype=F64).T @ np.asarray(q, dtype=F64)
    return np.asarray(kbar, dtype=F64) @ q_idx


def as_f32(x: np.ndarray) -> np.ndarray:
    """Round to float32 (nearest) and back to float64: the precision the block
    scores are stored in, in which the routing decision is taken."""
    return np.asarray(x, dtype=F64).astype(np.float32).astype(F64)


# ============================================================================
# 1.5-entmax   ([SR-SWA explainer] "稀疏路由" step 3; Peters et al. 2019)
# ============================================================================
# entmax_1.5(z) = argmax_{p in simplex} p.z + H^T_{1.5}(p); its solution is
# p_j = [z_j/2 - tau]_+^2 with tau fixed by sum_j p_j = 1.

def entmax15(z: np.ndarray) -> np.ndarray:
    """Exact 1.5-entmax by sorting (Peters et al. 2019).

    With u = z/2 sorted descending, for every prefix size r take the mean mu_r
    of the r largest, ss_r = sum_{i<=r} (u_(i) - mu_r)^2 and
    tau_r = mu_r - sqrt(max(0, (1 - ss_r) / r)); the support size r* is the
    largest r with tau_r <= u_(r); p_j = max(0, u_j - tau_{r*})^2.
    """
    tau = entmax15_threshold(z)
    u = np.asarray(z, dtype=F64) / 2.0
    return np.maximum(u - tau, 0.0) ** 2


def entmax15_threshold(z: np.ndarray) -> float:
    u = np.asarray(z, dtype=F64) / 2.0
    us = np.sort(u)[::-1]
    best_tau = None
    for r in range(1, len(us) + 1):
        top = us[:r]
        mu = top.mean()
        ss = float(np.sum((top - mu) ** 2))
        tau_r = mu - math.sqrt(max(0.0, (1.0 - ss) / r))
        if tau_r <= us[r - 1]:
            best_tau = tau_r
    return float(best_tau)


def entmax15_bisect(z: np.ndarray, iters: int = 200) -> np.ndarray:
    """1.5-entmax by bisection on tau: f(tau) = sum_j max(0, u_j - tau)^2 is
    continuous and non-increasing, f(u_max - 1) >= 1 > 0 = f(u_max), so the
    root lies in [u_max - 1, u_max] (Blondel, Martins & Niculae 2020)."""
    u = np.asarray(z, dtype=F64) / 2.0
    lo, hi = u.max() - 1.0, u.max()
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if np.sum(np.maximum(u - mid, 0.0) ** 2) >= 1.0:
            lo = mid
        else:
            hi = mid
        if hi - lo <= 1e-16 * max(1.0, abs(hi)):
            break
    return np.maximum(u - 0.5 * (lo + hi), 0.0) ** 2


def entmax15_bruteforce(z: np.ndarray) -> np.ndarray:
    """1.5-entmax by enumerating every support set S (small inputs only).

    On S the normalisation sum_{j in S} (u_j - tau)^2 = 1 is a quadratic in
    tau; its smaller root is the candidate.  The answer is the S whose
    candidate satisfies the optimality (KKT) conditions: u_j > tau on S and
    u_j <= tau off S.
    """
    u = np.asarray(z, dtype=F64) / 2.0
    N = len(u)
    assert N <= 14, "brute force is exponential"
    found = None
    for size in range(1, N + 1):
        for S in itertools.combinations(range(N), size):
            uS = u[list(S)]
            a, b, c = float(size), -2.0 * uS.sum(), float(np.sum(uS ** 2)) - 1.0
            disc = b * b - 4 * a * c
            if disc < 0:
                continue
            tau = (-b - math.sqrt(disc)) / (2 * a)
            inside = all(u[j] > tau for j in S)
            outside = all(u[j] <= tau for j in range(N) if j not in S)
            if inside and outside:
                assert found is None or np.allclose(found, tau), "two KKT points"
                found = tau
    return np.maximum(u - found, 0.0) ** 2


# ============================================================================
# Top-k selection and log bias   ([SR-SWA explainer] "稀疏路由" steps 3-4)
# ============================================================================
def topk_blocks(s: np.ndarray, k: int) -> List[int]:
    """The min(k, nb) blocks ranked first by (score descending, index
    ascending), returned in ascending index order."""
    order = sorted(range(len(s)), key=lambda j: (-float(s[j]), j))
    return sorted(order[:min(k, len(s))])


def route_unit(s: np.ndarray, k: int):
    """Routing of one unit from its block scores s [nb] (already in the
    decision precision): entmax over all blocks, then the top-k.

    Returns (idx int32 [k], prob float64 [k], bias float64 [k]); entries past
    min(k, nb) are (-1, 0, -inf).  bias = ln p, -inf where p = 0, with no
    renormalisation over the kept blocks.
    """
    s = np.asarray(s, dtype=F64)
    idx = np.full(k, -1, dtype=np.int32)
    prob = np.zeros(k, dtype=F64)
    bias = np.full(k, NEG_INF, dtype=F64)
    if len(s) == 0:
        return idx, prob, bias
    p = entmax15(s)
    sel = topk_blocks(s, k)
    for i, j in enumerate(sel):
        idx[i] = j
        prob[i] = p[j]
        bias[i] = math.log(p[j]) if p[j] > 0 else NEG_INF
    return idx, prob, bias


# ============================================================================
# Sparse decode   ([SR-SWA explainer] "稀疏路由" step 4, "环形缓冲")
# ============================================================================
def srswa_unit(q, k_prefix, v_prefix, m, sel_idx, sel_bias, k_window, v_window,
               scale, block: int = 32) -> np.ndarray:
    """SR-SWA decode of one unit: the tokens of every selected block (index >=
    0), each with its block's bias added after scaling, plus the window with
    bias 0, then plain softmax attention.  sel_bias None means bias 0."""
    Ks, Vs, bs = [], [], []
    for i, j in enumerate(sel_idx):
        j = int(j)
        if j < 0:
            continue
        lo, hi = j * block, min(j * block + block, m)
        bj = 0.0 if sel_bias is None else float(sel_bias[i])
        Ks.append(np.asarray(k_prefix[lo:hi], dtype=F64))
        Vs.append(np.asarray(v_prefix[lo:hi], dtype=F64))
        bs.append(np.full(hi - lo, bj))
    Ks.append(np.asarray(k_window, dtype=F64))
    Vs.append(np.asarray(v_window, dtype=F64))
    bs.append(np.zeros(len(k_window)))
    return attention(q, np.concatenate(Ks), np.concatenate(Vs), scale, np.concatenate(bs))


# ============================================================================
# Prefill-side routing   ([Unlimited OCR Works README mirror] SGLang server
# section, notes on the memory knobs: the prefill holds a temporary score
# tensor of about [tokens, context/32], one score per (prefill token, block))
# ============================================================================
# Readings (the page gives only that tensor's shape): every query of a prefill
# chunk is routed the way a decode query is (scores, 1.5-entmax, top-k, log
# bias), over the prefix blocks it may see causally -- the blocks all of whose
# prefix tokens come before the query's position.  A block that still holds
# the query or a later token is left to the local window.

def visible_blocks(t: int, m: int, block: int = 32) -> int:
    """Prefix blocks a query at absolute position t may route to: block j
    (tokens [32j, min(32j + 32, m))) counts when every one of its tokens is
    at a position < t.  Blocks are contiguous from 0, so this is a count."""
    return sum(1 for lo, hi in block_ranges(m, block) if hi <= t)


def prefill_route_unit(q_rows: np.ndarray, q_pos: int, proj: np.ndarray, kbar: np.ndarray,
                       m: int, k: int, block: int = 32):
    """Routing of the Tq queries of one unit's prefill chunk: query i sits at
    position q_pos + i and is routed over its visible blocks from its scores
    rounded to float32.  q_rows [Tq][D], kbar [nb][d].
    Returns idx int32 [Tq][k], prob [Tq][k], bias [Tq][k]."""
    Tq = len(q_rows)
    idx = np.full((Tq, k), -1, dtype=np.int32)
    prob = np.zeros((Tq, k), dtype=F64)
    bias = np.full((Tq, k), NEG_INF, dtype=F64)
    for i in range(Tq):
        nbv = visible_blocks(q_pos + i, m, block)
        s32 = as_f32(block_scores(q_rows[i], proj, kbar[:nbv]))
        idx[i], prob[i], bias[i] = route_unit(s32, k)
    return idx, prob, bias


# ============================================================================
# Windowed no-repeat n-gram ban   ([Unlimited OCR Works README mirror] SGLang
# client example: the custom logit processor with ngram_size 35, window_size
# 128 for one page / 1024 for several, page_token_id, eos_token_id and
# max_page_tokens, the per-page output cap; [Unlimited OCR blog] inference
# parameters no_repeat_ngram_size / ngram_window)
# ============================================================================
# Readings (the pages give the parameters only): the next token is banned
# (logit -inf) when it would complete an n-gram equal to one lying wholly in
# the last `window` generated tokens; the page guard, once the current page
# has produced max_page_tokens tokens (> 0), leaves only the page marker and
# end-of-sequence open.

def ngram_banned(gen: Sequence[int], n: int, window: int) -> List[int]:
    """Tokens the next step may not produce.  gen = the generated tokens so
    far.  Inside the last `window` of them, every earlier n-gram whose first
    n-1 tokens equal the last n-1 generated tokens bans its n-th token."""
    gen = list(gen)
    T = len(gen)
    w = gen[max(0, T - window):]
    if n < 1 or len(w) < n:
        return []
    tail = w[len(w) - (n - 1):] if n > 1 else []
    banned = []
    for p in range(0, len(w) - n + 1):
        if w[p:p + n - 1] == tail:
            banned.append(w[p + n - 1])
    return sorted(set(banned))


def ngram_process(logits: np.ndarray, gen: Sequence[int], n: int, window: int,
                  page_tokens: int, max_page_tokens: int, page_token: int, eos_token: int) -> np.ndarray:
    """The processed logits of one sequence (a copy): the page guard, then
    the n-gram ban."""
    out = np.array(logits, copy=True)
    if max_page_tokens > 0 and page_tokens >= max_page_tokens:
        keep = {page_token, eos_token}
        for v in range(len(out)):
            if v not in keep:
                out[v] = NEG_INF
    for v in ngram_banned(gen, n, window):
        out[v] = NEG_INF
    return out


# ============================================================================
# page2d two-axis rotary position embedding   ([SR-SWA explainer] section
# "2D 位置编码" (rotary encoding, config sparse_rope_mode page2d, with a token
# axis = offset within the page for the order inside a page and a page axis =
# page number, page_mod 2, for the order between pages) and its last question
# (the language model is DeepSeek-V2); rotary embedding itself: Su et al.,
# "RoFormer: Enhanced Transformer with Rotary Position Embedding" (2021): its
# 2-D case turns each pair of dimensions, its general form uses the
# frequencies 10000^(-2(i-1)/d))
# ============================================================================
# Readings (the page names the two axes and page_mod only):
# * a pair (a, b) turned by phi becomes (a cos phi - b sin phi,
#   a sin phi + b cos phi);
# * the pairs are (j, j + D/2), j < D/2 (the "rotate half" layout of the
#   DeepSeek-V2 / Llama code family);
# * pairs j < D/4 turn with the token axis, pairs j >= D/4 with the page
#   axis; each axis has the frequencies of a rotary embedding over D/2 dims,
#   theta_i = base^(-2 i / (D/2)) with i = j mod D/4, base 10000;
# * token-axis position = the offset; page-axis position = page mod page_mod
#   when page_mod > 0, else the page number.

def rope_page2d_angles(page: int, offset: int, D: int, page_mod: int, base: float = 10000.0) -> np.ndarray:
    """The angle of each of the D/2 rotation pairs for a token at (page, offset)."""
    quarter = D // 4
    pos_page = page % page_mod if page_mod > 0 else page
    phi = np.empty(D // 2, dtype=F64)
    for j in range(D // 2):
        i = j % quarter
        theta = float(base) ** (-2.0 * i / (D / 2))
        pos = offset if j < quarter else pos_page
        phi[j] = pos * theta
    return phi


def rope_page2d(x: np.ndarray, page: int, offset: int, page_mod: int, base: float = 10000.0) -> np.ndarray:
    """x [..., D] of one token (any leading dims, e.g. heads), rotated; float64."""
    x = np.asarray(x, dtype=F64)
    D = x.shape[-1]
    phi = rope_page2d_angles(page, offset, D, page_mod, base)
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[..., :D // 2], x[..., D // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


# ============================================================================
# Whole routing of a batch, and the certified-gap rule for near-ties
# ============================================================================
def route(q, k_prefix, prefix_len, proj, k: int, block: int = 32):
    """Index, score and route every unit.  q [B][H][D]; returns dict with
    kbar (list), scores64, scores32 (decision precision), idx, prob, bias."""
    B, H = q.shape[0], q.shape[1]
    res = {"kbar": {}, "s64": {}, "s32": {},
           "idx": np.full((B, H, k), -1, np.int32),
           "prob": np.zeros((B, H, k)), "bias": np.full((B, H, k), NEG_INF)}
    for b in range(B):
        m = int(prefix_len[b])
        for h in range(H):
            kb = block_index(k_prefix[b, h], m, proj, block)
            s64 = block_scores(q[b, h], proj, kb)
            s32 = as_f32(s64)
            i, p, bi = route_unit(s32, k)
            res["kbar"][b, h], res["s64"][b, h], res["s32"][b, h] = kb, s64, s32
            res["idx"][b, h], res["prob"][b, h], res["bias"][b, h] = i, p, bi
    return res


def score_error_bound(q: np.ndarray, proj: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """Per-block bound on how far a stored score s_j may lie from the exact
    value (P^T q) . kbar_j when it is evaluated the way the routing's stored
    scores are: the block key kbar_j is held in float32 (rounded once from a
    float64 or exact value), q_idx = P^T q and the dot product are
    accumulated in float64, and the result is rounded once to float32.

        eps_j = 2^-22 * sum_i |q_idx_i| |kbar_ji|  +  ulp32(s_j)

    Rounding kbar_ji to float32 moves the term q_idx_i kbar_ji by at most
    2^-24 |q_idx_i| |kbar_ji|; the float64 sums add errors some 2^29 times
    smaller for these magnitudes, which the factor 4 margin (2^-22) absorbs;
    the final rounding moves the value by half a float32 ulp of the
    pre-rounded value, at most one ulp of the exact one.  The bound is
    within a factor 8 of the largest error such an evaluation can make on
    the given values (tests/test_oracle_score_bound.py pins both sides)."""
    q_idx = np.asarray(proj, dtype=F64).T @ np.asarray(q, dtype=F64)
    s = np.asarray(kbar, dtype=F64) @ q_idx
    mag = np.abs(np.asarray(kbar, dtype=F64)) @ np.abs(q_idx)
    ulp = np.spacing(np.abs(s).astype(np.float32)).astype(F64)
    return 2.0 ** -22 * mag + ulp


def certified_selection(s: np.ndarray, eps: np.ndarray, k: int):
    """Which blocks every evaluation of the scores within the bounds selects,
    and which none does (the certified-gap reading of the selection where
    floating point decides it).  s = exact scores, eps = per-block bounds,
    selection = the first min(k, nb) blocks by (score desc, index asc).

    Block x is surely selected when fewer than k other blocks can reach its
    lowest value s_x - eps_x (a block that reaches it exactly may win the tie
    by index, so it counts); surely dropped when at least k blocks have a
    lowest value above its highest value s_x + eps_x.
    Returns (sure_in, sure_out) as boolean arrays [nb]."""
    s = np.asarray(s, dtype=F64)
    eps = np.asarray(eps, dtype=F64)
    lo, hi = s - eps, s + eps
    others = ~np.eye(len(s), dtype=bool)                      # pairs (x, y) with y != x
    rivals = ((hi[None, :] >= lo[:, None]) & others).sum(axis=1)
    above = ((lo[None, :] > hi[:, None]) & others).sum(axis=1)
    return rivals < k, above >= k


def ambiguous_boundary(s64: np.ndarray, eps: np.ndarray, k: int) -> bool:
    """True when the bounds leave the selected set open: fewer than
    min(k, nb) blocks are surely selected, so evaluations within the bounds
    may select different sets (certified_selection says which)."""
    sure_in, _ = certified_selection(s64, eps, k)
    return int(sure_in.sum()) < min(k, len(s64))


def selection_within_bounds(sel: np.ndarray, s64: np.ndarray, eps: np.ndarray, k: int) -> bool:
    """Whether a selected index list (ascending, -1 padding) is one that an
    evaluation within the bounds can give: min(k, nb) distinct blocks in
    ascending order, every surely selected block in it, no surely dropped
    one."""
    sure_in, sure_out = certified_selection(s64, eps, k)
    nb = len(s64)
    want = min(k, nb)
    sel = [int(j) for j in sel]
    picked = sel[:want]
    if any(j != -1 for j in sel[want:]):
        return False
    if any(j < 0 or j >= nb for j in picked) or picked != sorted(set(picked)) or len(picked) != want:
        return False
    return all(j in picked for j in np.nonzero(sure_in)[0]) and not any(sure_out[j] for j in picked)
