"""Pins of the oracle's certified score bound and of the selection rule built
on it, against exact rational arithmetic.  No GPU is used here.

Where floating point decides the routing's integer result (which blocks are
selected), the checker needs a bound on how far a stored block score can lie
from the exact one.  `score_error_bound` states one for the evaluation the
routing's stored scores get (block key held in float32, q_idx = P^T q and
the dot product accumulated in float64, one final rounding to float32).
These checks show, with the exact score computed in rationals
(fractions.Fraction), that

* the bound is sound: evaluations of that kind, in several summation orders
  and with or without fused multiply-adds, never leave it, also on inputs
  with heavy cancellation (score near 0 with large terms, q nearly in the
  null space of P^T), large magnitudes and short last blocks;
* the bound is tight: it is at most 8 times the largest error such an
  evaluation can make on the given values, and on a constructed input the
  error reaches more than 1/8 of it (1/16 on every block);
* the selection rule (`certified_selection`, `ambiguous_boundary`,
  `selection_within_bounds`) is sound against brute force over perturbed
  scores, and flags real near-tie pairs of blocks exactly when evaluations
  within the bounds can order them differently.

Each check takes the oracle routine it checks as an argument, so that
test_oracle_mutations.py can hand it a broken copy.
"""
from fractions import Fraction

import numpy as np

from long_context_decode_attn_amd import synth as S
from oracle import uocr_oracle as O

BLOCK = 32


# ----------------------------------------------------------------------------
# exact arithmetic and float64 evaluations of the score
# ----------------------------------------------------------------------------
def _bf16(x):
    return S.widen(S.store(np.asarray(x, np.float32), "bf16"), "bf16")


def _f32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def _fma(a, b, c):
    """a * b + c with one rounding to float64 (a fused multiply-add)."""
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def exact_qidx(q, P):
    D, d = P.shape
    return [sum(Fraction(float(P[t, i])) * Fraction(float(q[t])) for t in range(D)) for i in range(d)]


def exact_kbar(Kblk, P):
    """mean over the block's tokens of P^T k, exactly."""
    n, D = Kblk.shape
    col = [sum(Fraction(float(Kblk[r, t])) for r in range(n)) / n for t in range(D)]
    return [sum(Fraction(float(P[t, i])) * col[t] for t in range(D)) for i in range(P.shape[1])]


def exact_score(qidx_x, kbar_x):
    return sum(a * b for a, b in zip(qidx_x, kbar_x))


def _sum_seq(terms):
    acc = 0.0
    for t in terms:
        acc += t
    return acc


def _sum_tree(terms):
    terms = list(terms)
    while len(terms) > 1:
        terms = [terms[i] + terms[i + 1] if i + 1 < len(terms) else terms[i] for i in range(0, len(terms), 2)]
    return terms[0]


def _qidx64(q, P, how):
    """q_idx = P^T q in float64, in one of the orders a kernel may use."""
    D, d = P.shape
    out = np.empty(d)
    for i in range(d):
        prods = [float(P[t, i]) * float(q[t]) for t in range(D)]
        if how == "seq":
            out[i] = _sum_seq(prods)
        elif how == "slices8":      # D/8 slices of 8 terms, slices added in order
            out[i] = _sum_seq(_sum_seq(prods[s:s + 8]) for s in range(0, D, 8))
        elif how == "slices16":
            out[i] = _sum_seq(_sum_seq(prods[s:s + D // 8]) for s in range(0, D, D // 8))
        elif how == "fma":
            acc = 0.0
            for t in range(D):
                acc = _fma(float(P[t, i]), float(q[t]), acc)
            out[i] = acc
        else:
            raise ValueError(how)
    return out


def _kbar64(Kblk, P, how):
    """kbar of one block in float64 (before its float32 rounding)."""
    n, D = Kblk.shape
    d = P.shape[1]
    if how == "mean_then_project":          # column sums, times 1/n, then P^T
        inv = 1.0 / n
        col = [_sum_seq(float(Kblk[r, t]) for r in range(n)) * inv for t in range(D)]
        return np.array([_sum_tree([float(P[t, i]) * col[t] for t in range(D)]) for i in range(d)])
    if how == "project_then_mean":          # every token's P^T k, then the mean
        proj = [[_sum_seq(float(P[t, i]) * float(Kblk[r, t]) for t in range(D)) for i in range(d)]
                for r in range(n)]
        return np.array([_sum_seq(proj[r][i] for r in range(n)) / n for i in range(d)])
    raise ValueError(how)


def _dot64(qidx, kb32, how):
    """float64 dot product of q_idx with the float32-held block key."""
    d = len(qidx)
    if how == "seq":
        return _sum_seq(float(qidx[i]) * float(kb32[i]) for i in range(d))
    if how == "lanes8x4":                   # 8 lanes of 4 terms, then a tree over the lanes
        return _sum_tree([_sum_seq(float(qidx[i]) * float(kb32[i]) for i in range(4 * l, 4 * l + 4))
                          for l in range(d // 4)])
    if how == "fma":
        acc = 0.0
        for i in range(d):
            acc = _fma(float(qidx[i]), float(kb32[i]), acc)
        return acc
    raise ValueError(how)


EVALUATIONS = [("slices8", "mean_then_project", "lanes8x4"),
               ("seq", "mean_then_project", "seq"),
               ("slices16", "project_then_mean", "lanes8x4"),
               ("fma", "mean_then_project", "fma"),
               ("seq", "project_then_mean", "fma")]


def stored_scores(q, P, blocks, qidx_how, kbar_how, dot_how):
    """The stored (float32) scores of an evaluation of the stated kind."""
    qi = _qidx64(q, P, qidx_how)
    return np.array([_f32(_dot64(qi, _f32(_kbar64(Kb, P, kbar_how)), dot_how)) for Kb in blocks])


# ----------------------------------------------------------------------------
# input families
# ----------------------------------------------------------------------------
def _case(kind, D=128, d=32, nb=6, seed=0):
    """(q, P, blocks) with q and keys in bfloat16, P in float32."""
    rng = np.random.default_rng(seed)
    P = _f32(rng.standard_normal((D, d)) / np.sqrt(d))
    q = _bf16(rng.standard_normal(D))
    sizes = [BLOCK] * nb
    if kind == "short_blocks":
        sizes = [1, 3, 31, 7, BLOCK, 17][:nb]
    blocks = [rng.standard_normal((n, D)) for n in sizes]
    if kind == "planted":           # keys shifted by 0.5 q: scores near 0.5 |P^T q|^2
        blocks = [b + 0.5 * q for b in blocks]
    elif kind == "large":           # large keys, small query
        q = _bf16(q * 2.0 ** -9)
        blocks = [b * 2.0 ** 18 for b in blocks]
    elif kind == "cancel":          # scores near 0 with large terms: block means orthogonal to q_idx
        qi = P.T @ q
        u = np.linalg.lstsq(P.T, qi, rcond=None)[0]      # P^T u = q_idx
        for b in blocks:
            b *= 8.0
            mean_proj = P.T @ b.mean(axis=0)
            b -= (mean_proj @ qi) / (qi @ qi) * u     # remove the q_idx component of the mean
    elif kind == "null_q":          # q nearly in the null space of P^T: q_idx cancels
        z = rng.standard_normal(D) * 4.0
        z -= P @ np.linalg.lstsq(P, z, rcond=None)[0]
        q = _bf16(z)
    elif kind not in ("plain", "short_blocks"):
        raise ValueError(kind)
    return q, P, [_bf16(b) for b in blocks]


KINDS = [("plain", 128), ("plain", 64), ("planted", 128), ("large", 128), ("cancel", 128),
         ("null_q", 128), ("short_blocks", 64)]


def _oracle_kbar(blocks, P):
    return np.array([O.block_index(b, len(b), P)[0] for b in blocks])


# ----------------------------------------------------------------------------
# checks
# ----------------------------------------------------------------------------
def check_bound_sound(score_error_bound=O.score_error_bound):
    worst = 0.0
    for n, (kind, D) in enumerate(KINDS):
        q, P, blocks = _case(kind, D=D, seed=100 + n)
        qx = exact_qidx(q, P)
        s_exact = [exact_score(qx, exact_kbar(b, P)) for b in blocks]
        eps = score_error_bound(q, P, _oracle_kbar(blocks, P))
        assert np.all(eps > 0), kind
        for how in EVALUATIONS:
            got = stored_scores(q, P, blocks, *how)
            for j, (g, ex) in enumerate(zip(got, s_exact)):
                err = abs(Fraction(float(g)) - ex)
                assert err <= Fraction(float(eps[j])), (kind, how, j, float(err), eps[j])
                worst = max(worst, float(err) / eps[j])
        # the oracle's own decision values (exact score rounded once) lie inside too
        s32 = O.as_f32(O.block_scores(q, P, _oracle_kbar(blocks, P)))
        for j, ex in enumerate(s_exact):
            assert abs(Fraction(float(s32[j])) - ex) <= Fraction(float(eps[j])), (kind, j)
    return worst


def _half_ulp32(x):
    return np.spacing(np.abs(np.asarray(x, np.float64)).astype(np.float32)).astype(np.float64) / 2.0


def check_bound_tight(score_error_bound=O.score_error_bound):
    # (a) never more than 8 times the largest error the stated evaluation can
    # make on the given values: every key element rounded by a full half ulp
    # in the direction that adds up, plus half an ulp of the final rounding
    for n, (kind, D) in enumerate(KINDS):
        q, P, blocks = _case(kind, D=D, seed=200 + n)
        kb = _oracle_kbar(blocks, P)
        qi = P.T @ q
        s = kb @ qi
        worst = np.abs(qi) @ _half_ulp32(kb).T + _half_ulp32(s)
        eps = score_error_bound(q, P, kb)
        assert np.all(eps <= 8.0 * worst * (1 + 1e-9)), (kind, eps / worst)
    # (b) a constructed case where every key element's float32 rounding takes
    # almost a full half ulp in the same direction: the error reached is more
    # than 1/8 of the bound
    rng = np.random.default_rng(7)
    D, d = 128, 32
    P = _f32(rng.standard_normal((D, d)) / np.sqrt(d))
    q = _bf16(rng.standard_normal(D))
    qi64 = _qidx64(q, P, "seq")
    exps = rng.integers(-3, 3, size=(5, d))
    # 2^e (1 + 2^-24 - 2^-40): rounds down to 2^e, by almost half an ulp; the
    # sign makes q_idx_i * (rounded - exact) positive for every i
    mag = np.ldexp(1.0 + 2.0 ** -24 - 2.0 ** -40, exps)
    kbar = -np.sign(qi64)[None, :] * mag
    eps = score_error_bound(q, P, kbar)
    qx = exact_qidx(q, P)
    reached = []
    for j in range(len(kbar)):
        ex = exact_score(qx, [Fraction(float(v)) for v in kbar[j]])
        for how in ("seq", "lanes8x4", "fma"):
            got = _f32(_dot64(qi64, _f32(kbar[j]), how))
            err = abs(Fraction(float(got)) - ex)
            assert err <= Fraction(float(eps[j])), (j, how)
            reached.append(float(err) / eps[j])
    # the final rounding may take back up to half an ulp of what the keys'
    # rounding added, so not every block gets as far as the best one
    assert max(reached) > 1.0 / 8.0 and min(reached) > 1.0 / 16.0, reached
    # (c) an evaluation that forms q_idx in float32 (128 terms) leaves the
    # bound on some of the realistic inputs: the bound is no wider than the
    # float64 evaluation needs (and the kernels form q_idx in float64)
    outside = 0
    for n, (kind, D) in enumerate(KINDS):
        q, P, blocks = _case(kind, D=D, seed=100 + n)
        kb = _oracle_kbar(blocks, P)
        eps = score_error_bound(q, P, kb)
        qi32 = np.zeros(P.shape[1], np.float32)
        for t in range(P.shape[0]):
            qi32 = (qi32 + P[t].astype(np.float32) * np.float32(q[t])).astype(np.float32)
        qx = exact_qidx(q, P)
        for j, blk in enumerate(blocks):
            got = _f32(_dot64(qi32.astype(np.float64), _f32(kb[j]), "seq"))
            outside += abs(Fraction(float(got)) - exact_score(qx, exact_kbar(blk, P))) > Fraction(float(eps[j]))
    assert outside > 0


def check_selection_rule(certified_selection=O.certified_selection, ambiguous=O.ambiguous_boundary,
                         within=O.selection_within_bounds):
    rng = np.random.default_rng(11)

    def topk(v, k):
        order = sorted(range(len(v)), key=lambda j: (-float(v[j]), j))
        return sorted(order[:min(k, len(v))])

    # hand-made cases first: bounds that differ between blocks, where a block
    # ranked above the boundary pair can fall below it although that pair is
    # further apart than its own bounds
    cases = [(np.array([10.05, 10.0, 9.9]), np.array([0.2, 0.001, 0.001]), 2),
             (np.array([3.0, 1.0, 2.95, 0.0]), np.array([0.0, 0.01, 0.1, 0.5]), 1),
             (np.array([1.0, 1.0, 1.0]), np.zeros(3), 2)]
    for trial in range(300):
        nb = int(rng.integers(1, 9))
        k = int(rng.integers(1, nb + 2))
        s = np.round(rng.normal(size=nb) * 2.0, 1)       # frequent exact ties
        eps = rng.uniform(0.0, 0.3, size=nb) * (rng.random(nb) < 0.7)
        cases.append((s, eps, k))
    for s, eps, k in cases:
        nb = len(s)
        sure_in, sure_out = certified_selection(s, eps, k)
        outcomes = set()
        for _ in range(60):   # perturbations inside the bounds, corners included
            pick = rng.integers(0, 3, size=nb)
            if _ < 2 ** nb:   # every corner of the box first
                pick = np.array([(_ >> i) & 1 for i in range(nb)])
            delta = np.where(pick == 0, -eps, np.where(pick == 1, eps, rng.uniform(-1, 1, nb) * eps))
            sel = topk(s + delta, k)
            outcomes.add(tuple(sel))
            assert all(j in sel for j in np.nonzero(sure_in)[0]), (s, eps, k, sel)
            assert not any(sure_out[j] for j in sel), (s, eps, k, sel)
            padded = np.full(max(k, 1), -1)
            padded[:len(sel)] = sel
            assert within(padded, s, eps, k)
        if len(outcomes) > 1:
            assert ambiguous(s, eps, k), (s, eps, k, outcomes)
        if not ambiguous(s, eps, k):
            assert outcomes == {tuple(topk(s, k))}
        # completeness on the corners: a block not surely in can be pushed out,
        # one not surely out can be pulled in (no exact ties at the corners here)
        s2 = s + rng.uniform(-1e-6, 1e-6, nb)
        i2, o2 = certified_selection(s2, eps, k)
        for x in range(nb):
            down = s2 + eps
            down[x] = s2[x] - eps[x]
            up = s2 - eps
            up[x] = s2[x] + eps[x]
            if not i2[x]:
                assert x not in topk(down, k), (x, s2, eps, k)
            if not o2[x]:
                assert x in topk(up, k), (x, s2, eps, k)
    # a wrong selection is rejected: a surely dropped block, a duplicate, a
    # missing surely selected block, entries past min(k, nb)
    s = np.array([9.0, 8.0, 1.0, 0.5, 0.4])
    eps = np.full(5, 1e-3)
    assert within(np.array([0, 1]), s, eps, 2)
    assert not within(np.array([0, 2]), s, eps, 2)
    assert not within(np.array([1, 1]), s, eps, 2)
    assert not within(np.array([1, 0]), s, eps, 2)
    assert not within(np.array([0, 1, 3]), s, eps, 2)
    assert within(np.array([0, 1, 2, 3, 4, -1]), s, eps, 6)


def check_near_tie_pairs(score_error_bound=O.score_error_bound, ambiguous=O.ambiguous_boundary):
    """Pairs of real blocks whose exact scores differ by amounts from far
    below to far above their bounds: the second block is the first with one
    small key element moved by a few bfloat16 steps.  Whenever evaluations of
    the stated kind (or the oracle's own decision values) order the pair
    differently, the rule flags the boundary between them; when the gap
    exceeds the bounds it does not, and every evaluation orders them alike.
    Returns the number of pairs on which evaluations disagreed."""
    rng = np.random.default_rng(23)
    D, d = 64, 32
    P = _f32(rng.standard_normal((D, d)) / np.sqrt(d))
    flagged = certain = disagreements = 0
    for trial in range(160):
        q = _bf16(rng.standard_normal(D))
        a = _bf16(rng.standard_normal((BLOCK, D)))
        r, t = int(rng.integers(BLOCK)), int(rng.integers(D))
        tiny = 2.0 ** int(rng.integers(-24, -4))          # the element that moves is small,
        a[r, t] = tiny                                     # so its bfloat16 steps are small
        b = a.copy()
        b[r, t] = tiny * (1.0 + int(rng.integers(1, 4)) * 2.0 ** -7)
        blocks = [a, b]
        kb = _oracle_kbar(blocks, P)
        eps = score_error_bound(q, P, kb)
        s64 = kb @ (P.T @ q)
        orders = set()
        for how in (EVALUATIONS[0], EVALUATIONS[1], EVALUATIONS[3]):
            v = stored_scores(q, P, blocks, *how)
            orders.add(0 if v[0] >= v[1] else 1)          # equal scores: the lower index first
        s32 = O.as_f32(s64)
        orders.add(0 if s32[0] >= s32[1] else 1)
        amb = ambiguous(s64, eps, 1)
        if len(orders) > 1:
            disagreements += 1
            assert amb, (trial, s64, eps)
        if abs(s64[0] - s64[1]) > eps[0] + eps[1]:
            assert not amb and len(orders) == 1, (trial, s64, eps)
            certain += 1
        else:
            flagged += amb
    assert certain > 0 and flagged > 0 and disagreements > 0, (certain, flagged, disagreements)
    return disagreements


def test_score_bound_is_sound():
    assert check_bound_sound() <= 1.0


def test_score_bound_is_tight():
    check_bound_tight()


def test_selection_rule_against_brute_force():
    check_selection_rule()


def test_near_tie_pairs_are_flagged():
    check_near_tie_pairs()
