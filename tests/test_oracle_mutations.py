"""Planted mistakes: each test hands a pin a broken copy of one oracle
routine (a dropped term, an off-by-one, a wrong sign or index, a transposed
operand) and checks that the pin rejects it.  Mistakes are planted only in
these CPU copies, never in the GPU path."""
import math

import numpy as np
import pytest

from oracle import uocr_oracle as O
from tests import test_oracle_pins as T


def _fails(check, **broken):
    with pytest.raises(AssertionError):
        check(**broken)


def test_window_off_by_one_is_caught():
    _fails(T.check_ring, window_positions=lambda t, n: list(range(max(0, t - n + 1), t)))


def test_ring_read_from_wrong_slot_is_caught():
    def ring_window(ring, t):
        n = ring.shape[0]
        return np.stack([ring[(tau + 1) % n] for tau in O.window_positions(t, n)]) if t else ring[:0]
    _fails(T.check_ring, ring_window=ring_window)


def test_append_before_pointer_advance_is_caught():
    def ring_append(rk, rv, t_gen, k, v):
        n = rk.shape[2]
        for b in range(rk.shape[0]):
            t_gen[b] += 1
            rk[b, :, t_gen[b] % n] = k[b]
            rv[b, :, t_gen[b] % n] = v[b]
    _fails(T.check_ring, ring_append=ring_append)


def test_cache_law_without_min_is_caught():
    _fails(T.check_cache_law, cache_len=lambda m, n, t: m + n)


def test_attention_without_scale_is_caught():
    _fails(T.check_attention, attention=lambda q, K, V, s, bias=None: O.attention(q, K, V, 1.0, bias))


def test_attention_with_sign_error_is_caught():
    _fails(T.check_attention, attention=lambda q, K, V, s, bias=None: O.attention(-q, K, V, s, bias))


def test_attention_dropping_bias_is_caught():
    _fails(T.check_attention, attention=lambda q, K, V, s, bias=None: O.attention(q, K, V, s, None))


def test_rswa_missing_prefix_is_caught():
    def rswa_decode(q, Kp, Vp, pl, rk, rv, t, s):
        return O.rswa_decode(q, Kp, Vp, np.zeros_like(pl), rk, rv, t, s)
    _fails(T.check_rswa_reductions, rswa_decode=rswa_decode)


def test_block_mean_over_fixed_32_is_caught():
    def block_index(K, m, P, block=32):
        Pd = np.asarray(P, float)
        return np.array([(np.asarray(K, float)[lo:lo + block] @ Pd).sum(0) / block
                         for lo in range(0, m, block)])
    _fails(T.check_block_index, block_index=block_index)


def test_score_with_extra_temperature_is_caught():
    def block_scores(q, P, kbar):
        return O.block_scores(q, P, kbar) / math.sqrt(np.asarray(kbar).shape[1])
    _fails(T.check_block_index, block_scores=block_scores)


def test_block_index_mean_before_wrong_axis_is_caught():
    def block_index(K, m, P, block=32):
        Pd = np.asarray(P, float)
        return np.array([(np.asarray(K, float)[lo:min(lo + block, m)] @ Pd).mean(1).mean() * np.ones(Pd.shape[1])
                         for lo in range(0, m, block)])
    _fails(T.check_block_index, block_index=block_index)


def test_entmax_without_half_is_caught():
    def entmax(z):
        return O.entmax15(2 * np.asarray(z, float))
    _fails(T.check_entmax, entmax=entmax)


def test_entmax_as_softmax_is_caught():
    def entmax(z):
        e = np.exp(np.asarray(z, float) - np.max(z))
        return e / e.sum()
    _fails(T.check_entmax, entmax=entmax)


def test_entmax_as_sparsemax_is_caught():
    def sparsemax(z):
        z = np.asarray(z, float)
        zs = np.sort(z)[::-1]
        cs = np.cumsum(zs)
        r = np.arange(1, len(z) + 1)
        k = r[1 + r * zs > cs].max()
        tau = (cs[k - 1] - 1) / k
        return np.maximum(z - tau, 0)
    _fails(T.check_entmax, entmax=sparsemax)


def test_topk_with_wrong_tie_break_is_caught():
    def topk(s, k):
        order = sorted(range(len(s)), key=lambda j: (-float(s[j]), -j))
        return sorted(order[:min(k, len(s))])
    _fails(T.check_topk, topk_blocks=topk)


def test_topk_ascending_scores_is_caught():
    def topk(s, k):
        order = sorted(range(len(s)), key=lambda j: (float(s[j]), j))
        return sorted(order[:min(k, len(s))])
    _fails(T.check_topk, topk_blocks=topk)


def test_srswa_bias_before_scale_is_caught():
    def srswa_unit(q, K, V, m, sel, bias, wk, wv, scale, block=32):
        b2 = None if bias is None else np.asarray(bias, float) / scale
        return O.srswa_unit(q, K, V, m, sel, b2, wk, wv, scale, block)
    _fails(T.check_srswa, srswa_unit=srswa_unit)


def test_srswa_missing_window_is_caught():
    def srswa_unit(q, K, V, m, sel, bias, wk, wv, scale, block=32):
        return O.srswa_unit(q, K, V, m, sel, bias, wk[:0], wv[:0], scale, block)
    _fails(T.check_srswa, srswa_unit=srswa_unit)


def test_prefill_visibility_including_the_query_block_is_caught():
    _fails(T.check_prefill_route,
           visible_blocks=lambda t, m, block=32: sum(1 for lo, hi in O.block_ranges(m, block) if lo < t))


def test_prefill_route_ignoring_chunk_position_is_caught():
    def prefill_route_unit(q, q_pos, P, kbar, m, k, block=32):
        return O.prefill_route_unit(q, 0, P, kbar, m, k, block)
    _fails(T.check_prefill_route, prefill_route_unit=prefill_route_unit)


def test_ngram_window_counting_the_unmatched_tail_is_caught():
    def ngram_banned(gen, n, window):
        return O.ngram_banned(gen, n, window + 1)
    _fails(T.check_ngram, ngram_banned=ngram_banned)


def test_ngram_matching_one_token_short_is_caught():
    _fails(T.check_ngram, ngram_banned=lambda gen, n, window: O.ngram_banned(gen, max(n - 1, 1), window))


def _rope_variant(swap_axes=False, freq_over_d=False, flip_sin=False, no_mod=False, interleaved=False):
    def rope(x, page, offset, page_mod, base=10000.0):
        x = np.asarray(x, dtype=np.float64)
        D = x.shape[-1]
        q4 = D // 4
        pp = page if (no_mod or page_mod <= 0) else page % page_mod
        phi = np.empty(D // 2)
        for j in range(D // 2):
            i = j % q4
            theta = base ** (-2.0 * i / (D if freq_over_d else D / 2))
            first = j < q4
            phi[j] = (pp if first else offset) * theta if swap_axes else (offset if first else pp) * theta
        cs, sn = np.cos(phi), np.sin(phi) * (-1.0 if flip_sin else 1.0)
        if interleaved:
            a, b = x[..., 0::2], x[..., 1::2]
            out = np.empty_like(x)
            out[..., 0::2], out[..., 1::2] = a * cs - b * sn, a * sn + b * cs
            return out
        a, b = x[..., :D // 2], x[..., D // 2:]
        return np.concatenate([a * cs - b * sn, a * sn + b * cs], axis=-1)
    return rope


def test_rope_variant_without_mistake_passes():
    T.check_rope(rope_page2d=_rope_variant())


@pytest.mark.parametrize("mistake", ["swap_axes", "freq_over_d", "flip_sin", "no_mod", "interleaved"])
def test_rope_mistakes_are_caught(mistake):
    _fails(T.check_rope, rope_page2d=_rope_variant(**{mistake: True}))


# ----------------------------------------------------------------------------
# the certified score bound and the selection rule built on it
# ----------------------------------------------------------------------------
from tests import test_oracle_score_bound as B   # noqa: E402


def test_score_bound_too_loose_is_caught():
    _fails(B.check_bound_tight, score_error_bound=lambda q, P, kb: O.score_error_bound(q, P, kb) * 2.0 ** 8)


def test_score_bound_too_tight_is_caught():
    def too_tight(q, P, kb):
        qi = np.asarray(P, float).T @ np.asarray(q, float)
        s = np.asarray(kb, float) @ qi
        return 2.0 ** -26 * (np.abs(kb) @ np.abs(qi)) + np.spacing(np.abs(s).astype(np.float32)).astype(float) / 4
    _fails(B.check_bound_sound, score_error_bound=too_tight)


def test_score_bound_relative_to_the_score_is_caught():
    """A bound proportional to |s| instead of the sum of |terms| fails where
    the score cancels to near 0."""
    def relative(q, P, kb):
        qi = np.asarray(P, float).T @ np.asarray(q, float)
        s = np.asarray(kb, float) @ qi
        return 2.0 ** -22 * np.abs(s) + np.spacing(np.abs(s).astype(np.float32)).astype(float)
    _fails(B.check_bound_sound, score_error_bound=relative)


def test_selection_rule_comparing_only_ranks_k_and_k_plus_1_is_caught():
    """The pairwise reading (flag only when the blocks ranked k and k + 1 are
    within their bounds) misses swaps deeper in the ranking when the bounds
    differ between blocks."""
    def pairwise(s, eps, k):
        if len(s) <= k:
            return False
        order = sorted(range(len(s)), key=lambda j: (-float(s[j]), j))
        a, b = order[k - 1], order[k]
        return abs(s[a] - s[b]) <= eps[a] + eps[b]
    _fails(B.check_selection_rule, ambiguous=pairwise)


def test_selection_rule_ignoring_index_ties_is_caught():
    """Counting only rivals strictly above a block's lowest value forgets that
    an exact tie goes to the lower index."""
    def strict(s, eps, k):
        lo, hi = np.asarray(s) - eps, np.asarray(s) + eps
        others = ~np.eye(len(s), dtype=bool)
        return (((hi[None, :] > lo[:, None]) & others).sum(1) < k,
                ((lo[None, :] > hi[:, None]) & others).sum(1) >= k)
    _fails(B.check_selection_rule, certified_selection=strict)
