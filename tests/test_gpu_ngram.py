"""GPU parity of the windowed no-repeat n-gram ban and page guard
(uocr_ngram_ban) against the oracle, through the C ABI: the processed logits
must be bit-identical."""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import synth as S
from long_context_decode_attn_amd import uocr as U
from oracle import uocr_oracle as O
from tests._gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu


def _run(B, T, vocab, ngram, window, ring_cap, dtype, max_page=0, seed=3, phrase=40, page_tok=None, n_gen=None):
    hist = S.token_history(B, T, vocab, seed, phrase=phrase, repeat_p=0.5, lookback=max(window - phrase, 1))
    n_gen = np.full(B, T, np.int32) if n_gen is None else np.asarray(n_gen, np.int32)
    ring = np.zeros((B, ring_cap), np.int32)
    for b in range(B):
        for pos in range(max(0, n_gen[b] - ring_cap), n_gen[b]):
            ring[b, pos % ring_cap] = hist[b, pos]
    page_tokens = (np.arange(B, dtype=np.int32) * 7) % (2 * max(max_page, 1)) if page_tok is None else page_tok
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((B, vocab)).astype(np.float32)
    tl = torch.from_numpy(logits).cuda()
    if dtype == "bf16":
        tl = tl.to(torch.bfloat16)
        logits = tl.float().cpu().numpy()
    U.uocr_ngram_ban(torch.from_numpy(ring).cuda(), torch.from_numpy(n_gen).cuda(),
                     torch.from_numpy(np.asarray(page_tokens, np.int32)).cuda(), tl, ngram, window,
                     page_token=vocab - 1, eos_token=1, max_page_tokens=max_page)
    got = tl.float().cpu().numpy()
    banned_total = 0
    for b in range(B):
        want = O.ngram_process(logits[b].astype(np.float64), hist[b, :n_gen[b]].tolist(), ngram, window,
                               int(page_tokens[b]), max_page, vocab - 1, 1)
        assert np.array_equal(np.isneginf(got[b]), np.isneginf(want)), b
        fin = np.isfinite(want)
        assert np.array_equal(got[b][fin], want[fin].astype(np.float32)), b
        banned_total += int(np.isneginf(want).sum())
    return banned_total


@pytest.mark.parametrize("ngram,window,dtype", [(35, 128, "f32"), (35, 1024, "bf16"), (3, 64, "f32"),
                                                (1, 32, "bf16"), (2, 4096, "f32")])
def test_ngram_ban_matches_oracle(ngram, window, dtype):
    need_gpu()
    say("ngram", ngram, window, dtype)
    T = np.random.default_rng(ngram + window).integers(ngram, 1500, size=24)
    n = _run(B=24, T=1500, vocab=5000, ngram=ngram, window=window, ring_cap=max(window, 1100) + 37, dtype=dtype,
             phrase=max(3 * ngram, 8), n_gen=T)
    assert n > 0   # the repeated phrases produce bans


def test_ngram_ban_short_histories_and_ring_wrap():
    """Histories shorter than n and than the window, a ring that wrapped
    several times, a vocabulary of the pages' size."""
    need_gpu()
    say("ngram short/wrap")
    _run(B=6, T=3000, vocab=129280, ngram=35, window=1024, ring_cap=1024, dtype="bf16",
         n_gen=[0, 20, 34, 35, 1500, 3000])


def test_ngram_page_guard():
    """The per-page cap leaves only the page marker and end-of-sequence open
    (and the n-gram ban still applies to them)."""
    need_gpu()
    say("ngram page guard")
    _run(B=10, T=400, vocab=3000, ngram=4, window=128, ring_cap=128, dtype="f32", max_page=20, phrase=6,
         page_tok=np.array([0, 19, 20, 21, 500, 5, 20, 40, 1, 2], np.int32))
