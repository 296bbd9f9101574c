"""Seeded synthetic inputs for R-SWA / SR-SWA decode attention.

This module holds the input recipe only: workload shapes, random streams,
bf16 rounding of the drawn values and the planted-block construction used to
make routing non-trivial.  It contains none of the attention, routing or
entmax arithmetic; both the GPU path and the CPU checker read the same bits
produced here.

Workload shapes follow the pages' deployments: 256 visual tokens per page
(Unlimited OCR paper summary, lshu.cn, section 3.1 DeepEncoder), documents of
2 to 125 pages inside the 32K context, a generated-token window of n = 128
(same page, section 2.1 core design), up to 512 concurrent sequences (same
page, section 5.2 TPS), 32-token blocks and 16 routed blocks (Unlimited-OCR-2
explainer, nxmr.cn, section on sparse routing).  No document, image or trained
weight is used: every value is drawn from N(0, 1) (the index projection from
N(0, 1/32)) with numpy's PCG64 under a fixed seed.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

TOKENS_PER_PAGE = 256
BLOCK = 32
WINDOW = 128

# Independent random streams; the value is the first element of the
# SeedSequence spawn key, the second is the sequence index (or the step).
_S_PROJ, _S_QSTAR, _S_KP, _S_VP, _S_RING, _S_STEP, _S_PLANT, _S_Q, _S_MISC, _S_PREFILL = range(10)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    dtype: str            # "f32" or "bf16": storage type of q, k, v and out
    pages: int
    prompt: int           # prompt tokens appended to the visual tokens
    t0: int               # generated tokens before the first decode step
    steps: int
    seed: int
    sparse: bool = False
    window: int = WINDOW
    idx_dim: int = 32
    block: int = BLOCK
    topk: int = 16
    planted: int = 0      # planted relevant blocks per sequence
    planted_on_pages: bool = False   # one planted block per distinct page
    planted_noise: float = 1.0       # scale of the N(0, 1) part of planted keys
    fixed_query: bool = False        # same query every step (the planted q*)
    query_noise: bool = False        # with fixed_query: (q* + xi_t) / sqrt(2), xi_t ~ N(0, I) per step

    @property
    def prefix_len(self) -> int:
        return self.pages * TOKENS_PER_PAGE + self.prompt

    @property
    def n_blocks(self) -> int:
        return -(-self.prefix_len // self.block)

    @property
    def units(self) -> int:
        return self.batch * self.heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads.  Names say what they are; sizes are in the fields.
WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        # dense, CPU-sized, fp32: 2 pages + 16 prompt tokens, ring starts
        # empty and wraps three times in 512 steps
        Workload("dense-2p-b1-fp32", batch=1, heads=2, head_dim=64, dtype="f32",
                 pages=2, prompt=16, t0=0, steps=512, seed=1001),
        # dense steady state: 10 pages + 32 prompt, ring full at t = 6144
        Workload("dense-10p-b64", batch=64, heads=10, head_dim=128, dtype="bf16",
                 pages=10, prompt=32, t0=6144, steps=1000, seed=1002),
        # dense, high concurrency, short context: 1 page + 32 prompt
        Workload("dense-1p-b512", batch=512, heads=10, head_dim=128, dtype="bf16",
                 pages=1, prompt=32, t0=128, steps=1000, seed=1003),
        # dense companions of the two SR-SWA shapes: R-SWA over the whole
        # 40-page / 125-page prefix plus the window
        Workload("dense-40p-b32", batch=32, heads=10, head_dim=128, dtype="bf16",
                 pages=40, prompt=0, t0=128, steps=1000, seed=1006),
        Workload("dense-125p-b8", batch=8, heads=10, head_dim=128, dtype="bf16",
                 pages=125, prompt=0, t0=128, steps=2048, seed=1007),
        # SR-SWA at 40 pages: 320 blocks, 16 planted per sequence
        Workload("srswa-40p-b32", batch=32, heads=10, head_dim=128, dtype="bf16",
                 pages=40, prompt=0, t0=128, steps=1000, seed=1004, sparse=True,
                 planted=16, fixed_query=True),
        # SR-SWA at 125 pages (32000 tokens, 1000 blocks), 24 planted blocks on
        # 24 distinct pages; 2048 steps wrap the ring 16 times
        Workload("srswa-125p-b8", batch=8, heads=10, head_dim=128, dtype="bf16",
                 pages=125, prompt=0, t0=128, steps=2048, seed=1005, sparse=True,
                 planted=24, planted_on_pages=True, fixed_query=True),
        # the same two shapes with a per-step query (q* + xi_t) / sqrt(2), so
        # that the routing decision changes from step to step
        Workload("srswa-40p-b32-qnoise", batch=32, heads=10, head_dim=128, dtype="bf16",
                 pages=40, prompt=0, t0=128, steps=1000, seed=1004, sparse=True,
                 planted=16, fixed_query=True, query_noise=True),
        Workload("srswa-125p-b8-qnoise", batch=8, heads=10, head_dim=128, dtype="bf16",
                 pages=125, prompt=0, t0=128, steps=2048, seed=1005, sparse=True,
                 planted=24, planted_on_pages=True, fixed_query=True, query_noise=True),
        # wide routing: the planted blocks' own N(0, 1) part is scaled by 0.02,
        # so their scores lie within a fraction of each other and the 1.5-entmax
        # support holds every planted block (16 at 40 pages; 24 at 125 pages, of
        # which the top 16 are selected): each query reads 16 blocks, the
        # working set of about 16 x 32 reference tokens the pages describe
        Workload("srswa-40p-b32-wide", batch=32, heads=10, head_dim=128, dtype="bf16",
                 pages=40, prompt=0, t0=128, steps=1000, seed=1008, sparse=True,
                 planted=16, planted_noise=0.02, fixed_query=True),
        Workload("srswa-125p-b8-wide", batch=8, heads=10, head_dim=128, dtype="bf16",
                 pages=125, prompt=0, t0=128, steps=2048, seed=1009, sparse=True,
                 planted=24, planted_on_pages=True, planted_noise=0.02, fixed_query=True),
    ]
}


# ----------------------------------------------------------------------------
# bf16 storage
# ----------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even);
    returns the 16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Storage form of float32 values: float32 for "f32", uint16 bf16 bits for "bf16"."""
    return np.ascontiguousarray(x32, dtype=np.float32) if dtype == "f32" else to_bf16_bits(x32)


def widen(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements."""
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    return bf16_bits_to_f32(stored).astype(np.float64)


NAN_BITS = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0)}


def nan_fill(shape, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.full(shape, np.nan, dtype=np.float32)
    return np.full(shape, 0x7FC0, dtype=np.uint16)


# ----------------------------------------------------------------------------
# random streams
# ----------------------------------------------------------------------------
def _gen(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=tuple(key))))


def normal32(seed: int, shape, *key: int) -> np.ndarray:
    return _gen(seed, *key).standard_normal(size=shape, dtype=np.float32)


# ----------------------------------------------------------------------------
# static state: prefix K/V, projection, planted blocks, fixed queries
# ----------------------------------------------------------------------------
def projection(w: Workload) -> np.ndarray:
    """Index projection P [head_dim][idx_dim], float32, entries N(0, 1/idx_dim)."""
    p = normal32(w.seed, (w.head_dim, w.idx_dim), _S_PROJ, 0)
    return (p * np.float32(1.0 / math.sqrt(w.idx_dim))).astype(np.float32)


def planted_blocks(w: Workload, b: int) -> np.ndarray:
    """Sorted block indices whose keys carry the planted query shift."""
    if w.planted == 0:
        return np.zeros(0, dtype=np.int64)
    g = _gen(w.seed, _S_PLANT, b)
    if w.planted_on_pages:
        per_page = TOKENS_PER_PAGE // w.block
        pages = [(i * w.pages) // w.planted for i in range(w.planted)]
        blocks = [p * per_page + int(g.integers(0, per_page)) for p in pages]
        return np.array(sorted(blocks), dtype=np.int64)
    return np.sort(g.choice(w.n_blocks, size=w.planted, replace=False)).astype(np.int64)


def fixed_query_f32(w: Workload, b: int) -> np.ndarray:
    """The planted query q*[h][D] of sequence b, already rounded to storage precision."""
    q = normal32(w.seed, (w.heads, w.head_dim), _S_QSTAR, b)
    return widen(store(q, w.dtype), w.dtype).astype(np.float32)


def prefix_kv_seq(w: Workload, b: int, m_cap: Optional[int] = None):
    """Prefix K and V of sequence b as storage arrays [H][m_cap][D]; planted
    blocks get k <- round(k + 0.5 q*_h)."""
    m = w.prefix_len
    m_cap = m if m_cap is None else m_cap
    k = normal32(w.seed, (w.heads, m, w.head_dim), _S_KP, b)
    v = normal32(w.seed, (w.heads, m, w.head_dim), _S_VP, b)
    if w.planted:
        qs = fixed_query_f32(w, b)
        for blk in planted_blocks(w, b):
            lo, hi = blk * w.block, min(blk * w.block + w.block, m)
            if w.planted_noise != 1.0:
                k[:, lo:hi, :] *= np.float32(w.planted_noise)
            k[:, lo:hi, :] += np.float32(0.5) * qs[:, None, :]
    ks, vs = store(k, w.dtype), store(v, w.dtype)
    if m_cap > m:
        pad = nan_fill((w.heads, m_cap - m, w.head_dim), w.dtype)
        ks = np.concatenate([ks, pad], axis=1)
        vs = np.concatenate([vs, pad], axis=1)
    return ks, vs


def prefix_kv(w: Workload, m_cap: Optional[int] = None):
    """Prefix K, V storage arrays [B][H][m_cap][D] (padding beyond m is NaN)."""
    m_cap = w.prefix_len if m_cap is None else m_cap
    shape = (w.batch, w.heads, m_cap, w.head_dim)
    dt = np.float32 if w.dtype == "f32" else np.uint16
    K = np.empty(shape, dtype=dt)
    V = np.empty(shape, dtype=dt)
    for b in range(w.batch):
        K[b], V[b] = prefix_kv_seq(w, b, m_cap)
    return K, V


# ----------------------------------------------------------------------------
# generated tokens: history before t0 and per-step inputs
# ----------------------------------------------------------------------------
def history_token(w: Workload, tau: int):
    """k, v of generated token tau for every (b, h): storage arrays [B][H][D].
    Tokens tau < t0 form the initial ring, tokens >= t0 are appended by steps."""
    k = normal32(w.seed, (w.batch, w.heads, w.head_dim), _S_RING, tau, 0)
    v = normal32(w.seed, (w.batch, w.heads, w.head_dim), _S_RING, tau, 1)
    return store(k, w.dtype), store(v, w.dtype)


def step_query(w: Workload, step: int) -> np.ndarray:
    """Query of decode step `step` (0-based), storage array [B][H][D]: the
    planted q* (fixed_query), (q* + xi_t) / sqrt(2) with xi_t ~ N(0, I) drawn
    per step (fixed_query and query_noise), or N(0, 1)."""
    if w.fixed_query:
        q = np.stack([fixed_query_f32(w, b) for b in range(w.batch)]).astype(np.float32)
        if w.query_noise:
            xi = normal32(w.seed, (w.batch, w.heads, w.head_dim), _S_Q, step)
            q = ((q + xi) * np.float32(1.0 / math.sqrt(2.0))).astype(np.float32)
        return store(q, w.dtype)
    return store(normal32(w.seed, (w.batch, w.heads, w.head_dim), _S_Q, step), w.dtype)


def prefill_queries(w: Workload, tq: int, chunk: int = 0) -> np.ndarray:
    """Queries of a prefill chunk, storage array [B][H][tq][D].  Query i of a
    sequence is, by i mod 4: the planted q* plus N(0, 1/4) noise (routes to
    the planted blocks), plain N(0, 1), q* itself, or N(0, 1) scaled by 1e-3
    (nearly flat scores: many blocks tie for the entmax support).  Without
    planted queries every kind is N(0, 1), scaled as above."""
    z = normal32(w.seed, (w.batch, w.heads, tq, w.head_dim), _S_PREFILL, chunk)
    kind = np.arange(tq) % 4
    q = z.copy()
    if w.fixed_query:
        qs = np.stack([fixed_query_f32(w, b) for b in range(w.batch)]).astype(np.float32)[:, :, None, :]
        q = np.where((kind == 0)[None, None, :, None], qs + np.float32(0.5) * z, q)
        q = np.where((kind == 2)[None, None, :, None], np.broadcast_to(qs, q.shape), q)
    q = np.where((kind == 3)[None, None, :, None], z * np.float32(1e-3), q)
    return store(q.astype(np.float32), w.dtype)


def token_history(batch: int, n_tokens: int, vocab: int, seed: int, phrase: int = 40, repeat_p: float = 0.3,
                  lookback: int = 0):
    """Generated-token histories [batch][n_tokens] int32 with repetition, the
    way an OCR decode loops: the text is built from random phrases of
    `phrase` tokens, and with probability repeat_p a phrase copies an earlier
    stretch (starting at most `lookback` tokens back when lookback > 0), so
    long n-grams recur."""
    g = _gen(seed, _S_MISC, 7)
    out = np.empty((batch, n_tokens), dtype=np.int32)
    for b in range(batch):
        seq = []
        while len(seq) < n_tokens:
            if seq and g.random() < repeat_p:
                lo = max(0, len(seq) - lookback) if lookback > 0 else 0
                start = int(g.integers(lo, max(lo + 1, len(seq) - phrase + 1)))
                seq.extend(seq[start:start + phrase])
            else:
                seq.extend(g.integers(0, vocab, size=phrase).tolist())
        out[b] = seq[:n_tokens]
    return out


def step_inputs(w: Workload, step: int):
    """(q, k_new, v_new) of decode step `step`; k_new, v_new are token t0+step."""
    k, v = history_token(w, w.t0 + step)
    return step_query(w, step), k, v


def initial_ring(w: Workload, t0=None):
    """Ring K/V [B][H][n][D] holding, for sequence b, tokens max(0, t0_b-n) ..
    t0_b-1 in slot tau mod n (slots never written are NaN) and the generated
    count t_gen[B] = t0.  t0 defaults to w.t0 for every sequence."""
    n = w.window
    t0s = np.full((w.batch,), w.t0, dtype=np.int64) if t0 is None else np.asarray(t0, dtype=np.int64)
    Kr = nan_fill((w.batch, w.heads, n, w.head_dim), w.dtype)
    Vr = nan_fill((w.batch, w.heads, n, w.head_dim), w.dtype)
    lo = int(max(0, (t0s - n).min())) if len(t0s) else 0
    hi = int(t0s.max()) if len(t0s) else 0
    for tau in range(lo, hi):
        seqs = [b for b in range(w.batch) if t0s[b] - n <= tau < t0s[b]]
        if not seqs:
            continue
        k, v = history_token(w, tau)
        for b in seqs:
            Kr[b, :, tau % n, :] = k[b]
            Vr[b, :, tau % n, :] = v[b]
    return Kr, Vr, t0s.astype(np.int32)


def step_pool(w: Workload, steps: int):
    """Stacked per-step inputs for `steps` consecutive steps: q, k_new, v_new
    as storage arrays [steps][B][H][D]."""
    qs, ks, vs = [], [], []
    for s in range(steps):
        q, k, v = step_inputs(w, s)
        qs.append(q)
        ks.append(k)
        vs.append(v)
    return np.stack(qs), np.stack(ks), np.stack(vs)


def random_scores(seed: int, units: int, nb_cap: int, spread: float = 1.0) -> np.ndarray:
    """Block scores [units][nb_cap] float32 for exercising the selection step
    on its own: N(0, spread^2)."""
    return (normal32(seed, (units, nb_cap), _S_MISC, 0) * np.float32(spread)).astype(np.float32)


def random_selection(seed: int, units: int, n_blocks: int, k: int, live: int):
    """A routing result for exercising sparse decode on its own: per unit, k
    distinct ascending block indices (-1 padding when n_blocks < k) and a
    log-weight bias per entry; `live` entries chosen at random get a bias drawn
    from U(-5, 0), the rest -inf.  Returns (idx int32 [units][k],
    bias float32 [units][k])."""
    g = _gen(seed, _S_MISC, 1)
    idx = np.full((units, k), -1, dtype=np.int32)
    bias = np.full((units, k), -np.inf, dtype=np.float32)
    for u in range(units):
        sel = np.sort(g.choice(n_blocks, size=min(k, n_blocks), replace=False))
        idx[u, :len(sel)] = sel
        order = g.permutation(len(sel))[:live]
        bias[u, order] = g.uniform(-5.0, 0.0, size=len(order)).astype(np.float32)
    return idx, bias


def rope_rows(seed: int, batch: int, heads: int, tokens: int, head_dim: int, dtype: str) -> np.ndarray:
    """Rows to be rotated (queries or keys), storage array [B][H][T][D], N(0, 1)."""
    return store(normal32(seed, (batch, heads, tokens, head_dim), _S_MISC, 2), dtype)


def page_positions(seed: int, batch: int, tokens: int, page_tokens: int = 256, first_page: int = 0,
                   start_offset: int = 0):
    """(page, offset) int32 [B][T] of T consecutive tokens of a multi-page
    document: each page holds a number of tokens drawn from
    U[page_tokens/2, 3 page_tokens/2]; the offset restarts at 0 on every new
    page.  Sequence b starts on page first_page + b at offset start_offset."""
    g = _gen(seed, _S_MISC, 3)
    page = np.empty((batch, tokens), dtype=np.int32)
    offset = np.empty((batch, tokens), dtype=np.int32)
    lo, hi = max(1, page_tokens // 2), max(1, page_tokens // 2) + page_tokens
    for b in range(batch):
        p, o = first_page + b, start_offset
        length = max(int(g.integers(lo, hi + 1)), o + 1)
        for t in range(tokens):
            if o >= length:
                p, o = p + 1, 0
                length = int(g.integers(lo, hi + 1))
            page[b, t], offset[b, t] = p, o
            o += 1
    return page, offset
