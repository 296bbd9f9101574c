"""Decode steps over several per-layer states, replayed from HIP graphs.

A decoder that generates one token runs the decode step once per layer, each
layer with its own prefix, ring, generated-token counts and block keys.  This
module keeps L such states on the device (clones of one seeded state) and
runs steps in turn over them: global step i goes to layer i mod L.  The steps
are captured in HIP graphs (the way a serving loop launches decode steps) of
G = 2 L steps, two per layer, so that the double-buffered generated-token
counts of the fused steps return to the buffer they started from and a graph
can be replayed any number of times.

Every graph step reads its (q, k_new, v_new) from an input slot of its own
and, with the fused steps, writes its output (and, for SR-SWA, its
selection) into an output slot of its own, so that each step of a replay can
be inspected afterwards.  All
arithmetic runs in the library's kernels; this module only allocates, copies
and sequences.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import synth as S
from .session import DecodeSession, to_device

INFINITY_CACHE_BYTES = 256 * 2 ** 20


def layers_for(step_bytes: int, minimum: int = 12) -> int:
    """Layers to cycle so that the steps' combined working set is at least
    twice the 256 MB Infinity Cache: a layer's bytes have left the cache before
    the same layer runs again."""
    need = -(-2 * INFINITY_CACHE_BYTES // max(int(step_bytes), 1))
    return max(minimum, need)


class LayeredDecoder:
    def __init__(self, w: S.Workload, layers: int, num_splits: int = 0, fused: bool = True,
                 base: Optional[DecodeSession] = None, device: str = "cuda", rope: bool = False):
        self.w = w
        self.fused = fused
        # page2d RoPE fused into the steps: each sequence's new token at
        # (page, offset) positions of a seeded multi-page document
        self.rope = None
        if rope:
            assert fused, "RoPE is fused into the step kernels only"
            page, offset = S.page_positions(3, w.batch, 1, first_page=w.pages - 1, start_offset=17)
            self.rope = (torch.from_numpy(np.ascontiguousarray(page[:, 0])).to(device),
                         torch.from_numpy(np.ascontiguousarray(offset[:, 0])).to(device), 2, 10000.0)
        if base is None:
            base = DecodeSession(w, device=device, num_splits=num_splits, fused=fused)
        self.layers: List[DecodeSession] = [base] + [base.clone() for _ in range(layers - 1)]
        self.L = layers
        self.G = 2 * layers
        B, H, D = w.batch, w.heads, w.head_dim
        dt = base.shape.torch_dtype
        G = self.G
        self.q = torch.zeros((G, B, H, D), dtype=dt, device=device)
        self.k = torch.zeros((G, B, H, D), dtype=dt, device=device)
        self.v = torch.zeros((G, B, H, D), dtype=dt, device=device)
        self.out = torch.zeros((G, B, H, D), dtype=dt, device=device)
        if w.sparse:
            k = base.route.topk
            self.sel_idx = torch.zeros((G, B, H, k), dtype=torch.int32, device=device)
            self.sel_prob = torch.zeros((G, B, H, k), dtype=torch.float32, device=device)
            self.sel_bias = torch.zeros((G, B, H, k), dtype=torch.float32, device=device)
        self.graph = None

    # -- per-layer one-time work ------------------------------------------
    def build_index(self) -> None:
        if self.w.sparse:
            for s in self.layers:
                s.build_index()

    # -- steps -------------------------------------------------------------
    def _step(self, g: int, layer: int) -> None:
        s = self.layers[layer]
        if self.fused:
            sel = (self.sel_idx[g], self.sel_prob[g], self.sel_bias[g]) if self.w.sparse else None
            s.fused_step(self.q[g], self.k[g], self.v[g], out=self.out[g], sel=sel, rope=self.rope)
        else:   # one launch per row; outputs stay in the session's own buffers
            s.step(self.q[g], self.k[g], self.v[g])

    def order(self, n: int) -> List[int]:
        """Layer of each of the n steps of a graph: for the full graph, step g
        on layer g mod L (every layer twice); for a shorter tail, each layer
        twice in a row, so that its counts return to their first buffer."""
        if n == self.G:
            return [g % self.L for g in range(n)]
        return [g // 2 for g in range(n)]

    def run_eager(self, n: int) -> None:
        """n steps launched one by one from the host (inputs from the slots)."""
        for i in range(n):
            self._step(i % self.G, i % self.L)

    def capture(self, n: Optional[int] = None) -> torch.cuda.CUDAGraph:
        """A HIP graph of n (default G) steps; step g reads and writes slot g."""
        n = self.G if n is None else n
        assert 0 < n <= self.G
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i, layer in enumerate(self.order(n)):
                self._step(i, layer)
        if n % 2 == 1 and self.fused:
            # the last layer stepped once: its counts moved to the other
            # buffer; point the session back at the buffer the graphs read
            s = self.layers[self.order(n)[-1]]
            s.t_gen, s.t_gen_next = s.t_gen_next, s.t_gen
        if n == self.G:
            self.graph = g
        return g

    def fix_tail_counts(self, n: int) -> None:
        """After a replay of an n-step tail graph in which the last layer
        stepped once (n odd), copy that layer's advanced count into the buffer
        the graphs read, so that the next replay does not repeat a ring slot."""
        if n % 2 == 1 and self.fused:
            s = self.layers[self.order(n)[-1]]
            s.t_gen.copy_(s.t_gen_next)

    # -- inputs ------------------------------------------------------------
    def fill_inputs(self, steps) -> None:
        """Copy per-step inputs (a list of (q, k, v) storage arrays from synth)
        into the first len(steps) input slots."""
        for g, (q, k, v) in enumerate(steps):
            self.q[g].copy_(to_device(q, self.w.dtype))
            self.k[g].copy_(to_device(k, self.w.dtype))
            self.v[g].copy_(to_device(v, self.w.dtype))

    def fill_pool(self, pool_n: int = 64) -> None:
        """Inputs for timing: slot g gets step g of a seeded pool."""
        n = min(pool_n, self.G)
        self.fill_inputs([S.step_inputs(self.w, i) for i in range(n)])
        for g in range(n, self.G):
            self.q[g].copy_(self.q[g % n])
            self.k[g].copy_(self.k[g % n])
            self.v[g].copy_(self.v[g % n])

    def live_blocks(self, g: int) -> int:
        """Selected blocks with a finite bias (the blocks the sparse step
        reads) in output slot g."""
        si = self.sel_idx[g].cpu().numpy()
        sb = self.sel_bias[g].cpu().numpy()
        return int(np.sum((si >= 0) & np.isfinite(sb)))
