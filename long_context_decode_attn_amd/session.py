"""Device-resident decode state of one synthetic workload, driven through the
C entry points of libuocr.so.

A session owns the buffers of one layer's decode state on the GPU (prefix
K/V, ring K/V, generated-token counts, index projection, block index, routing
outputs, workspaces) and runs one decode step as the pages describe it:
append the new token to the ring, then (SR-SWA) score the prefix blocks,
select them with 1.5-entmax top-k, and attend over the selected blocks plus
the window with the log bias, or (R-SWA) attend over the whole prefix plus the
window.  All arithmetic happens in the HIP kernels; this module only moves
seeded inputs to the device and sequences the calls.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import synth as S
from . import uocr as U


def to_device(stored: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Storage array from synth (float32, or uint16 bf16 bits) -> device tensor."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32)).to(device)
    bits = np.ascontiguousarray(stored, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(bits).to(device).view(torch.bfloat16)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> exact float64 values on the host."""
    return t.detach().float().cpu().numpy().astype(np.float64)


class DecodeSession:
    def __init__(self, w: S.Workload, device="cuda", prefix_cap: Optional[int] = None,
                 num_splits: int = 0, prefix_kv=None, ring=None, fused: bool = False):
        self.w = w
        self.device = device
        self.fused = fused
        cap = w.prefix_len if prefix_cap is None else prefix_cap
        self.shape = U.Shape.of(w, cap)
        self.route = U.Route(w.block, w.idx_dim, w.topk)
        self.num_splits = num_splits
        B, H, D, n = w.batch, w.heads, w.head_dim, w.window
        dt = self.shape.torch_dtype
        Kp, Vp = S.prefix_kv(w, cap) if prefix_kv is None else prefix_kv
        self.k_prefix = to_device(Kp, w.dtype, device)
        self.v_prefix = to_device(Vp, w.dtype, device)
        del Kp, Vp
        self.prefix_len = torch.full((B,), w.prefix_len, dtype=torch.int32, device=device)
        Kr, Vr, t_gen = S.initial_ring(w) if ring is None else ring
        self.k_ring = to_device(Kr, w.dtype, device)
        self.v_ring = to_device(Vr, w.dtype, device)
        self.t_gen = torch.from_numpy(np.asarray(t_gen, dtype=np.int32)).to(device)
        self.t_gen_next = torch.empty_like(self.t_gen)  # second buffer of the fused steps
        self.out = torch.empty((B, H, D), dtype=dt, device=device)
        if w.sparse:
            k = self.route.topk
            self.proj = torch.from_numpy(S.projection(w)).to(device)
            self.kbar = torch.empty((B, H, self.shape.nb_cap, w.idx_dim), dtype=torch.float32, device=device)
            self.scores = torch.empty((B, H, self.shape.nb_cap), dtype=torch.float32, device=device)
            self.sel_idx = torch.empty((B, H, k), dtype=torch.int32, device=device)
            self.sel_prob = torch.empty((B, H, k), dtype=torch.float32, device=device)
            self.sel_bias = torch.empty((B, H, k), dtype=torch.float32, device=device)
            self.workspace = U.alloc_workspace(U.uocr_srswa_workspace_bytes(self.shape, self.route, num_splits),
                                               device)
        else:
            self.workspace = U.alloc_workspace(U.uocr_rswa_workspace_bytes(self.shape, num_splits), device)

    def clone(self) -> "DecodeSession":
        """An independent copy of the whole device state (another layer's
        buffers with the same contents)."""
        c = object.__new__(DecodeSession)
        c.__dict__.update(self.__dict__)
        for k, v in self.__dict__.items():
            if isinstance(v, torch.Tensor):
                setattr(c, k, v.clone())
        return c

    # -- one-time work after prefill ---------------------------------------
    def build_index(self) -> None:
        U.uocr_block_index_build(self.shape, self.route, self.k_prefix, self.prefix_len, self.proj, self.kbar)

    # -- the rows of one decode step ----------------------------------------
    def append(self, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
        U.uocr_ring_append(self.shape, self.k_ring, self.v_ring, k_new, v_new, self.t_gen)

    def prefill_route(self, q: torch.Tensor, q_pos: torch.Tensor):
        """Routing of a prefill chunk q [B][H][tq][D] whose query 0 sits at
        position q_pos[b] (int32 [B]); returns (idx, prob, bias) [B][H][tq][k]."""
        B, H, tq, k = q.shape[0], q.shape[1], q.shape[2], self.route.topk
        idx = torch.empty((B, H, tq, k), dtype=torch.int32, device=q.device)
        prob = torch.empty((B, H, tq, k), dtype=torch.float32, device=q.device)
        bias = torch.empty((B, H, tq, k), dtype=torch.float32, device=q.device)
        U.uocr_prefill_route(self.shape, self.route, q, q_pos, self.proj, self.kbar, self.prefix_len,
                             idx, prob, bias)
        return idx, prob, bias

    def score(self, q: torch.Tensor) -> None:
        U.uocr_block_score(self.shape, self.route, q, self.proj, self.kbar, self.prefix_len, self.scores)

    def select(self) -> None:
        U.uocr_entmax15_topk(self.shape, self.route, self.scores, self.prefix_len, self.sel_idx,
                             self.sel_prob, self.sel_bias)

    def attend(self, q: torch.Tensor) -> None:
        if self.w.sparse:
            U.uocr_srswa_decode(self.shape, self.route, q, self.k_prefix, self.v_prefix, self.prefix_len,
                                self.sel_idx, self.sel_bias, self.k_ring, self.v_ring, self.t_gen, self.out,
                                self.workspace, self.num_splits)
        else:
            U.uocr_rswa_decode(self.shape, q, self.k_prefix, self.v_prefix, self.prefix_len, self.k_ring,
                               self.v_ring, self.t_gen, self.out, self.workspace, self.num_splits)

    def fused_step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, out=None, sel=None,
                   rope=None) -> None:
        """The whole step in one launch; the generated-token counts move to
        the other buffer, which becomes `t_gen`.  out (and, for SR-SWA, sel =
        (idx, prob, bias)) default to the session's own buffers; rope = None
        or (page, offset, page_mod, base) turns q and k_new by page2d RoPE."""
        out = self.out if out is None else out
        if self.w.sparse:
            si, sp, sb = (self.sel_idx, self.sel_prob, self.sel_bias) if sel is None else sel
            U.uocr_srswa_step(self.shape, self.route, q, k_new, v_new, self.k_prefix, self.v_prefix,
                              self.prefix_len, self.proj, self.kbar, self.k_ring, self.v_ring, self.t_gen,
                              self.t_gen_next, si, sp, sb, out, self.num_splits, rope=rope)
        else:
            U.uocr_rswa_step(self.shape, q, k_new, v_new, self.k_prefix, self.v_prefix, self.prefix_len,
                             self.k_ring, self.v_ring, self.t_gen, self.t_gen_next, out, self.workspace,
                             self.num_splits, rope=rope)
        self.t_gen, self.t_gen_next = self.t_gen_next, self.t_gen

    def step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor) -> torch.Tensor:
        """One decode step: append, (route,) attend.  Returns `out` (reused)."""
        if self.fused:
            self.fused_step(q, k_new, v_new)
            return self.out
        self.append(k_new, v_new)
        if self.w.sparse:
            self.score(q)
            self.select()
        self.attend(q)
        return self.out
