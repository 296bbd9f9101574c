"""Shared helpers of the GPU parity tests (not collected as tests)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import synth as S
from long_context_decode_attn_amd import uocr as U
from oracle import uocr_oracle as O

BF16_MAX_ABS, BF16_REL_L2 = 2e-2, 1e-2
F32_MAX_ABS, F32_REL_L2 = 1e-4, 1e-4


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    U.load_library()  # raises if the HIP library is missing: no silent fallback


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    max_abs, rel = (F32_MAX_ABS, F32_REL_L2) if dtype == "f32" else (BF16_MAX_ABS, BF16_REL_L2)
    err = np.abs(got - ref).max() if got.size else 0.0
    nrm = np.linalg.norm(ref)
    rl2 = np.linalg.norm(got - ref) / nrm if nrm > 0 else np.linalg.norm(got - ref)
    assert err <= max_abs and rl2 <= rel, f"{what}: max-abs {err:.3e} (<= {max_abs}), rel-L2 {rl2:.3e} (<= {rel})"
    return err, rl2


class HostMirror:
    """The oracle's copy of one workload's decode state (float64)."""

    def __init__(self, w: S.Workload, prefix_cap=None, prefix_kv=None, ring=None):
        self.w = w
        Kp, Vp = S.prefix_kv(w, prefix_cap) if prefix_kv is None else prefix_kv
        self.Kp = S.widen(Kp, w.dtype)
        self.Vp = S.widen(Vp, w.dtype)
        Kr, Vr, t_gen = S.initial_ring(w) if ring is None else ring
        self.Kr = S.widen(Kr, w.dtype)
        self.Vr = S.widen(Vr, w.dtype)
        self.t_gen = np.asarray(t_gen, np.int64).copy()
        self.prefix_len = np.full(w.batch, w.prefix_len)

    def append(self, k_new, v_new):
        O.ring_append(self.Kr, self.Vr, self.t_gen, S.widen(k_new, self.w.dtype), S.widen(v_new, self.w.dtype))

    def window(self, b, h):
        t = int(self.t_gen[b])
        return O.ring_window(self.Kr[b, h], t), O.ring_window(self.Vr[b, h], t)
