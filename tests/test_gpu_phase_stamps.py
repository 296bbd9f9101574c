"""The stamping library (libuocr_stamps.so, the kernels with the fused
SR-SWA step's phase stamps compiled in) computes exactly what libuocr.so
computes, and its stamps are in the order the step's phases run.  The
stamping library runs in a child process (a process loads one of the two)."""
import os
import subprocess
import sys

import numpy as np
import pytest

from long_context_decode_attn_amd import synth as S
from long_context_decode_attn_amd import uocr as U
from tests._gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name,steps", [("srswa-40p-b32", 3), ("srswa-125p-b8-wide", 2)])
def test_stamping_library_matches_and_orders_phases(name, steps, tmp_path):
    need_gpu()
    if not os.path.exists(U.STAMPS_LIB_PATH):
        pytest.fail("libuocr_stamps.so is missing: build with `python -m long_context_decode_attn_amd.build`")
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from phase_stamps_child import run_steps
    say("phase stamps", name, steps)
    w = S.WORKLOADS[name]
    plain = run_steps(w, steps)
    path = str(tmp_path / "child.npz")
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "phase_stamps_child.py"), name,
                        str(steps), path], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    child = np.load(path)
    for key in ("out", "sel_idx", "sel_bias", "t_gen", "k_ring"):
        assert np.array_equal(plain[key], child[key]), f"{key} differs between the two libraries"
    st = child["stamps"]
    W = 8
    t = st - st[:, :1]
    for a, b in ((0, 5), (5, 6), (6, 1), (1, 2), (2, 7), (7, 4)):
        assert (t[:, b] >= t[:, a]).all(), f"slot {b} before slot {a}"
    assert (t[:, 17:16 + W] >= t[:, 1:2]).all(), "a window share ended before the scores were in LDS"
    # wave 0 publishes the selection and then stamps as the others do, when
    # it has waited for the flag: no order between slot 2 and slots 32 + w
    assert (t[:, 33:32 + W] >= t[:, 1:2]).all(), "a wave had a selection before the scores were in LDS"
    assert (t[:, 48:48 + W] <= t[:, 56:56 + W]).all(), "a wave merged its groups before its live blocks"
    assert (t[:, 56:56 + W] <= t[:, 7:8]).all(), "the merge barrier passed before a wave got there"
    assert (t[:, 4] < 100 * 1000).all(), "a workgroup ran for more than a millisecond"
    assert ((st[:, 3] & 0xF) < 8).all()
