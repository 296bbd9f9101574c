"""Child process of tests/test_gpu_phase_stamps.py (not a test): runs the
fused SR-SWA step of a named workload on libuocr_stamps.so and saves the
step's outputs and the phase stamps of its units.

    python tests/phase_stamps_child.py WORKLOAD STEPS OUT.npz
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from long_context_decode_attn_amd import synth as S  # noqa: E402
from long_context_decode_attn_amd import uocr as U  # noqa: E402
from long_context_decode_attn_amd.session import DecodeSession  # noqa: E402


def run_steps(w, steps):
    """The workload's first `steps` fused steps on a fresh seeded session;
    returns the last step's output, selection and counts as host arrays."""
    from long_context_decode_attn_amd.session import to_device
    sess = DecodeSession(w, fused=True)
    sess.build_index()
    for i in range(steps):
        q, k, v = S.step_inputs(w, i)
        sess.fused_step(to_device(q, w.dtype), to_device(k, w.dtype), to_device(v, w.dtype))
    torch.cuda.synchronize()
    return {"out": sess.out.view(torch.int16 if w.dtype == "bf16" else torch.int32).cpu().numpy(),
            "sel_idx": sess.sel_idx.cpu().numpy(), "sel_bias": sess.sel_bias.view(torch.int32).cpu().numpy(),
            "t_gen": sess.t_gen.cpu().numpy(), "k_ring": sess.k_ring.view(torch.int16 if w.dtype == "bf16"
                                                                            else torch.int32).cpu().numpy()}


def main():
    name, steps, path = sys.argv[1], int(sys.argv[2]), sys.argv[3]
    U.use_phase_stamps()
    U.load_library()
    torch.cuda.set_device(0)
    w = S.WORKLOADS[name]
    res = run_steps(w, steps)
    res["stamps"] = U.uocr_phase_stamps(w.units).astype(np.int64)
    np.savez(path, **res)
    print("saved", path, flush=True)


if __name__ == "__main__":
    main()
