"""The measurement kernels of include/uocr_calib.h on the GPU: they run on
small inputs, reject bad arguments, and the in-kernel merge computes what it
claims (the last workgroup to arrive sums every partial of its unit and
leaves the counter at 0), in each of its three modes."""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import uocr as U
from tests._gpu_common import need_gpu

pytestmark = pytest.mark.gpu


def test_calibration_kernels_run():
    need_gpu()
    src = torch.ones(1 << 22, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    for nt in (False, True):
        U.uocr_calib_read(src, nt, sink)
    U.uocr_calib_empty(80, 512)
    sk = torch.zeros(16, dtype=torch.int32, device="cuda")
    U.uocr_calib_pull(src, 1 << 16, 16, 512, True, sk)
    st = torch.zeros(320, dtype=torch.int64, device="cuda")
    U.uocr_calib_start(320, 512, st)
    torch.cuda.synchronize()
    assert (sink == 0).all() and (sk == 0).all()     # the loads' hash never matches
    t = st.cpu().numpy()
    assert (t > 0).all() and t.max() - t.min() < 100_000_000   # all within a second of each other
    with pytest.raises(U.UocrError):
        U.uocr_calib_empty(0, 512)
    with pytest.raises(U.UocrError):
        U.uocr_calib_empty(8, 100)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_in_kernel_merge_is_right(mode):
    need_gpu()
    units, split = 37, 5
    part = torch.zeros(units * split * 130, dtype=torch.float32, device="cuda")
    cnt = torch.zeros(units, dtype=torch.int32, device="cuda")
    out = torch.zeros(units * 130, dtype=torch.float32, device="cuda")
    for _ in range(3):   # the counters must come back to 0 after every launch
        out.zero_()
        U.uocr_calib_exchange(mode, units, split, part, cnt, out)
        torch.cuda.synchronize()
        o = out.view(units, 130).cpu().numpy()
        if mode == 2:
            want = np.full((units, 130), float(split))
        else:
            want = split * (split + 1) / 2 + split * np.arange(130, dtype=np.float64)[None, :].repeat(units, 0)
        assert np.array_equal(o, want.astype(np.float32))
        assert (cnt == 0).all()
