"""bench.py on the host: the refusal of more than one GPU, and the byte model
behind its roofline against the per-unit figures of the measurement plan
(bytes each step must move at the pages' shapes: bf16, D = 128, n = 128)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from long_context_decode_attn_amd import synth as S  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_document_length_override_refuses_a_prefix_without_room_for_the_planted_blocks():
    # 1 page holds 8 blocks, fewer than the 16 planted ones of the 40-page workload
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "srswa-40p-b32", "--pages",
                        "1", "--batch", "8", "--no-cpu-baseline"], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "out of range" in r.stderr and r.stdout == ""


def test_document_length_override_bytes_scale_with_the_pages():
    """The dense step's bytes follow the prefix; the sparse step's block keys
    follow it at 128 B per 32 tokens while its window and selected blocks do not."""
    w = S.WORKLOADS["dense-40p-b32"]
    small, big = w.replace(pages=2, batch=8), w.replace(pages=125, batch=8)
    d = lambda x: bench.algorithmic_bytes(x)["uocr_rswa_decode"] / x.units
    assert d(big) - d(small) == (125 - 2) * 256 * 2 * 128 * 2
    ws = S.WORKLOADS["srswa-40p-b32"]
    ss, sb = ws.replace(pages=2, batch=8), ws.replace(pages=125, batch=8)
    keys = lambda x: bench.algorithmic_bytes(x)["uocr_block_score"] / x.units
    assert abs((keys(sb) - keys(ss)) - (sb.n_blocks - ss.n_blocks) * 128) <= 8 * (sb.n_blocks - ss.n_blocks)
    sd = lambda x: bench.algorithmic_bytes(x)["uocr_srswa_decode"] / x.units
    assert sd(sb) == sd(ss)


# bytes per unit per step: append 1,024 B; dense decode q + 2 (m + w) D 2 + out;
# sparse decode q + selection + 2 (512 + w) D 2 + out = 328,320 B
@pytest.mark.parametrize("name,per_unit,kernel", [
    ("dense-10p-b64", 1_394_176, None),            # 2720 tokens per unit
    ("dense-1p-b512", 214_528, None),              # 416 tokens
    ("dense-40p-b32", 5_309_952, None),            # 10368 tokens
    ("dense-125p-b8", 16_451_072, None),           # 32128 tokens
    ("srswa-40p-b32", 328_320, "uocr_srswa_decode"),
    ("srswa-125p-b8", 328_320, "uocr_srswa_decode"),
])
def test_algorithmic_bytes_follow_the_per_unit_figures(name, per_unit, kernel):
    w = S.WORKLOADS[name]
    b = bench.algorithmic_bytes(w)   # every selected block counted (the nominal figure)
    got = b[kernel] if kernel else b["uocr_ring_append"] + b["uocr_rswa_decode"]
    assert abs(got / w.units - per_unit) <= 2.0, (name, got / w.units, per_unit)


def test_sparse_full_step_bytes():
    """Full SR-SWA step at 40 pages: 372,992 B per unit (119.4 MB per step),
    within the accounting of the score round trip (nb x 4 B written, then read)."""
    w = S.WORKLOADS["srswa-40p-b32"]
    b = bench.algorithmic_bytes(w)
    step = sum(b.values())
    assert abs(step / w.units - 372_992) / 372_992 < 2e-3
    assert abs(step / 1e6 - 119.4) < 0.3


def test_counters_and_profiles_belong_to_this_kernel_source():
    """The HBM traffic bench.py reports and the rocprofv3 summaries under
    profiles/ name the kernel source they were taken on (a sha256 prefix of
    uocr_kernels.hip); they must name the one in the tree, so that an edit of
    the kernels is followed by new measurements."""
    h = bench.kernel_source_hash()
    assert bench.COUNTER_TRAFFIC and all(rec[0] == h for rec in bench.COUNTER_TRAFFIC.values())
    prof = os.path.join(ROOT, "profiles")
    names = sorted(f for f in os.listdir(prof) if f.endswith(".txt"))
    assert names
    for f in names:
        with open(os.path.join(prof, f)) as fh:
            assert f"kernel source sha256[:16]: {h}" in fh.read(), f
