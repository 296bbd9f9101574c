"""The C ABI on the CPU: the library loads, exports every entry point the
header declares, and rejects invalid arguments with the documented status
before launching anything.  No kernel runs here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from long_context_decode_attn_amd import uocr as U
    try:
        return U, U.load_library()
    except RuntimeError as e:  # not built in this checkout
        pytest.skip(str(e))


def _declared():
    """Every function name declared in include/*.h."""
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(uocr_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    U, lib = _lib()
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(U.EXPORTED) == names


def test_version_and_status_strings():
    U, lib = _lib()
    assert U.uocr_version() == 10000
    for code in range(0, -8, -1):
        assert U.uocr_status_string(code) not in ("", "unknown status")
    assert U.uocr_status_string(-99) == "unknown status"


def _shape(U, **kw):
    base = dict(batch=2, heads=3, head_dim=128, prefix_cap=320, window=128, dtype=1, scale=0.088)
    base.update(kw)
    return U._Shape(**base)


FAKE = ctypes.c_void_p(0x10000)       # 16-byte aligned, never dereferenced
ODD = ctypes.c_void_p(0x10004)


def _rswa(lib, sh, q=FAKE, ws=None, wsb=0, splits=1, out=FAKE):
    return lib.uocr_rswa_decode(ctypes.byref(sh), q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, out, ws, wsb, splits, None)


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 7, -3), ("batch", 0, -2), ("heads", -1, -2), ("head_dim", 96, -6), ("prefix_cap", -1, -2),
    ("prefix_cap", (1 << 20) + 1, -2), ("window", 0, -2), ("window", 1025, -2), ("scale", float("inf"), -2),
])
def test_shape_validation(field, value, status):
    U, lib = _lib()
    sh = _shape(U, **{field: value})
    assert _rswa(lib, sh) == status
    assert U.uocr_last_error()


def test_null_alignment_and_workspace_errors():
    U, lib = _lib()
    sh = _shape(U)
    assert lib.uocr_rswa_decode(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 1, None) == -1
    assert _rswa(lib, sh, q=None) == -1
    assert _rswa(lib, sh, q=ODD) == -5
    assert _rswa(lib, sh, out=ODD) == -5
    # more than one split needs a workspace of the queried size
    need = lib.uocr_rswa_workspace_bytes(ctypes.byref(sh), 4)
    assert need > 0
    assert _rswa(lib, sh, splits=4) == -1
    assert _rswa(lib, sh, splits=4, ws=FAKE, wsb=need - 1) == -4
    assert _rswa(lib, sh, splits=-1) == -2
    assert lib.uocr_rswa_workspace_bytes(ctypes.byref(sh), 1) == 0


def test_route_validation():
    U, lib = _lib()
    sh = _shape(U)
    for block, idx, k, status in [(16, 32, 16, -6), (32, 64, 16, -6), (32, 32, 0, -2), (32, 32, 65, -2)]:
        r = U._Route(block, idx, k)
        assert lib.uocr_block_score(ctypes.byref(sh), ctypes.byref(r), FAKE, FAKE, FAKE, FAKE, FAKE, None) == status
        assert lib.uocr_entmax15_topk(ctypes.byref(sh), ctypes.byref(r), FAKE, FAKE, FAKE, None, FAKE, None) == status
    big = _shape(U, prefix_cap=4097 * 32)
    r = U._Route(32, 32, 16)
    assert lib.uocr_entmax15_topk(ctypes.byref(big), ctypes.byref(r), FAKE, FAKE, FAKE, None, FAKE, None) == -6
    def srswa(route, sel=FAKE, ws=None, wsb=0, splits=1):
        return lib.uocr_srswa_decode(ctypes.byref(sh), route, FAKE, FAKE, FAKE, FAKE, sel, None, FAKE, FAKE, FAKE,
                                     FAKE, ws, wsb, splits, None)
    assert srswa(None) == -1
    assert srswa(ctypes.byref(r), sel=None) == -1
    assert srswa(ctypes.byref(r), splits=-1) == -2
    # several workgroups per unit need the workspace uocr_srswa_workspace_bytes gives
    need = lib.uocr_srswa_workspace_bytes(ctypes.byref(sh), ctypes.byref(r), 4)
    assert need == U.uocr_srswa_workspace_bytes(U.Shape(2, 3, 128, 320), U.Route(), 4) > 0
    assert lib.uocr_srswa_workspace_bytes(ctypes.byref(sh), ctypes.byref(r), 1) == 0
    assert lib.uocr_srswa_splits(ctypes.byref(sh), ctypes.byref(r), 0) == 8      # 6 units: about 256 workgroups
    assert srswa(ctypes.byref(r), splits=4) == -1
    assert srswa(ctypes.byref(r), ws=FAKE, wsb=need - 1, splits=4) == -4
    assert srswa(ctypes.byref(r), ws=ODD, wsb=need, splits=4) == -5
    assert lib.uocr_ring_append(ctypes.byref(sh), FAKE, FAKE, FAKE, ODD, FAKE, None) == -5
    assert lib.uocr_block_index_build(ctypes.byref(sh), ctypes.byref(r), FAKE, FAKE, None, FAKE, None) == -1


def test_prefill_route_validation():
    U, lib = _lib()
    sh = _shape(U)
    r = U._Route(32, 32, 16)
    call = lambda tq, q=FAKE, qpos=FAKE, idx=FAKE: lib.uocr_prefill_route(
        ctypes.byref(sh), ctypes.byref(r), q, tq, qpos, FAKE, FAKE, FAKE, idx, None, FAKE, None)
    assert call(-1) == -2
    assert call((1 << 20) + 1) == -2
    assert call(0, q=None, qpos=None, idx=None) == 0      # nothing to do, nothing launched
    assert call(8, q=None) == -1
    assert call(8, qpos=None) == -1
    assert call(8, q=ODD) == -5
    big = _shape(U, batch=4096, heads=64)
    assert lib.uocr_prefill_route(ctypes.byref(big), ctypes.byref(r), FAKE, 4096, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  None, FAKE, None) == -2    # outputs beyond 2^31 entries


def test_ngram_ban_validation():
    U, lib = _lib()
    call = lambda **kw: lib.uocr_ngram_ban(*[kw.get(k, d) for k, d in [
        ("batch", 2), ("tokens", FAKE), ("ring_cap", 128), ("n_gen", FAKE), ("page_tokens", FAKE), ("ngram", 35),
        ("window", 128), ("page_token", 7), ("eos_token", 1), ("max_page_tokens", 0), ("logits", FAKE),
        ("vocab", 1000), ("dtype", 0), ("stream", None)]])
    assert call(window=129) == -2              # ring shorter than the window
    assert call(window=0) == -2
    assert call(window=4097, ring_cap=5000) == -2
    assert call(ngram=0) == -2
    assert call(dtype=5) == -3
    assert call(max_page_tokens=10, page_tokens=None) == -1
    assert call(max_page_tokens=10, page_token=1000) == -2
    assert call(tokens=None) == -1
    assert call(logits=ctypes.c_void_p(0x10002)) == -5  # float32 logits need 4-byte alignment
    assert call(batch=0, tokens=None, n_gen=None, logits=None) == 0


def test_block_index_range_validation():
    U, lib = _lib()
    sh, r = _shape(U), U._Route(32, 32, 16)          # prefix_cap 320: nb_cap 10

    def call(first, last, k=FAKE, kbar=FAKE):
        return lib.uocr_block_index_range(ctypes.byref(sh), ctypes.byref(r), k, FAKE, FAKE, kbar, first, last, None)

    assert call(-1, 4) == -2
    assert call(5, 4) == -2
    assert call(0, 11) == -2
    assert call(3, 3, k=None, kbar=None) == 0      # empty range: nothing to do
    assert call(0, 10, k=None) == -1
    assert call(2, 7, kbar=ODD) == -5
    assert lib.uocr_block_index_range(None, ctypes.byref(r), FAKE, FAKE, FAKE, FAKE, 0, 1, None) == -1


def test_rope_page2d_validation():
    U, lib = _lib()
    sh = _shape(U)

    def call(sh=sh, x=FAKE, y=None, tokens=64, page=FAKE, offset=FAKE, page_mod=2, base=10000.0):
        return lib.uocr_rope_page2d(ctypes.byref(sh), x, y, tokens, page, offset, page_mod, base, None)

    assert call(tokens=-1) == -2
    assert call(tokens=(1 << 20) + 1) == -2
    assert call(page_mod=-1) == -2
    assert call(base=0.0) == -2
    assert call(base=float("nan")) == -2
    assert call(base=float("inf")) == -2
    assert call(x=None) == -1
    assert call(page=None) == -1
    assert call(offset=None) == -1
    assert call(x=ODD) == -5                    # rows are read as 16-byte chunks
    assert call(y=ODD) == -5
    assert call(y=FAKE) == -2                   # y is x
    assert call(page=ctypes.c_void_p(0x10002)) == -5
    assert call(sh=_shape(U, head_dim=96)) == -6
    assert call(sh=_shape(U, dtype=3)) == -3
    assert call(tokens=0, x=None, page=None, offset=None) == 0   # nothing to do
    assert lib.uocr_rope_page2d(None, FAKE, None, 4, FAKE, FAKE, 2, 10000.0, None) == -1


def test_split_geometry():
    U, lib = _lib()
    for B, H, m in [(64, 10, 2592), (512, 10, 288), (1, 2, 528), (32, 10, 10240), (8, 10, 32000), (1, 1, 0)]:
        sh = U.Shape(B, H, 128, m)
        S = U.uocr_rswa_splits(sh)
        assert 1 <= S <= max(1, -(-(m + 128) // 32))
        assert U.uocr_rswa_splits(sh, 10 ** 6) <= -(-(m + 128) // 16)
    # sparse decode: workgroups per unit, enough for ~256 workgroups when the
    # units alone do not fill the chip
    r = U.Route()
    assert U.uocr_srswa_splits(U.Shape(8, 10, 128, 32000), r) == 4       # 80 units -> 320 workgroups
    assert U.uocr_srswa_splits(U.Shape(32, 10, 128, 10240), r) == 1      # 320 units
    assert U.uocr_srswa_splits(U.Shape(1, 2, 128, 528), r) == 8          # at most 8 per unit
    assert U.uocr_srswa_splits(U.Shape(8, 10, 128, 32000), r, 1) == 1
    assert U.uocr_srswa_splits(U.Shape(8, 10, 128, 32000), r, 99) == 64


def test_product_path_has_no_oracle_or_fallback():
    """Nothing in the package imports the oracle, and the binding has no
    CPU path: every compute function goes through libuocr.so."""
    pkg = os.path.join(ROOT, "long_context_decode_attn_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "uocr_oracle" not in text, f


def test_static_workspace_refuses_a_split_count_that_does_not_fit():
    """uocr_rswa_decode_static: an explicit split count whose partials exceed
    the library's static workspace is refused before anything is launched."""
    U, lib = _lib()
    sh = U._Shape(1 << 14, 64, 128, 1 << 17, 128, 1, 0.088)   # 2^20 units x 16 splits: 8 GiB of partials
    rc = lib.uocr_rswa_decode_static(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert rc == -4, rc
    assert "static" in lib.uocr_last_error().decode()
    # invalid arguments are refused as by uocr_rswa_decode
    assert lib.uocr_rswa_decode_static(ctypes.byref(_shape(U)), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                                       None) == -1
    assert lib.uocr_rswa_decode_static(ctypes.byref(_shape(U)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1,
                                       None) == -2


def test_phase_stamps_only_in_the_stamping_library():
    """uocr_phase_stamps: libuocr.so records no stamps and says so (before
    any HIP call); libuocr_stamps.so, built from the same sources with the
    stamps compiled in, exports the same entry points."""
    import numpy as np
    U, lib = _lib()
    buf = np.zeros((4, 64), dtype=np.uint64)
    p = ctypes.c_void_p(buf.ctypes.data)
    assert lib.uocr_phase_stamps(None, 4, None) == -1
    assert lib.uocr_phase_stamps(p, 0, None) == -2
    assert lib.uocr_phase_stamps(p, 4097, None) == -2
    assert lib.uocr_phase_stamps(p, 4, None) == -6
    assert "libuocr_stamps.so" in lib.uocr_last_error().decode()
    if not os.path.exists(U.STAMPS_LIB_PATH):
        pytest.skip("libuocr_stamps.so is not built in this checkout")
    stamped = ctypes.CDLL(U.STAMPS_LIB_PATH)
    for n in _declared():
        assert hasattr(stamped, n), n
