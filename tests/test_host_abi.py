"""Host-side checks of libhsakv's C ABI: no GPU needed, nothing is launched.

Every call here fails validation on the host (or is a pure helper), so no
kernel is ever enqueued.
"""

import ctypes
import re
import os
import subprocess

import pytest

hs = pytest.importorskip("block_sparse_rank_amd.hsakv")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20          # 16-byte aligned stand-in address; never dereferenced here


def _dims(**over):
    base = dict(H=12, d=128, Lq=4680, tokens_per_frame=1560, Psize=8, P=32, Kp=4, Binter=128,
                Bintra=64, Bq=64, r=256, dtype="bf16")
    base.update(over)
    return hs.make_dims(**base)


def test_header_declares_exactly_the_exports():
    with open(os.path.join(ROOT, "include", "hsakv.h")) as f:
        hdr = f.read()
    declared = set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", hdr, re.M))
    assert declared == set(hs.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", hs.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert declared <= exported
    for name in declared:
        assert hasattr(hs._lib, name)


def test_version_and_status_strings():
    assert hs.version() == 1
    for code in range(-8, 1):
        assert hs.status_str(code) and hs.status_str(code) != "unknown status"
    assert hs.status_str(-99) == "unknown status"
    assert hs._lib.hsakv_last_hip_error() == 0


@pytest.mark.parametrize("name", ["tiny", "wan1.3b-480p", "wan1.3b-480p-60s", "wan14b-480p",
                                  "wan14b-720p-90s"])
def test_workloads_validate(name):
    import synth
    s = synth.shape(name)
    d = hs.make_dims(H=s.H, d=s.d, Lq=s.Lq, tokens_per_frame=s.tokens_per_frame, Psize=s.Psize,
                     P=s.P, Kp=s.Kp, Binter=s.Binter, Bintra=s.Bintra, Bq=s.Bq, r=s.r,
                     dtype=s.dtype)
    assert hs.validate(d) == hs.OK
    for e in (hs.ENTRY_GATHER, hs.ENTRY_SELECT, hs.ENTRY_SPARSE, hs.ENTRY_LINEAR, hs.ENTRY_FORWARD):
        assert hs.workspace_bytes(d, e) > 0
        assert hs.workspace_bytes(d, e) % 256 == 0
    assert hs.workspace_bytes(d, 99) == 0


@pytest.mark.parametrize("over,code", [
    (dict(dtype=7), hs.ERR_BAD_DTYPE),
    (dict(H=0), hs.ERR_BAD_DIMS),
    (dict(Lq=0), hs.ERR_BAD_DIMS),
    (dict(Kp=0), hs.ERR_BAD_DIMS),
    (dict(P=-1), hs.ERR_BAD_DIMS),
    (dict(d=96), hs.ERR_UNSUPPORTED),
    (dict(Bq=32), hs.ERR_UNSUPPORTED),
    (dict(Binter=100), hs.ERR_UNSUPPORTED),
    (dict(Bintra=1024), hs.ERR_UNSUPPORTED),
    (dict(r=100), hs.ERR_UNSUPPORTED),
    (dict(Kp=65), hs.ERR_UNSUPPORTED),
    (dict(H=300, d=64), hs.ERR_UNSUPPORTED),
    (dict(tokens_per_frame=1 << 28), hs.ERR_BAD_DIMS),
    (dict(Kp=44), hs.ERR_UNSUPPORTED),            # NB_max above 4096
])
def test_validation_errors(over, code):
    d = _dims(**over)
    assert hs.validate(d) == code
    assert hs.workspace_bytes(d, hs.ENTRY_FORWARD) == 0


def test_null_dims():
    assert hs._lib.hsakv_validate(None) == hs.ERR_NULL_ARG


def _expect(code, fn, *args, **kw):
    with pytest.raises(hs.HsakvError) as ei:
        fn(*args, **kw)
    assert ei.value.status == code


def test_entry_points_reject_before_launch():
    d = _dims()
    H = d.H
    # bad dims first
    _expect(hs.ERR_UNSUPPORTED, hs.hkv_page_summary, _dims(d=96), FAKE, FAKE, stream=0)
    # null pointers
    _expect(hs.ERR_NULL_ARG, hs.hkv_page_summary, d, None, FAKE, stream=0)
    _expect(hs.ERR_NULL_ARG, hs.hkv_gather, d, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None,
            FAKE, None, stream=0)
    # misalignment
    _expect(hs.ERR_MISALIGNED, hs.hkv_page_summary, d, FAKE + 2, FAKE, stream=0)
    _expect(hs.ERR_MISALIGNED, hs.hsa_fuse, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8, stream=0)
    # tau outside (0, 1], NaN included
    for bad in (0.0, 1.5, float("nan"), -0.2):
        tau = [0.5] * H
        tau[3] = bad
        _expect(hs.ERR_BAD_TAU, hs.hsa_select, d, FAKE, FAKE, FAKE, FAKE, tau, FAKE, FAKE,
                stream=0)
    # workspace missing, too small, misaligned
    st = hs._lib.hkv_gather(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE,
                            FAKE, None, 0, None)
    assert st == hs.ERR_WORKSPACE
    need = hs.workspace_bytes(d, hs.ENTRY_GATHER)
    st = hs._lib.hkv_gather(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE, need - 1, None)
    assert st == hs.ERR_WORKSPACE
    st = hs._lib.hkv_gather(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE + 16, need, None)
    assert st == hs.ERR_WORKSPACE
    # forward: null struct members
    _expect(hs.ERR_NULL_ARG, hs.hsa_forward, d, [0.5] * H, 0, {"q": FAKE}, {"out": FAKE}, None,
            stream=0)
    # no launch happened, so no HIP error was recorded
    assert hs._lib.hsakv_last_hip_error() == 0


def test_python_binding_fails_loudly_without_library(tmp_path):
    """The binding raises at import when libhsakv.so is absent (no fallback path)."""
    import shutil
    import sys
    pkg = tmp_path / "block_sparse_rank_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "block_sparse_rank_amd", "hsakv.py"), pkg / "hsakv.py")
    (pkg / "__init__.py").write_text("")
    code = "import block_sparse_rank_amd.hsakv"
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode != 0 and "not built" in r.stderr
