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


def _shape_dims(name):
    import synth
    s = synth.shape(name)
    return hs.make_dims(H=s.H, d=s.d, Lq=s.Lq, tokens_per_frame=s.tokens_per_frame, Psize=s.Psize, P=s.P,
                        Kp=s.Kp, Binter=s.Binter, Bintra=s.Bintra, Bq=s.Bq, r=s.r, dtype=s.dtype)


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
    assert hs.version() == 6
    for code in range(-9, 1):
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
    for e in (hs.ENTRY_GATHER, hs.ENTRY_SELECT, hs.ENTRY_SPARSE, hs.ENTRY_LINEAR, hs.ENTRY_FORWARD,
              hs.ENTRY_SUMMARY, hs.ENTRY_COMMIT):
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
    # E and F past 2^31 bytes (32-bit byte offsets in the projection):
    # r = 1024, L = 8 * 131072 + 64 columns of bf16
    (dict(r=1024, Kp=8, tokens_per_frame=16384, Binter=512, Lq=64), hs.ERR_UNSUPPORTED),
])
def test_validation_errors(over, code):
    d = _dims(**over)
    assert hs.validate(d) == code
    assert hs.workspace_bytes(d, hs.ENTRY_FORWARD) == 0


def test_projection_byte_limit_boundary():
    """r * L * 2 bytes just below 2^31 validates; the first r above does not."""
    d = _dims(r=992, Kp=8, tokens_per_frame=16384, Binter=512, Lq=64)
    assert 992 * d.L * 2 < 2 ** 31 and hs.validate(d) == hs.OK
    d = _dims(r=1024, Kp=8, tokens_per_frame=16384, Binter=512, Lq=64)
    assert 1024 * d.L * 2 >= 2 ** 31 and hs.validate(d) == hs.ERR_UNSUPPORTED


def test_static_sparse_rejects_what_exceeds_its_scratch():
    """The allocation-free attention refuses dims whose plan and partials
    need more than its fixed scratch, on the host, before any launch."""
    big = _dims(H=96, Lq=10800, tokens_per_frame=3600, Kp=6, r=512)
    assert hs.validate(big) == hs.OK
    assert hs.workspace_bytes(big, hs.ENTRY_SPARSE_STATIC) > hs.STATIC_SCRATCH_BYTES
    _expect(hs.ERR_TOO_LARGE, hs.hsa_sparse_attn_static, big, *([FAKE] * 9), stream=0)
    d13, d720 = (_shape_dims(n) for n in ("wan1.3b-480p", "wan14b-720p-90s"))
    for d in (d13, d720):
        assert hs.workspace_bytes(d, hs.ENTRY_SPARSE_STATIC) <= hs.STATIC_SCRATCH_BYTES
    # 1.3B 480p: one split range per work-group on both entry points; the
    # 720p 40-head shape gives hsa_sparse_attn five ranges per work-group
    # (more partials) while the allocation-free entry keeps one
    assert hs.workspace_bytes(d13, hs.ENTRY_SPARSE) == hs.workspace_bytes(d13, hs.ENTRY_SPARSE_STATIC)
    assert hs.workspace_bytes(d720, hs.ENTRY_SPARSE) > hs.workspace_bytes(d720, hs.ENTRY_SPARSE_STATIC)
    assert hs._lib.hsakv_last_hip_error() == 0


def test_page_commit_rejects_before_launch():
    d = _dims(P=2)
    Tp = d.Tp
    _expect(hs.ERR_BAD_DIMS, hs.hkv_page_commit, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 2 * Tp - 5, 0,
            stream=0)
    _expect(hs.ERR_BAD_DIMS, hs.hkv_page_commit, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 0, 0, stream=0)
    _expect(hs.ERR_BAD_DIMS, hs.hkv_page_commit, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, -3, 0, stream=0)
    _expect(hs.ERR_NULL_ARG, hs.hkv_page_commit, d, FAKE, FAKE, FAKE, FAKE, None, FAKE, 10, 0, 0, stream=0)
    _expect(hs.ERR_MISALIGNED, hs.hkv_page_commit, d, FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 0, 0,
            stream=0)
    # nothing to commit: returns at once, nothing enqueued
    assert hs._lib.hkv_page_commit(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, 0, 5, 0, None, 0,
                                   None) == 0
    # a commit that completes a page needs the page-mean scratch
    need = hs.workspace_bytes(d, hs.ENTRY_COMMIT)
    assert need >= 32 * d.H * d.d * 4
    for ws_ptr, nbytes in ((None, 0), (FAKE, 32 * d.H * d.d * 4 - 1), (FAKE + 16, need)):
        st = hs._lib.hkv_page_commit(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, Tp - 50, 0,
                                     ws_ptr, nbytes, None)
        assert st == hs.ERR_WORKSPACE
    st = hs._lib.hkv_page_summary(ctypes.byref(d), FAKE, FAKE, FAKE, hs.workspace_bytes(d, hs.ENTRY_SUMMARY) - 1,
                                  None)
    assert st == hs.ERR_WORKSPACE
    assert hs._lib.hsakv_last_hip_error() == 0


def test_sparse_plan_and_compute_reject_before_launch():
    d = _dims()
    need = hs.workspace_bytes(d, hs.ENTRY_SPARSE)
    assert hs._lib.hsa_sparse_plan(ctypes.byref(_dims(dtype="f32")), FAKE, FAKE, FAKE, FAKE, need, None) == \
        hs.ERR_BAD_DTYPE
    assert hs._lib.hsa_sparse_plan(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, need - 1, None) == hs.ERR_WORKSPACE
    assert hs._lib.hsa_sparse_plan(ctypes.byref(d), None, FAKE, FAKE, FAKE, need, None) == hs.ERR_NULL_ARG
    assert hs._lib.hsa_sparse_compute(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16,
                                      need, None) == hs.ERR_WORKSPACE
    assert hs._lib.hsa_sparse_compute(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                      need, None) == hs.ERR_NULL_ARG
    assert hs._lib.hsakv_last_hip_error() == 0


def test_backward_rejects_before_launch():
    d = _dims()
    need = hs.workspace_bytes(d, hs.ENTRY_BACKWARD)
    # gate partials, dO_l hi and lo, dK', dV' slice partials and hi / lo parts
    assert need >= 3 * d.Lq * d.H * 4 + 2 * d.Lq * d.H * d.d * 2 + 2 * d.r * d.H * d.d * 4
    args = [FAKE] * 17
    lib = hs._lib.hsa_backward_params
    assert lib(ctypes.byref(_dims(dtype="f32")), *args, FAKE, need, None, None) == hs.ERR_BAD_DTYPE
    assert lib(ctypes.byref(d), *args, FAKE, need - 1, None, None) == hs.ERR_WORKSPACE
    assert lib(ctypes.byref(d), *args, FAKE + 16, need, None, None) == hs.ERR_WORKSPACE
    for i in range(17):
        a = list(args)
        a[i] = None
        assert lib(ctypes.byref(d), *a, FAKE, need, None, None) == hs.ERR_NULL_ARG, i
    a = list(args)
    a[8] = FAKE + 4      # k_low
    assert lib(ctypes.byref(d), *a, FAKE, need, None, None) == hs.ERR_MISALIGNED
    a = list(args)
    a[6] = FAKE + 4      # w_g is read 16 bytes at a time
    assert lib(ctypes.byref(d), *a, FAKE, need, None, None) == hs.ERR_MISALIGNED
    assert lib(ctypes.byref(_dims(d=96)), *args, FAKE, need, None, None) == hs.ERR_UNSUPPORTED
    # key rows of 2^31 bytes or more: (Kp Tp + Lq) H d 2 = (8 * 16384 + 4680) * 8192 * 2
    big = _dims(H=64, Kp=8, tokens_per_frame=2048, Binter=512, r=32)
    assert hs.validate(big) == hs.OK
    assert lib(ctypes.byref(big), *args, FAKE, hs.workspace_bytes(big, hs.ENTRY_BACKWARD), None, None) == \
        hs.ERR_UNSUPPORTED
    # a fork with a stream needs both events
    half = hs.Fork()
    half.stream = FAKE
    assert lib(ctypes.byref(d), *args, FAKE, need, None, ctypes.byref(half)) == hs.ERR_NULL_ARG
    assert hs._lib.hsakv_last_hip_error() == 0


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
    st = hs._lib.hkv_gather(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, None, None, FAKE, FAKE, FAKE, FAKE,
                            FAKE, None, 0, None)
    assert st == hs.ERR_WORKSPACE
    need = hs.workspace_bytes(d, hs.ENTRY_GATHER)
    st = hs._lib.hkv_gather(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, None, None, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE, need - 1, None)
    assert st == hs.ERR_WORKSPACE
    st = hs._lib.hkv_gather(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, None, None, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE + 16, need, None)
    assert st == hs.ERR_WORKSPACE
    # forward: null struct members
    _expect(hs.ERR_NULL_ARG, hs.hsa_forward, d, [0.5] * H, 0, {"q": FAKE}, {"out": FAKE}, None,
            stream=0)
    # forward: a fork with a stream but no events
    full = {n: FAKE for n, _ in hs.Inputs._fields_}
    half_fork = hs.Fork(FAKE, None, None)
    _expect(hs.ERR_NULL_ARG, hs.hsa_forward, d, [0.5] * H, 0, full, {"out": FAKE}, None,
            stream=0, fork=half_fork)
    # forward: every argument valid but the workspace one byte short, or
    # misaligned: rejected on the host, nothing is enqueued
    need = hs.workspace_bytes(d, hs.ENTRY_FORWARD)
    for ws_ptr, nbytes in ((FAKE, need - 1), (FAKE + 16, need), (None, need)):
        st = hs._lib.hsa_forward(ctypes.byref(d), ctypes.cast(hs._host_f32([0.5] * H), ctypes.c_void_p),
                                 0, None, None, ctypes.byref(hs.Inputs(*[FAKE] * len(hs.Inputs._fields_))),
                                 ctypes.byref(hs.Outputs(FAKE)), ws_ptr, nbytes, None, None)
        assert st == hs.ERR_WORKSPACE
    # an unknown retrieval policy
    _expect(hs.ERR_UNSUPPORTED, hs.hsa_forward, d, [0.5] * H, 0, full, {"out": FAKE}, None, stream=0,
            policy=9)
    _expect(hs.ERR_UNSUPPORTED, hs.hkv_gather, d, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE,
            None, stream=0, policy=-1)
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
