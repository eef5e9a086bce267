"""The allocation-free sparse attention (hsa_sparse_attn_static) against the
workspace entry point hsa_sparse_attn, through the C ABI, on the same inputs:
the results are equal bit for bit. Calls follow one another on one GPU, the
later ones on smaller inputs, so each runs over the scratch contents its
predecessor left behind. Where the workspace entry gives each work-group
several split ranges (more than 8 heads, more than 1024 tiles per group),
the allocation-free entry keeps one: both are then compared with the oracle."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from block_sparse_rank_amd import hsakv as hs  # noqa: E402
from gpu_util import Case, compare, dev, host, pack_selection  # noqa: E402


def _both(c):
    _, n_sel, k_hist, v_hist = c.gather(c.page_summary())
    cnt, idx, _, _ = c.select(k_hist, n_sel)
    ref = c.sparse(k_hist, v_hist, n_sel, cnt, idx)
    s = c.s
    got = torch.full((s.Lq, s.H, s.d), float("nan"), dtype=torch.float32, device="cuda")
    hs.hsa_sparse_attn_static(c.d, c.t["q"], k_hist, v_hist, c.t["k_intra"], c.t["v_intra"], n_sel,
                              cnt, idx, got)
    torch.cuda.synchronize()
    return host(ref), host(got)


def test_static_scratch_equals_workspace_entry_on_shrinking_inputs():
    shapes = [
        synth.shape("wan1.3b-480p"),
        synth.shape("tiny").with_(dtype="bf16", clustered=True, tau_law="uniform", seed=7),
        synth.shape("tiny").with_(dtype="bf16", H=3, d=64, Lq=77, tokens_per_frame=25, Psize=4,
                                  clustered=True, tau_law="uniform", seed=19),
        synth.shape("tiny"),                                   # float32 path
    ]
    sizes = [hs.workspace_bytes(_dims(s), hs.ENTRY_SPARSE) for s in shapes]
    assert sizes[0] > sizes[1] >= sizes[2]
    for s in shapes:
        print(f"[static] {s.name} {s.dtype} H={s.H} Lq={s.Lq}", flush=True)
        ref, got = _both(Case(s))
        assert np.all(np.isfinite(got))
        assert ref.tobytes() == got.tobytes(), s.name


def test_static_one_range_and_workspace_two_ranges_both_match_the_oracle():
    # nine heads, 1032 tiles per group: hsa_sparse_attn runs two split ranges
    # per work-group, hsa_sparse_attn_static one (its partials stay in scratch)
    s = synth.shape("tiny").with_(dtype="bf16", H=9, d=64, Lq=512, tokens_per_frame=2048, Kp=4, P=6,
                                  Binter=64, r=64, clustered=True, tau_law="uniform", seed=35)
    d = _dims(s)
    assert hs.workspace_bytes(d, hs.ENTRY_SPARSE) > hs.workspace_bytes(d, hs.ENTRY_SPARSE_STATIC)
    assert hs.workspace_bytes(d, hs.ENTRY_SPARSE_STATIC) <= hs.STATIC_SCRATCH_BYTES
    print(f"[static] {s.name} bf16 H={s.H} Lq={s.Lq} Kp={s.Kp} Tp={s.Tp}", flush=True)
    c = Case(s)
    ref = c.oracle()
    _, n_sel, k_hist, v_hist = c.gather(c.page_summary())
    cnt, idx = (dev(x) for x in pack_selection(ref["sel"], c.d.NB_max))
    o_ws = host(c.sparse(k_hist, v_hist, n_sel, cnt, idx))
    o_st = torch.full((s.Lq, s.H, s.d), float("nan"), dtype=torch.float32, device="cuda")
    hs.hsa_sparse_attn_static(c.d, c.t["q"], k_hist, v_hist, c.t["k_intra"], c.t["v_intra"], n_sel,
                              cnt, idx, o_st)
    torch.cuda.synchronize()
    o_st = host(o_st)
    assert np.all(np.isfinite(o_st))
    compare("o_sparse(workspace entry, two ranges)", o_ws, ref["o_sparse"], s.dtype)
    compare("o_sparse(static entry, one range)", o_st, ref["o_sparse"], s.dtype)


def _dims(s):
    return hs.make_dims(H=s.H, d=s.d, Lq=s.Lq, tokens_per_frame=s.tokens_per_frame, Psize=s.Psize,
                        P=s.P, Kp=s.Kp, Binter=s.Binter, Bintra=s.Bintra, Bq=s.Bq, r=s.r,
                        dtype=s.dtype)
