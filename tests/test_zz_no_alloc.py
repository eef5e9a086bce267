"""The allocation-free sparse attention (hsa_sparse_attn_static) against the
workspace entry point hsa_sparse_attn, through the C ABI, on the same inputs:
the results are equal bit for bit. Calls follow one another on one GPU, the
later ones on smaller inputs, so each runs over the scratch contents its
predecessor left behind."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from block_sparse_rank_amd import hsakv as hs  # noqa: E402
from gpu_util import Case, host  # noqa: E402


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


def _dims(s):
    return hs.make_dims(H=s.H, d=s.d, Lq=s.Lq, tokens_per_frame=s.tokens_per_frame, Psize=s.Psize,
                        P=s.P, Kp=s.Kp, Binter=s.Binter, Bintra=s.Bintra, Bq=s.Bq, r=s.r,
                        dtype=s.dtype)
