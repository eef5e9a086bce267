"""The online softmax's running-max raise on inputs built to take it.

The attention kernels raise a row's running max only when a score passes it
by more than 8 (log2 units), and then rescale O and the row sum; on the
seeded workloads that branch is rare. Here the keys that come late in a
row's order are made several times larger, so that most rows (not all: the
raise is per query) take the branch after their first tiles:
  * the low-rank branch: the projection rows of the last 64 projected keys
    of E and F scaled by 4 (exact in bf16), the third tile's by 2;
  * the sparse branch: the chunk's own keys scaled by 4, so the chunk blocks
    (after the history blocks in a row's order) score far above the history.
Both are compared with the oracle on the same inputs (the sparse branch on
the oracle's own selection)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from gpu_util import Case, compare, dev, host, pack_selection  # noqa: E402


def _scaled(bits: np.ndarray, factor: float) -> np.ndarray:
    """bf16 bit patterns times a power of two (exact)."""
    return synth.round_bf16_bits(synth.bf16_bits_to_f32(bits) * np.float32(factor))


def _shape():
    return synth.shape("tiny").with_(dtype="bf16", H=2, d=128, r=256, Lq=200, tokens_per_frame=16, Kp=2, P=6,
                                     clustered=True, tau_law="uniform", seed=41)


def test_lowrank_attention_raises_running_max():
    s = _shape()
    ch = synth.draw_chunk(s)
    for name in ("E", "F"):
        m = ch[name].copy()
        m[128:192] = _scaled(m[128:192], 2.0)
        m[192:256] = _scaled(m[192:256], 4.0)
        ch[name] = m
    c = Case(s, chunk=ch)
    ref = c.oracle()
    _, n_sel, k_hist, v_hist = c.gather(c.page_summary())
    o, kl, _ = c.linear(k_hist, v_hist, n_sel)
    compare("k_low", host(kl), ref["k_low"], "f32", max_abs=2e-3, rel=1e-5)
    compare("o_linear", host(o), ref["o_linear"], s.dtype)


def test_sparse_attention_raises_running_max():
    s = _shape()
    ch = synth.draw_chunk(s)
    ch["k_intra"] = _scaled(ch["k_intra"], 4.0)
    c = Case(s, chunk=ch)
    ref = c.oracle()
    _, n_sel, k_hist, v_hist = c.gather(c.page_summary())
    cnt, idx = pack_selection(ref["sel"], c.d.NB_max)
    o = c.sparse(k_hist, v_hist, n_sel, dev(cnt), dev(idx))
    compare("o_sparse", host(o), ref["o_sparse"], s.dtype)
