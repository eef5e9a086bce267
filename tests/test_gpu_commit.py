"""GPU parity of the page commit (hkv_page_commit) and of a multi-chunk
rollout: each chunk's forward retrieves from the pages finalised so far,
then its own K/V are committed to the pool. Everything is compared with the
oracle doing the same sequence; pool rows bit for bit, page means within
float32 rounding (and bit for bit with hkv_page_summary of the same pages)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402
from block_sparse_rank_amd import hsakv as hs  # noqa: E402
from gpu_util import Case, compare, dev, dims_of, host  # noqa: E402


def _commit_case(s, P_cap, n, n_chunks, fill0, seed):
    """n_chunks commits of n tokens into an empty pool of P_cap pages,
    starting at history position fill0; GPU against the oracle."""
    rng = np.random.default_rng(seed)
    d = dims_of(s.with_(P=P_cap))
    st = np.uint16 if s.dtype == "bf16" else np.float32
    shape = (P_cap, s.Tp, s.H, s.d)
    pk, pv = np.zeros(shape, st), np.zeros(shape, st)
    km = np.full((P_cap, s.H, s.d), -7.0)
    pp = np.full(P_cap, -1, np.int32)
    tk, tv = dev(pk), dev(pv)
    tkm = dev(km.astype(np.float32))
    tpp = dev(pp)
    fill = fill0
    finalised = []
    for c in range(n_chunks):
        x = rng.standard_normal((2, n, s.H, s.d)).astype(np.float32)
        kc = synth.round_bf16_bits(x[0]) if s.dtype == "bf16" else x[0]
        vc = synth.round_bf16_bits(x[1]) if s.dtype == "bf16" else x[1]
        prompt = c % 3
        pk, pv, km, pp, done = oracle.page_commit(pk, pv, km, pp, kc, vc, fill, prompt)
        hs.hkv_page_commit(d, tk, tv, tkm, tpp, dev(kc), dev(vc), n, fill, prompt)
        fill += n
        finalised += done
    torch.cuda.synchronize()
    assert host(tk).tobytes() == pk.tobytes() and host(tv).tobytes() == pv.tobytes()
    assert host(tpp).tolist() == pp.tolist()
    got = host(tkm)
    untouched = [p for p in range(P_cap) if p not in finalised]
    assert np.all(got[untouched] == np.float32(-7.0))
    if finalised:
        compare("page_kmean(committed)", got[finalised], km[finalised], "f32", max_abs=1e-5, rel=1e-6)
        # the same bits as the page summary of the final pool
        ref = torch.empty((P_cap, s.H, s.d), dtype=torch.float32, device="cuda")
        hs.hkv_page_summary(d, tk, ref)
        assert host(ref)[finalised].tobytes() == got[finalised].tobytes()
    return finalised


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_commit_sequence_three_frame_chunks_into_eight_frame_pages(dtype):
    # pages of 8 frames, chunks of 3 frames (the pages' setting), 7 tokens per frame
    s = synth.shape("tiny").with_(dtype=dtype, H=2, d=64, tokens_per_frame=7, Psize=8)
    fin = _commit_case(s, P_cap=4, n=21, n_chunks=8, fill0=0, seed=1)
    assert fin == [0, 1, 2]


def test_commit_of_a_full_shape_chunk_into_480p_pages():
    """A Wan-1.3B 480p chunk (4680 tokens, 12 heads, d 128) committed across
    the end of a 12480-token page."""
    s = synth.shape("wan1.3b-480p")
    fin = _commit_case(s, P_cap=2, n=s.Lq, n_chunks=1, fill0=s.Tp - 1000, seed=2)
    assert fin == [0]


def test_commit_errors_leave_the_pool_untouched():
    s = synth.shape("tiny")
    d = dims_of(s.with_(P=2))
    pk = torch.zeros((2, s.Tp, s.H, s.d), device="cuda")
    km = torch.zeros((2, s.H, s.d), device="cuda")
    pp = torch.zeros(2, dtype=torch.int32, device="cuda")
    kc = torch.ones((10, s.H, s.d), device="cuda")
    with pytest.raises(hs.HsakvError) as ei:
        hs.hkv_page_commit(d, pk, pk, km, pp, kc, kc, 10, 2 * s.Tp - 5, 0)
    assert ei.value.status == hs.ERR_BAD_DIMS
    hs.hkv_page_commit(d, pk, pk, km, pp, kc, kc, 0, 7, 0)           # nothing to commit
    torch.cuda.synchronize()
    assert float(pk.abs().sum()) == 0.0 and float(km.abs().sum()) == 0.0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rollout_forward_then_commit(dtype):
    """Four chunks: each forward sees the pages finalised so far (dims P), then
    its chunk's keys and values are committed; retrieval, gathered rows and
    the output follow the oracle's rollout."""
    base = synth.shape("tiny").with_(dtype=dtype, clustered=dtype == "bf16",
                                     tau_law="uniform" if dtype == "bf16" else "alt")
    P0, P_cap = 4, 12
    s0 = base.with_(P=P0)
    pk0, pv0 = synth.draw_pool(s0)
    st = pk0.dtype
    pk = np.zeros((P_cap,) + pk0.shape[1:], st)
    pv = np.zeros_like(pk)
    pk[:P0], pv[:P0] = pk0, pv0
    pp = np.full(P_cap, -1, np.int32)
    pp[:P0] = synth.page_prompts(s0)
    km = np.zeros((P_cap, base.H, base.d))
    km[:P0] = np.stack([oracle.page_summary(oracle.as_f64(pk0[p], dtype)[None])[0] for p in range(P0)])
    d_cap = dims_of(base.with_(P=P_cap))
    tk, tv = dev(pk), dev(pv)
    tpp = dev(pp)
    tkm = torch.empty((P_cap, base.H, base.d), dtype=torch.float32, device="cuda")
    hs.hkv_page_summary(dims_of(base.with_(P=P0)), tk, tkm)
    fill = P0 * base.Tp
    for c in range(4):
        P = fill // base.Tp
        s = base.with_(P=P, seed=100 + c)
        ch = synth.draw_chunk(s)
        ch["page_prompt"] = pp[:P].copy()
        cur = 0
        ref = oracle.forward(dtype=dtype, q=ch["q"], k_intra=ch["k_intra"], v_intra=ch["v_intra"],
                             pool_k=pk[:P], pool_v=pv[:P], page_prompt=pp[:P], cur_prompt=cur, E=ch["E"],
                             F=ch["F"], w_g=ch["w_g"], b_g=ch["b_g"], tau=ch["tau"], Kp=s.Kp,
                             Binter=s.Binter, Bintra=s.Bintra, Bq=s.Bq, page_kmean=km[:P])
        c_gpu = Case(s, chunk=ch, pool=(pk[:P], pv[:P]), cur_prompt=cur)
        c_gpu.t["pool_k"], c_gpu.t["pool_v"], c_gpu.t["page_prompt"] = tk, tv, tpp
        outs = c_gpu.forward(tkm)
        n = int(host(outs["n_sel"])[0])
        assert n == ref["n_sel"] and host(outs["page_idx"])[:n].tolist() == ref["page_idx"].tolist()
        tol = dict(max_abs=2e-2, mean_abs=2e-3, rel=1e-2) if dtype == "bf16" else dict(max_abs=1e-4, rel=1e-5)
        compare(f"rollout out chunk {c}", oracle.as_f64(host(outs["out"]), dtype), ref["out"], "f32", **tol)
        # commit the chunk's own keys and values under the current prompt
        pk, pv, km, pp, done = oracle.page_commit(pk, pv, km, pp, ch["k_intra"], ch["v_intra"], fill, cur)
        hs.hkv_page_commit(d_cap, tk, tv, tkm, tpp, c_gpu.t["k_intra"], c_gpu.t["v_intra"], s.Lq, fill, cur)
        fill += s.Lq
        torch.cuda.synchronize()
        assert host(tpp).tolist() == pp.tolist()
        assert host(tk).tobytes() == pk.tobytes()
        compare(f"page_kmean after chunk {c}", host(tkm)[:fill // base.Tp], km[:fill // base.Tp], "f32",
                max_abs=1e-5, rel=1e-6)
