"""GPU parity, stage by stage, on tiny workloads and their edge cases.

Every stage runs through the C ABI (libhsakv.so) on cuda:0 and is compared
with the float64 oracle on the same seeded inputs. The sparse attention is
fed the oracle's own selection so that its output compares on identical
masks; the gate is fed the oracle's two branches.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402
from block_sparse_rank_amd import hsakv as hs  # noqa: E402
from gpu_util import (Case, check_selection, compare, dev, expected_sparse, host,  # noqa: E402
                      pack_selection, ws)


def _variant(name, **over):
    return synth.shape("tiny").with_(**over) if name == "tiny" else synth.shape(name, **over)


# (id, shape, extra Case kwargs). Shapes span several tiles and ragged tails.
VARIANTS = [
    ("tiny", _variant("tiny"), {}),
    ("tiny-bf16", _variant("tiny", dtype="bf16", clustered=True, tau_law="uniform", seed=7), {}),
    ("ragged-Lq200-Tp96", _variant("tiny", Lq=200, tokens_per_frame=12, seed=11), {}),
    ("odd-Lq77-Tp100", _variant("tiny", Lq=77, tokens_per_frame=25, Psize=4, seed=12), {}),
    ("one-page-match", _variant("tiny", P=3, seed=13), dict(page_prompt=[1, 0, 1])),
    ("no-page-match", _variant("tiny", seed=14), dict(cur_prompt=5)),
    ("H1-d128", _variant("tiny", H=1, d=128, seed=15), {}),
    ("bf16-d128-r64", _variant("tiny", dtype="bf16", d=128, H=3, r=64, Kp=3, P=8,
                               clustered=True, tau_law="uniform", seed=16), {}),
    ("kp4-binter256", _variant("tiny", Kp=4, P=8, Binter=256, Lq=130, seed=17), {}),
    ("bf16-one-page", _variant("tiny", dtype="bf16", P=3, clustered=True, tau_law="uniform",
                               seed=18), dict(page_prompt=[1, 0, 1])),
    ("bf16-odd-Lq77", _variant("tiny", dtype="bf16", Lq=77, tokens_per_frame=25, Psize=4,
                               clustered=True, tau_law="uniform", seed=19), {}),
    ("bf16-no-page", _variant("tiny", dtype="bf16", H=4, d=128, clustered=True,
                              tau_law="uniform", seed=20), dict(cur_prompt=9)),
    # low-rank projection with 256 x 256 tiles (r >= 128, H*d a multiple of 256):
    # rows past r inside a tile, a split whose history and chunk parts both end in partial 64-key steps
    ("bf16-r128-seam", _variant("tiny", dtype="bf16", H=2, d=128, r=128, Lq=200, tokens_per_frame=13,
                                clustered=True, tau_law="uniform", seed=25), {}),
    # two row tiles, the second ragged
    ("bf16-r320-hd256", _variant("tiny", dtype="bf16", H=4, d=64, r=320, Lq=136, tokens_per_frame=13,
                                 P=8, Kp=3, clustered=True, tau_law="uniform", seed=26), {}),
    # three and four 64-key steps per split (the ring of five half-stages wraps), a split across the seam;
    # with r128-seam and r320-hd256 (one and two steps) every fill state of the ring
    ("bf16-r128-long", _variant("tiny", dtype="bf16", H=2, d=128, r=128, Lq=1000, tokens_per_frame=250,
                                clustered=True, tau_law="uniform", seed=27), {}),
    # eight slots out of 24 pages: the retrieval's slot order over more chosen pages
    ("kp8-p24", _variant("tiny", Kp=8, P=24, seed=28), {}),
    # 160-token pages: 128-row history blocks straddle page seams while no block
    # spans more than two pages (the gather's two-page path)
    ("bf16-tp160", _variant("tiny", dtype="bf16", tokens_per_frame=20, Kp=3, P=6, clustered=True,
                            tau_law="uniform", seed=29), {}),
    # the limits the 720p workload crosses, at a size the oracle finishes in
    # seconds: 129 query blocks (more than 128) and 1129 tiles per head (more
    # than 1024) take the plan's wide row grouping (64-word bitmasks, four
    # rows per lane); 1129 blocks per row take the 32-items-per-lane
    # selection; r = 512 on the 256 x 256 projection (two row tiles)
    ("bf16-limits", _variant("tiny", dtype="bf16", H=2, d=128, Lq=8256, tokens_per_frame=4000, Kp=2,
                             P=3, Binter=64, r=512, clustered=True, tau_law="uniform", seed=31),
     dict(tau=[0.35, 0.42])),
    # 257 query blocks (more than 256): the plan keeps four consecutive rows
    # per group
    ("bf16-consecutive-rows", _variant("tiny", dtype="bf16", H=1, d=64, Lq=16448, tokens_per_frame=16, Kp=1,
                                       P=2, r=64, clustered=True, tau_law="uniform", seed=33),
     dict(tau=[0.35])),
    # nine heads and 1032 tiles per group: the attention runs two split ranges
    # per work-group (more than 1024 tiles per group and more than 8 heads)
    ("bf16-two-ranges", _variant("tiny", dtype="bf16", H=9, d=64, Lq=512, tokens_per_frame=2048, Kp=4, P=6,
                                 Binter=64, r=64, clustered=True, tau_law="uniform", seed=35), {}),
]


@pytest.fixture(scope="module", params=VARIANTS, ids=[v[0] for v in VARIANTS])
def case(request):
    _, s, kw = request.param
    torch.manual_seed(0)
    c = Case(s, **kw)
    c.ref = c.oracle()
    return c


def test_page_summary(case):
    km = case.page_summary()
    ref = np.stack([oracle.page_summary(oracle.as_f64(case.pool_k[p], case.s.dtype)[None])[0]
                    for p in range(case.s.P)])
    compare("page_kmean", host(km), ref, "f32", max_abs=1e-5, rel=1e-6)


def test_retrieval_and_gather(case):
    s, ref = case.s, case.ref
    km = case.page_summary()
    page_idx, n_sel, k_hist, v_hist = case.gather(km)
    n = int(host(n_sel)[0])
    assert n == ref["n_sel"]
    pi = host(page_idx)
    assert pi[:n].tolist() == ref["page_idx"].tolist()
    assert np.all(pi[n:] == -1)
    Lh = n * s.Tp
    assert host(k_hist)[:Lh].tobytes() == ref["k_hist"].tobytes()
    assert host(v_hist)[:Lh].tobytes() == ref["v_hist"].tobytes()
    # rows past the present slots are not written
    assert np.all(host(k_hist)[Lh:].view(np.uint8) == 0)


def test_selection(case):
    s, ref = case.s, case.ref
    _, n_sel, k_hist, _ = case.gather(case.page_summary())
    cnt, idx, mask, mass = case.select(k_hist, n_sel)
    NB = len(ref["blocks"])
    compare("block_mass", host(mass)[:, :, :NB], ref["mass"], "f32", max_abs=1e-6, rel=1e-5)
    differ = check_selection(host(cnt), host(idx), ref["mass"], ref["sel"], ref_tau(case))
    print(f"selection rows differing at the boundary: {len(differ)}")
    m = host(mask)[:, :, :NB]
    for h in range(s.H):
        for i in range(len(ref["qblocks"])):
            ids = host(idx)[h, i, :host(cnt)[h, i]]
            assert np.flatnonzero(m[h, i]).tolist() == ids.tolist()


def ref_tau(case):
    return [float(t) for t in case.ch["tau"]]


def test_sparse_attention_on_oracle_masks(case):
    s, ref = case.s, case.ref
    _, n_sel, k_hist, v_hist = case.gather(case.page_summary())
    cnt, idx = pack_selection(ref["sel"], case.d.NB_max)
    o = case.sparse(k_hist, v_hist, n_sel, dev(cnt), dev(idx))
    compare("o_sparse", host(o), ref["o_sparse"], s.dtype)


def test_linear_branch(case):
    s, ref = case.s, case.ref
    _, n_sel, k_hist, v_hist = case.gather(case.page_summary())
    o, kl, vl = case.linear(k_hist, v_hist, n_sel)
    tol = dict(max_abs=1e-4, rel=1e-5) if s.dtype == "f32" else dict(max_abs=2e-3, rel=1e-5)
    compare("k_low", host(kl), ref["k_low"], "f32", **tol)
    compare("v_low", host(vl), ref["v_low"], "f32", **tol)
    compare("o_linear", host(o), ref["o_linear"], s.dtype)


def test_gate_and_fuse_on_oracle_branches(case):
    s, ref = case.s, case.ref
    o_s = dev(ref["o_sparse"].astype(np.float32))
    o_l = dev(ref["o_linear"].astype(np.float32))
    out, gate = case.fuse(o_s, o_l)
    compare("gate", host(gate), ref["gate"], "f32", max_abs=1e-6, rel=1e-6)
    want = oracle.fuse(ref["gate"], ref["o_sparse"].astype(np.float32).astype(np.float64),
                       ref["o_linear"].astype(np.float32).astype(np.float64))
    got = oracle.as_f64(host(out), s.dtype)
    compare("out(fuse)", got, want, s.dtype)


def test_forward_end_to_end(case):
    s, ref = case.s, case.ref
    km = case.page_summary()
    outs = case.forward(km)
    n = int(host(outs["n_sel"])[0])
    assert n == ref["n_sel"] and host(outs["page_idx"])[:n].tolist() == ref["page_idx"].tolist()
    cnt, idx = host(outs["sel_count"]), host(outs["sel_idx"])
    differ = check_selection(cnt, idx, ref["mass"], ref["sel"], ref_tau(case))
    print(f"rows at the boundary: {len(differ)} of {s.H * len(ref['qblocks'])}")
    # a row whose (valid) set differs at the boundary is checked against
    # attention over its own set; every other row against the oracle
    want_s = expected_sparse(s, case.ch, ref, cnt, idx, differ)
    compare("o_linear(fwd)", host(outs["o_linear"]), ref["o_linear"], s.dtype)
    compare("o_sparse(fwd)", host(outs["o_sparse"]), want_s, s.dtype)
    compare("gate(fwd)", host(outs["gate"]), ref["gate"], "f32", max_abs=1e-6, rel=1e-6)
    got = oracle.as_f64(host(outs["out"]), s.dtype)
    compare("out(fwd)", got, oracle.fuse(ref["gate"], want_s, ref["o_linear"]), s.dtype)


def test_forward_matches_stages(case):
    """hsa_forward against the entry points called one after another on the same
    inputs. The forward pools the history keys inside the gather and runs the
    low-rank branch on a second stream; neither may change a result: pages,
    gathered rows, selection and both branches agree bit for bit. The gate and
    the gated output differ from hsa_fuse's by rounding only (the gate's dot
    product is summed in another order)."""
    s = case.s
    km = case.page_summary()
    f = case.forward(km)
    page_idx, n_sel, k_hist, v_hist = case.gather(km)
    n = int(host(n_sel)[0])
    assert int(host(f["n_sel"])[0]) == n
    assert host(f["page_idx"])[:n].tolist() == host(page_idx)[:n].tolist()
    rows = n * s.Tp
    assert host(f["k_hist"])[:rows].tobytes() == host(k_hist)[:rows].tobytes()
    assert host(f["v_hist"])[:rows].tobytes() == host(v_hist)[:rows].tobytes()
    cnt, idx, _, _ = case.select(k_hist, n_sel)
    c, fi, si = host(cnt), host(f["sel_idx"]), host(idx)
    assert np.array_equal(host(f["sel_count"]), c)
    for h in range(s.H):
        for i in range(c.shape[1]):
            assert np.array_equal(fi[h, i, :c[h, i]], si[h, i, :c[h, i]]), (h, i)
    o_s = case.sparse(k_hist, v_hist, n_sel, cnt, idx)
    assert host(f["o_sparse"]).tobytes() == host(o_s).tobytes()
    o_l, _, _ = case.linear(k_hist, v_hist, n_sel)
    assert host(f["o_linear"]).tobytes() == host(o_l).tobytes()
    out, gate = case.fuse(o_s, o_l)
    g_f, g_s = host(f["gate"]), host(gate)
    assert np.max(np.abs(g_f - g_s)) <= 1e-6
    a, b = oracle.as_f64(host(f["out"]), s.dtype), oracle.as_f64(host(out), s.dtype)
    ulp = 2.0 ** -7 if s.dtype == "bf16" else 2.0 ** -20
    assert np.all(np.abs(a - b) <= ulp * np.abs(b) + 1e-6)


def test_forward_with_only_out(case):
    """With only `out` requested every intermediate lives in the workspace (as
    in the bench): the output is the same, bit for bit, as with all outputs."""
    km = case.page_summary()
    full = host(case.forward(km)["out"])
    bare = host(case.forward(km, debug=False)["out"])
    assert full.tobytes() == bare.tobytes()


def test_sparse_plan_then_compute_equals_entry_point(case):
    """The attention in its two exported parts gives the bits of hsa_sparse_attn."""
    s = case.s
    if s.dtype != "bf16":
        pytest.skip("the plan/compute split is the bf16 path")
    _, n_sel, k_hist, v_hist = case.gather(case.page_summary())
    cnt, idx, _, _ = case.select(k_hist, n_sel)
    ref = case.sparse(k_hist, v_hist, n_sel, cnt, idx)
    w = ws(case.d, hs.ENTRY_SPARSE)
    o = torch.full((s.Lq, s.H, s.d), float("nan"), dtype=torch.float32, device="cuda")
    hs.hsa_sparse_plan(case.d, n_sel, cnt, idx, w)
    hs.hsa_sparse_compute(case.d, case.t["q"], k_hist, v_hist, case.t["k_intra"], case.t["v_intra"], n_sel, o, w)
    assert host(o).tobytes() == host(ref).tobytes()


def test_forward_on_one_stream_equals_forked(case):
    """Without a fork every stage runs on the caller's stream: the same
    results, bit for bit, as with the low-rank branch on the fork's stream."""
    km = case.page_summary()
    a = case.forward(km)
    b = case.forward(km, fork=None)
    for k in ("out", "o_sparse", "o_linear", "sel_count", "k_hist"):
        assert host(a[k]).tobytes() == host(b[k]).tobytes(), k


def test_forward_is_deterministic(case):
    km = case.page_summary()
    a = host(case.forward(km)["out"])
    b = host(case.forward(km)["out"])
    assert a.tobytes() == b.tobytes()


def test_forward_from_two_threads():
    """bf16 forwards from two host threads, each on its own stream, workspace
    and fork: every result equals the one-thread result bit for bit."""
    import threading
    s = _variant("tiny", dtype="bf16", clustered=True, tau_law="uniform", seed=30)
    c = Case(s)
    km = c.page_summary()
    ref = host(c.forward(km, debug=False)["out"]).tobytes()
    torch.cuda.synchronize()
    results, errors = [], []

    def worker():
        try:
            st = torch.cuda.Stream()
            fk = hs.fork_create()
            with torch.cuda.stream(st):
                outs = [c.forward(km, debug=False, fork=fk)["out"] for _ in range(3)]
            st.synchronize()
            hs.fork_destroy(fk)
            results.extend(host(o).tobytes() for o in outs)
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker) for _ in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    assert len(results) == 6 and all(r == ref for r in results)


# ---------------------------------------------------------------------------
# special cases with closed forms on the GPU

def test_tau_one_is_dense_attention():
    s = synth.shape("tiny").with_(seed=21)
    ch = synth.draw_chunk(s)
    ch["tau"] = np.ones(s.H, np.float32)
    c = Case(s, chunk=ch)
    ref = c.oracle()
    _, n_sel, k_hist, v_hist = c.gather(c.page_summary())
    cnt, idx, _, _ = c.select(k_hist, n_sel)
    NB = len(ref["blocks"])
    assert np.all(host(cnt) == NB)
    o = c.sparse(k_hist, v_hist, n_sel, cnt, idx)
    q = oracle.as_f64(ch["q"], s.dtype)
    K = np.concatenate([ref["k_hist"], ch["k_intra"]]).astype(np.float64)
    V = np.concatenate([ref["v_hist"], ch["v_intra"]]).astype(np.float64)
    for h in range(s.H):
        dense = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(np.ascontiguousarray(a[:, h]))[None, None] for a in (q, K, V)))[0, 0]
        compare(f"dense h{h}", host(o)[:, h], dense.numpy(), "f32")


def test_zero_query_selects_lowest_ids():
    s = synth.shape("tiny").with_(seed=22)
    ch = synth.draw_chunk(s)
    ch["q"] = np.zeros_like(ch["q"])
    ch["tau"] = np.array([0.35, 0.6], np.float32)   # tau * 6 blocks is not an integer
    c = Case(s, chunk=ch)
    _, n_sel, k_hist, _ = c.gather(c.page_summary())
    cnt, idx, _, mass = c.select(k_hist, n_sel)
    NB = 6
    assert np.all(host(mass)[:, :, :NB] == np.float32(1.0 / NB))
    for h, t in enumerate(ch["tau"]):
        k = int(np.ceil(t * NB))
        assert np.all(host(cnt)[h] == k)
        assert np.all(host(idx)[h, :, :k] == np.arange(k))


def test_duplicate_page_tie_goes_to_lower_index():
    s = synth.shape("tiny").with_(Kp=1, seed=23)
    ch = synth.draw_chunk(s)
    pk, pv = synth.draw_pool(s)
    c0 = Case(s, chunk=ch, pool=(pk, pv))
    best = int(c0.oracle()["page_idx"][0])
    # copy the best page to the highest candidate index above it
    cands = [p for p in range(s.P) if ch["page_prompt"][p] == s.cur_prompt and p > best]
    if not cands:
        pytest.skip("best page is the last candidate")
    dup = cands[-1]
    pk2, pv2 = pk.copy(), pv.copy()
    pk2[dup] = pk[best]
    pv2[dup] = pv[best]
    c = Case(s, chunk=ch, pool=(pk2, pv2))
    ref = c.oracle()
    assert ref["page_idx"].tolist() == [best]
    km = c.page_summary()
    kmh = host(km)
    assert kmh[dup].tobytes() == kmh[best].tobytes()
    page_idx, n_sel, _, _ = c.gather(km)
    assert host(n_sel)[0] == 1 and host(page_idx)[0] == best


def test_nan_page_scores_rank_last():
    """Page means holding NaN or infinities give scores that are not numbers:
    such pages rank below every finite page and the slot count stays min(Kp,
    candidates), as in the oracle's rule."""
    s = synth.shape("tiny").with_(P=12, Kp=4, seed=32)
    ch = synth.draw_chunk(s)
    c = Case(s, chunk=ch, page_prompt=np.zeros(12, np.int32))
    km = c.page_summary()
    kmh = host(km).copy()
    kmh[1, 0, 3] = np.nan
    kmh[4, 1, 0] = np.inf
    kmh[4, 1, 1] = -np.inf
    kmh[7] = np.nan
    kmh[9, 0, 0] = np.inf                 # +inf alone: ranks first
    km_bad = dev(kmh.astype(np.float32))
    qbar = oracle.chunk_query_mean(oracle.as_f64(ch["q"], s.dtype))
    for Kp, prompts in ((4, np.zeros(12, np.int32)), (11, np.zeros(12, np.int32)),
                        (2, np.array([1, 0, 1, 1, 0, 1, 1, 0, 1, 1, 1, 1], np.int32))):
        s2 = s.with_(Kp=Kp)
        c2 = Case(s2, chunk=dict(ch), pool=(c.pool_k, c.pool_v), page_prompt=prompts)
        want, n = oracle.retrieve(kmh.astype(np.float64), prompts, s.cur_prompt, qbar, Kp)
        page_idx, n_sel, _, _ = c2.gather(km_bad)
        assert int(host(n_sel)[0]) == n
        pi = host(page_idx)
        assert pi[:n].tolist() == want.tolist(), (Kp, pi, want)
        assert np.all(pi[n:] == -1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nonfinite_query_scores(dtype):
    """A query holding +inf makes the chunk mean infinite in that column, so
    every page score is +inf, -inf or NaN by the sign of the page means
    there: the kernel takes these pages' scores from the exact terms and
    ranks them as the oracle does (NaN as -inf, ties to the lower page)."""
    s = synth.shape("tiny").with_(P=12, Kp=4, dtype=dtype, seed=37)
    ch = synth.draw_chunk(s)
    q = ch["q"].copy()
    q[5, 0, 3] = 0x7F80 if dtype == "bf16" else np.float32(np.inf)   # +inf (bfloat16 bits)
    ch["q"] = q
    prompts = np.zeros(12, np.int32)
    c = Case(s, chunk=ch, page_prompt=prompts)
    km = c.page_summary()
    kmh = host(km).astype(np.float64)
    qbar = oracle.chunk_query_mean(oracle.as_f64(ch["q"], s.dtype))
    assert np.isinf(qbar[0, 3])
    want, n = oracle.retrieve(kmh, prompts, s.cur_prompt, qbar, s.Kp)
    page_idx, n_sel, _, _ = c.gather(km)
    assert int(host(n_sel)[0]) == n
    assert host(page_idx)[:n].tolist() == want.tolist(), (host(page_idx), want)


@pytest.mark.parametrize("policy", ["two_stage", "page_only", "prompt_only", "recent", "random",
                                    "mismatched"])
@pytest.mark.parametrize("Kp,seed", [(4, 0), (3, 987654321)])
def test_retrieval_policies(policy, Kp, seed):
    """Every retrieval policy on a 12-page pool with three prompts: the pages
    chosen and the gathered rows equal the oracle's."""
    s = synth.shape("tiny").with_(P=12, Kp=Kp, seed=34)
    prompts = np.array([p % 3 for p in range(12)], np.int32)
    c = Case(s, page_prompt=prompts, cur_prompt=1)
    km = c.page_summary()
    kmh = host(km).astype(np.float64)
    qbar = oracle.chunk_query_mean(oracle.as_f64(c.ch["q"], s.dtype))
    want, n = oracle.retrieve(kmh, prompts, 1, qbar, Kp, policy, seed)
    page_idx, n_sel, k_hist, _ = c.gather(km, policy=policy, seed=seed)
    assert int(host(n_sel)[0]) == n
    assert host(page_idx)[:n].tolist() == want.tolist(), (policy, host(page_idx), want)
    assert host(k_hist)[:n * s.Tp].tobytes() == np.concatenate([c.pool_k[p] for p in want]).tobytes()


@pytest.mark.parametrize("policy", ["two_stage", "page_only", "recent", "random"])
def test_retrieval_over_more_pages_than_threads(policy):
    """1100 pages, more than the 1024 pages one ranking pass covers, and Kp =
    64: the chosen pages lie on both sides of the pass boundary (the recency
    policy takes the newest candidates, all above it) and their slots, in
    ascending page order, equal the oracle's."""
    P, Kp = 1100, 64
    s = synth.shape("tiny").with_(P=P, Kp=Kp, tokens_per_frame=1, Psize=8, seed=36)
    prompts = np.array([p % 2 for p in range(P)], np.int32)
    c = Case(s, page_prompt=prompts, cur_prompt=0)
    km = c.page_summary()
    kmh = host(km).astype(np.float64)
    qbar = oracle.chunk_query_mean(oracle.as_f64(c.ch["q"], s.dtype))
    want, n = oracle.retrieve(kmh, prompts, 0, qbar, Kp, policy, 5)
    assert n == Kp and want.max() >= 1024 and (policy == "recent" or want.min() < 1024)
    page_idx, n_sel, k_hist, _ = c.gather(km, policy=policy, seed=5)
    assert int(host(n_sel)[0]) == n
    assert host(page_idx).tolist() == want.tolist(), (policy, host(page_idx), want)
    assert host(k_hist).tobytes() == np.concatenate([c.pool_k[p] for p in want]).tobytes()


@pytest.mark.parametrize("policy", ["recent", "random", "mismatched"])
def test_forward_with_other_policies(policy):
    s = synth.shape("tiny").with_(dtype="bf16", P=10, Kp=3, clustered=True, tau_law="uniform", seed=35)
    prompts = np.array([p % 2 for p in range(10)], np.int32)
    c = Case(s, page_prompt=prompts)
    ref = c.oracle(policy=policy, seed=77)
    outs = c.forward(c.page_summary(), policy=policy, seed=77)
    n = int(host(outs["n_sel"])[0])
    assert n == ref["n_sel"] and host(outs["page_idx"])[:n].tolist() == ref["page_idx"].tolist()
    cnt, idx = host(outs["sel_count"]), host(outs["sel_idx"])
    differ = check_selection(cnt, idx, ref["mass"], ref["sel"], [float(t) for t in c.ch["tau"]])
    want_s = expected_sparse(s, c.ch, ref, cnt, idx, differ)
    compare(f"out({policy})", oracle.as_f64(host(outs["out"]), s.dtype),
            oracle.fuse(ref["gate"], want_s, ref["o_linear"]), s.dtype)


def test_gate_limits_isolate_branches():
    s = synth.shape("tiny").with_(seed=24)
    for bias, branch in ((1e3, "o_sparse"), (-1e3, "o_linear")):
        ch = synth.draw_chunk(s)
        ch["b_g"] = np.full(s.H, bias, np.float32)
        c = Case(s, chunk=ch)
        outs = c.forward(c.page_summary())
        assert host(outs["out"]).tobytes() == host(outs[branch]).tobytes()
