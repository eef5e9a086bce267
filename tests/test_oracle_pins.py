"""Pins of the float64 oracle to facts fixed outside the oracle itself.

Each pin is a closed form, a brute force on tiny inputs, a library routine
that a special case reduces to (torch's CPU scaled_dot_product_attention in
float64, scipy's expit), an invariant of the definition, or a hand-worked
fixture under tests/golden/. None of them re-runs the oracle's own formula.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sdpa(q, k, v, mask=None):
    """Library dense attention, float64, scale 1/sqrt(d). q [n][d], k/v [m][d]."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m)[0, 0].numpy()


# ---------------------------------------------------------------------------
# O1-O6 page summary, retrieval, gather

def test_page_summary_closed_forms():
    Tp, H, d = 12, 2, 3
    const = np.full((1, Tp, H, d), 2.5)
    ramp = np.broadcast_to(np.arange(Tp, dtype=np.float64)[None, :, None, None], (1, Tp, H, d))
    got = oracle.page_summary(np.concatenate([const, ramp]))
    assert np.array_equal(got[0], np.full((H, d), 2.5))
    assert np.allclose(got[1], (Tp - 1) / 2.0, rtol=0, atol=1e-15)


@pytest.mark.parametrize("case", _golden("retrieval_hand.json")["cases"])
def test_retrieval_hand_worked(case):
    kmean = np.array(case["page_mean"], dtype=np.float64)[:, None, :]   # one head
    # a chunk whose every query equals the stated mean, so the chunk mean is exact
    q = np.tile(np.array(case["query_mean"], dtype=np.float64)[None, None, :], (7, 1, 1))
    qbar = oracle.chunk_query_mean(q)
    assert np.array_equal(qbar, np.array(case["query_mean"], dtype=np.float64)[None, :])
    idx, n = oracle.retrieve(kmean, np.array(case["page_prompt"]), case["cur_prompt"], qbar, case["Kp"])
    assert idx.tolist() == case["page_idx"]
    assert n == len(case["page_idx"])
    # ranking is invariant to a positive rescaling of Q
    idx2, _ = oracle.retrieve(kmean, np.array(case["page_prompt"]), case["cur_prompt"], 3.75 * qbar, case["Kp"])
    assert idx2.tolist() == case["page_idx"]


def _brute_topk(scores, cand, Kp):
    """Best subset of size min(Kp, |cand|) by total score; ties to the lexicographically smallest set."""
    k = min(Kp, len(cand))
    best = None
    for sub in itertools.combinations(sorted(cand), k):
        tot = sum(scores[p] for p in sub)
        key = (-tot, sub)
        if best is None or key < best:
            best = key
    return list(best[1]) if best else []


@pytest.mark.parametrize("seed", range(300))
def test_retrieval_brute_force(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(1, 9))
    H, d = 2, 4
    Kp = int(rng.integers(1, 5))
    kmean = rng.standard_normal((P, H, d))
    if P > 2 and seed % 3 == 0:              # a duplicated page forces an exact tie
        kmean[P - 1] = kmean[0]
    prompts = rng.integers(0, 3, size=P)
    cur = int(rng.integers(0, 3))
    qbar = rng.standard_normal((H, d))
    cand = [p for p in range(P) if prompts[p] == cur]
    scores = {p: float(np.tensordot(kmean[p], qbar, axes=2)) for p in cand}
    want = _brute_topk(scores, cand, Kp)
    idx, n = oracle.retrieve(kmean, prompts, cur, qbar, Kp)
    assert idx.tolist() == want and n == len(want)


def test_retrieval_duplicate_tie_goes_low():
    kmean = np.zeros((6, 1, 2))
    kmean[1] = kmean[4] = [[1.0, 0.0]]
    kmean[2] = [[0.5, 0.0]]
    idx, n = oracle.retrieve(kmean, np.zeros(6, np.int32), 0, np.array([[1.0, 0.0]]), 1)
    assert idx.tolist() == [1] and n == 1


def test_retrieval_nan_scores_rank_last():
    """Pages whose score is not a number rank below every finite score; among
    themselves the lower page goes first (worked by hand: finite scores of
    pages 0, 2, 4 are 1, 3, 2)."""
    kmean = np.zeros((5, 1, 2))
    kmean[0] = [[1.0, 0.0]]
    kmean[1] = [[np.nan, 0.0]]
    kmean[2] = [[3.0, 0.0]]
    kmean[3] = [[np.inf, -np.inf]]        # inf - inf: NaN
    kmean[4] = [[2.0, 0.0]]
    q = np.array([[1.0, 1.0]])
    prompts = np.zeros(5, np.int32)
    assert oracle.retrieve(kmean, prompts, 0, q, 2)[0].tolist() == [2, 4]
    assert oracle.retrieve(kmean, prompts, 0, q, 3)[0].tolist() == [0, 2, 4]
    assert oracle.retrieve(kmean, prompts, 0, q, 4)[0].tolist() == [0, 1, 2, 4]
    idx, n = oracle.retrieve(kmean, prompts, 0, q, 5)
    assert idx.tolist() == [0, 1, 2, 3, 4] and n == 5
    # only NaN candidates: the lowest indices
    assert oracle.retrieve(kmean, np.array([1, 0, 1, 0, 1], np.int32), 0, q, 1)[0].tolist() == [1]


def test_gather_is_a_bit_copy():
    s = synth.shape("tiny")
    pk, _ = synth.draw_pool(s)
    bits = synth.round_bf16_bits(pk)
    for arr in (pk, bits):
        out = oracle.gather(arr, np.array([4, 0], dtype=np.int32))
        assert out.dtype == arr.dtype and out.shape == (2 * s.Tp, s.H, s.d)
        assert out[:s.Tp].tobytes() == arr[4].tobytes()
        assert out[s.Tp:].tobytes() == arr[0].tobytes()
    assert oracle.gather(pk, np.zeros(0, np.int32)).shape == (0, s.H, s.d)


# ---------------------------------------------------------------------------
# O7-O8 block tables and pooling

@pytest.mark.parametrize("case", _golden("workload_blocks.json")["cases"])
def test_block_table_workloads(case):
    blocks = oracle.block_table(case["Lh"], case["Lq"], 128, 64)
    nbh = sum(1 for s, e in blocks if s < case["Lh"])
    assert nbh == case["NBh"]
    assert len(blocks) - nbh == case["NBc"]
    if case["NBh"]:
        assert blocks[nbh - 1][1] - blocks[nbh - 1][0] == case["last_hist"]
    assert blocks[-1][1] - blocks[-1][0] == case["last_intra"]
    assert blocks[-1][1] == case["Lh"] + case["Lq"]
    # the blocks tile [0, Lh + Lq) exactly, in order
    assert blocks[0][0] == 0
    assert all(a[1] == b[0] for a, b in zip(blocks, blocks[1:]))
    assert len(oracle.query_blocks(case["Lq"], 64)) == case["NQB"]


def test_pool_closed_forms():
    L, H, d = 300, 2, 3
    x = np.broadcast_to(np.arange(L, dtype=np.float64)[:, None, None], (L, H, d)).copy()
    ranges = [(0, 128), (128, 256), (256, 300)]
    kb = oracle.pool_blocks(x, ranges)
    for b, (s, e) in enumerate(ranges):         # mean of an arithmetic run s..e-1
        assert np.allclose(kb[:, b, :], (s + e - 1) / 2.0, rtol=0, atol=1e-12)
    c = np.full((L, H, d), -1.25)
    assert np.array_equal(oracle.pool_blocks(c, ranges), np.full((H, 3, d), -1.25))


# ---------------------------------------------------------------------------
# O9-O10 block mass and selection

def test_block_mass_is_a_softmax():
    rng = np.random.default_rng(0)
    qb, kb = rng.standard_normal((3, 5, 16)), rng.standard_normal((3, 9, 16))
    m = oracle.block_mass(qb, kb)
    want = scipy.special.softmax(np.einsum("hid,hbd->hib", qb, kb) / 4.0, axis=-1)
    assert np.allclose(m, want, rtol=1e-13, atol=1e-15)
    assert np.allclose(m.sum(-1), 1.0, atol=1e-14)


@pytest.mark.parametrize("tau", [0.35, 0.6, 0.9, 0.999])
def test_zero_query_gives_uniform_mass(tau):
    nb = 6
    qb = np.zeros((1, 1, 8))
    kb = np.random.default_rng(1).standard_normal((1, nb, 8))
    m = oracle.block_mass(qb, kb)
    assert np.allclose(m, 1.0 / nb, rtol=0, atol=1e-16)
    sel = oracle.select_row(m[0, 0], tau)
    assert sel.tolist() == list(range(math.ceil(tau * nb)))


@pytest.mark.parametrize("case", _golden("selection_hand.json")["cases"])
def test_selection_hand_worked(case):
    assert oracle.select_row(np.array(case["mass"]), case["tau"]).tolist() == case["selected"]


@pytest.mark.parametrize("seed", range(200))
def test_selection_brute_force(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(1, 11))
    mass = rng.dirichlet(np.full(nb, 0.7))
    tau = float(np.float32(rng.uniform(0.05, 0.999)))
    # every subset: smallest cardinality reaching tau, then the heaviest of those
    best = None
    for k in range(1, nb + 1):
        for sub in itertools.combinations(range(nb), k):
            tot = float(mass[list(sub)].sum())
            if abs(tot - tau) < 1e-6:
                pytest.skip("a subset sits on the boundary; float32 decides it")
            if tot >= tau and (best is None or (k, -tot, sub) < best):
                best = (k, -tot, sub)
        if best is not None:
            break
    got = oracle.select_row(mass, tau)
    assert got.tolist() == list(best[2])


@pytest.mark.parametrize("seed", range(50))
def test_selection_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(2, 400))
    mass = rng.dirichlet(np.full(nb, 2.0))
    prev = set()
    for tau in (0.35, 0.5, 0.6, 0.75, 0.9, 0.99):
        s = oracle.select_row(mass, tau)
        tot = mass[s].sum()
        assert tot >= tau - 1e-6                       # reaches tau
        assert tot - mass[s].min() < tau + 1e-6        # minimal: dropping the lightest fails
        assert prev <= set(s.tolist())                 # nested as tau grows
        assert list(s) == sorted(s)
        prev = set(s.tolist())
    assert oracle.select_row(mass, 1.0).tolist() == list(range(nb))


# ---------------------------------------------------------------------------
# O11 sparse attention

def _rand_qkv(rng, Lq, L, H, d):
    return (rng.standard_normal((Lq, H, d)), rng.standard_normal((L, H, d)),
            rng.standard_normal((L, H, d)))


def test_sparse_all_blocks_is_dense_attention():
    rng = np.random.default_rng(3)
    Lh, Lq, H, d = 300, 130, 2, 16
    q, K, V = _rand_qkv(rng, Lq, Lh + Lq, H, d)
    blocks = oracle.block_table(Lh, Lq, 128, 64)
    qblocks = oracle.query_blocks(Lq, 64)
    sel = [[np.arange(len(blocks))] * len(qblocks) for _ in range(H)]
    got = oracle.sparse_attention(q, K, V, sel, blocks, qblocks)
    for h in range(H):
        assert np.allclose(got[:, h], _sdpa(q[:, h], K[:, h], V[:, h]), rtol=1e-12, atol=1e-13)


def test_sparse_mask_is_masked_dense_attention():
    rng = np.random.default_rng(4)
    Lh, Lq, H, d = 256, 200, 2, 16
    q, K, V = _rand_qkv(rng, Lq, Lh + Lq, H, d)
    blocks = oracle.block_table(Lh, Lq, 128, 64)
    qblocks = oracle.query_blocks(Lq, 64)
    sel = [[np.sort(rng.choice(len(blocks), size=int(rng.integers(1, len(blocks) + 1)), replace=False))
            for _ in qblocks] for _ in range(H)]
    got = oracle.sparse_attention(q, K, V, sel, blocks, qblocks)
    for h in range(H):
        for i, (qs, qe) in enumerate(qblocks):
            mask = np.zeros((qe - qs, Lh + Lq), dtype=bool)
            for b in sel[h][i]:
                mask[:, blocks[b][0]:blocks[b][1]] = True
            want = _sdpa(q[qs:qe, h], K[:, h], V[:, h], mask)
            assert np.allclose(got[qs:qe, h], want, rtol=1e-12, atol=1e-13)


def test_sparse_constant_values_and_single_token_block():
    rng = np.random.default_rng(5)
    Lh, Lq, H, d = 128, 65, 1, 8           # the last chunk block holds one key
    q, K, V = _rand_qkv(rng, Lq, Lh + Lq, H, d)
    blocks = oracle.block_table(Lh, Lq, 128, 64)
    qblocks = oracle.query_blocks(Lq, 64)
    assert blocks[-1] == (Lh + 64, Lh + 65)
    Vc = np.full_like(V, 0.375)
    sel = [[np.array([0, 2])] * len(qblocks)]
    assert np.allclose(oracle.sparse_attention(q, K, Vc, sel, blocks, qblocks), 0.375, atol=1e-15)
    sel1 = [[np.array([len(blocks) - 1])] * len(qblocks)]
    got = oracle.sparse_attention(q, K, V, sel1, blocks, qblocks)
    assert np.allclose(got[:, 0], np.broadcast_to(V[Lh + 64, 0], (Lq, d)), atol=1e-15)


# ---------------------------------------------------------------------------
# O12 linear branch

def test_linear_identity_projection_is_dense_attention():
    rng = np.random.default_rng(6)
    L, Lq, H, d = 96, 40, 2, 16
    q, K, V = _rand_qkv(rng, Lq, L, H, d)
    I = np.eye(L)
    o_l, kl, vl = oracle.linear_branch(q, K, V, I, I)
    assert np.array_equal(kl, K) and np.array_equal(vl, V)
    for h in range(H):
        assert np.allclose(o_l[:, h], _sdpa(q[:, h], K[:, h], V[:, h]), rtol=1e-12, atol=1e-13)


def test_linear_one_hot_rows_attend_chosen_keys():
    rng = np.random.default_rng(7)
    L, Lq, H, d = 50, 20, 2, 8
    q, K, V = _rand_qkv(rng, Lq, L, H, d)
    pick_k = np.array([3, 17, 41, 0, 9])
    pick_v = np.array([5, 5, 22, 49, 1])
    E = np.zeros((5, L)); E[np.arange(5), pick_k] = 1.0
    F = np.zeros((5, L)); F[np.arange(5), pick_v] = 1.0
    o_l, _, _ = oracle.linear_branch(q, K, V, E, F)
    for h in range(H):
        want = _sdpa(q[:, h], K[pick_k, h], V[pick_v, h])
        assert np.allclose(o_l[:, h], want, rtol=1e-12, atol=1e-13)


def test_active_columns_skip_absent_slots():
    cols = oracle.active_projection_columns(n_sel=1, Kp=3, Tp=4, Lq=2)
    assert cols.tolist() == [0, 1, 2, 3, 12, 13]
    assert oracle.active_projection_columns(0, 2, 4, 3).tolist() == [8, 9, 10]
    assert oracle.active_projection_columns(2, 2, 4, 1).tolist() == list(range(9))


# ---------------------------------------------------------------------------
# O13 gate and fusion

def test_gate_matches_expit_and_isolates_branches():
    rng = np.random.default_rng(8)
    Lq, H, d = 30, 3, 8
    q = rng.standard_normal((Lq, H, d))
    w = rng.standard_normal((H, d))
    b = rng.standard_normal(H)
    g = oracle.gate(q, w, b)
    want = scipy.special.expit(np.stack([q[:, h] @ w[h] + b[h] for h in range(H)], axis=1))
    assert np.allclose(g, want, rtol=1e-14, atol=0)
    o_s, o_l = rng.standard_normal((Lq, H, d)), rng.standard_normal((Lq, H, d))
    big = np.full(H, 1e3)
    assert np.array_equal(oracle.fuse(oracle.gate(q, w * 0, big), o_s, o_l), o_s)
    assert np.array_equal(oracle.fuse(oracle.gate(q, w * 0, -big), o_s, o_l), o_l)
    half = oracle.fuse(oracle.gate(q, w * 0, np.zeros(H)), o_s, o_l)
    assert np.allclose(half, 0.5 * (o_s + o_l), rtol=0, atol=1e-15)
    assert np.all(np.isfinite(oracle.gate(q * 1e4, w, b)))


# ---------------------------------------------------------------------------
# whole forward on the tiny workload

def _tiny_forward(**over):
    s = synth.shape("tiny")
    ch = synth.draw_chunk(s)
    ch.update(over)
    pk, pv = synth.draw_pool(s)
    return s, ch, pk, pv, oracle.forward(
        dtype=s.dtype, q=ch["q"], k_intra=ch["k_intra"], v_intra=ch["v_intra"], pool_k=pk,
        pool_v=pv, page_prompt=ch["page_prompt"], cur_prompt=s.cur_prompt, E=ch["E"], F=ch["F"],
        w_g=ch["w_g"], b_g=ch["b_g"], tau=ch["tau"], Kp=s.Kp, Binter=s.Binter, Bintra=s.Bintra,
        Bq=s.Bq)


def test_tiny_forward_structure():
    s, ch, pk, pv, r = _tiny_forward()
    assert r["n_sel"] == 2
    assert set(r["page_idx"].tolist()) <= {0, 2, 4}           # prompt ids p mod 2, current 0
    assert list(r["page_idx"]) == sorted(r["page_idx"])
    assert r["k_hist"].tobytes() == np.concatenate([pk[p] for p in r["page_idx"]]).tobytes()
    assert len(r["blocks"]) == 6 and len(r["qblocks"]) == 4
    for i in range(4):                                        # head 1 has tau = 1.0
        assert r["sel"][1][i].tolist() == list(range(6))
    assert r["out"].shape == (s.Lq, s.H, s.d)
    q = oracle.as_f64(ch["q"], s.dtype)
    K = np.concatenate([r["k_hist"], ch["k_intra"]]).astype(np.float64)
    V = np.concatenate([r["v_hist"], ch["v_intra"]]).astype(np.float64)
    assert np.allclose(r["o_sparse"][:, 1], _sdpa(q[:, 1], K[:, 1], V[:, 1]), rtol=1e-12, atol=1e-13)


def test_tiny_forward_gate_limits():
    s = synth.shape("tiny")
    _, _, _, _, hi = _tiny_forward(b_g=np.full(s.H, 1e3, np.float32))
    assert np.array_equal(hi["out"], hi["o_sparse"])
    _, _, _, _, lo = _tiny_forward(b_g=np.full(s.H, -1e3, np.float32))
    assert np.array_equal(lo["out"], lo["o_linear"])


# ---------------------------------------------------------------------------
# whole forward: how the branches are wired (key order, E against K and F
# against V, the columns of absent slots). Every expected value below is
# built by the test itself from the pool pages and the chunk, never from the
# oracle's own intermediates.

def _forward_f32(s, ch, pk, pv, **kw):
    return oracle.forward(
        dtype=s.dtype, q=ch["q"], k_intra=ch["k_intra"], v_intra=ch["v_intra"], pool_k=pk,
        pool_v=pv, page_prompt=ch["page_prompt"], cur_prompt=s.cur_prompt, E=ch["E"], F=ch["F"],
        w_g=ch["w_g"], b_g=ch["b_g"], tau=ch["tau"], Kp=s.Kp, Binter=s.Binter, Bintra=s.Bintra,
        Bq=s.Bq, **kw)


def _keys_by_hand(pk, pv, ch, page_idx):
    """[history pages in slot order ; chunk] along tokens, float64, built here."""
    K = np.concatenate([pk[int(p)] for p in page_idx] + [ch["k_intra"]]).astype(np.float64)
    V = np.concatenate([pv[int(p)] for p in page_idx] + [ch["v_intra"]]).astype(np.float64)
    return K, V


def test_forward_identity_projection_is_history_then_chunk():
    """r = L and E = F = I with every slot present: the projected keys and
    values are the key sequence itself, history slots first, then the chunk,
    and the low-rank branch is dense attention over it."""
    s = synth.shape("tiny").with_(seed=41)
    ch = synth.draw_chunk(s)
    pk, pv = synth.draw_pool(s)
    L = s.L
    ch["E"] = np.eye(L, dtype=np.float32)
    ch["F"] = np.eye(L, dtype=np.float32)
    r = _forward_f32(s, ch, pk, pv)
    assert r["n_sel"] == s.Kp
    K, V = _keys_by_hand(pk, pv, ch, r["page_idx"])
    assert np.array_equal(r["k_low"], K) and np.array_equal(r["v_low"], V)
    q = ch["q"].astype(np.float64)
    for h in range(s.H):
        assert np.allclose(r["o_linear"][:, h], _sdpa(q[:, h], K[:, h], V[:, h]),
                           rtol=1e-12, atol=1e-13)


def test_forward_one_hot_projection_with_an_absent_slot():
    """One matching page for Kp = 2 slots: slot 1 is absent and its E/F
    columns face no key. One-hot rows of E and of F (different columns for
    the two) pick a history token of the present slot, a chunk token, and a
    column of the absent slot (a zero row of K' or V')."""
    s = synth.shape("tiny").with_(P=3, seed=42)
    ch = synth.draw_chunk(s)
    ch["page_prompt"] = np.array([1, 0, 1], np.int32)      # only page 1 matches prompt 0
    pk, pv = synth.draw_pool(s)
    Tp, Lq, L = s.Tp, s.Lq, s.L
    assert L == 2 * Tp + Lq
    ek = [5, 2 * Tp + 44, Tp + 2, 127, 2 * Tp + 255]       # slot 0 t5, chunk t44, absent, slot 0 t127, chunk t255
    fv = [17, 2 * Tp + 4, Tp + 100, 2 * Tp, 0]
    E = np.zeros((len(ek), L), np.float32)
    F = np.zeros((len(fv), L), np.float32)
    E[np.arange(len(ek)), ek] = 1.0
    F[np.arange(len(fv)), fv] = 1.0
    ch["E"], ch["F"] = E, F
    r = _forward_f32(s.with_(r=len(ek)), ch, pk, pv)
    assert r["n_sel"] == 1 and r["page_idx"].tolist() == [1]

    def pick(col, page, chunk):
        if col < Tp:
            return page[col].astype(np.float64)
        if col >= 2 * Tp:
            return chunk[col - 2 * Tp].astype(np.float64)
        return np.zeros(page.shape[1:])                     # absent slot

    Kw = np.stack([pick(c, pk[1], ch["k_intra"]) for c in ek])
    Vw = np.stack([pick(c, pv[1], ch["v_intra"]) for c in fv])
    assert np.array_equal(r["k_low"], Kw) and np.array_equal(r["v_low"], Vw)
    q = ch["q"].astype(np.float64)
    for h in range(s.H):
        assert np.allclose(r["o_linear"][:, h], _sdpa(q[:, h], Kw[:, h], Vw[:, h]),
                           rtol=1e-12, atol=1e-13)


def _blocks_by_hand(Lh, Lq, Binter, Bintra):
    hist = [(a, min(a + Binter, Lh)) for a in range(0, Lh, Binter)]
    chunk = [(Lh + a, Lh + min(a + Bintra, Lq)) for a in range(0, Lq, Bintra)]
    return hist + chunk


@pytest.mark.parametrize("tau0,P,prompts", [(0.35, 6, None), (0.6, 3, [1, 0, 1])])
def test_forward_sparse_branch_is_masked_attention_over_history_then_chunk(tau0, P, prompts):
    """A tau < 1 head: the forward's block masses are the softmax of pooled
    logits over test-built blocks of [history ; chunk], and its sparse output
    is dense attention masked to the tokens of the forward's selected blocks
    of that same sequence."""
    s = synth.shape("tiny").with_(P=P, seed=43)
    ch = synth.draw_chunk(s)
    if prompts is not None:
        ch["page_prompt"] = np.array(prompts, np.int32)
    ch["tau"] = np.array([tau0, 1.0], np.float32)
    pk, pv = synth.draw_pool(s)
    r = _forward_f32(s, ch, pk, pv)
    K, V = _keys_by_hand(pk, pv, ch, r["page_idx"])
    Lh = r["n_sel"] * s.Tp
    blocks = _blocks_by_hand(Lh, s.Lq, s.Binter, s.Bintra)
    q = ch["q"].astype(np.float64)
    for h in range(s.H):
        kb = np.stack([K[a:b, h].mean(axis=0) for a, b in blocks])
        for i in range(-(-s.Lq // s.Bq)):
            q0, q1 = i * s.Bq, min((i + 1) * s.Bq, s.Lq)
            qb = q[q0:q1, h].mean(axis=0)
            want_mass = scipy.special.softmax(kb @ qb / math.sqrt(s.d))
            assert np.allclose(r["mass"][h, i], want_mass, rtol=1e-12, atol=1e-15)
            ids = r["sel"][h][i]
            if tau0 < 1.0 and h == 0:
                assert len(ids) < len(blocks)               # a real subset
            mask = np.zeros((q1 - q0, K.shape[0]), dtype=bool)
            for b in ids:
                mask[:, blocks[b][0]:blocks[b][1]] = True
            want = _sdpa(q[q0:q1, h], K[:, h], V[:, h], mask)
            assert np.allclose(r["o_sparse"][q0:q1, h], want, rtol=1e-12, atol=1e-13)


def test_bf16_decode_is_exact():
    x = np.array([1.0, -2.5, 3.140625, 1e-3], dtype=np.float32)
    bits = synth.round_bf16_bits(x)
    back = oracle.as_f64(bits, "bf16")
    assert back[0] == 1.0 and back[1] == -2.5 and back[2] == 3.140625
    assert abs(back[3] - 1e-3) < 1e-3 * 2 ** -8
    # round-to-nearest-even on a hand-made tie: 1 + 2^-8 sits halfway between
    # 1 and 1 + 2^-7, and goes to the even mantissa, 1
    assert oracle.as_f64(synth.round_bf16_bits(np.array([1 + 2 ** -8], np.float32)), "bf16")[0] == 1.0


# ---------------------------------------------------------------------------
# page commit

def _empty_pool(P, Tp, H, d):
    return (np.zeros((P, Tp, H, d), np.float32), np.zeros((P, Tp, H, d), np.float32),
            np.full((P, H, d), -7.0), np.full(P, -1, np.int32))


def test_commit_within_one_page_finalises_nothing():
    P, Tp, H, d = 3, 8, 2, 4
    pk, pv, km, pp = _empty_pool(P, Tp, H, d)
    k = np.arange(1, 5 * H * d + 1, dtype=np.float32).reshape(5, H, d)
    v = -k
    # tokens 2..6: the page's last token (7) is still missing
    nk, nv, nkm, npp, done = oracle.page_commit(pk, pv, km, pp, k, v, fill=2, cur_prompt=5)
    assert done == []
    assert np.array_equal(nk[0, 2:7], k) and np.array_equal(nv[0, 2:7], v)
    assert np.all(nk[0, :2] == 0) and np.all(nk[0, 7] == 0) and np.all(nk[1:] == 0)
    assert np.array_equal(nkm, km) and np.array_equal(npp, pp)
    assert np.all(pk == 0)                       # inputs untouched


def test_commit_across_a_page_end_finalises_it():
    """Tokens 6..10 of 8-token pages: page 0 fills (tokens 6, 7 close it),
    page 1 receives tokens 8..10 and stays open."""
    P, Tp, H, d = 3, 8, 1, 2
    pk, pv, km, pp = _empty_pool(P, Tp, H, d)
    first = np.full((6, H, d), 2.0, np.float32)
    pk, pv, km, pp, done = oracle.page_commit(pk, pv, km, pp, first, first, fill=0, cur_prompt=1)
    assert done == []
    ramp = np.arange(5, dtype=np.float32)[:, None, None] * np.ones((5, H, d), np.float32)
    pk, pv, km, pp, done = oracle.page_commit(pk, pv, km, pp, ramp, ramp, fill=6, cur_prompt=4)
    assert done == [0]
    # page 0 = six 2.0 tokens, then ramp values 0 and 1: mean (12 + 0 + 1) / 8
    assert np.allclose(km[0], 13.0 / 8.0, rtol=0, atol=1e-15)
    assert pp.tolist() == [4, -1, -1]
    assert np.array_equal(km[1], np.full((H, d), -7.0))
    assert np.array_equal(pk[1, :3, 0, 0], [2.0, 3.0, 4.0])


def test_commit_of_chunks_equals_commit_of_their_concatenation():
    """Three-frame chunks into eight-frame pages (the pages' 480p setting in
    miniature): committing chunk by chunk equals committing all at once, and
    after 8 chunks exactly 3 pages are finalised."""
    rng = np.random.default_rng(9)
    P, Tp, H, d, n = 4, 16, 2, 4, 6          # a frame of 2 tokens; page = 8 frames, chunk = 3
    pk, pv, km, pp = _empty_pool(P, Tp, H, d)
    chunks = [rng.standard_normal((n, H, d)).astype(np.float32) for _ in range(8)]
    fill, all_done = 0, []
    for c in chunks:
        pk, pv, km, pp, done = oracle.page_commit(pk, pv, km, pp, c, -c, fill, cur_prompt=3)
        fill += n
        all_done += done
    assert all_done == [0, 1, 2]
    qk, qv, qkm, qpp, qdone = oracle.page_commit(*_empty_pool(P, Tp, H, d), np.concatenate(chunks),
                                                 -np.concatenate(chunks), 0, cur_prompt=3)
    assert qdone == [0, 1, 2]
    assert np.array_equal(qk, pk) and np.array_equal(qv, pv)
    assert np.array_equal(qkm[:3], km[:3]) and qpp.tolist() == pp.tolist() == [3, 3, 3, -1]
    # a finalised page's mean is the page summary of the page
    assert np.allclose(km[1], oracle.page_summary(pk[1:2].astype(np.float64))[0], rtol=0, atol=1e-15)
    with pytest.raises(ValueError):
        oracle.page_commit(pk, pv, km, pp, chunks[0], chunks[0], P * Tp - 2, 0)


# ---------------------------------------------------------------------------
# retrieval policies

def test_splitmix64_published_outputs():
    """The first outputs of SplitMix64 seeded with 0, as published with the
    generator's reference implementation."""
    assert oracle.splitmix64_at(0, 0) == 0xE220A8397B1DCDAF
    assert oracle.splitmix64_at(0, 1) == 0x6E789E6AA1B965F4
    assert oracle.splitmix64_at(0, 2) == 0x06C45D188009454F
    # output i of seed s is output i + 1 of seed s - golden ratio increment
    g = 0x9E3779B97F4A7C15
    assert oracle.splitmix64_at((5 - g) % 2 ** 64, 4) == oracle.splitmix64_at(5, 3)


def _policy_pool():
    # scores with qbar = e0 (one head): pages 0..5 score 1, -1, 0, 2, 1, 3
    kmean = np.zeros((6, 1, 2))
    kmean[:, 0, 0] = [1.0, -1.0, 0.0, 2.0, 1.0, 3.0]
    prompts = np.array([0, 1, 0, 0, 1, 1], np.int32)   # current prompt 0: pages 0, 2, 3
    return kmean, prompts, np.array([[1.0, 0.0]])


@pytest.mark.parametrize("policy,Kp,want", [
    ("two_stage", 2, [0, 3]),          # matching 0, 2, 3 by score 1, 0, 2: 3 then 0
    ("page_only", 2, [3, 5]),          # all pages: 5 (3), 3 (2)
    ("page_only", 3, [0, 3, 5]),       # then the tie 0/4 at 1 goes to 0
    ("prompt_only", 2, [2, 3]),        # two most recent matching
    ("recent", 2, [4, 5]),
    ("recent", 9, [0, 1, 2, 3, 4, 5]),
    ("mismatched", 2, [4, 5]),         # pages 1, 4, 5 of other prompts: 5 (3), 4 (1)
    ("mismatched", 4, [1, 4, 5]),
])
def test_retrieval_policies_hand_worked(policy, Kp, want):
    kmean, prompts, q = _policy_pool()
    idx, n = oracle.retrieve(kmean, prompts, 0, q, Kp, policy)
    assert idx.tolist() == want and n == len(want)


def test_random_policy_follows_its_keys():
    kmean, prompts, q = _policy_pool()
    for seed in (0, 1, 12345):
        keys = [oracle.splitmix64_at(seed, p) >> 40 for p in range(6)]
        want = sorted(sorted(range(6), key=lambda p: (-keys[p], p))[:3])
        assert oracle.retrieve(kmean, prompts, 0, q, 3, "random", seed)[0].tolist() == want
    a = oracle.retrieve(kmean, prompts, 0, q, 3, "random", 7)[0].tolist()
    assert a == oracle.retrieve(kmean, prompts, 0, q, 3, "random", 7)[0].tolist()
    with pytest.raises(ValueError):
        oracle.retrieve(kmean, prompts, 0, q, 3, "nearest")


# ---------------------------------------------------------------------------
# backward of the learned parameters: finite differences of the loss
# sum(d_out * O) through the forward's own gate, branch and fusion

def _bwd_case(seed=11, Lq=9, H=2, d=4, L=7, r=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Lq, H, d))
    K = rng.standard_normal((L, H, d))
    V = rng.standard_normal((L, H, d))
    E = rng.standard_normal((r, L)) / math.sqrt(L)
    F = rng.standard_normal((r, L)) / math.sqrt(L)
    w = rng.standard_normal((H, d)) / math.sqrt(d)
    b = rng.standard_normal(H) * 0.3
    o_s = rng.standard_normal((Lq, H, d)) * 0.1
    d_out = rng.standard_normal((Lq, H, d))
    return q, K, V, E, F, w, b, o_s, d_out


def _loss(q, K, V, E, F, w, b, o_s, d_out):
    o_l, _, _ = oracle.linear_branch(q, K, V, E, F)
    return float(np.sum(d_out * oracle.fuse(oracle.gate(q, w, b), o_s, o_l)))


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_backward_matches_finite_differences(seed):
    args = list(_bwd_case(seed))
    got = oracle.backward_params(*args)
    names = {3: "d_E", 4: "d_F", 5: "d_wg", 6: "d_bg"}
    eps = 1e-6
    for pos, name in names.items():
        base = args[pos]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            up, dn = base.copy(), base.copy()
            up[idx] += eps
            dn[idx] -= eps
            a_up, a_dn = list(args), list(args)
            a_up[pos], a_dn[pos] = up, dn
            num[idx] = (_loss(*a_up) - _loss(*a_dn)) / (2 * eps)
        assert np.allclose(got[name], num, rtol=1e-6, atol=1e-8), name


def test_backward_special_cases():
    q, K, V, E, F, w, b, o_s, d_out = _bwd_case(14)
    zero = oracle.backward_params(q, K, V, E, F, w, b, o_s, 0 * d_out)
    for k in ("d_wg", "d_bg", "d_E", "d_F"):
        assert np.array_equal(zero[k], 0 * zero[k])
    # a saturated gate (g = 1): no gradient reaches the gate or the low-rank branch
    sat = oracle.backward_params(q, K, V, E, F, 0 * w, np.full(len(b), 1e3), o_s, d_out)
    for k in ("d_wg", "d_bg", "d_E", "d_F"):
        assert np.all(sat[k] == 0)
    # g = 1/2 exactly (w = b = 0): db = sum_t <d_out, O_s - O_l> / 4
    half = oracle.backward_params(q, K, V, E, F, 0 * w, 0 * b, o_s, d_out)
    want = np.einsum("thd,thd->h", d_out, o_s - half["o_linear"]) / 4.0
    assert np.allclose(half["d_bg"], want, rtol=1e-13, atol=1e-14)
