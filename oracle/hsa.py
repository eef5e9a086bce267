"""Plain float64 CPU oracle of WorldAttention's HSA forward over an HKV active set.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU
baseline may import this module. The product path never calls it, and this
module imports nothing from the HIP path (nor torch): it is NumPy only.

What it follows. The pages are five web pages about the paper "WorldAttention:
An Efficient Attention Architecture for Interactive Video World Models"
(arXiv 2609.34606). The technical content is in the ai4snews news summary
(English and Chinese editions, same six paragraphs): the HKV paragraph
(semantic pages of Psize = 8 frames, two-stage prompt-level then page-level
retrieval of a top-Kp active cache), the HSA paragraph (a Linformer-style
low-rank global branch and a head-adaptive block-sparse branch that keeps,
per head, the fewest blocks whose cumulative attention mass reaches tau_h,
with Binter = 128 for history and Bintra = 64 inside the chunk, fused by
learned gates) and the kernel paragraph (KV reorganisation and contiguous
copies dominate). The open-questions paragraph states that Top-1 prompt
retrieval is what is used. The Linformer paper (cited on the mlsanity map)
defines the low-rank projection.

The pages give no equations. Every step below states the reading it takes
where they are silent; the readings are numbered R1..R28 and listed, with
reasons, in the design notes of this repository.

Decision precision. Page ranking and block selection turn floating point
into integers. The pages fix no precision, so both sides take those
decisions in the kernels' float32: the oracle computes scores and masses in
float64 and rounds them to float32 before ranking and before comparing
cumulative mass with tau_h.

Parity pins: every function here is pinned by a test in tests/ against
closed forms, brute force or library routines (see each docstring). The
whole forward at the full workloads has no printed worked example on the
pages: beyond those pins, parity there is unpinned and the oracle is the
definition.
"""

from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

__all__ = [
    "as_f64",
    "page_summary",
    "chunk_query_mean",
    "prompt_filter",
    "page_scores",
    "retrieve",
    "gather",
    "block_table",
    "query_blocks",
    "concat_keys",
    "pool_blocks",
    "block_mass",
    "select_row",
    "select",
    "sparse_attention_row",
    "sparse_attention",
    "active_projection_columns",
    "linear_branch",
    "gate",
    "fuse",
    "forward",
    "page_commit",
    "POLICIES",
    "splitmix64_at",
    "backward_params",
]


# ---------------------------------------------------------------------------
# values

def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage values -> float64, exactly. bf16 arrives as uint16 bit patterns."""
    if dtype == "bf16":
        if x.dtype != np.uint16:
            raise TypeError("bf16 tensors are passed as uint16 bit patterns")
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        if x.dtype != np.float32:
            raise TypeError("f32 tensors are passed as float32")
        return x.astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# HKV: page summary and two-stage retrieval (news summary, HKV paragraph;
# open-questions paragraph for Top-1; project page, second figure caption)

def page_summary(pool_k: np.ndarray) -> np.ndarray:
    """O1. Page-mean key kbar[p, h, :] = mean over the page's tokens.

    Commit-time metadata of each semantic page (reading R2).
    pool_k: [P][Tp][H][d] float64 -> [P][H][d] float64.
    """
    return pool_k.mean(axis=1)


def chunk_query_mean(q: np.ndarray) -> np.ndarray:
    """O2. Chunk-mean query qbar[h, :] over the chunk's Lq tokens. [Lq][H][d] -> [H][d]."""
    return q.mean(axis=0)


def prompt_filter(page_prompt: np.ndarray, cur_prompt: int) -> List[int]:
    """O3. Prompt-level stage: the pages tagged with the current prompt, ascending.

    Reading R1: prompt matching is equality of integer prompt ids (the one
    matching prompt is the Top-1 prompt the pages say is used).
    """
    return [p for p in range(len(page_prompt)) if int(page_prompt[p]) == int(cur_prompt)]


def page_scores(page_kmean: np.ndarray, qbar: np.ndarray, pages: Sequence[int]) -> Dict[int, float]:
    """O4. Page-level score s_p = sum over heads and dims of kbar[p] * qbar (reading R2).

    Returned rounded to float32: the ranking decision is taken in the
    kernels' precision. A score that is not a number (a page mean or a query
    holding an infinity or a NaN) is taken as -infinity, so such a page
    ranks below every page with a number (reading R24).
    """
    out = {}
    for p in pages:
        s = float(np.sum(page_kmean[p] * qbar))
        out[p] = -math.inf if math.isnan(s) else float(np.float32(s))
    return out


# Retrieval policies: the method's two-stage retrieval and the alternatives
# the pages compare it with under the same page budget (news summary, HKV
# paragraph, Table 6: page-only, prompt-only, recent-page, random-page and
# mismatched-page retrieval; Table 5: a sliding window of recent frames,
# which is the recent-page policy).
POLICIES = ("two_stage", "page_only", "prompt_only", "recent", "random", "mismatched")


def splitmix64_at(seed: int, i: int) -> int:
    """Output i (0-based) of the SplitMix64 generator seeded with `seed`
    (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
    OOPSLA 2014): state seed + (i + 1) * 0x9E3779B97F4A7C15 mod 2^64, then
    the generator's output mix."""
    M = (1 << 64) - 1
    z = (seed + (i + 1) * 0x9E3779B97F4A7C15) & M
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
    return z ^ (z >> 31)


def retrieve(page_kmean: np.ndarray, page_prompt: np.ndarray, cur_prompt: int,
             qbar: np.ndarray, Kp: int, policy: str = "two_stage",
             seed: int = 0) -> Tuple[np.ndarray, int]:
    """O3-O5. Retrieval of Kp pages.

    two_stage (the method): candidates are the prompt-matching pages; they
    are ordered by score, higher first, equal scores to the lower page
    index; the first min(Kp, |candidates|) are kept and put in ascending
    page order, which is their slot order in the active cache (reading R3).
    The alternatives change only the candidates and the ranking key
    (reading R27): page_only ranks every page by score; prompt_only keeps the
    Kp most recent (highest-index) matching pages; recent the Kp most recent
    pages; random every page by the top 24 bits of SplitMix64 output p for
    the given seed (so a draw is reproducible); mismatched ranks the pages of
    other prompts by score.
    Returns (page_idx int32 [n_sel], n_sel).
    """
    P = len(page_prompt)
    if policy in ("two_stage", "prompt_only"):
        cand = prompt_filter(page_prompt, cur_prompt)
    elif policy == "mismatched":
        match = set(prompt_filter(page_prompt, cur_prompt))
        cand = [p for p in range(P) if p not in match]
    elif policy in ("page_only", "recent", "random"):
        cand = list(range(P))
    else:
        raise ValueError(policy)
    if policy in ("two_stage", "page_only", "mismatched"):
        s = page_scores(page_kmean, qbar, cand)
    elif policy in ("prompt_only", "recent"):
        s = {p: float(p) for p in cand}
    else:
        s = {p: float(splitmix64_at(seed, p) >> 40) for p in cand}
    ranked = sorted(cand, key=lambda p: (-s[p], p))
    chosen = sorted(ranked[:Kp])
    return np.array(chosen, dtype=np.int32), len(chosen)


def gather(pool: np.ndarray, page_idx: np.ndarray) -> np.ndarray:
    """O6. Active-cache assembly (news summary, kernel paragraph: contiguous copies).

    Slot s holds pool page page_idx[s]; slots are stacked along tokens:
    out[s*Tp + t] = pool[page_idx[s], t] (reading R4). Works on any storage
    type, bit for bit. pool: [P][Tp][H][d] -> [n_sel*Tp][H][d].
    """
    P, Tp = pool.shape[0], pool.shape[1]
    out = np.empty((len(page_idx) * Tp,) + pool.shape[2:], dtype=pool.dtype)
    for s, p in enumerate(page_idx):
        out[s * Tp:(s + 1) * Tp] = pool[int(p)]
    return out


# ---------------------------------------------------------------------------
# HSA sparse branch (news summary, HSA paragraph)

def block_table(Lh: int, Lq: int, Binter: int, Bintra: int) -> List[Tuple[int, int]]:
    """O7. Key blocks as [start, end) token ranges of the key sequence [history; chunk].

    History keys are tiled by Binter, the chunk's keys by Bintra; the last
    block of each part may be ragged. Ids run over history first, then the
    chunk (reading R5).
    """
    blocks = []
    for b in range(-(-Lh // Binter)):
        blocks.append((b * Binter, min((b + 1) * Binter, Lh)))
    for j in range(-(-Lq // Bintra)):
        blocks.append((Lh + j * Bintra, Lh + min((j + 1) * Bintra, Lq)))
    return blocks


def query_blocks(Lq: int, Bq: int) -> List[Tuple[int, int]]:
    """O7. Query blocks [start, end) of size Bq, the last ragged (reading R6)."""
    return [(i * Bq, min((i + 1) * Bq, Lq)) for i in range(-(-Lq // Bq))]


def concat_keys(hist: np.ndarray, intra: np.ndarray) -> np.ndarray:
    """O7. The key (or value) sequence: retrieved history followed by the chunk's own."""
    return np.concatenate([hist, intra], axis=0)


def pool_blocks(x: np.ndarray, ranges: Sequence[Tuple[int, int]]) -> np.ndarray:
    """O8. Block pooling: the mean over each block's valid tokens (reading R7).

    x: [L][H][d] -> [H][n_blocks][d].
    """
    H, d = x.shape[1], x.shape[2]
    out = np.empty((H, len(ranges), d), dtype=np.float64)
    for b, (s, e) in enumerate(ranges):
        out[:, b, :] = x[s:e].mean(axis=0)
    return out


def block_mass(qb: np.ndarray, kb: np.ndarray) -> np.ndarray:
    """O9. Block attention mass: softmax over all key blocks of the pooled logits.

    z[h, i, b] = <qb[h, i], kb[h, b]> / sqrt(d), and the mass of a row
    (h, i) is the softmax of z over b, history and chunk blocks jointly
    (readings R8, R11). qb: [H][NQB][d], kb: [H][NB][d] -> [H][NQB][NB].
    """
    d = qb.shape[-1]
    z = np.matmul(qb, np.swapaxes(kb, 1, 2)) / math.sqrt(d)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def select_row(mass: np.ndarray, tau: float) -> np.ndarray:
    """O10. Head-adaptive minimal block set of one (head, query block) row.

    Blocks are ranked by mass, larger first, equal masses to the lower
    block id. The set is the shortest prefix of that ranking whose
    cumulative mass reaches tau (>=, so tau = 1.00 is reachable); at least
    one block is kept; tau >= 1 keeps every block; if rounding keeps the
    total below tau, every block is kept (reading R9). Masses and
    cumulative sums are compared in float32, the kernels' precision.
    Returns the selected block ids, ascending, int32.
    """
    nb = mass.shape[0]
    tau32 = np.float32(tau)
    if tau32 >= np.float32(1.0):
        return np.arange(nb, dtype=np.int32)
    m32 = mass.astype(np.float32)
    order = sorted(range(nb), key=lambda b: (-float(m32[b]), b))
    c = 0.0
    for k, b in enumerate(order, start=1):
        c += float(m32[b])
        if np.float32(c) >= tau32:
            return np.array(sorted(order[:k]), dtype=np.int32)
    return np.arange(nb, dtype=np.int32)


def select(mass: np.ndarray, tau: Sequence[float]) -> List[List[np.ndarray]]:
    """O10 for every row: sel[h][i] = selected block ids of row (h, i)."""
    H, NQB = mass.shape[0], mass.shape[1]
    return [[select_row(mass[h, i], float(tau[h])) for i in range(NQB)] for h in range(H)]


def _tokens_of(ids: Sequence[int], blocks: Sequence[Tuple[int, int]]) -> np.ndarray:
    parts = [np.arange(blocks[b][0], blocks[b][1]) for b in ids]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def sparse_attention_row(q: np.ndarray, K: np.ndarray, V: np.ndarray, h: int,
                         qrange: Tuple[int, int], ids: Sequence[int],
                         blocks: Sequence[Tuple[int, int]]) -> np.ndarray:
    """O11 for one row: exact softmax attention of the row's queries over the
    tokens of its selected blocks only, scale 1/sqrt(d), no mask
    (readings R10, R11). Returns [rows][d].
    """
    d = q.shape[-1]
    J = _tokens_of(ids, blocks)
    qs = q[qrange[0]:qrange[1], h, :]
    kj = K[J, h, :]
    vj = V[J, h, :]
    logits = qs @ kj.T / math.sqrt(d)
    logits = logits - logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w /= w.sum(axis=1, keepdims=True)
    return w @ vj


def sparse_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                     sel: Sequence[Sequence[Sequence[int]]],
                     blocks: Sequence[Tuple[int, int]],
                     qblocks: Sequence[Tuple[int, int]]) -> np.ndarray:
    """O11 for every row. q: [Lq][H][d]; K, V: [L][H][d] -> O_s [Lq][H][d]."""
    out = np.zeros(q.shape, dtype=np.float64)
    for h in range(q.shape[1]):
        for i, qr in enumerate(qblocks):
            out[qr[0]:qr[1], h, :] = sparse_attention_row(q, K, V, h, qr, sel[h][i], blocks)
    return out


# ---------------------------------------------------------------------------
# HSA linear branch (news summary, HSA paragraph; Linformer projection)

def active_projection_columns(n_sel: int, Kp: int, Tp: int, Lq: int) -> np.ndarray:
    """O12. Columns of E and F that face the present keys.

    E and F have L = Kp*Tp + Lq columns in key order: slot s owns columns
    [s*Tp, (s+1)*Tp), the chunk owns the last Lq. Columns of absent slots
    (s >= n_sel) are skipped (reading R12).
    """
    return np.concatenate([np.arange(n_sel * Tp), Kp * Tp + np.arange(Lq)])


def linear_branch(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                  E_act: np.ndarray, F_act: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """O12. Linformer-style low-rank global attention, one E and one F shared by heads.

    K'_h = E_act K_h and V'_h = F_act V_h (each r x d), then
    O_l = softmax(q K'^T / sqrt(d)) V' per head (reading R12).
    Returns (O_l [Lq][H][d], K' [r][H][d], V' [r][H][d]).
    """
    Lq, H, d = q.shape
    r = E_act.shape[0]
    Kp_ = np.empty((r, H, d))
    Vp_ = np.empty((r, H, d))
    out = np.empty((Lq, H, d))
    for h in range(H):
        kh = E_act @ K[:, h, :]
        vh = F_act @ V[:, h, :]
        Kp_[:, h, :] = kh
        Vp_[:, h, :] = vh
        logits = q[:, h, :] @ kh.T / math.sqrt(d)
        logits = logits - logits.max(axis=1, keepdims=True)
        w = np.exp(logits)
        w /= w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ vh
    return out, Kp_, Vp_


# ---------------------------------------------------------------------------
# gated fusion (news summary, HSA paragraph: learned gates)

def gate(q: np.ndarray, w_g: np.ndarray, b_g: np.ndarray) -> np.ndarray:
    """O13. Per-token, per-head sigmoid gate g = sigma(<q[t,h], w_g[h]> + b_g[h]) (reading R13).

    Evaluated in the overflow-free form. [Lq][H][d] -> [Lq][H].
    """
    x = np.einsum("thd,hd->th", q, w_g) + b_g[None, :]
    g = np.empty_like(x)
    pos = x >= 0
    g[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    g[~pos] = ex / (1.0 + ex)
    return g


def fuse(g: np.ndarray, o_s: np.ndarray, o_l: np.ndarray) -> np.ndarray:
    """O13. Convex combination O = g O_s + (1 - g) O_l (reading R13)."""
    gg = g[:, :, None]
    return gg * o_s + (1.0 - gg) * o_l


# ---------------------------------------------------------------------------
# the whole chunk-layer

def forward(*, dtype: str, q, k_intra, v_intra, pool_k, pool_v, page_prompt, cur_prompt: int,
            E, F, w_g, b_g, tau, Kp: int, Binter: int, Bintra: int, Bq: int,
            page_kmean=None, heads=None, rows=None, policy: str = "two_stage",
            seed: int = 0) -> Dict[str, object]:
    """O1-O13 for one chunk-layer, returning every intermediate.

    Tensors arrive in their storage type (bf16 as uint16 bits, f32 as
    float32) and are upcast exactly. `page_kmean` may be passed in (it is
    commit-time metadata); otherwise it is computed from the pool.
    `heads` restricts the per-head stages to a subset (retrieval always uses
    every head); `rows` further restricts the sparse branch to a list of
    (h, i) rows. The pool may be a [P][Tp][H][d] array or a callable
    returning page p's [Tp][H][d] storage array. `policy` and `seed` select
    the retrieval policy (two-stage by default).
    """
    qf = as_f64(q, dtype)
    Lq, H, d = qf.shape
    P = len(page_prompt)

    def page(arr, p):
        return arr(p) if callable(arr) else arr[p]

    if page_kmean is None:
        page_kmean = np.stack([page_summary(as_f64(page(pool_k, p), dtype)[None])[0]
                               for p in range(P)])
    qbar = chunk_query_mean(qf)
    page_idx, n_sel = retrieve(page_kmean, page_prompt, cur_prompt, qbar, Kp, policy, seed)

    hsel = list(range(H)) if heads is None else list(heads)
    Tp = page(pool_k, 0).shape[0]
    k_hist = np.concatenate([page(pool_k, int(p))[:, hsel] for p in page_idx]) if n_sel else \
        np.zeros((0, len(hsel), d), dtype=page(pool_k, 0).dtype)
    v_hist = np.concatenate([page(pool_v, int(p))[:, hsel] for p in page_idx]) if n_sel else \
        np.zeros((0, len(hsel), d), dtype=page(pool_v, 0).dtype)
    Lh = n_sel * Tp

    K = concat_keys(as_f64(k_hist, dtype), as_f64(k_intra, dtype)[:, hsel])
    V = concat_keys(as_f64(v_hist, dtype), as_f64(v_intra, dtype)[:, hsel])
    qh = qf[:, hsel]
    blocks = block_table(Lh, Lq, Binter, Bintra)
    qblocks = query_blocks(Lq, Bq)
    kb = pool_blocks(K, blocks)
    qb = pool_blocks(qh, qblocks)
    mass = block_mass(qb, kb)
    tau_h = [float(tau[h]) for h in hsel]
    sel = select(mass, tau_h)

    if rows is None:
        o_s = sparse_attention(qh, K, V, sel, blocks, qblocks)
    else:
        o_s = {}
        for (h, i) in rows:
            hi = hsel.index(h)
            o_s[(h, i)] = sparse_attention_row(qh, K, V, hi, qblocks[i], sel[hi][i], blocks)

    cols = active_projection_columns(n_sel, Kp, Tp, Lq)
    E_act = as_f64(E, dtype)[:, cols]
    F_act = as_f64(F, dtype)[:, cols]
    o_l, k_low, v_low = linear_branch(qh, K, V, E_act, F_act)
    g = gate(qh, np.asarray(w_g, np.float64)[hsel], np.asarray(b_g, np.float64)[hsel])
    out = fuse(g, o_s, o_l) if rows is None else None

    return {
        "page_kmean": page_kmean, "qbar": qbar, "page_idx": page_idx, "n_sel": n_sel,
        "k_hist": k_hist, "v_hist": v_hist, "heads": hsel, "blocks": blocks, "qblocks": qblocks,
        "qb": qb, "kb": kb, "mass": mass, "sel": sel, "o_sparse": o_s, "o_linear": o_l,
        "k_low": k_low, "v_low": v_low, "gate": g, "out": out,
    }


# ---------------------------------------------------------------------------
# HKV page commit (news summary, HKV paragraph: history KV pairs partitioned
# into semantic pages of Psize frames, each page indexed for the prompt-level
# and page-level retrieval stages; project page, second figure caption)

def page_commit(pool_k: np.ndarray, pool_v: np.ndarray, page_kmean: np.ndarray,
                page_prompt: np.ndarray, k_chunk: np.ndarray, v_chunk: np.ndarray,
                fill: int, cur_prompt: int):
    """Append one chunk's keys and values to the page pool and finalise the
    pages it completes.

    The history is one token sequence cut into pages of Tp tokens, page p
    holding tokens [p Tp, (p + 1) Tp); `fill` tokens are already committed,
    so the chunk's token j becomes history token fill + j (reading R25). A
    page is finalised by the commit that writes its last token: its
    page-mean key (the metadata the page-level stage scores) is the mean of
    its Tp keys, and it is tagged with that commit's prompt id (reading R26).
    Pages not completed keep their mean and tag.

    pool_k, pool_v: [P][Tp][H][d] storage arrays (bf16 bits or float32);
    page_kmean [P][H][d] float64; page_prompt [P] int; k_chunk, v_chunk
    [n][H][d] storage arrays. Returns new (pool_k, pool_v, page_kmean,
    page_prompt, finalised page ids); the inputs are not modified.
    """
    P, Tp = pool_k.shape[0], pool_k.shape[1]
    n = k_chunk.shape[0]
    if fill < 0 or fill + n > P * Tp:
        raise ValueError("the chunk does not fit in the pool")
    pk, pv = pool_k.copy(), pool_v.copy()
    km, pp = np.array(page_kmean, dtype=np.float64), np.array(page_prompt).copy()
    for j in range(n):
        t = fill + j
        pk[t // Tp, t % Tp] = k_chunk[j]
        pv[t // Tp, t % Tp] = v_chunk[j]
    done = [p for p in range(P) if fill < (p + 1) * Tp <= fill + n]
    dtype = "bf16" if pk.dtype == np.uint16 else "f32"
    for p in done:
        km[p] = page_summary(as_f64(pk[p], dtype)[None])[0]
        pp[p] = cur_prompt
    return pk, pv, km, pp, done


# ---------------------------------------------------------------------------
# backward of the learned parameters (news summary, HSA paragraph: the gates
# are learned; the Linformer projections E and F are the low-rank branch's
# parameters)

def backward_params(q: np.ndarray, K: np.ndarray, V: np.ndarray, E_act: np.ndarray, F_act: np.ndarray,
                    w_g: np.ndarray, b_g: np.ndarray, o_s: np.ndarray, d_out: np.ndarray) -> Dict[str, np.ndarray]:
    """Gradients of a loss with upstream gradient d_out = dLoss/dO with
    respect to the gate parameters w_g [H][d], b_g [H] and the projections
    E_act, F_act [r][L_act] (reading R28: the sparse branch has no learned
    parameter and is held fixed).

    With O = g O_s + (1 - g) O_l and g = sigma(x), x = <q, w_g[h]> + b_g[h]:
      dLoss/dx = <d_out, O_s - O_l> g (1 - g),
      dw_g[h] = sum_t dx[t, h] q[t, h],  db_g[h] = sum_t dx[t, h];
    and for the low-rank branch, with dO_l = (1 - g) d_out, P = softmax(S),
    S = q K'^T / sqrt(d), K' = E_act K_h, V' = F_act V_h (per head):
      dV' = P^T dO_l,  dS = P * (dO_l V'^T - rowsum(dO_l * O_l)),
      dK' = dS^T q / sqrt(d),
      dE_act = sum_h dK'_h K_h^T,  dF_act = sum_h dV'_h V_h^T.
    Inputs float64: q [Lq][H][d], K, V [L_act][H][d], o_s, d_out [Lq][H][d].
    """
    Lq, H, d = q.shape
    r = E_act.shape[0]
    x = np.einsum("thd,hd->th", q, w_g) + b_g[None, :]
    g = gate(q, w_g, b_g)
    o_l, k_low, v_low = linear_branch(q, K, V, E_act, F_act)
    dx = np.einsum("thd,thd->th", d_out, o_s - o_l) * g * (1.0 - g)
    d_wg = np.einsum("th,thd->hd", dx, q)
    d_bg = dx.sum(axis=0)
    dE = np.zeros_like(E_act)
    dF = np.zeros_like(F_act)
    dKl = np.empty((r, H, d))
    dVl = np.empty((r, H, d))
    for h in range(H):
        dol = (1.0 - g[:, h])[:, None] * d_out[:, h, :]
        logits = q[:, h, :] @ k_low[:, h, :].T / math.sqrt(d)
        logits = logits - logits.max(axis=1, keepdims=True)
        P = np.exp(logits)
        P /= P.sum(axis=1, keepdims=True)
        dV = P.T @ dol
        dP = dol @ v_low[:, h, :].T
        Dt = np.sum(dol * o_l[:, h, :], axis=1, keepdims=True)
        dS = P * (dP - Dt)
        dK = dS.T @ q[:, h, :] / math.sqrt(d)
        dKl[:, h, :] = dK
        dVl[:, h, :] = dV
        dE += dK @ K[:, h, :].T
        dF += dV @ V[:, h, :].T
    del x
    return {"d_wg": d_wg, "d_bg": d_bg, "d_E": dE, "d_F": dF, "d_klow": dKl, "d_vlow": dVl, "gate": g,
            "o_linear": o_l, "k_low": k_low, "v_low": v_low}
