"""Helpers of the GPU parity tests: device upload, the HIP path stage by
stage through the C ABI, and the comparison rules against the oracle.

Comparison rules (per-stage):
  * page_idx, n_sel: exactly equal; gathered K/V: bit for bit.
  * selection: identical sets, except blocks at the tau boundary: a block in
    the symmetric difference is allowed when the oracle's cumulative mass of
    the blocks ranked ahead of it is within 1e-4 of tau, or its mass is
    within 1e-4 of the oracle's last selected block.
  * floating outputs: float32 max-abs <= 1e-4 and relative Frobenius
    <= 1e-5; bf16 max-abs <= 2e-2, mean-abs <= 2e-3 and relative Frobenius
    <= 1e-2. The reference norm is printed beside every check.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
from block_sparse_rank_amd import hsakv as hs

BOUNDARY = 1e-4
TOL = {
    "f32": dict(max_abs=1e-4, mean_abs=None, rel=1e-5),
    "bf16": dict(max_abs=2e-2, mean_abs=2e-3, rel=1e-2),
}


def dims_of(s: synth.Shape) -> hs.Dims:
    return hs.make_dims(H=s.H, d=s.d, Lq=s.Lq, tokens_per_frame=s.tokens_per_frame,
                        Psize=s.Psize, P=s.P, Kp=s.Kp, Binter=s.Binter, Bintra=s.Bintra,
                        Bq=s.Bq, r=s.r, dtype=s.dtype)


def dev(arr: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    """Storage array -> device tensor with the same bits."""
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array (bf16 as uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def tdtype(s: synth.Shape):
    return torch.bfloat16 if s.dtype == "bf16" else torch.float32


def ws(d: hs.Dims, entry: int) -> torch.Tensor:
    n = hs.workspace_bytes(d, entry)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def compare(name: str, got: np.ndarray, ref: np.ndarray, dtype: str, **over) -> dict:
    tol = dict(TOL[dtype])
    tol.update(over)
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    diff = np.abs(got - ref)
    ref_norm = float(np.linalg.norm(ref))
    stats = dict(max_abs=float(diff.max()) if diff.size else 0.0,
                 mean_abs=float(diff.mean()) if diff.size else 0.0,
                 rel=float(np.linalg.norm(got - ref) / ref_norm) if ref_norm > 0 else 0.0,
                 ref_norm=ref_norm, ref_rms=float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0)
    print(f"[{name}] max_abs={stats['max_abs']:.3e} mean_abs={stats['mean_abs']:.3e} "
          f"rel={stats['rel']:.3e} |ref|={ref_norm:.4e} rms(ref)={stats['ref_rms']:.3e}", flush=True)
    assert stats["max_abs"] <= tol["max_abs"], (name, stats)
    if tol.get("mean_abs") is not None:
        assert stats["mean_abs"] <= tol["mean_abs"], (name, stats)
    if tol.get("rel") is not None:
        assert stats["rel"] <= tol["rel"], (name, stats)
    return stats


def check_selection(cnt: np.ndarray, idx: np.ndarray, mass: np.ndarray, sel, tau) -> list:
    """GPU selection (counts, ids) against the oracle's under the boundary rule.

    Returns the list of (h, i) rows whose sets differ (each allowed)."""
    H, NQB, NB = mass.shape
    differ = []
    for h in range(H):
        for i in range(NQB):
            c = int(cnt[h, i])
            assert 1 <= c <= NB, (h, i, c)
            ids = idx[h, i, :c]
            assert np.all(np.diff(ids) > 0) and ids[0] >= 0 and ids[-1] < NB, (h, i)
            g = set(ids.tolist())
            o = set(np.asarray(sel[h][i]).tolist())
            if g == o:
                continue
            m32 = mass[h, i].astype(np.float32)
            order = sorted(range(NB), key=lambda b: (-float(m32[b]), b))
            rank = {b: k for k, b in enumerate(order)}
            csum = np.cumsum([float(m32[b]) for b in order])
            p_last = float(m32[order[len(o) - 1]])
            for b in g ^ o:
                c_before = csum[rank[b]] - float(m32[b])
                ok = abs(c_before - float(tau[h])) <= BOUNDARY or abs(float(m32[b]) - p_last) <= BOUNDARY
                assert ok, f"row ({h},{i}) block {b}: not a boundary block"
            differ.append((h, i))
    return differ


def masked_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, ids, blocks) -> np.ndarray:
    """Library check, independent of the oracle: float64 attention of q [n][d]
    over the tokens of blocks `ids` of K, V [L][d] (torch's SDPA)."""
    J = np.concatenate([np.arange(blocks[b][0], blocks[b][1]) for b in ids])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(K[J]), t(V[J]))[0, 0].numpy()


def expected_sparse(s, ch, ref, cnt, idx, differ) -> np.ndarray:
    """The oracle's O_s, with each boundary row (h, i) in `differ` replaced by
    the library check of attention over the GPU's own (valid) set."""
    want = ref["o_sparse"].copy()
    if differ:
        q = oracle.as_f64(ch["q"], s.dtype)
        K = np.concatenate([oracle.as_f64(ref["k_hist"], s.dtype), oracle.as_f64(ch["k_intra"], s.dtype)])
        V = np.concatenate([oracle.as_f64(ref["v_hist"], s.dtype), oracle.as_f64(ch["v_intra"], s.dtype)])
        for (h, i) in differ:
            q0, q1 = ref["qblocks"][i]
            want[q0:q1, h] = masked_attention(q[q0:q1, h], K[:, h], V[:, h], idx[h, i, :cnt[h, i]].tolist(),
                                              ref["blocks"])
    return want


def pack_selection(sel, NB_max: int):
    """Oracle selection lists -> (sel_count [H][NQB], sel_idx [H][NQB][NB_max]) int32."""
    H, NQB = len(sel), len(sel[0])
    cnt = np.zeros((H, NQB), np.int32)
    idx = np.zeros((H, NQB, NB_max), np.int32)
    for h in range(H):
        for i in range(NQB):
            ids = np.asarray(sel[h][i], np.int32)
            cnt[h, i] = len(ids)
            idx[h, i, :len(ids)] = ids
    return cnt, idx


_FORK = None


def default_fork() -> "hs.Fork":
    """One fork (second stream and two events) for this process's tests, as a
    caller that keeps one for its forwards would."""
    global _FORK
    if _FORK is None:
        _FORK = hs.fork_create()
    return _FORK


class Case:
    """Inputs of one chunk-layer on the host (storage arrays) and on the device."""

    def __init__(self, s: synth.Shape, chunk: dict | None = None, pool=None, cur_prompt=None,
                 page_prompt=None, tau=None):
        self.s = s
        self.d = dims_of(s)
        assert hs.validate(self.d) == hs.OK
        self.ch = chunk if chunk is not None else synth.draw_chunk(s)
        if page_prompt is not None:
            self.ch["page_prompt"] = np.asarray(page_prompt, np.int32)
        if tau is not None:
            self.ch["tau"] = np.asarray(tau, np.float32)
        self.cur_prompt = s.cur_prompt if cur_prompt is None else cur_prompt
        self.pool_k, self.pool_v = pool if pool is not None else synth.draw_pool(s)
        ch = self.ch
        self.t = {k: dev(ch[k]) for k in ("q", "k_intra", "v_intra", "E", "F", "w_g", "b_g",
                                          "page_prompt")}
        self.t["pool_k"] = dev(self.pool_k)
        self.t["pool_v"] = dev(self.pool_v)

    # -- oracle ---------------------------------------------------------------
    def oracle(self, **kw) -> dict:  # noqa: D401 - keyword arguments go to oracle.forward
        s, ch = self.s, self.ch
        return oracle.forward(
            dtype=s.dtype, q=ch["q"], k_intra=ch["k_intra"], v_intra=ch["v_intra"],
            pool_k=self.pool_k, pool_v=self.pool_v, page_prompt=ch["page_prompt"],
            cur_prompt=self.cur_prompt, E=ch["E"], F=ch["F"], w_g=ch["w_g"], b_g=ch["b_g"],
            tau=ch["tau"], Kp=s.Kp, Binter=s.Binter, Bintra=s.Bintra, Bq=s.Bq, **kw)

    # -- HIP path, stage by stage ---------------------------------------------------
    def page_summary(self) -> torch.Tensor:
        s = self.s
        km = torch.empty((s.P, s.H, s.d), dtype=torch.float32, device="cuda")
        hs.hkv_page_summary(self.d, self.t["pool_k"], km)
        return km

    def gather(self, page_kmean: torch.Tensor, policy=None, seed=0):
        s, d = self.s, self.d
        page_idx = torch.full((s.Kp,), -7, dtype=torch.int32, device="cuda")
        n_sel = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        k_hist = torch.zeros((s.Kp * s.Tp, s.H, s.d), dtype=tdtype(s), device="cuda")
        v_hist = torch.zeros_like(k_hist)
        hs.hkv_gather(d, self.t["pool_k"], self.t["pool_v"], page_kmean, self.t["page_prompt"],
                      self.cur_prompt, self.t["q"], page_idx, n_sel, k_hist, v_hist,
                      ws(d, hs.ENTRY_GATHER), policy=policy, seed=seed)
        return page_idx, n_sel, k_hist, v_hist

    def select(self, k_hist, n_sel, tau=None):
        s, d = self.s, self.d
        cnt = torch.zeros((s.H, d.NQB), dtype=torch.int32, device="cuda")
        idx = torch.full((s.H, d.NQB, d.NB_max), -1, dtype=torch.int32, device="cuda")
        mask = torch.zeros((s.H, d.NQB, d.NB_max), dtype=torch.uint8, device="cuda")
        mass = torch.zeros((s.H, d.NQB, d.NB_max), dtype=torch.float32, device="cuda")
        hs.hsa_select(d, self.t["q"], k_hist, self.t["k_intra"], n_sel,
                      self.ch["tau"] if tau is None else tau, cnt, idx, mask, mass,
                      ws(d, hs.ENTRY_SELECT))
        return cnt, idx, mask, mass

    def sparse(self, k_hist, v_hist, n_sel, cnt, idx):
        s, d = self.s, self.d
        o = torch.full((s.Lq, s.H, s.d), float("nan"), dtype=torch.float32, device="cuda")
        hs.hsa_sparse_attn(d, self.t["q"], k_hist, v_hist, self.t["k_intra"], self.t["v_intra"],
                           n_sel, cnt, idx, o, ws(d, hs.ENTRY_SPARSE))
        return o

    def linear(self, k_hist, v_hist, n_sel):
        s, d = self.s, self.d
        o = torch.full((s.Lq, s.H, s.d), float("nan"), dtype=torch.float32, device="cuda")
        kl = torch.zeros((s.r, s.H, s.d), dtype=torch.float32, device="cuda")
        vl = torch.zeros_like(kl)
        hs.hsa_linear_branch(d, self.t["q"], k_hist, v_hist, self.t["k_intra"], self.t["v_intra"],
                             n_sel, self.t["E"], self.t["F"], o, kl, vl, ws(d, hs.ENTRY_LINEAR))
        return o, kl, vl

    def fuse(self, o_s, o_l):
        s, d = self.s, self.d
        out = torch.zeros((s.Lq, s.H, s.d), dtype=tdtype(s), device="cuda")
        gate = torch.zeros((s.Lq, s.H), dtype=torch.float32, device="cuda")
        hs.hsa_fuse(d, self.t["q"], self.t["w_g"], self.t["b_g"], o_s, o_l, out, gate)
        return out, gate

    def forward(self, page_kmean, debug=True, fork="default", policy=None, seed=0, tiers=None):
        s, d = self.s, self.d
        outs = {"out": torch.zeros((s.Lq, s.H, s.d), dtype=tdtype(s), device="cuda")}
        if debug:
            outs.update(
                page_idx=torch.zeros((s.Kp,), dtype=torch.int32, device="cuda"),
                n_sel=torch.zeros((1,), dtype=torch.int32, device="cuda"),
                sel_count=torch.zeros((s.H, d.NQB), dtype=torch.int32, device="cuda"),
                sel_idx=torch.zeros((s.H, d.NQB, d.NB_max), dtype=torch.int32, device="cuda"),
                o_sparse=torch.zeros((s.Lq, s.H, s.d), dtype=torch.float32, device="cuda"),
                o_linear=torch.zeros((s.Lq, s.H, s.d), dtype=torch.float32, device="cuda"),
                gate=torch.zeros((s.Lq, s.H), dtype=torch.float32, device="cuda"),
                k_hist=torch.zeros((s.Kp * s.Tp, s.H, s.d), dtype=tdtype(s), device="cuda"),
                v_hist=torch.zeros((s.Kp * s.Tp, s.H, s.d), dtype=tdtype(s), device="cuda"),
            )
        ins = {k: self.t[k] for k in ("q", "k_intra", "v_intra", "pool_k", "pool_v", "E", "F",
                                      "w_g", "b_g", "page_prompt")}
        ins["page_kmean"] = page_kmean
        if fork == "default":
            fork = default_fork()
        hs.hsa_forward(d, self.ch["tau"], self.cur_prompt, ins, outs, ws(d, hs.ENTRY_FORWARD),
                       fork=fork, policy=policy, seed=seed, tiers=tiers)
        return outs
