"""GPU parity of the backward of the learned parameters (hsa_backward_params)
with the oracle's backward_params: gradients of the gate weights and biases
and of the projections E and F for a seeded upstream gradient.

Two bars, both element by element over every output:

* stage: the GPU backward is fed the oracle's forward values (K', V', the
  low-rank output and the sparse output, rounded once to float32), so only
  its own arithmetic differs from the float64 oracle. Its float32 sums over
  at most Lq tokens and H d columns, the float32 exp / log of the recomputed
  probabilities and the bf16 hi + lo split of dK', dV' (remainder rounded at
  2^-9 of a part already 2^-9 below the value, so 2^-18 relative) keep the
  relative Frobenius error well below 2e-5; the largest element error stays
  below 1e-4 of the largest reference element.
* end to end: the GPU backward is fed the GPU forward's own saved values
  (bf16 products in the forward), against the oracle on its own forward; the
  bar is the bf16 one of the forward tests, relative to the reference's
  scale: Frobenius 1e-2, largest element error 2e-2 of the largest element.
  Rows whose sparse block set differs from the oracle's at the tau boundary
  get the oracle-side sparse output of attention over the GPU's own set
  (torch SDPA in float64), as in the forward tests.

Columns of E and F facing absent slots are exactly zero.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402
from block_sparse_rank_amd import hsakv as hs  # noqa: E402
from gpu_util import Case, check_selection, default_fork, dev, expected_sparse, host, ws  # noqa: E402

STAGE = dict(rel=2e-5, max_rel=1e-4)
E2E = dict(rel=1e-2, max_rel=2e-2)


def _v(name, **over):
    return synth.shape("tiny").with_(**over)


# (id, shape, Case keyword arguments, b_g override or None). All bf16 (the
# entry point's storage type).
VARIANTS = [
    ("tiny-bf16", _v("tiny", dtype="bf16", clustered=True, tau_law="uniform", seed=7), {}, None),
    ("d128-r64-kp3", _v("tiny", dtype="bf16", d=128, H=3, r=64, Kp=3, P=8, clustered=True,
                        tau_law="uniform", seed=16), {}, None),
    # two 256-row tiles of r, the second ragged; H d = 256
    ("r320-hd256", _v("tiny", dtype="bf16", H=4, d=64, r=320, Lq=136, tokens_per_frame=13, P=8, Kp=3,
                      clustered=True, tau_law="uniform", seed=26), {}, None),
    # 104-token pages: 64-column tiles straddle the slot seams and the history/chunk seam
    ("r128-seam", _v("tiny", dtype="bf16", H=2, d=128, r=128, Lq=200, tokens_per_frame=13,
                     clustered=True, tau_law="uniform", seed=25), {}, None),
    # Lq = 77 queries: a ragged last query slice and ragged E/F column tile
    ("odd-Lq77", _v("tiny", dtype="bf16", Lq=77, tokens_per_frame=25, Psize=4, clustered=True,
                    tau_law="uniform", seed=19), {}, None),
    # no page of the current prompt: every history column of E and F is absent
    ("no-page", _v("tiny", dtype="bf16", H=4, d=128, clustered=True, tau_law="uniform", seed=20),
     dict(cur_prompt=9), None),
    # one matching page for two slots; saturated and offset gates
    ("one-page-gates", _v("tiny", dtype="bf16", P=3, H=3, clustered=True, tau_law="uniform", seed=18),
     dict(page_prompt=[1, 0, 1]), [9.0, -9.0, 0.7]),
]


def _rel_compare(name, got, ref, rel, max_rel):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name
    scale = float(np.abs(ref).max())
    nrm = float(np.linalg.norm(ref))
    e_max = float(np.abs(got - ref).max())
    e_rel = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got))
    print(f"[{name}] rel={e_rel:.3e} max_abs={e_max:.3e} max|ref|={scale:.3e}", flush=True)
    if nrm == 0:
        assert e_max == 0.0, name
        return
    assert e_rel <= rel, (name, e_rel)
    assert e_max <= max_rel * scale, (name, e_max, scale)


def _active_cols(s, n_sel):
    return oracle.active_projection_columns(n_sel, s.Kp, s.Tp, s.Lq)


def _backward(d, s, t, k_hist, v_hist, n_sel, k_low, v_low, o_s, o_l, d_out, w_g, b_g, fork=None):
    out = dict(d_wg=torch.full((s.H, s.d), float("nan"), device="cuda"),
               d_bg=torch.full((s.H,), float("nan"), device="cuda"),
               d_E=torch.full((s.r, s.L), float("nan"), device="cuda"),
               d_F=torch.full((s.r, s.L), float("nan"), device="cuda"))
    hs.hsa_backward_params(d, t["q"], k_hist, v_hist, t["k_intra"], t["v_intra"], n_sel, w_g, b_g,
                           k_low, v_low, o_s, o_l, d_out, out["d_wg"], out["d_bg"], out["d_E"], out["d_F"],
                           ws(d, hs.ENTRY_BACKWARD), fork=fork)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def _check(tag, s, got, want, n_sel, bar):
    cols = _active_cols(s, n_sel)
    absent = np.setdiff1d(np.arange(s.L), cols)
    for k in ("d_E", "d_F"):
        assert np.all(got[k][:, absent] == 0.0), f"{k}: absent columns not zero"
        _rel_compare(f"{tag} {k}", got[k][:, cols], want[k], **bar)
    _rel_compare(f"{tag} d_wg", got["d_wg"], want["d_wg"], **bar)
    _rel_compare(f"{tag} d_bg", got["d_bg"], want["d_bg"], **bar)


def _setup(s, kw, bg):
    c = Case(s, **kw)
    if bg is not None:
        c.ch["b_g"] = np.asarray(bg, np.float32)
        c.t["b_g"] = dev(c.ch["b_g"])
    return c


@pytest.mark.parametrize("vid,s,kw,bg", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_backward_stage_and_end_to_end(vid, s, kw, bg):
    print(f"[backward] {vid} H={s.H} d={s.d} Lq={s.Lq} Tp={s.Tp} Kp={s.Kp} r={s.r}", flush=True)
    c = _setup(s, kw, bg)
    up = synth.draw_upstream(s)
    ch = c.ch
    ref = c.oracle()
    n_sel = ref["n_sel"]
    qf = oracle.as_f64(ch["q"], s.dtype)
    K = oracle.concat_keys(oracle.as_f64(ref["k_hist"], s.dtype), oracle.as_f64(ch["k_intra"], s.dtype))
    V = oracle.concat_keys(oracle.as_f64(ref["v_hist"], s.dtype), oracle.as_f64(ch["v_intra"], s.dtype))
    cols = _active_cols(s, n_sel)
    E_act = oracle.as_f64(ch["E"], s.dtype)[:, cols]
    F_act = oracle.as_f64(ch["F"], s.dtype)[:, cols]
    w_g = np.asarray(ch["w_g"], np.float64)
    b_g = np.asarray(ch["b_g"], np.float64)
    d_out = oracle.as_f64(up["d_out"], s.dtype)

    # the oracle's own history cache (host-built from its retrieval) on the device
    k_hist = np.zeros((s.Kp * s.Tp, s.H, s.d), np.uint16)
    v_hist = np.zeros_like(k_hist)
    k_hist[:n_sel * s.Tp] = ref["k_hist"]
    v_hist[:n_sel * s.Tp] = ref["v_hist"]
    t_kh, t_vh = dev(k_hist), dev(v_hist)
    t_ns = dev(np.asarray([n_sel], np.int32))
    t_do = dev(up["d_out"])

    # stage bar: oracle forward values in, float32-rounded
    want = oracle.backward_params(qf, K, V, E_act, F_act, w_g, b_g, ref["o_sparse"], d_out)
    f32 = lambda a: dev(np.ascontiguousarray(a, np.float32))  # noqa: E731
    got = _backward(c.d, s, c.t, t_kh, t_vh, t_ns, f32(want["k_low"]), f32(want["v_low"]),
                    f32(ref["o_sparse"]), f32(want["o_linear"]), t_do, c.t["w_g"], c.t["b_g"])
    _check(f"{vid} stage", s, got, want, n_sel, STAGE)
    # a second call, on two streams (the fork): the same bits
    again = _backward(c.d, s, c.t, t_kh, t_vh, t_ns, f32(want["k_low"]), f32(want["v_low"]),
                      f32(ref["o_sparse"]), f32(want["o_linear"]), t_do, c.t["w_g"], c.t["b_g"],
                      fork=default_fork())
    for k in got:
        assert got[k].tobytes() == again[k].tobytes(), f"{k}: not the same bits with the fork"

    # end to end: the GPU forward's own saved values in
    km = c.page_summary()
    outs = c.forward(km)
    o_l_gpu, kl_gpu, vl_gpu = c.linear(outs["k_hist"], outs["v_hist"], outs["n_sel"])
    assert int(host(outs["n_sel"])[0]) == n_sel
    cnt, idx = host(outs["sel_count"]), host(outs["sel_idx"])
    differ = check_selection(cnt, idx, ref["mass"], ref["sel"], [float(x) for x in ch["tau"]])
    o_s_ref = expected_sparse(s, ch, ref, cnt, idx, differ)
    want_e = oracle.backward_params(qf, K, V, E_act, F_act, w_g, b_g, o_s_ref, d_out)
    got_e = _backward(c.d, s, c.t, outs["k_hist"], outs["v_hist"], outs["n_sel"], kl_gpu, vl_gpu,
                      outs["o_sparse"], o_l_gpu, t_do, c.t["w_g"], c.t["b_g"])
    _check(f"{vid} e2e", s, got_e, want_e, n_sel, E2E)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["wan1.3b-480p", "wan14b-480p"])
def test_backward_full_shape(name):
    """Wan-1.3B- and Wan-14B-shaped 480p (H = 12 or 40, d = 128, Lq = 4680,
    four 12480-token slots, r = 256) at the stage bar, every element of every
    gradient. The history cache comes from the oracle's own retrieval; the
    sparse branch's output is the seeded stand-in (the backward holds it
    fixed, so any values exercise the same arithmetic)."""
    s = synth.shape(name)
    print(f"[backward] {name} generating", flush=True)
    c = Case(s)
    ch = c.ch
    up = synth.draw_upstream(s)
    km = np.stack([oracle.page_summary(oracle.as_f64(c.pool_k[p], s.dtype)[None])[0] for p in range(s.P)])
    qf = oracle.as_f64(ch["q"], s.dtype)
    page_idx, n_sel = oracle.retrieve(km, ch["page_prompt"], c.cur_prompt, oracle.chunk_query_mean(qf), s.Kp)
    kh = oracle.gather(c.pool_k, page_idx)
    vh = oracle.gather(c.pool_v, page_idx)
    K = oracle.concat_keys(oracle.as_f64(kh, s.dtype), oracle.as_f64(ch["k_intra"], s.dtype))
    V = oracle.concat_keys(oracle.as_f64(vh, s.dtype), oracle.as_f64(ch["v_intra"], s.dtype))
    cols = _active_cols(s, n_sel)
    E_act = oracle.as_f64(ch["E"], s.dtype)[:, cols]
    F_act = oracle.as_f64(ch["F"], s.dtype)[:, cols]
    o_s = up["o_sparse"].astype(np.float64)
    print(f"[backward] {name} oracle", flush=True)
    want = oracle.backward_params(qf, K, V, E_act, F_act, np.asarray(ch["w_g"], np.float64),
                                  np.asarray(ch["b_g"], np.float64), o_s, oracle.as_f64(up["d_out"], s.dtype))
    del K, V
    k_hist = np.zeros((s.Kp * s.Tp, s.H, s.d), np.uint16)
    v_hist = np.zeros_like(k_hist)
    k_hist[:n_sel * s.Tp] = kh
    v_hist[:n_sel * s.Tp] = vh
    f32 = lambda a: dev(np.ascontiguousarray(a, np.float32))  # noqa: E731
    print(f"[backward] {name} GPU", flush=True)
    got = _backward(c.d, s, c.t, dev(k_hist), dev(v_hist), dev(np.asarray([n_sel], np.int32)),
                    f32(want["k_low"]), f32(want["v_low"]), f32(up["o_sparse"]), f32(want["o_linear"]),
                    dev(up["d_out"]), c.t["w_g"], c.t["b_g"], fork=default_fork())
    _check(f"{name} stage", s, got, want, n_sel, STAGE)
