"""hsa_forward captured in a HIP graph (through torch.cuda.CUDAGraph) and
replayed: every replay equals the eager call bit for bit. The call records
and waits on its fork's events, so with a fork the capture spans both
streams; the library launches no memset and allocates nothing, so the graph
holds only its kernels and the event edges. Between replays the test runs its
own eager work (an eager forward into other buffers, fills of the graph's
outputs) and synchronises, then checks the replay's outputs again.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from block_sparse_rank_amd import hsakv as hs  # noqa: E402
from gpu_util import Case, default_fork, host, tdtype, ws  # noqa: E402

CASES = [
    ("bf16-d128-r64", synth.shape("tiny").with_(dtype="bf16", d=128, H=3, r=64, Kp=3, P=8, clustered=True,
                                                tau_law="uniform", seed=16)),
    ("bf16-r128-long", synth.shape("tiny").with_(dtype="bf16", H=2, d=128, r=128, Lq=1000, tokens_per_frame=100,
                                                 clustered=True, tau_law="uniform", seed=27)),
    ("tiny-f32", synth.shape("tiny")),
    ("wan1.3b-480p", synth.shape("wan1.3b-480p")),
]


def _outs(c):
    s, d = c.s, c.d
    return dict(
        out=torch.zeros((s.Lq, s.H, s.d), dtype=tdtype(s), device="cuda"),
        page_idx=torch.zeros((s.Kp,), dtype=torch.int32, device="cuda"),
        n_sel=torch.zeros((1,), dtype=torch.int32, device="cuda"),
        sel_count=torch.zeros((s.H, d.NQB), dtype=torch.int32, device="cuda"),
        sel_idx=torch.zeros((s.H, d.NQB, d.NB_max), dtype=torch.int32, device="cuda"),
        o_sparse=torch.zeros((s.Lq, s.H, s.d), dtype=torch.float32, device="cuda"),
        o_linear=torch.zeros((s.Lq, s.H, s.d), dtype=torch.float32, device="cuda"),
        gate=torch.zeros((s.Lq, s.H), dtype=torch.float32, device="cuda"),
    )


@pytest.mark.timeout(600)
@pytest.mark.parametrize("use_fork", [True, False], ids=["fork", "one-stream"])
@pytest.mark.parametrize("cid,s", CASES, ids=[c[0] for c in CASES])
def test_forward_graph_replays_equal_eager(cid, s, use_fork):
    print(f"[graph] {cid} fork={use_fork}", flush=True)
    c = Case(s)
    km = c.page_summary()
    ins = {k: c.t[k] for k in ("q", "k_intra", "v_intra", "pool_k", "pool_v", "E", "F", "w_g", "b_g",
                               "page_prompt")}
    ins["page_kmean"] = km
    fork = default_fork() if use_fork else None
    w_eager, w_graph = ws(c.d, hs.ENTRY_FORWARD), ws(c.d, hs.ENTRY_FORWARD)
    eager = _outs(c)
    hs.hsa_forward(c.d, c.ch["tau"], c.cur_prompt, ins, eager, w_eager, fork=fork)
    torch.cuda.synchronize()
    want = {k: host(v).copy() for k, v in eager.items()}

    got = _outs(c)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=cap):
        hs.hsa_forward(c.d, c.ch["tau"], c.cur_prompt, ins, got, w_graph, fork=fork)
    torch.cuda.synchronize()
    for rep in range(3):
        for v in got.values():
            v.fill_(7)                       # the replay must rewrite every output
        other = _outs(c)
        hs.hsa_forward(c.d, c.ch["tau"], c.cur_prompt, ins, other, w_eager, fork=fork)   # eager work between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in got.items():
            a, b = host(v), want[k]
            if k == "sel_idx":   # ids past a row's count are not outputs
                cnt = want["sel_count"]
                keep = np.arange(a.shape[-1])[None, None, :] < cnt[:, :, None]
                a, b = a[keep], b[keep]
            assert a.tobytes() == b.tobytes(), f"replay {rep}: {k} differs from the eager call"
        assert host(other["out"]).tobytes() == want["out"].tobytes()
    del g
    torch.cuda.synchronize()
    print(f"[graph] {cid}: 3 replays equal the eager call (n_sel {int(want['n_sel'][0])})", flush=True)
