"""GPU parity of tiered pages: the gather and the forward reading pages
through a page table (some in HBM slots, the rest only in the pinned host
store) equal the gather and forward over an all-HBM pool, bit for bit; a
rollout with the slot planner between forwards keeps the HBM pool at its
slot count while every forward still equals the all-HBM one."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from block_sparse_rank_amd import hsakv as hs  # noqa: E402
from gpu_util import Case, dev, host  # noqa: E402


class Tiered:
    """A host store with every page and an HBM pool of `slots` pages."""

    def __init__(self, c, slots):
        s = c.s
        st = c.pool_k.dtype
        self.slots = slots
        self.hk = hs.HostStore(c.pool_k.shape, st)
        self.hv = hs.HostStore(c.pool_v.shape, st)
        self.hk.array[:] = c.pool_k
        self.hv.array[:] = c.pool_v
        td = torch.bfloat16 if s.dtype == "bf16" else torch.float32
        self.pk = torch.zeros((slots, s.Tp, s.H, s.d), dtype=td, device="cuda")
        self.pv = torch.zeros_like(self.pk)
        self.table = torch.full((s.P,), -1, dtype=torch.int32, device="cuda")
        self.tiers = hs.Tiers(self.table.data_ptr(), self.hk.device, self.hv.device)
        self.pl = hs.TierPlacement(s.P, slots)
        self.now = 0

    def want(self, c, pages):
        self.now += 1
        pp, ps, up, uv = hs.hkv_tier_plan(self.pl, self.now, pages)
        hs.hkv_tier_apply(c.d, self.tiers, self.pk, self.pv, self.slots, pp, ps, up, uv)
        torch.cuda.synchronize()
        return pp

    def free(self):
        torch.cuda.synchronize()
        self.hk.free()
        self.hv.free()


def _shape(dtype):
    return synth.shape("tiny").with_(dtype=dtype, P=8, Kp=3, clustered=dtype == "bf16",
                                     tau_law="uniform" if dtype == "bf16" else "alt", seed=36)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("resident", [[], [0, 2, 4], [1, 3, 5, 7]])
def test_tiered_gather_equals_all_hbm(dtype, resident):
    s = _shape(dtype)
    c = Case(s, page_prompt=np.zeros(s.P, np.int32))
    km = c.page_summary()
    ref = c.gather(km)
    t = Tiered(c, slots=4)
    try:
        t.want(c, resident)
        tab = host(t.table)
        assert sorted(np.flatnonzero(tab >= 0).tolist()) == sorted(resident)
        for p in resident:
            assert host(t.pk)[tab[p]].tobytes() == c.pool_k[p].tobytes()
        # the HBM pool argument is the slot pool: non-resident pages come from the host store
        page_idx = torch.full((s.Kp,), -7, dtype=torch.int32, device="cuda")
        n_sel = torch.zeros(1, dtype=torch.int32, device="cuda")
        k_hist = torch.zeros((s.Kp * s.Tp, s.H, s.d), dtype=t.pk.dtype, device="cuda")
        v_hist = torch.zeros_like(k_hist)
        ws = torch.empty(hs.workspace_bytes(c.d, hs.ENTRY_GATHER), dtype=torch.uint8, device="cuda")
        hs.hkv_gather(c.d, t.pk, t.pv, km, c.t["page_prompt"], c.cur_prompt, c.t["q"], page_idx, n_sel, k_hist,
                      v_hist, ws, tiers=t.tiers)
        torch.cuda.synchronize()
        assert host(page_idx).tolist() == host(ref[0]).tolist()
        assert host(k_hist).tobytes() == host(ref[2]).tobytes()
        assert host(v_hist).tobytes() == host(ref[3]).tobytes()
        # the forward (gather with the history keys pooled on the way) too
        full = c.forward(km)
        c2_t = dict(c.t)
        c.t["pool_k"], c.t["pool_v"] = t.pk, t.pv
        tiered = c.forward(km, tiers=t.tiers)
        c.t.update(c2_t)
        for k in ("out", "o_sparse", "o_linear", "k_hist", "sel_idx"):
            assert host(tiered[k]).tobytes() == host(full[k]).tobytes(), k
    finally:
        t.free()


def test_rollout_with_slot_planner_keeps_hbm_flat():
    """Six chunk-layers over a 8-page pool with 3 HBM slots: before each
    forward the planner holds the pages the previous forward retrieved; the
    results equal the all-HBM forwards and the HBM pool never grows."""
    s = _shape("bf16")
    pool = synth.draw_pool(s)
    prompts = np.zeros(s.P, np.int32)
    t = None
    try:
        last = []
        for k in range(6):
            ch = synth.draw_chunk(s.with_(seed=200 + k))
            c = Case(s, chunk=ch, pool=pool, page_prompt=prompts)
            if t is None:
                t = Tiered(c, slots=3)
            km = c.page_summary()
            t.want(c, last)
            full = c.forward(km)
            c.t["pool_k"], c.t["pool_v"] = t.pk, t.pv
            tiered = c.forward(km, tiers=t.tiers)
            assert host(tiered["out"]).tobytes() == host(full["out"]).tobytes()
            n = int(host(full["n_sel"])[0])
            last = host(full["page_idx"])[:n].tolist()
            assert t.pk.shape[0] == 3 and int((host(t.table) >= 0).sum()) <= 3
    finally:
        if t is not None:
            t.free()
