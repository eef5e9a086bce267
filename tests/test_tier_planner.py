"""Host-only checks of the HBM slot planner (hkv_tier_plan): hand-worked
least-recently-used cases and invariants over random request sequences,
against a plain simulation of the rule written here. No GPU is touched."""

import numpy as np
import pytest

hs = pytest.importorskip("block_sparse_rank_amd.hsakv")


def _plan(pl, now, want):
    return hs.hkv_tier_plan(pl, now, want)


def test_lru_hand_worked():
    pl = hs.TierPlacement(P=6, slots=2)
    pp, ps, up, uv = _plan(pl, 1, [0, 1])
    assert pp.tolist() == [0, 1] and ps.tolist() == [0, 1]
    assert up.tolist() == [0, 1] and uv.tolist() == [0, 1]
    # page 2 wanted: both slots were used at time 1, the lower slot goes
    pp, ps, up, uv = _plan(pl, 2, [2])
    assert pp.tolist() == [2] and ps.tolist() == [0]
    assert list(zip(up.tolist(), uv.tolist())) == [(0, -1), (2, 0)]
    # pages 1 (resident) and 3: page 1 is wanted now, so page 2's slot goes
    pp, ps, up, uv = _plan(pl, 3, [1, 3])
    assert pp.tolist() == [3] and ps.tolist() == [0]
    assert list(zip(up.tolist(), uv.tolist())) == [(2, -1), (3, 0)]
    assert pl.slot_of_page.tolist() == [-1, 1, -1, 0, -1, -1]
    assert pl.page_of_slot.tolist() == [3, 1]


def test_more_wanted_pages_than_slots():
    pl = hs.TierPlacement(P=5, slots=2)
    pp, ps, _, _ = _plan(pl, 1, [4, 2, 0])
    assert pp.tolist() == [4, 2] and ps.tolist() == [0, 1]       # page 0 stays in the host store
    assert pl.slot_of_page[0] == -1
    pp, _, _, _ = _plan(pl, 1, [])
    assert len(pp) == 0


def test_rejects_bad_pages():
    pl = hs.TierPlacement(P=3, slots=1)
    with pytest.raises(hs.HsakvError) as ei:
        _plan(pl, 1, [3])
    assert ei.value.status == hs.ERR_BAD_DIMS


def _simulate(P, slots, seq):
    """The planner's rule, written out: per request list, wanted pages become
    the most recent; a missing page takes a free slot or the least recently
    used slot whose page is not wanted now (ties to the lower slot)."""
    slot_of = [-1] * P
    page_of = [-1] * slots
    last = [0] * P
    out = []
    for now, want in seq:
        for p in want:
            last[p] = now
        pro = []
        for p in want:
            if slot_of[p] >= 0:
                continue
            free = [s for s in range(slots) if page_of[s] < 0]
            if free:
                s = free[0]
            else:
                cands = [s for s in range(slots) if last[page_of[s]] < now]
                if not cands:
                    break
                s = min(cands, key=lambda x: (last[page_of[x]], x))
                slot_of[page_of[s]] = -1
            slot_of[p] = s
            page_of[s] = p
            pro.append((p, s))
        out.append(pro)
    return out, slot_of, page_of


@pytest.mark.parametrize("seed", range(40))
def test_random_sequences_follow_the_rule(seed):
    rng = np.random.default_rng(seed)
    P, slots = int(rng.integers(2, 20)), int(rng.integers(1, 8))
    seq = [(t + 1, rng.choice(P, size=int(rng.integers(0, min(6, P + 1))), replace=False).tolist())
           for t in range(30)]
    want_out, slot_of, page_of = _simulate(P, slots, seq)
    pl = hs.TierPlacement(P, slots)
    for (now, want), pro in zip(seq, want_out):
        pp, ps, up, uv = _plan(pl, now, want)
        assert list(zip(pp.tolist(), ps.tolist())) == pro
        # the table updates replay to the new placement
        assert all(pl.slot_of_page[p] == v for p, v in zip(up.tolist(), uv.tolist()) if v >= 0)
        resident = [p for p in range(P) if pl.slot_of_page[p] >= 0]
        assert len(resident) <= slots
        for p in resident:
            assert pl.page_of_slot[pl.slot_of_page[p]] == p
    assert pl.slot_of_page.tolist() == slot_of and pl.page_of_slot.tolist() == page_of
