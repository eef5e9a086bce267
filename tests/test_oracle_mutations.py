"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutation edits the oracle's source text (a dropped term, a wrong sign,
a wrong index, a transposed operand, a flipped tie rule), loads the edited
copy as a throwaway module on the CPU, and runs the pins of
test_oracle_pins.py against it. The real oracle is never modified.
"""

import os
import types

import numpy as np
import pytest

import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "hsa.py")

_SEL = pins._golden("selection_hand.json")["cases"]
_RET = pins._golden("retrieval_hand.json")["cases"]
_BLK = pins._golden("workload_blocks.json")["cases"]


def _all(fn, cases):
    return lambda: [fn(c) for c in cases]


MUTATIONS = [
    ("block mass without 1/sqrt(d)",
     "z = np.matmul(qb, np.swapaxes(kb, 1, 2)) / math.sqrt(d)",
     "z = np.matmul(qb, np.swapaxes(kb, 1, 2))",
     [pins.test_block_mass_is_a_softmax]),
    ("block mass softmax over query blocks",
     "z = z - z.max(axis=-1, keepdims=True)\n    e = np.exp(z)\n    return e / e.sum(axis=-1, keepdims=True)",
     "z = z - z.max(axis=-2, keepdims=True)\n    e = np.exp(z)\n    return e / e.sum(axis=-2, keepdims=True)",
     [pins.test_block_mass_is_a_softmax]),
    ("selection with > instead of >=",
     "if np.float32(c) >= tau32:", "if np.float32(c) > tau32:",
     [_all(pins.test_selection_hand_worked, _SEL)]),
    ("selection ties to the higher id",
     "key=lambda b: (-float(m32[b]), b)", "key=lambda b: (-float(m32[b]), -b)",
     [_all(pins.test_selection_hand_worked, _SEL)]),
    ("selection keeps one block too many",
     "return np.array(sorted(order[:k]), dtype=np.int32)",
     "return np.array(sorted(order[:k + 1]), dtype=np.int32)",
     [_all(pins.test_selection_hand_worked, _SEL)]),
    ("selection ranks lightest first",
     "key=lambda b: (-float(m32[b]), b)", "key=lambda b: (float(m32[b]), b)",
     [_all(pins.test_selection_hand_worked, _SEL)]),
    ("retrieval ties to the higher page",
     "ranked = sorted(cand, key=lambda p: (-s[p], p))", "ranked = sorted(cand, key=lambda p: (-s[p], -p))",
     [pins.test_retrieval_duplicate_tie_goes_low]),
    ("retrieval keeps slots in rank order",
     "chosen = sorted(ranked[:Kp])", "chosen = list(ranked[:Kp])",
     [_all(pins.test_retrieval_hand_worked, _RET)]),
    ("retrieval ignores the prompt stage",
     "if int(page_prompt[p]) == int(cur_prompt)]", "]",
     [_all(pins.test_retrieval_hand_worked, _RET)]),
    ("retrieval score with a flipped sign",
     "s = float(np.sum(page_kmean[p] * qbar))", "s = float(np.sum(-page_kmean[p] * qbar))",
     [_all(pins.test_retrieval_hand_worked, _RET)]),
    ("history blocks tiled by Bintra",
     "blocks.append((b * Binter, min((b + 1) * Binter, Lh)))",
     "blocks.append((b * Bintra, min((b + 1) * Bintra, Lh)))",
     [_all(pins.test_block_table_workloads, _BLK)]),
    ("chunk blocks not offset by the history",
     "blocks.append((Lh + j * Bintra, Lh + min((j + 1) * Bintra, Lq)))",
     "blocks.append((j * Bintra, min((j + 1) * Bintra, Lq)))",
     [_all(pins.test_block_table_workloads, _BLK)]),
    ("pooling drops the last token of a block",
     "out[:, b, :] = x[s:e].mean(axis=0)", "out[:, b, :] = x[s:max(s + 1, e - 1)].mean(axis=0)",
     [pins.test_pool_closed_forms]),
    ("sparse attention without 1/sqrt(d)",
     "logits = qs @ kj.T / math.sqrt(d)", "logits = qs @ kj.T",
     [pins.test_sparse_all_blocks_is_dense_attention]),
    ("sparse attention over one block too few",
     "parts = [np.arange(blocks[b][0], blocks[b][1]) for b in ids]",
     "parts = [np.arange(blocks[b][0], blocks[b][1]) for b in ids[:-1]] or [np.arange(0, 1)]",
     [pins.test_sparse_mask_is_masked_dense_attention]),
    ("sparse attention normalises over the wrong axis",
     "w /= w.sum(axis=1, keepdims=True)\n    return w @ vj", "w /= w.sum(axis=0, keepdims=True)\n    return w @ vj",
     [pins.test_sparse_all_blocks_is_dense_attention]),
    ("linear branch projects V with E",
     "vh = F_act @ V[:, h, :]", "vh = E_act @ V[:, h, :]",
     [pins.test_linear_one_hot_rows_attend_chosen_keys]),
    ("linear branch without 1/sqrt(d)",
     "logits = q[:, h, :] @ kh.T / math.sqrt(d)", "logits = q[:, h, :] @ kh.T",
     [pins.test_linear_identity_projection_is_dense_attention]),
    ("active columns keep absent slots",
     "return np.concatenate([np.arange(n_sel * Tp), Kp * Tp + np.arange(Lq)])",
     "return np.concatenate([np.arange(Kp * Tp), Kp * Tp + np.arange(Lq)])",
     [pins.test_active_columns_skip_absent_slots]),
    ("gate without the bias",
     'x = np.einsum("thd,hd->th", q, w_g) + b_g[None, :]', 'x = np.einsum("thd,hd->th", q, w_g)',
     [pins.test_gate_matches_expit_and_isolates_branches]),
    ("fusion with the branches swapped",
     "return gg * o_s + (1.0 - gg) * o_l", "return gg * o_l + (1.0 - gg) * o_s",
     [pins.test_gate_matches_expit_and_isolates_branches]),
    ("forward projects K with F and V with E",
     "E_act = as_f64(E, dtype)[:, cols]\n    F_act = as_f64(F, dtype)[:, cols]",
     "E_act = as_f64(F, dtype)[:, cols]\n    F_act = as_f64(E, dtype)[:, cols]",
     [pins.test_forward_one_hot_projection_with_an_absent_slot]),
    ("key sequence puts the chunk before the history",
     "return np.concatenate([hist, intra], axis=0)", "return np.concatenate([intra, hist], axis=0)",
     [pins.test_forward_identity_projection_is_history_then_chunk,
      lambda: pins.test_forward_sparse_branch_is_masked_attention_over_history_then_chunk(0.35, 6, None)]),
    ("forward keeps the absent slots' columns",
     "cols = active_projection_columns(n_sel, Kp, Tp, Lq)", "cols = np.arange(n_sel * Tp + Lq)",
     [pins.test_forward_one_hot_projection_with_an_absent_slot]),
    ("forward pools the chunk keys as history blocks",
     "blocks = block_table(Lh, Lq, Binter, Bintra)", "blocks = block_table(Lh, Lq, Binter, Binter)",
     [lambda: pins.test_forward_sparse_branch_is_masked_attention_over_history_then_chunk(0.35, 6, None)]),
    ("commit finalises a page one token early",
     "done = [p for p in range(P) if fill < (p + 1) * Tp <= fill + n]",
     "done = [p for p in range(P) if fill < (p + 1) * Tp <= fill + n + 1]",
     [pins.test_commit_within_one_page_finalises_nothing,
      pins.test_commit_across_a_page_end_finalises_it]),
    ("commit writes the chunk one token late",
     "        t = fill + j\n", "        t = fill + j + 1\n",
     [pins.test_commit_within_one_page_finalises_nothing]),
    ("prompt-only keeps the oldest matching pages",
     "        s = {p: float(p) for p in cand}", "        s = {p: -float(p) for p in cand}",
     [lambda: pins.test_retrieval_policies_hand_worked("prompt_only", 2, [2, 3])]),
    ("mismatched keeps the matching pages",
     "        cand = [p for p in range(P) if p not in match]", "        cand = sorted(match)",
     [lambda: pins.test_retrieval_policies_hand_worked("mismatched", 2, [4, 5])]),
    ("SplitMix64 with a wrong shift",
     "z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M", "z = ((z ^ (z >> 28)) * 0x94D049BB133111EB) & M",
     [pins.test_splitmix64_published_outputs]),
    ("backward drops the softmax row term",
     "        dS = P * (dP - Dt)", "        dS = P * dP",
     [lambda: pins.test_backward_matches_finite_differences(11)]),
    ("backward gates the low-rank gradient with g",
     "        dol = (1.0 - g[:, h])[:, None] * d_out[:, h, :]", "        dol = g[:, h][:, None] * d_out[:, h, :]",
     [lambda: pins.test_backward_matches_finite_differences(11)]),
    ("page summary sums instead of averaging",
     "return pool_k.mean(axis=1)", "return pool_k.sum(axis=1)",
     [pins.test_page_summary_closed_forms]),
]


@pytest.mark.parametrize("name,old,new,checks", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, checks, monkeypatch):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mutant = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mutant.__dict__)
    monkeypatch.setattr(pins, "oracle", mutant)
    caught = False
    for check in checks:
        try:
            check()
        except (AssertionError, IndexError, ValueError):
            caught = True
    assert caught, f"no pin caught: {name}"


def test_unmutated_copy_passes_every_check(monkeypatch):
    with open(SRC) as f:
        src = f.read()
    copy = types.ModuleType("oracle_copy")
    exec(compile(src, "oracle_copy", "exec"), copy.__dict__)
    monkeypatch.setattr(pins, "oracle", copy)
    for _, _, _, checks in MUTATIONS:
        for check in checks:
            check()
    np.testing.assert_equal(True, True)
