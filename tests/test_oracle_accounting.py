"""Pins for the accounting helpers: every number below is printed on a page."""

import math

from oracle import accounting as C


def _pct(x):
    return round(100 * x, 1)


def test_table_4_1(golden):
    for case in golden("accounting_examples.json")["table_4_1"]:
        row = C.table_4_1_row(case["lengths"], case["L"])
        for key in ("T", "fixed", "padding", "packs", "packed", "pack_padding", "saved"):
            assert row[key] == case[key], (key, case["cite"])
        assert _pct(row["waste"]) == case["waste_pct"]
        assert _pct(row["saved_frac"]) == case["saved_pct"]
        if "pack_waste_pct" in case:
            assert _pct(row["pack_waste"]) == case["pack_waste_pct"]
        if "score_elements_fixed" in case:
            assert row["score_elements_fixed"] == case["score_elements_fixed"]
            assert row["score_elements_packed"] == case["score_elements_packed"]
            assert _pct(row["score_elements_packed"] / row["score_elements_fixed"]) == case["score_ratio_pct"]
        assert math.isclose(C.waste(case["lengths"], case["L"]), row["waste"])


def test_two_ledgers_counts(golden):
    case = golden("accounting_examples.json")["two_ledgers"]
    ls = case["lengths"]
    assert C.token_slots_padded(ls) == case["token_positions"]["padded"]
    assert sum(ls) == case["token_positions"]["segments"] == case["token_positions"]["whole_pack"]
    assert C.dense_slots(ls) == case["dense_score_slots"]["padded"]
    assert C.segment_slots(ls) == case["dense_score_slots"]["segments"]
    assert C.whole_pack_slots(ls) == case["dense_score_slots"]["whole_pack"]
    assert C.causal_pairs(ls) == case["causal_pairs"]["segments"]
    assert C.causal_pairs([sum(ls)]) == case["causal_pairs"]["whole_pack"]
    assert C.causal_pairs([sum(ls)]) - C.causal_pairs(ls) == case["causal_pairs"]["cross"]


def test_length_grouping_counts(golden):
    case = golden("accounting_examples.json")["length_grouping"]
    assert sum(C.token_slots_padded(b) for b in case["batches_original"]) == case["slots_original"]
    assert sum(C.token_slots_padded(b) for b in case["batches_grouped"]) == case["slots_grouped"]
    assert C.segment_slots(case["lengths"]) == case["sum_sq"]
    assert sum(C.dense_slots(b) for b in case["batches_original"]) == case["dense_original"]


def test_long_context_waste(golden):
    case = golden("accounting_examples.json")["long_context_waste"]
    N, L = len(case["lengths"]), case["L"]
    assert N * L == case["fixed"]
    assert sum(case["lengths"]) == case["real"]
    assert N * L - sum(case["lengths"]) == case["padding"]
    assert _pct(C.waste(case["lengths"], L)) == case["waste_pct"]


def test_occupancy_4k_window(golden):
    """Block-diagonal share of a 4096 window of ten 400-token documents plus the
    96-token remainder: (10 * 400^2 + 96^2) / 4096^2 = 9.59%, the page's ~10%."""
    case = golden("accounting_examples.json")["occupancy_4k"]
    ls = [case["doc_len"]] * case["docs"] + [case["window"] - case["docs"] * case["doc_len"]]
    share = C.segment_slots(ls) / C.whole_pack_slots(ls)
    assert abs(100 * share - case["claimed_pct"]) < 0.5
    assert round(100 * share, 2) == 9.59


def test_eta_and_useful_flops():
    assert C.eta([2, 8, 3, 7], 8) == 20 / 32
    # 19 causal pairs for [3,2,4], 4 d H FLOPs each
    assert C.useful_flops([3, 2, 4], heads=2, head_dim=64) == 19 * 4 * 64 * 2
    assert C.useful_flops([3, 2, 4], heads=1, head_dim=64, causal=False) == 29 * 4 * 64
