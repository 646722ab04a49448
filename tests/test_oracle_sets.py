"""Pins of the oracle's frame sets (CPU only).

The article's frame-7 example, hand-derived tables for the diagram geometry and the
frame-7 geometry, the partition and anchor statements of the article's method section,
time reversal, and the 768p key counts worked out by hand.
"""
import itertools

import numpy as np
import pytest

from oracle import sets
from tests.goldens import load, parse_ranges, table_sets


def _sets(f, F, C, R=1):
    return (sets.softmax_frames(f, F, C, R), sets.forward_frames(f, F, C, R),
            sets.backward_frames(f, F, C, R))


def test_frame7_printed_example():
    g = load("frame7_worked_example.json")
    s, fw, bw = _sets(g["query_frame"], g["frames"], g["chunk_frames"], g["neighbor_chunks"])
    assert s == g["softmax"]
    assert fw == g["forward"]
    assert bw == g["backward"]


@pytest.mark.parametrize("name", ["diagram_f16_c2_table.json", "worked_f15_c1_table.json"])
def test_hand_tables(name):
    g, rows = table_sets(name)
    for f, want in rows.items():
        s, fw, bw = _sets(f, g["frames"], g["chunk_frames"], g["neighbor_chunks"])
        assert s == want["softmax"], (name, f)
        assert fw == want["forward"], (name, f)
        assert bw == want["backward"], (name, f)


@pytest.mark.parametrize("name", ["diagram_f16_c2_table.json", "worked_f15_c1_table.json"])
def test_code_matrix_matches_table(name):
    g, rows = table_sets(name)
    codes = sets.code_matrix(g["frames"], g["chunk_frames"], g["neighbor_chunks"])
    want = np.zeros_like(codes)
    for f, r in rows.items():
        want[f, r["softmax"]] = sets.SOFTMAX
        want[f, r["forward"]] = sets.FORWARD
        want[f, r["backward"]] = sets.BACKWARD
    np.testing.assert_array_equal(codes, want)


GEOMS = [(F, C, R) for F in range(3, 41) for C in range(1, 8) for R in (1, 2)]


@pytest.mark.parametrize("F,C,R", GEOMS[::3])
def test_partition_and_anchors(F, C, R):
    """Window frames stay in softmax, the rest enter linear memory once, anchors are
    read by every frame and read every frame (method section, paragraphs 1-2)."""
    allf = set(range(F))
    for f in range(F):
        s, fw, bw = map(set, _sets(f, F, C, R))
        assert {0, F - 1} <= s
        if f in (0, F - 1):
            assert s == allf and not fw and not bw
            continue
        assert s | fw | bw == allf
        assert not (s & fw) and not (s & bw) and not (fw & bw)
        assert not ({0, F - 1} & (fw | bw))
        # forward memory lies strictly before the query, backward strictly after
        assert all(g < f for g in fw) and all(g > f for g in bw)
        # own chunk and the R chunks on each side are in the window (clipped)
        c = f // C
        for cc in range(max(0, c - R), min(-(-F // C) - 1, c + R) + 1):
            assert set(range(cc * C, min(F, (cc + 1) * C))) <= s


@pytest.mark.parametrize("F,C", [(F, C) for F in range(3, 41) for C in range(1, 8) if F % C == 0])
def test_time_reversal(F, C):
    for f in range(F):
        s, fw, bw = _sets(f, F, C)
        rs, rfw, rbw = _sets(F - 1 - f, F, C)
        assert sorted(F - 1 - g for g in s) == rs
        assert sorted(F - 1 - g for g in fw) == rbw
        assert sorted(F - 1 - g for g in bw) == rfw


def test_short_last_chunk():
    # F = 11, C = 5: chunks {0-4}, {5-9}, {10}; frame 10 is an anchor; frame 7 is in
    # chunk 1 whose window is chunks 0..2 = every frame.
    s, fw, bw = _sets(7, 11, 5)
    assert s == list(range(11)) and fw == [] and bw == []
    s, fw, bw = _sets(2, 11, 5)
    assert s == list(range(10)) + [10] and fw == [] and bw == []
    # F = 13, C = 5: chunk 2 = {10, 11, 12}; frame 11 sees 5..12 and anchor 0
    s, fw, bw = _sets(11, 13, 5)
    assert s == [0] + list(range(5, 13)) and fw == [1, 2, 3, 4] and bw == []


def test_768p_key_counts():
    g = load("p768_key_counts.json")
    F, T, C, L = g["frames"], g["tokens_per_frame"], g["chunk_frames"], g["text_len"]
    total = 0
    for grp in g["keys_per_query_by_frame_group"]:
        for f in parse_ranges(grp["frames"]):
            keys = len(sets.softmax_frames(f, F, C)) * T + L
            assert keys == grp["keys"], f
            total += T * keys
    assert total == g["pairs_per_head"]


def test_codes_are_int8_partition_codes():
    for F, C in itertools.product((3, 7, 16, 60), (1, 2, 5)):
        codes = sets.code_matrix(F, C)
        assert codes.dtype == np.int8 and codes.shape == (F, F)
        assert set(np.unique(codes)) <= {sets.SOFTMAX, sets.FORWARD, sets.BACKWARD}
        assert (codes[0] == sets.SOFTMAX).all() and (codes[F - 1] == sets.SOFTMAX).all()
