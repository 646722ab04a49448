"""Loaders for the hand-written fixtures under tests/golden/ (no arithmetic of the layer)."""
from __future__ import annotations

import json
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def parse_ranges(text: str) -> list[int]:
    """"0,2-7,15" -> [0, 2, 3, 4, 5, 6, 7, 15]; "" -> []."""
    out: list[int] = []
    for part in filter(None, (p.strip() for p in text.split(","))):
        if "-" in part:
            a, b = part.split("-")
            out.extend(range(int(a), int(b) + 1))
        else:
            out.append(int(part))
    return out


def table_sets(name: str) -> tuple[dict, dict[int, dict[str, list[int]]]]:
    """Per-query-frame {softmax, forward, backward} frame lists of a hand table."""
    g = load(name)
    rows: dict[int, dict[str, list[int]]] = {}
    for row in g["rows"]:
        for f in row["query_frames"]:
            rows[f] = {k: parse_ranges(row[k]) for k in ("softmax", "forward", "backward")}
    assert sorted(rows) == list(range(g["frames"])), name
    return g, rows
