"""Reader for tests/golden/hand_vectors.txt (hand-derived IBP vectors)."""
from __future__ import annotations

import os
import re

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_vectors.txt")


def _words(spec: str) -> np.ndarray:
    out: list[int] = []
    for tok in spec.split():
        m = re.fullmatch(r"ALL\(([0-9A-Fa-f]+),(\d+)\)", tok)
        if m:
            out.extend([int(m.group(1), 16)] * int(m.group(2)))
            continue
        m = re.fullmatch(r"SET\((\d+),([0-9A-Fa-f]+)\)", tok)
        if m:
            out[int(m.group(1))] = int(m.group(2), 16)
            continue
        out.append(int(tok, 16))
    return np.array(out, dtype=np.uint32)


def _bits(spec: str) -> set[int]:
    out: set[int] = set()
    for tok in spec.split():
        m = re.fullmatch(r"CHUNKS\((\d+),(\d+),(\d+),(\d+)-(\d+)\)", tok)
        if m:
            start, size, count, lo, hi = map(int, m.groups())
            for c in range(count):
                out.update(range(start + size * c + lo, start + size * c + hi + 1))
            continue
        if "-" in tok:
            a, b = map(int, tok.split("-"))
            out.update(range(a, b + 1))
        else:
            out.add(int(tok))
    return out


def load() -> list[dict]:
    cases: list[dict] = []
    cur: dict | None = None
    with open(GOLDEN) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split(":", 1))
            if key == "case":
                cur = {"case": val}
                cases.append(cur)
                continue
            assert cur is not None
            if key in ("W", "M", "tensor_bits", "L", "R", "record_words"):
                cur[key] = int(val)
            elif key in ("mask", "bitval", "x", "record", "record_head", "record_last"):
                cur[key] = _words(val)
            elif key == "one_bits":
                cur[key] = _bits(val)
            else:
                cur[key] = val
    return cases
