"""Readers for the hand-written fixtures under tests/golden/."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FMT = {"f32": 0, "i8": 1, "i4": 2, "i2": 3}


def dequant_table():
    """[(fmt, bytes, [values])] from dequant_table.txt."""
    out = []
    with open(os.path.join(GOLDEN, "dequant_table.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            left, right = line.split("->")
            fmt, hexb = left.split()
            vals = [float(v) for v in right.split()]
            out.append((FMT[fmt], bytes.fromhex(hexb), vals))
    return out


def worked_examples():
    """List of dicts: name, fmt, O, I, S, w (uint8 [O, rb]), scales (or None), x, y and
    A (the bound magnitude sum_i |scale * q * x|, float64 [S, O])."""
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                cur = {"name": rest, "w": [], "x": [], "y": [], "A": []}
            elif key == "end":
                cur["w"] = np.array([list(bytes.fromhex(h)) for h in cur["w"]], dtype=np.uint8)
                cur["x"] = np.array(cur["x"], dtype=np.float32)
                cur["y"] = np.array(cur["y"], dtype=np.float32)
                cur["A"] = np.array(cur["A"], dtype=np.float64)
                cases.append(cur)
                cur = None
            elif key == "fmt":
                cur["fmt"] = FMT[rest]
            elif key in ("O", "I", "S"):
                cur[key] = int(rest)
            elif key == "w":
                cur["w"].append(rest)
            elif key == "scales":
                cur["scales"] = None if rest == "none" else np.array(
                    [float(v) for v in rest.split()], dtype=np.float32)
            elif key in ("x", "y", "A"):
                cur[key].append([float(v) for v in rest.split()])
            else:
                raise ValueError("bad fixture line: %r" % line)
    return cases


def group_scale_examples():
    """List of dicts like worked_examples plus gs and gscales (float32 [O, ng])."""
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "group_scale_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                cur = {"name": rest, "w": [], "x": [], "y": [], "A": [], "gscales": []}
            elif key == "end":
                cur["w"] = np.array([list(bytes.fromhex(h)) for h in cur["w"]], dtype=np.uint8)
                cur["x"] = np.array(cur["x"], dtype=np.float32)
                cur["y"] = np.array(cur["y"], dtype=np.float32)
                cur["A"] = np.array(cur["A"], dtype=np.float64)
                cur["gscales"] = np.array(cur["gscales"], dtype=np.float32)
                cases.append(cur)
                cur = None
            elif key == "fmt":
                cur["fmt"] = FMT[rest]
            elif key in ("O", "I", "S", "gs"):
                cur[key] = int(rest)
            elif key == "w":
                cur["w"].append(rest)
            elif key == "gscales":
                cur["gscales"].append([float(v) for v in rest.split()])
            elif key in ("x", "y", "A"):
                cur[key].append([float(v) for v in rest.split()])
            else:
                raise ValueError("bad fixture line: %r" % line)
    return cases
