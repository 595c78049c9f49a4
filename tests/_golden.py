"""Loader for tests/golden/q4_0_blocks.txt (hand-worked Q4_0 blocks)."""

from dataclasses import dataclass
from pathlib import Path
from typing import List, Optional

import numpy as np

GOLDEN = Path(__file__).resolve().parent / "golden" / "q4_0_blocks.txt"


@dataclass
class Block:
    name: str
    x: np.ndarray            # 32 fp32 inputs
    dbits: int               # expected fp16 scale bits
    hex: str                 # expected 18 bytes
    deq: Optional[np.ndarray]


@dataclass
class GemvCase:
    block: str
    y: float
    S: float


def _f32(tok: str) -> np.float32:
    if tok.lower().startswith("0x"):
        return np.array([int(tok, 16)], dtype=np.uint32).view(np.float32)[0]
    return np.float32(tok)


def load():
    blocks: List[Block] = []
    gemvs: List[GemvCase] = []
    cur = None
    for raw in GOLDEN.read_text().splitlines():
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "block":
            cur = {"name": tok[1], "x": np.zeros(32, np.float32), "deq": None}
        elif tok[0] == "x":
            for t in tok[1:]:
                if t == "ramp":
                    cur["x"] = (np.arange(32) - 16).astype(np.float32)
                else:
                    key, val = t.split("=")
                    if key == "all":
                        cur["x"] = np.full(32, _f32(val), np.float32)
                    else:
                        cur["x"][int(key)] = _f32(val)
        elif tok[0] == "d":
            cur["dbits"] = int(tok[1], 16)
        elif tok[0] == "hex":
            cur["hex"] = tok[1].lower()
        elif tok[0] == "deq":
            cur["deq"] = np.array([np.float32(v) for v in tok[1:]], np.float32)
        elif tok[0] == "end":
            blocks.append(Block(**cur))
            cur = None
        elif tok[0] == "gemv":
            kv = dict(t.split("=") for t in tok[3:])
            gemvs.append(GemvCase(tok[1], float(kv["y"]), float(kv["S"])))
        else:
            raise ValueError(f"bad golden line: {raw!r}")
    return blocks, gemvs
