"""Planted packed layers for the GPU parity tests.

Each blob starts from an oracle-quantized layer (its idx, U, V and codes) and
overwrites parts of it, so that one term of the layer or one corner of the
format dominates the output:

* lowrank_only: every INT4 nibble is 8 (code 0) and every INT8 code 0, so the
  output is the low-rank term t U^T alone (MiniCPM5-2B-Hadamard-GSQ model
  card, Mathematical Foundations 2: the runtime equation's (X B^T) A^T).
* edge_codes: the extreme codes the clip ranges allow, -8 and -128 (INT4
  equation of the same section; Spark-X2.5-4B-Hadamard-GSQ card, Tier A),
  whole groups and rows at those codes, all-zero groups (scale 0) and all-zero
  INT8 rows (scale 0).
* scale_range: random codes with INT4 group scales spread over the bf16 range
  by row class (normal, in [2^-20, 2^-14), in (63, 256]), INT8 row scales over
  [2^-30, 2^10], and U = 0 so that each class is checked on its own scale.

Only the oracle's layout (oracle.layout) and plain numpy are used here; the
reference output of every planted blob is oracle.forward on that blob.
"""
from __future__ import annotations

import numpy as np

import oracle

NAMES = ("idx", "q4", "s4", "q8", "s8", "U", "V")


def parts(blob: np.ndarray, lay) -> dict:
    """Copies of the sub-buffers of a packed blob (oracle layout)."""
    L = oracle.layout(lay.N, lay.K, lay.r, lay.n_seg)
    n4, n8, K, N, r = L["N4"], L["N8"], lay.K, lay.N, lay.r
    spec = {
        "idx": (np.int32, (N,)), "q4": (np.uint8, (n4, K // 2)), "s4": (np.uint16, (n4, K // 64)),
        "q8": (np.int8, (n8, K)), "s8": (np.float32, (n8,)), "U": (np.uint16, (N, r)),
        "V": (np.uint16, (lay.n_seg * r, K)),
    }
    out = {}
    for name in NAMES:
        dt, shape = spec[name]
        off = L["off_" + name]
        nb = int(np.prod(shape)) * np.dtype(dt).itemsize
        out[name] = blob[off:off + nb].view(dt).reshape(shape).copy()
    return out


def pack(p: dict, lay) -> np.ndarray:
    """A blob with the given sub-buffers at the oracle layout's offsets."""
    L = oracle.layout(lay.N, lay.K, lay.r, lay.n_seg)
    blob = np.zeros(L["blob_bytes"], dtype=np.uint8)
    for name in NAMES:
        raw = np.ascontiguousarray(p[name]).view(np.uint8).reshape(-1)
        off = L["off_" + name]
        blob[off:off + raw.size] = raw
    return blob


def lowrank_only(blob: np.ndarray, lay) -> np.ndarray:
    p = parts(blob, lay)
    p["q4"][:] = 0x88
    p["q8"][:] = 0
    return pack(p, lay)


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 bits of fp64 values (the oracle's rounding)."""
    return oracle.bf16_round_bits(v)


def edge_codes(blob: np.ndarray, lay, seed: int = 11) -> np.ndarray:
    p = parts(blob, lay)
    rng = np.random.default_rng(seed)
    q4, s4, q8, s8 = p["q4"], p["s4"], p["q8"], p["s8"]
    n4, n8 = q4.shape[0], q8.shape[0]
    KG = lay.K // 64
    # INT4: every 5th row entirely at code -8 (nibble 0), every 7th at code +7
    # (nibble 15), and 10 % of the remaining bytes set to 0x00 / 0xFF / 0x0F
    q4[::5] = 0x00
    q4[3::7] = 0xFF
    mask = rng.random(q4.shape) < 0.1
    q4[mask] = rng.choice(np.array([0x00, 0xFF, 0x0F, 0xF0], dtype=np.uint8), size=int(mask.sum()))
    # all-zero groups: scale 0 with code 0 (nibble 8) in every 4th group of every 3rd row
    for row in range(1, n4, 3):
        for g in range(row % 4, KG, 4):
            s4[row, g] = 0
            q4[row, 32 * g:32 * (g + 1)] = 0x88
    # INT8: rows at -128 throughout, rows alternating -128 / 127, sprinkled
    # extremes, and all-zero rows with scale 0
    q8[::6] = -128
    q8[2::6, 0::2] = -128
    q8[2::6, 1::2] = 127
    mask = rng.random(q8.shape) < 0.1
    q8[mask] = rng.choice(np.array([-128, 127], dtype=np.int8), size=int(mask.sum()))
    zr = np.arange(4, n8, 6)
    q8[zr] = 0
    s8[zr] = 0.0
    return pack(p, lay)


# row classes of scale_range (by INT4 row index modulo 3)
SCALE_CLASSES = ("normal", "tiny [2^-20, 2^-14)", "large (63, 256]")


def scale_range(blob: np.ndarray, lay, seed: int = 12) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The blob, the class of each INT4 packed row and the scale exponent of each INT8 row."""
    p = parts(blob, lay)
    rng = np.random.default_rng(seed)
    n4, n8 = p["q4"].shape[0], p["q8"].shape[0]
    KG = lay.K // 64
    p["q4"][:] = rng.integers(0, 256, size=p["q4"].shape, dtype=np.uint8)
    p["q8"][:] = rng.integers(-128, 128, size=p["q8"].shape, dtype=np.int8)
    cls = np.arange(n4) % 3
    s = np.empty((n4, KG))
    s[cls == 0] = 2.0 ** rng.uniform(-8, -6, size=((cls == 0).sum(), KG))
    s[cls == 1] = 2.0 ** rng.uniform(-20, -14, size=((cls == 1).sum(), KG))
    s[cls == 2] = rng.uniform(63.5, 256.0, size=((cls == 2).sum(), KG))
    p["s4"][:] = _bf16_bits(s)
    e8 = rng.uniform(-30, 10, size=n8)
    p["s8"][:] = (2.0 ** e8).astype(np.float32)
    p["U"][:] = 0
    return pack(p, lay), cls, e8


def class_columns(blob: np.ndarray, lay, cls: np.ndarray) -> list[np.ndarray]:
    """Output columns of the INT4 rows of each scale class, then of the INT8 rows."""
    idx = parts(blob, lay)["idx"]
    n4 = cls.size
    cols = [np.sort(idx[:n4][cls == c]) for c in range(len(SCALE_CLASSES))]
    cols.append(np.sort(idx[n4:]))
    return cols
