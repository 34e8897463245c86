"""Seeded synthetic inputs for the DV-SSQ linear layer.

This module is shared by the oracle's tests, the GPU tests and the benchmark.
It draws numbers and rounds them to the storage types the layer reads; it
holds none of the layer's arithmetic (no rotation, no quantizer, no SVD, no
forward pass).

Random numbers come from SplitMix64 used as a counter-based generator: the
value for element i of a stream is mix64(key + (i + 1) * GAMMA), where mix64
is the SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) and key is derived from the seed
and a text tag naming the stream.  Uniforms take the top 53 bits; normals come
from the Box-Muller transform in fp64.

Workload shapes follow the two model cards: Spark-X2.5-4B (hidden 2560,
intermediate 10240, H_256 blocks; "Myric/Spark-X2.5-4B-GGUF", section "The
model") and MiniCPM5-2B (hidden 2048 = 2^11, H_2048; "MiniCPM5-2B-Hadamard-GSQ"
model card, Executive Overview).  Weights are N(0, std^2) with 1 % of the input
columns scaled by 20 as outliers, then rounded to bf16 (the BF16 checkpoint the
cards quantize); activations are N(0, 1) rounded to bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
    return z


def _tag_hash(tag: str) -> int:
    """FNV-1a 64-bit hash of the tag text."""
    h = 0xCBF29CE484222325
    for byte in tag.encode("utf-8"):
        h ^= byte
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def stream_key(seed: int, tag: str) -> np.uint64:
    with np.errstate(over="ignore"):
        base = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) * GAMMA + np.uint64(_tag_hash(tag))
    return _mix64(np.array([base], dtype=np.uint64))[0]


def raw_u64(seed: int, tag: str, n: int, start: int = 0) -> np.ndarray:
    """Elements start .. start+n-1 of the 64-bit stream (seed, tag)."""
    key = stream_key(seed, tag)
    ctr = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(key + ctr * GAMMA)


def uniform(seed: int, tag: str, n: int) -> np.ndarray:
    """n uniforms in the open interval (0, 1), fp64."""
    v = raw_u64(seed, tag, n)
    return ((v >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normal(seed: int, tag: str, n: int) -> np.ndarray:
    """n standard normals, fp64, by Box-Muller over consecutive uniform pairs."""
    npair = (n + 1) // 2
    u = uniform(seed, tag, 2 * npair)
    rad = np.sqrt(-2.0 * np.log(u[0::2]))
    ang = 2.0 * math.pi * u[1::2]
    out = np.empty(2 * npair, dtype=np.float64)
    out[0::2] = rad * np.cos(ang)
    out[1::2] = rad * np.sin(ang)
    return out[:n]


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even) in one step; uint16 bits.

    Inputs are rounded straight from fp64, never through fp32, so there is no
    double rounding.  Normal range: 8 significant bits; below 2^-126 the grid
    is the fixed bf16 subnormal quantum 2^-133.  Overflow gives +-inf.
    """
    a = np.asarray(v, dtype=np.float64)
    mag = np.abs(a)
    _, e = np.frexp(mag)                      # mag = f * 2^e, f in [0.5, 1)
    q = np.maximum(e.astype(np.int64) - 8, -133)
    m = np.rint(np.ldexp(mag, -q))            # rint is round-half-even
    r = np.ldexp(m, q)
    r = np.where(mag == 0.0, 0.0, r)
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)              # exact: r has <= 8 significant bits
    bits = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.signbit(a), bits | np.uint16(0x8000), bits)
    bits = np.where(np.isnan(a), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Layer:
    """One DV-SSQ layer: N output features, K input features, n_seg stacked
    projections of N/n_seg rows each that share the input."""
    name: str
    N: int
    K: int
    block: int
    r: int
    n_seg: int = 1
    w_std: float = 0.02
    n_outlier: int = 0      # outlier input columns (x20), shared by all segments
    outlier_tag: str = ""   # layers that read the same input share this tag


@dataclass(frozen=True)
class Workload:
    name: str
    layers: tuple
    m_decode: tuple = ()
    m_prefill: tuple = ()
    description: str = ""
    extra: dict = field(default_factory=dict)


def _outliers(K: int) -> int:
    return int(round(0.01 * K))


WORKLOADS = {
    "tiny": Workload(
        "tiny",
        (Layer("tiny", N=512, K=256, block=256, r=4, n_outlier=4, outlier_tag="tiny"),),
        m_decode=(1, 4),
        description="K=256, N=512, one H_256 block, 64 INT8 rows, r=4",
    ),
    "spark_up": Workload(
        "spark_up",
        (Layer("spark_up", N=10240, K=2560, block=256, r=16,
               n_outlier=_outliers(2560), outlier_tag="spark_hidden"),),
        m_decode=(1, 4, 16),
        description="Spark-shaped up_proj decode, K=2560, N=10240, r=16",
    ),
    "spark_down": Workload(
        "spark_down",
        (Layer("spark_down", N=2560, K=10240, block=256, r=16, w_std=0.01,
               n_outlier=_outliers(10240), outlier_tag="spark_inter"),),
        m_decode=(1, 8, 32),
        description="Spark-shaped down_proj decode, K=10240, N=2560, r=16",
    ),
    "spark_gateup": Workload(
        "spark_gateup",
        (Layer("spark_gateup", N=2 * 10240, K=2560, block=256, r=24, n_seg=2,
               n_outlier=_outliers(2560), outlier_tag="spark_hidden"),),
        m_prefill=(512, 2048),
        description="Spark-shaped fused gate+up prefill, K=2560, N=2x10240, r=24",
    ),
    "minicpm": Workload(
        "minicpm",
        (
            Layer("minicpm_gate", N=6144, K=2048, block=2048, r=16,
                  n_outlier=_outliers(2048), outlier_tag="minicpm_hidden"),
            Layer("minicpm_up", N=6144, K=2048, block=2048, r=16,
                  n_outlier=_outliers(2048), outlier_tag="minicpm_hidden"),
            Layer("minicpm_down", N=2048, K=6144, block=2048, r=16,
                  n_outlier=_outliers(6144), outlier_tag="minicpm_inter"),
        ),
        m_decode=(1,),
        m_prefill=(4096,),
        description="MiniCPM-shaped MLP, hidden 2048 with H_2048, intermediate 6144, r=16",
        extra={"r_variant": 32},
    ),
}


def outlier_columns(seed: int, layer: Layer) -> np.ndarray:
    """Sorted outlier column indices, drawn without replacement."""
    if layer.n_outlier == 0:
        return np.zeros(0, dtype=np.int64)
    u = uniform(seed, "outlier_cols/" + (layer.outlier_tag or layer.name), layer.K)
    order = np.argsort(u, kind="stable")
    return np.sort(order[: layer.n_outlier])


def weights_bf16(seed: int, layer: Layer) -> np.ndarray:
    """uint16 bf16 bits, shape [N][K]; rows s*N/n_seg .. are segment s."""
    ns = layer.N // layer.n_seg
    cols = outlier_columns(seed, layer)
    out = np.empty((layer.N, layer.K), dtype=np.uint16)
    for s in range(layer.n_seg):
        w = normal(seed, f"W/{layer.name}/{s}", ns * layer.K).reshape(ns, layer.K)
        w *= layer.w_std
        if cols.size:
            w[:, cols] *= 20.0
        out[s * ns:(s + 1) * ns] = to_bf16_bits(w)
    return out


def activations_bf16(seed: int, tag: str, M: int, K: int) -> np.ndarray:
    """uint16 bf16 bits, shape [M][K], N(0, 1).  Row m is the same for every M."""
    rows = [to_bf16_bits(normal(seed, f"x/{tag}/{m}", K)) for m in range(M)]
    return np.stack(rows) if rows else np.zeros((0, K), dtype=np.uint16)


def sketch(seed: int, layer: Layer, seg: int, l: int) -> np.ndarray:
    """Gaussian test matrix Omega [K][l] (fp64) for the randomized SVD."""
    return normal(seed, f"Omega/{layer.name}/{seg}", layer.K * l).reshape(layer.K, l)


def random_packed_parts(seed: int, N: int, K: int, r: int, n_seg: int = 1) -> dict:
    """Random but well-formed packed-layer contents (for timing only).

    Codes and factors are random draws of the right types and ranges; the tier
    split is a random choice of N/(8*n_seg) rows per segment.  Nothing here is
    a quantization of anything.
    """
    ns = N // n_seg
    n8s = ns // 8
    i4, i8 = [], []
    for s in range(n_seg):
        u = uniform(seed, f"tier/{s}", ns)
        pick = np.sort(np.argsort(u, kind="stable")[:n8s])
        mask = np.zeros(ns, dtype=bool)
        mask[pick] = True
        i4.append(np.nonzero(~mask)[0] + s * ns)
        i8.append(np.nonzero(mask)[0] + s * ns)
    idx = np.concatenate(i4 + i8).astype(np.int32)
    n4 = N - n8s * n_seg
    n8 = n8s * n_seg
    rb = lambda tag, n: raw_u64(seed, tag, n)
    q4 = (rb("q4", (n4 * K // 2 + 7) // 8).view(np.uint8)[: n4 * K // 2]).reshape(n4, K // 2)
    q8 = (rb("q8", (n8 * K + 7) // 8).view(np.int8)[: n8 * K]).reshape(n8, K)
    s4 = to_bf16_bits(0.002 + 0.004 * uniform(seed, "s4", n4 * (K // 64))).reshape(n4, K // 64)
    s8 = (0.0002 + 0.0004 * uniform(seed, "s8", n8)).astype(np.float32)
    U = to_bf16_bits(0.01 * normal(seed, "U", N * r)).reshape(N, r)
    V = to_bf16_bits(0.01 * normal(seed, "V", n_seg * r * K)).reshape(n_seg * r, K)
    return dict(idx=idx, q4=q4, s4=s4, q8=q8, s8=s8, U=U, V=V)


# Query gains per attention head (cycled over the heads).  With unit-variance
# q and k and the logit scale 1.1 / sqrt(head_dim), the logits of a head have
# a spread of about 1.1 x gain: from heads where no key falls 12 nats below
# the row maximum to heads where most keys do.
ATTN_Q_GAINS = (0.5, 1.0, 3.0, 6.0)


def attention_qkv(seed: int, tag: str, B: int, Mq: int, Nk: int, Hq: int, Hkv: int, D: int,
                  gains=ATTN_Q_GAINS):
    """uint16 bf16 bits: q [B][Mq][Hq][D], k and v [B][Nk][Hkv][D]; N(0, 1)
    draws, q scaled per head by gains[h % len(gains)]."""
    g = np.array([gains[h % len(gains)] for h in range(Hq)], dtype=np.float64)
    q = normal(seed, f"attn/{tag}/q", B * Mq * Hq * D).reshape(B, Mq, Hq, D) * g[None, None, :, None]
    k = normal(seed, f"attn/{tag}/k", B * Nk * Hkv * D).reshape(B, Nk, Hkv, D)
    v = normal(seed, f"attn/{tag}/v", B * Nk * Hkv * D).reshape(B, Nk, Hkv, D)
    return to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v)
