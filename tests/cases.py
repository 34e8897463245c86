"""Shared helpers for the GPU parity tests: oracle-quantized layers (cached per
session), device upload, and the parity metric."""
from __future__ import annotations

import functools

import numpy as np

import oracle
import synth

TOL = 5e-3          # max|y_gpu - y_ref| / max|y_ref|


def all_layers():
    out = {}
    for wl in synth.WORKLOADS.values():
        for lay in wl.layers:
            out[lay.name] = lay
    # the MiniCPM r = 32 variant of every projection
    for lay in synth.WORKLOADS["minicpm"].layers:
        v = synth.Layer(lay.name + "_r32", lay.N, lay.K, lay.block, 32, lay.n_seg, lay.w_std,
                        lay.n_outlier, lay.outlier_tag)
        out[v.name] = v
    return out


LAYERS = all_layers()

# small shapes that exercise tails and corner parameters
EXTRA = {
    "ragged_b64_r1": synth.Layer("ragged_b64_r1", N=520, K=768, block=64, r=1, n_outlier=8,
                                 outlier_tag="ragged_b64"),
    "k192_b64": synth.Layer("k192_b64", N=136, K=192, block=64, r=3, n_outlier=2,
                            outlier_tag="k192"),
    "b128_r64": synth.Layer("b128_r64", N=96, K=256, block=128, r=64, n_outlier=3,
                            outlier_tag="b128"),
    "seg2_b512_r32": synth.Layer("seg2_b512_r32", N=2 * 264, K=512, block=512, r=32, n_seg=2,
                                 n_outlier=5, outlier_tag="seg2_b512"),
    "b1024_tail": synth.Layer("b1024_tail", N=8 * 45, K=1024, block=1024, r=8, n_outlier=10,
                              outlier_tag="b1024"),
    "b2048_ragged": synth.Layer("b2048_ragged", N=8 * 37, K=4096, block=2048, r=12, n_outlier=41,
                                outlier_tag="b2048"),
    "seg2_small": synth.Layer("seg2_small", N=2 * 256, K=256, block=256, r=24, n_seg=2,
                              n_outlier=3, outlier_tag="seg2_small"),
    # a small gated MLP block: fused gate+up (I = 256) and its down projection
    "mlp_tiny_gu": synth.Layer("mlp_tiny_gu", N=2 * 256, K=256, block=256, r=4, n_seg=2, n_outlier=3,
                               outlier_tag="mlp_tiny"),
    "mlp_tiny_dn": synth.Layer("mlp_tiny_dn", N=256, K=256, block=256, r=4),
}
LAYERS.update(EXTRA)


@functools.lru_cache(maxsize=None)
def quantized(name: str, seed: int = 0):
    lay = LAYERS[name]
    blob = oracle.quantize_layer(lay, seed=seed, power_iters=2)
    return lay, blob


@functools.lru_cache(maxsize=None)
def activations(name: str, M: int, seed: int = 0):
    lay = LAYERS[name]
    return synth.activations_bf16(seed, lay.outlier_tag or lay.name, M, lay.K)


def rel_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    den = np.abs(y_ref).max()
    return float(np.abs(y_gpu - y_ref).max() / (den if den > 0 else 1.0))


def to_device_bf16(bits: np.ndarray, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)
    return t.view(torch.bfloat16)


def from_device_bf16(t) -> np.ndarray:
    import torch
    bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
    return synth.bf16_bits_to_f64(bits)


def sample_columns(lay, blob, n_random: int = 96, seed: int = 1) -> np.ndarray:
    """Output columns for sampled parity: random ones, both ends, and some INT8-tier rows."""
    L = oracle.layout(lay.N, lay.K, lay.r, lay.n_seg)
    idx = blob[L["off_idx"]:L["off_idx"] + 4 * lay.N].view(np.int32)
    rng = np.random.default_rng(seed)
    cols = set(rng.choice(lay.N, size=min(n_random, lay.N), replace=False).tolist())
    cols |= {0, lay.N - 1, lay.N // max(lay.n_seg, 1) - 1, lay.N // max(lay.n_seg, 1)}
    n8 = L["N8"]
    cols |= set(idx[L["N4"]:][:: max(1, n8 // 16)].tolist())    # INT8 rows
    cols |= set(idx[:L["N4"]][:: max(1, L["N4"] // 16)].tolist())  # INT4 rows
    return np.array(sorted(c for c in cols if 0 <= c < lay.N), dtype=np.int32)


@functools.lru_cache(maxsize=None)
def planted_blob(name: str, kind: str):
    """(layer, blob, extra) of a planted variant of an oracle-quantized layer
    (tests/planted.py): kind is lowrank, edge or scales; extra is the INT4 row
    class array for scales, else None."""
    import planted
    lay, blob = quantized(name)
    if kind == "lowrank":
        return lay, planted.lowrank_only(blob, lay), None
    if kind == "edge":
        return lay, planted.edge_codes(blob, lay), None
    if kind == "scales":
        b, cls, _ = planted.scale_range(blob, lay)
        return lay, b, cls
    raise ValueError(kind)
