"""ctypes wrapper around the fp64 CPU oracle (dvssq_oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg.  The product library never imports it.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dvssq_oracle.cpp")
LIB = os.path.join(HERE, "liboracle_dvssq.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (plain -O2, no fast-math, no FP contraction)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-pthread", SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=False)
        L = C.CDLL(LIB)
        P = C.c_void_p
        i32, i64, f64 = C.c_int, C.c_int64, C.c_double
        sig = {
            "orc_bf16_from_double": (C.c_uint16, [f64]),
            "orc_bf16_to_double": (f64, [C.c_uint16]),
            "orc_layout": (i32, [i32, i32, i32, i32, P]),
            "orc_fwht_rows": (i32, [P, i64, i64, i32]),
            "orc_rank_rows": (i32, [P, i64, i64, P, P]),
            "orc_quant_int8_row": (i32, [P, i64, P, P]),
            "orc_quant_int4_row": (i32, [P, i64, P, P]),
            "orc_svd_jacobi": (i32, [P, i64, i64, P, P, P]),
            "orc_svd_lowrank": (i32, [P, i64, i64, i32, P, i32, i32, i32, P, P, P]),
            "orc_quantize": (i32, [P, i32, i32, i32, i32, i32, P, i32, i32, i32, P, P]),
            "orc_unpack": (i32, [P, i32, i32, i32, i32, P, P, P, P]),
            "orc_forward": (i32, [P, i32, i32, i32, i32, i32, P, i32, P, i32]),
            "orc_forward_cols": (i32, [P, i32, i32, i32, i32, i32, P, i32, P, i32, P, i32]),
            "orc_rotate_x": (i32, [P, i32, i32, i32, P]),
            "orc_kvbss_attention": (i32, [P, P, P, i32, i32, i32, i32, i32, i32, i32, f64, f64, P, i64, P, i32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _chk(rc, what):
    if rc < 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")
    return rc


LAYOUT_FIELDS = ("N4", "N8", "off_idx", "off_q4", "off_s4", "off_q8", "off_s8", "off_U", "off_V",
                 "blob_bytes", "algo_bytes")


def layout(N, K, r, n_seg=1) -> dict:
    out = np.zeros(11, dtype=np.int64)
    _chk(lib().orc_layout(N, K, r, n_seg, _p(out)), "layout")
    return dict(zip(LAYOUT_FIELDS, (int(v) for v in out)))


def bf16_from_double(v: float) -> int:
    return int(lib().orc_bf16_from_double(float(v)))


def bf16_to_double(h: int) -> float:
    return float(lib().orc_bf16_to_double(int(h)))


def fwht_rows(X: np.ndarray, b: int) -> np.ndarray:
    X = np.ascontiguousarray(X, dtype=np.float64).copy()
    rows = X.shape[0] if X.ndim == 2 else 1
    K = X.shape[-1]
    _chk(lib().orc_fwht_rows(_p(X), rows, K, b), "fwht")
    return X


def rank_rows(W: np.ndarray):
    W = np.ascontiguousarray(W, dtype=np.float64)
    N, K = W.shape
    S = np.zeros(N)
    order = np.zeros(N, dtype=np.int32)
    _chk(lib().orc_rank_rows(_p(W), N, K, _p(S), _p(order)), "rank_rows")
    return S, order


def quant_int8_row(w: np.ndarray):
    w = np.ascontiguousarray(w, dtype=np.float64)
    q = np.zeros(w.size, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    _chk(lib().orc_quant_int8_row(_p(w), w.size, _p(q), _p(s)), "quant_int8_row")
    return q, float(s[0])


def quant_int4_row(w: np.ndarray):
    w = np.ascontiguousarray(w, dtype=np.float64)
    q = np.zeros(w.size, dtype=np.int8)
    s = np.zeros(w.size // 64, dtype=np.uint16)
    _chk(lib().orc_quant_int4_row(_p(w), w.size, _p(q), _p(s)), "quant_int4_row")
    return q, s


def svd_jacobi(A: np.ndarray):
    A = np.ascontiguousarray(A, dtype=np.float64)
    m, n = A.shape
    U = np.zeros((m, n))
    S = np.zeros(n)
    V = np.zeros((n, n))
    sweeps = _chk(lib().orc_svd_jacobi(_p(A), m, n, _p(U), _p(S), _p(V)), "svd_jacobi")
    return U, S, V, sweeps


def svd_lowrank(R: np.ndarray, r: int, omega=None, power_iters: int = 4, full: bool = False):
    R = np.ascontiguousarray(R, dtype=np.float64)
    n, k = R.shape
    A = np.zeros((n, r))
    B = np.zeros((r, k))
    S = np.zeros(r)
    if full:
        om, l = None, 0
    else:
        om = np.ascontiguousarray(omega, dtype=np.float64)
        l = om.shape[1]
    _chk(lib().orc_svd_lowrank(_p(R), n, k, r, _p(om) if om is not None else None, l,
                               power_iters, int(full), _p(A), _p(B), _p(S)), "svd_lowrank")
    return A, B, S


def quantize(W_bf16: np.ndarray, r: int, block: int, n_seg: int = 1, omega=None,
             power_iters: int = 4, full_svd: bool = False, want_diag: bool = False):
    """Quantize W (uint16 bf16 bits [N][K]) into a packed blob (uint8 array)."""
    W = np.ascontiguousarray(W_bf16, dtype=np.uint16)
    N, K = W.shape
    L = layout(N, K, r, n_seg)
    blob = np.zeros(L["blob_bytes"], dtype=np.uint8)
    l = 0
    om = None
    if not full_svd:
        om = np.ascontiguousarray(omega, dtype=np.float64)
        l = om.shape[-1]
    diag = np.zeros(4 * n_seg) if want_diag else None
    _chk(lib().orc_quantize(_p(W), N, K, r, block, n_seg, _p(om) if om is not None else None, l,
                            power_iters, int(full_svd), _p(blob),
                            _p(diag) if diag is not None else None), "quantize")
    if want_diag:
        return blob, diag.reshape(n_seg, 4)
    return blob


def unpack(blob: np.ndarray, N, K, r, n_seg=1):
    idx = np.zeros(N, dtype=np.int32)
    What = np.zeros((N, K))
    U = np.zeros((N, r))
    V = np.zeros((n_seg * r, K))
    _chk(lib().orc_unpack(_p(blob), N, K, r, n_seg, _p(idx), _p(What), _p(U), _p(V)), "unpack")
    return idx, What, U, V


def forward(blob: np.ndarray, N, K, r, block, n_seg, x_bf16: np.ndarray, nthreads: int = 0):
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M = x.shape[0]
    y = np.zeros((M, N))
    _chk(lib().orc_forward(_p(blob), N, K, r, block, n_seg, _p(x), M, _p(y), nthreads), "forward")
    return y


def forward_cols(blob: np.ndarray, N, K, r, block, n_seg, x_bf16: np.ndarray, cols,
                 nthreads: int = 0):
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    M = x.shape[0]
    y = np.zeros((M, cols.size))
    _chk(lib().orc_forward_cols(_p(blob), N, K, r, block, n_seg, _p(x), M, _p(cols), cols.size,
                                _p(y), nthreads), "forward_cols")
    return y


def rotate_x(x_bf16: np.ndarray, block: int) -> np.ndarray:
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x.shape
    xr = np.zeros((M, K))
    _chk(lib().orc_rotate_x(_p(x), M, K, block, _p(xr)), "rotate_x")
    return xr


def quantize_layer(layer, seed: int = 0, power_iters: int = 4, want_diag: bool = False):
    """Quantize one synthetic layer of synth.WORKLOADS (tiny uses the exact SVD)."""
    import synth

    W = synth.weights_bf16(seed, layer)
    full = layer.N // layer.n_seg <= 1024 and layer.K <= 1024
    omega = None
    if not full:
        l = layer.r + 8
        omega = np.stack([synth.sketch(seed, layer, s, l) for s in range(layer.n_seg)])
    return quantize(W, layer.r, layer.block, layer.n_seg, omega=omega, power_iters=power_iters,
                    full_svd=full, want_diag=want_diag)


# ------------------------------------------------------------------ gated MLP block (test infrastructure)
# The Spark model page describes the feed-forward block as gate, up and down
# projections with GELU (Spark-X2.5-4B GGUF page, "The model": GELU FFN; ASHQ1
# page, Architecture: ffn_gate / ffn_up / ffn_down).  Readings: GELU is the
# exact x * Phi(x); the gate and up projections are the two segments of one
# fused layer (segment 0 = gate, segment 1 = up); every tensor between the
# projections is bf16, as in the BF16 model: the layer outputs are rounded to
# bf16, gelu(gate) * up is computed exactly and rounded to bf16, and that is
# the down projection's input.

def bf16_round_bits(v: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 rounding of fp64 values (this module's C rounding), as bits."""
    f = np.frompyfunc(lambda t: int(lib().orc_bf16_from_double(float(t))), 1, 1)
    return np.asarray(f(np.asarray(v, dtype=np.float64)), dtype=np.uint16)


def bf16_bits_value(bits: np.ndarray) -> np.ndarray:
    f = np.frompyfunc(lambda h: float(lib().orc_bf16_to_double(int(h))), 1, 1)
    return np.asarray(f(np.asarray(bits, dtype=np.uint16)), dtype=np.float64)


def gelu(x: np.ndarray) -> np.ndarray:
    """GELU(x) = x Phi(x) with the standard normal CDF Phi(x) = erfc(-x / sqrt 2) / 2
    (the same function as (1 + erf(x / sqrt 2)) / 2, without its cancellation for
    negative x, where 1 + erf loses every digit below Phi ~ 1e-16)."""
    import scipy.special
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * scipy.special.erfc(-x / np.sqrt(2.0))


def mlp_intermediate(y_gate_up: np.ndarray) -> np.ndarray:
    """bf16 bits of gelu(gate) * up from the fused layer's fp64 output [M][2I]."""
    I = y_gate_up.shape[1] // 2
    g = bf16_bits_value(bf16_round_bits(y_gate_up[:, :I]))
    u = bf16_bits_value(bf16_round_bits(y_gate_up[:, I:]))
    return bf16_round_bits(gelu(g) * u)


def mlp_forward(gu_blob: np.ndarray, gu: tuple, down_blob: np.ndarray, down: tuple, x_bf16: np.ndarray,
                nthreads: int = 0) -> np.ndarray:
    """y = down(bf16(gelu(bf16(gate(x))) * bf16(up(x)))) in fp64, with gate and up
    the two segments of the fused layer gu = (N, K, r, block) and down = (N, K, r, block)."""
    N, K, r, b = gu
    y_gu = forward(gu_blob, N, K, r, b, 2, x_bf16, nthreads)
    h = mlp_intermediate(y_gu)
    Nd, Kd, rd, bd = down
    return forward(down_blob, Nd, Kd, rd, bd, 1, h, nthreads)


def mlp_forward_cols(gu_blob: np.ndarray, gu: tuple, down_blob: np.ndarray, down: tuple, x_bf16: np.ndarray,
                     cols, nthreads: int = 0) -> np.ndarray:
    """mlp_forward restricted to output columns cols of the down projection."""
    N, K, r, b = gu
    y_gu = forward(gu_blob, N, K, r, b, 2, x_bf16, nthreads)
    h = mlp_intermediate(y_gu)
    Nd, Kd, rd, bd = down
    return forward_cols(down_blob, Nd, Kd, rd, bd, 1, h, cols, nthreads)


# ------------------------------------------------------------------ dense materialization (test infrastructure)
# The Spark card's Quickstart & Inference Guide offers materialize_weights(),
# which turns the quantized MLP weights into plain BF16 for generation.  Reading: the dense weight of the
# layer in the original input domain, W = (W_hat + U V_seg) H^T (H symmetric,
# so H^T = H), so that x W^T is the layer's forward; rows in original output
# order, rounded once to bf16.

def materialize(blob: np.ndarray, N, K, r, block, n_seg=1) -> np.ndarray:
    """fp64 dense weight [N][K] (original output order, original input domain)."""
    idx, What, U, V = unpack(blob, N, K, r, n_seg)
    seg = idx // (N // n_seg)
    Wr = What + np.einsum("pi,pik->pk", U, V.reshape(n_seg, r, K)[seg])
    W = np.empty_like(Wr)
    W[idx] = fwht_rows(Wr, block)
    return W


# ------------------------------------------------------------------ KV-BSS attention (test infrastructure)
# Spark-X2.5-4B-Hadamard-GSQ card, section 2 (KV-BSS); Spark-X2.5-4B discussion
# 14, Mathematical Formulation and the eager attention change.

KVBSS_TAU = 1.10      # focus factor
KVBSS_HAZE = 12.0     # nats below the row maximum at which logits are dropped


def kvbss_attention(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, scale: float, haze: float,
                    window: int = 0, rows=None, nthreads: int = 0) -> np.ndarray:
    """Causal grouped-query attention with the KV-BSS logit scale and haze mask, fp64.

    q [B][Mq][Hq][D], k and v [B][Nk][Hkv][D] (uint16 bf16 bits).  Returns
    o [B][Mq][Hq][D], or [len(rows)][D] for the flattened query rows
    (b * Mq + i) * Hq + h listed in rows.  haze = inf turns the mask off."""
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v = np.ascontiguousarray(v_bits, dtype=np.uint16)
    B, Mq, Hq, D = q.shape
    _, Nk, Hkv, _ = k.shape
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = B * Mq * Hq if r is None else r.size
    o = np.zeros((n, D))
    _chk(lib().orc_kvbss_attention(_p(q), _p(k), _p(v), B, Mq, Nk, Hq, Hkv, D, window, float(scale), float(haze),
                                   _p(r) if r is not None else None, n, _p(o), nthreads), "kvbss_attention")
    return o.reshape(B, Mq, Hq, D) if r is None else o
