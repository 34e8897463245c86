"""Pins for the fp64 oracle against what the model cards and mathematics fix.

Each test checks the oracle against something other than itself: a closed
form, a library routine for a special case, brute force on a small input, the
cards' printed constants (tests/golden/), or an invariant.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def exact_bf16(v: float) -> int:
    """Round a double to bf16 by exact rational arithmetic (reference for pins)."""
    if v == 0:
        return 0x8000 if np.signbit(v) else 0
    sign = 0x8000 if v < 0 else 0
    a = Fraction(abs(v))
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    # a in [1, 2): 7 fraction bits for normals; fixed quantum 2^-133 below 2^-126
    q = max(e - 7, -133)
    m = Fraction(abs(v)) / Fraction(2) ** q
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * Fraction(2) ** q
    with np.errstate(over="ignore"):
        f = np.float32(float(val))
    return sign | (int(f.view(np.uint32)) >> 16)


# ------------------------------------------------------------------ number types

def test_bf16_rounding_matches_exact_rational():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(300) * 10.0 ** rng.integers(-40, 38, 300))
    # exact ties between neighbours, both parities, and subnormal-range values
    vals += [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -127 * 1.5, 2 ** -133,
             3 * 2 ** -134, 2 ** -140, 1.0, -2.5, 3.0e38, 3.4e38]
    for v in vals:
        want = exact_bf16(float(v))
        assert oracle.bf16_from_double(v) == want, v
    got = synth.to_bf16_bits(np.array(vals))
    assert [int(g) for g in got] == [exact_bf16(float(v)) for v in vals]


def test_bf16_known_values():
    assert oracle.bf16_from_double(1.0) == 0x3F80
    assert oracle.bf16_from_double(1 + 2 ** -8) == 0x3F80      # tie -> even
    assert oracle.bf16_from_double(1 + 3 * 2 ** -8) == 0x3F82  # tie -> even
    assert oracle.bf16_from_double(-2.0) == 0xC000
    assert oracle.bf16_to_double(0x3F81) == 1 + 2 ** -7


# ------------------------------------------------------------------ Hadamard / FWHT

def test_sylvester_h8_golden():
    H8 = np.loadtxt(os.path.join(GOLD, "sylvester_h8.txt"))
    got = oracle.fwht_rows(np.eye(8), 8) * np.sqrt(8)
    np.testing.assert_array_equal(got, H8)


@pytest.mark.parametrize("b", [2, 4, 8, 16, 64, 256, 2048])
def test_hadamard_closed_form(b):
    H = oracle.fwht_rows(np.eye(b), b)            # row i = e_i H = row i of H
    ref = scipy.linalg.hadamard(b) / np.sqrt(b)   # Sylvester, natural order
    np.testing.assert_allclose(H, ref, atol=1e-15, rtol=0)
    Hu = np.rint(H * np.sqrt(b))
    np.testing.assert_array_equal(Hu @ Hu.T, b * np.eye(b))   # H H^T = b I (unnormalized)


@pytest.mark.parametrize("b,nblk", [(64, 3), (256, 2), (2048, 1)])
def test_fwht_against_dense(b, nblk):
    rng = np.random.default_rng(b)
    X = rng.standard_normal((5, b * nblk))
    got = oracle.fwht_rows(X, b)
    Hb = scipy.linalg.hadamard(b) / np.sqrt(b)
    HK = scipy.linalg.block_diag(*([Hb] * nblk))
    np.testing.assert_allclose(got, X @ HK, atol=1e-12 * np.abs(X).max() * np.sqrt(b), rtol=0)


def test_fwht_involution_parseval_and_dispersion():
    rng = np.random.default_rng(3)
    b = 256
    X = rng.standard_normal((7, 4 * b))
    X[:, 5] *= 50.0                                  # a coordinate-aligned outlier
    Y = oracle.fwht_rows(X, b)
    np.testing.assert_allclose(oracle.fwht_rows(Y, b), X, atol=1e-12)
    for blk in range(4):
        sl = slice(blk * b, (blk + 1) * b)
        np.testing.assert_allclose((Y[:, sl] ** 2).sum(1), (X[:, sl] ** 2).sum(1), rtol=1e-13)
        # MiniCPM card, Mathematical Foundations 1: max_j |x'_j| <= (1/sqrt(d)) sum_i |x_i|
        bound = np.abs(X[:, sl]).sum(1) / np.sqrt(b)
        assert np.all(np.abs(Y[:, sl]).max(1) <= bound * (1 + 1e-13))


def test_fwht_special_vectors():
    b = 256
    for i in [0, 1, 77, 255]:
        e = np.zeros(b)
        e[i] = 1.0
        y = oracle.fwht_rows(e[None], b)[0]
        np.testing.assert_array_equal(np.abs(y), np.full(b, 1 / 16))   # exact for b = 256
        assert y[0] == 1 / 16
    y = oracle.fwht_rows(np.ones((1, b)), b)[0]
    np.testing.assert_allclose(y, np.eye(b)[0] * np.sqrt(b), atol=1e-13)


def test_rotation_identity():
    # MiniCPM card, Mathematical Foundations 1: (X H)(W H)^T = X W^T
    rng = np.random.default_rng(4)
    K = 512
    X = rng.standard_normal((3, K))
    W = rng.standard_normal((40, K))
    lhs = oracle.fwht_rows(X, 256) @ oracle.fwht_rows(W, 256).T
    ref = X @ W.T
    assert np.abs(lhs - ref).max() <= 1e-12 * np.abs(ref).max()


# ------------------------------------------------------------------ salience

def test_salience_ranking_brute_force():
    rng = np.random.default_rng(5)
    W = rng.standard_normal((64, 128))
    W[10] = W[3]                                   # an exact tie: lower index first
    S, order = oracle.rank_rows(W)
    np.testing.assert_allclose(S, (W ** 2).sum(1), rtol=1e-14)
    ref = sorted(range(64), key=lambda n: (-sum(float(v) ** 2 for v in W[n]), n))
    assert list(order) == ref
    assert list(order).index(3) < list(order).index(10)
    # row energies are invariant under the rotation
    S2, _ = oracle.rank_rows(oracle.fwht_rows(W, 128))
    np.testing.assert_allclose(S2, S, rtol=1e-12)


def test_salient_counts_match_card():
    gold = json.load(open(os.path.join(GOLD, "page_constants.json")))
    for n, want in gold["salient_counts"]["value"].items():
        assert oracle.layout(int(n), 256, 4)["N8"] == want
    assert oracle.layout(512, 256, 4)["N8"] == 64


# ------------------------------------------------------------------ quantizers

def test_int4_quantizer_properties():
    gold = json.load(open(os.path.join(GOLD, "page_constants.json")))
    G = gold["int4_group_size"]["value"]
    lo, hi = gold["int4_clip"]["value"]
    rng = np.random.default_rng(6)
    w = rng.standard_normal(16 * G) * 0.02
    w[G:2 * G] = 0.0                               # an all-zero group
    w[5] = 0.9                                     # an outlier inside group 0
    q, s = oracle.quant_int4_row(w)
    sv = np.array([oracle.bf16_to_double(int(h)) for h in s])
    assert q.min() >= lo and q.max() <= hi
    for g in range(16):
        wg, qg = w[g * G:(g + 1) * G], q[g * G:(g + 1) * G]
        if g == 1:
            assert sv[g] == 0 and not qg.any()
            continue
        amax = np.abs(wg).max()
        assert abs(sv[g] - amax / 7.0) <= 2 ** -8 * amax / 7.0      # bf16 unit roundoff 2^-8
        assert np.abs(wg - qg * sv[g]).max() <= sv[g] / 2 + 1e-18   # per-element error <= s/2
        assert np.abs(qg).max() == 7                                 # absmax maps to +-7


def test_int4_on_grid_is_exact():
    rng = np.random.default_rng(7)
    s = 2.0 ** -6
    q0 = rng.integers(-7, 8, 256)
    for g in range(4):
        q0[g * 64] = 7                              # make max|w| = 7 s in every group
    w = q0 * s
    q, sc = oracle.quant_int4_row(w)
    np.testing.assert_array_equal(q, q0)
    assert all(oracle.bf16_to_double(int(h)) == s for h in sc)


def test_int8_quantizer_properties():
    rng = np.random.default_rng(8)
    w = rng.standard_normal(1024) * 0.05
    q, s = oracle.quant_int8_row(w)
    amax = np.abs(w).max()
    assert abs(s - amax / 127) <= 2 ** -24 * amax / 127 * 2
    assert q.min() >= -128 and q.max() <= 127 and np.abs(q).max() == 127
    assert np.abs(w - q.astype(np.float64) * s).max() <= s / 2 * (1 + 1e-12)
    q0, s0 = oracle.quant_int8_row(np.zeros(64))
    assert s0 == 0 and not q0.any()
    grid = rng.integers(-127, 128, 512).astype(np.float64)
    grid[0] = 127
    qg, sg = oracle.quant_int8_row(grid * 2.0 ** -10)
    np.testing.assert_array_equal(qg, grid.astype(np.int8))


# ------------------------------------------------------------------ SVD

def test_jacobi_svd_against_library():
    rng = np.random.default_rng(9)
    A = rng.standard_normal((60, 24))
    U, S, V, sweeps = oracle.svd_jacobi(A)
    np.testing.assert_allclose(S, np.linalg.svd(A, compute_uv=False), rtol=1e-12)
    np.testing.assert_allclose(U.T @ U, np.eye(24), atol=1e-12)
    np.testing.assert_allclose(V.T @ V, np.eye(24), atol=1e-12)
    np.testing.assert_allclose(U @ np.diag(S) @ V.T, A, atol=1e-12)
    assert np.all(np.diff(S) <= 0)
    for j in range(24):                             # sign rule on right vectors
        assert V[np.abs(V[:, j]).argmax(), j] > 0


def test_lowrank_full_is_eckart_young():
    rng = np.random.default_rng(10)
    R = rng.standard_normal((80, 40)) @ np.diag(np.linspace(2, 0.1, 40)) @ rng.standard_normal((40, 40))
    r = 6
    A, B, S = oracle.svd_lowrank(R, r, full=True)
    sig = np.linalg.svd(R, compute_uv=False)
    err2 = np.linalg.norm(R - A @ B) ** 2
    assert abs(err2 - (sig[r:] ** 2).sum()) <= 1e-10 * (sig ** 2).sum()
    # A B equals the explicit r-term sum sum_i sigma_i u_i v_i^T
    U, Sl, Vt = np.linalg.svd(R)
    ref = sum(Sl[i] * np.outer(U[:, i], Vt[i]) for i in range(r))
    np.testing.assert_allclose(A @ B, ref, atol=1e-10)
    # sqrt(Sigma) on both sides: columns of A and rows of B have equal norms
    np.testing.assert_allclose(np.linalg.norm(A, axis=0), np.sqrt(S), rtol=1e-10)
    np.testing.assert_allclose(np.linalg.norm(B, axis=1), np.sqrt(S), rtol=1e-10)
    # wide matrix takes the transposed route
    A2, B2, S2 = oracle.svd_lowrank(R.T.copy(), r, full=True)
    np.testing.assert_allclose(S2, S, rtol=1e-10)
    np.testing.assert_allclose(A2 @ B2, (A @ B).T, atol=1e-10)


def test_randomized_recovers_exact_low_rank():
    rng = np.random.default_rng(11)
    n, k, rank, r = 300, 200, 5, 8
    R = rng.standard_normal((n, rank)) @ rng.standard_normal((rank, k))
    omega = rng.standard_normal((k, r + 8))
    A, B, S = oracle.svd_lowrank(R, r, omega=omega, power_iters=2)
    assert np.abs(R - A @ B).max() <= 1e-12 * np.abs(R).max()
    assert np.all(S[rank:] <= 1e-10 * S[0])


def test_randomized_close_to_optimal():
    rng = np.random.default_rng(12)
    n, k, r = 400, 256, 8
    R = rng.standard_normal((n, k)) * 0.01 + rng.standard_normal((n, 3)) @ rng.standard_normal((3, k))
    A, B, S = oracle.svd_lowrank(R, r, omega=rng.standard_normal((k, r + 8)), power_iters=4)
    sig = np.linalg.svd(R, compute_uv=False)
    np.testing.assert_allclose(S[:3], sig[:3], rtol=1e-9)
    assert np.linalg.norm(R - A @ B) <= 1.05 * np.sqrt((sig[r:] ** 2).sum())


# ------------------------------------------------------------------ packing + forward

def _decode_blob_numpy(blob, N, K, r, n_seg):
    """Independent decode of the packed format from the byte layout."""
    L = oracle.layout(N, K, r, n_seg)
    n4, n8 = L["N4"], L["N8"]
    idx = blob[L["off_idx"]:L["off_idx"] + 4 * N].view(np.int32)
    q4 = blob[L["off_q4"]:L["off_q4"] + n4 * K // 2].reshape(n4, K // 2)
    runs = q4.reshape(n4, K // 8, 4)      # 4 bytes per run of 8 codes
    codes = np.concatenate([(runs & 0xF), (runs >> 4)], axis=2).astype(np.int64).reshape(n4, K) - 8
    s4 = synth.bf16_bits_to_f64(blob[L["off_s4"]:L["off_s4"] + 2 * n4 * K // 64].view(np.uint16)).reshape(n4, K // 64)
    q8 = blob[L["off_q8"]:L["off_q8"] + n8 * K].view(np.int8).reshape(n8, K).astype(np.float64)
    s8 = blob[L["off_s8"]:L["off_s8"] + 4 * n8].view(np.float32).astype(np.float64)
    What = np.concatenate([codes * np.repeat(s4, 64, axis=1), q8 * s8[:, None]])
    U = synth.bf16_bits_to_f64(blob[L["off_U"]:L["off_U"] + 2 * N * r].view(np.uint16)).reshape(N, r)
    V = synth.bf16_bits_to_f64(blob[L["off_V"]:L["off_V"] + 2 * n_seg * r * K].view(np.uint16)).reshape(n_seg * r, K)
    return idx.copy(), What, U, V


def test_layout_is_aligned_and_disjoint():
    for (N, K, r, ns) in [(512, 256, 4, 1), (10240, 2560, 16, 1), (20480, 2560, 24, 2), (2048, 6144, 32, 1)]:
        L = oracle.layout(N, K, r, ns)
        n4, n8 = L["N4"], L["N8"]
        sizes = [4 * N, n4 * K // 2, n4 * K // 64 * 2, n8 * K, 4 * n8, 2 * N * r, 2 * ns * r * K]
        offs = [L[k] for k in ("off_idx", "off_q4", "off_s4", "off_q8", "off_s8", "off_U", "off_V")]
        assert all(o % 256 == 0 for o in offs)
        for i in range(6):
            assert offs[i] + sizes[i] <= offs[i + 1]
        assert offs[6] + sizes[6] <= L["blob_bytes"]
        assert L["algo_bytes"] == sum(sizes)
        assert n8 == N // 8


@pytest.fixture(scope="module")
def tiny_case():
    lay = synth.WORKLOADS["tiny"].layers[0]
    W = synth.weights_bf16(0, lay)
    blob, diag = oracle.quantize(W, lay.r, lay.block, full_svd=True, want_diag=True)
    return lay, W, blob, diag


def test_packed_tiers_and_index(tiny_case):
    lay, W, blob, _ = tiny_case
    idx, What, U, V = oracle.unpack(blob, lay.N, lay.K, lay.r)
    idx2, What2, U2, V2 = _decode_blob_numpy(blob, lay.N, lay.K, lay.r, 1)
    np.testing.assert_array_equal(idx, idx2)
    np.testing.assert_array_equal(What, What2)
    np.testing.assert_array_equal(U, U2)
    np.testing.assert_array_equal(V, V2)
    n8 = lay.N // 8
    assert sorted(idx) == list(range(lay.N))
    assert np.all(np.diff(idx[:-n8]) > 0) and np.all(np.diff(idx[-n8:]) > 0)
    Wd = synth.bf16_bits_to_f64(W)
    energy = (Wd ** 2).sum(1)
    top = np.lexsort((np.arange(lay.N), -energy))[:n8]
    assert set(idx[-n8:]) == set(top)
    # every dequantized row sits within half a step of the rotated weight
    Wrot = oracle.fwht_rows(Wd, lay.block)
    err = np.abs(Wrot[idx] - What)
    assert err[:-n8].max() <= np.abs(Wrot).max() / 7 / 2 * 1.01


def test_pack_roundtrip_via_file(tmp_path, tiny_case):
    lay, W, blob, _ = tiny_case
    p = tmp_path / "blob.bin"
    blob.tofile(p)
    back = np.fromfile(p, dtype=np.uint8)
    np.testing.assert_array_equal(back, blob)
    blob2 = oracle.quantize(W, lay.r, lay.block, full_svd=True)
    np.testing.assert_array_equal(blob2, blob)          # deterministic


def test_svd_reduces_residual(tiny_case):
    _, _, _, diag = tiny_case
    fr, f64, fbf, _ = diag[0]
    assert f64 < fr and fbf < fr


def test_tiny_residual_eckart_young(tiny_case):
    lay, W, blob, _ = tiny_case
    idx, What, U, V = oracle.unpack(blob, lay.N, lay.K, lay.r)
    Wrot = oracle.fwht_rows(synth.bf16_bits_to_f64(W), lay.block)
    R = np.empty_like(Wrot)
    R[idx] = Wrot[idx] - What
    sig = np.linalg.svd(R, compute_uv=False)
    A, B, S = oracle.svd_lowrank(R, lay.r, full=True)
    np.testing.assert_allclose(S, sig[:lay.r], rtol=1e-10)
    err2 = np.linalg.norm(R - A @ B) ** 2
    assert abs(err2 - (sig[lay.r:] ** 2).sum()) <= 1e-10 * (sig ** 2).sum()
    # the stored factors are these, rounded to bf16
    np.testing.assert_allclose(U, A[idx], atol=np.abs(A).max() * 2 ** -8)
    np.testing.assert_allclose(V, B, atol=np.abs(B).max() * 2 ** -8)


def test_forward_dense_brute_force(tiny_case):
    lay, W, blob, _ = tiny_case
    x = synth.activations_bf16(0, "tiny", 4, lay.K)
    y = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, 1, x)
    idx, What, U, V = _decode_blob_numpy(blob, lay.N, lay.K, lay.r, 1)
    H = scipy.linalg.hadamard(lay.K) / np.sqrt(lay.K)
    xd = synth.bf16_bits_to_f64(x)
    ref = np.zeros_like(y)
    ref[:, idx] = (xd @ H) @ (What + U @ V).T
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()
    # two routes: un-rotate the weights instead of rotating x (H symmetric, orthonormal)
    ref2 = np.zeros_like(y)
    ref2[:, idx] = xd @ ((What + U @ V) @ H.T).T
    assert np.abs(y - ref2).max() <= 1e-12 * np.abs(ref).max()
    # quantized layer approximates the bf16 layer
    ytrue = xd @ synth.bf16_bits_to_f64(W).T
    assert np.abs(y - ytrue).max() <= 0.1 * np.abs(ytrue).max()


def test_forward_cols_matches_forward(tiny_case):
    lay, W, blob, _ = tiny_case
    x = synth.activations_bf16(0, "tiny", 3, lay.K)
    y = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, 1, x)
    cols = np.array([0, 5, 511, 100, 64])
    yc = oracle.forward_cols(blob, lay.N, lay.K, lay.r, lay.block, 1, x, cols)
    np.testing.assert_array_equal(yc, y[:, cols])


def test_two_segment_layer():
    # fused gate+up reading: each segment is its own projection
    lay = synth.Layer("seg2", N=2 * 256, K=256, block=256, r=4, n_seg=2, n_outlier=3, outlier_tag="seg2")
    W = synth.weights_bf16(0, lay)
    blob = oracle.quantize(W, lay.r, lay.block, n_seg=2, full_svd=True)
    single = [oracle.quantize(W[s * 256:(s + 1) * 256], lay.r, lay.block, full_svd=True) for s in range(2)]
    x = synth.activations_bf16(0, "seg2", 3, lay.K)
    y = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, 2, x)
    for s in range(2):
        ys = oracle.forward(single[s], 256, lay.K, lay.r, lay.block, 1, x)
        np.testing.assert_array_equal(y[:, s * 256:(s + 1) * 256], ys)
    idx, _, _, _ = oracle.unpack(blob, lay.N, lay.K, lay.r, 2)
    n8 = 2 * 32
    assert np.all(idx[:224] < 256) and np.all(idx[224:448] >= 256)
    assert np.all(idx[448:480] < 256) and np.all(idx[480:] >= 256)


def test_planted_mistakes_are_caught(tiny_case):
    """The dense brute-force pin fails when a term of the forward is dropped or
    an operand is transposed (mistakes planted in a copy of the oracle's
    decoded values, on the CPU)."""
    lay, W, blob, _ = tiny_case
    x = synth.activations_bf16(0, "tiny", 2, lay.K)
    y = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, 1, x)
    idx, What, U, V = _decode_blob_numpy(blob, lay.N, lay.K, lay.r, 1)
    xr = oracle.fwht_rows(synth.bf16_bits_to_f64(x), lay.block)
    variants = {
        "drop low-rank": xr @ What.T,
        "drop rotation": synth.bf16_bits_to_f64(x) @ (What + U @ V).T,
        "sign of residual": xr @ (What - U @ V).T,
    }
    for name, bad in variants.items():
        ref = np.zeros_like(y)
        ref[:, idx] = bad
        assert np.abs(y - ref).max() > 1e-6 * np.abs(y).max(), name


# ------------------------------------------------------------------ gated MLP block

def test_gelu_closed_forms():
    """GELU(x) = x Phi(x): tabulated normal-CDF values, the odd-part identity
    GELU(x) - GELU(-x) = x (Phi(x) + Phi(-x) = 1), its limits, and Phi as the
    integral of the normal density (a different route than erf)."""
    import scipy.integrate
    assert oracle.gelu(np.array([0.0]))[0] == 0.0
    # Phi(1) = 0.8413447460685429, Phi(2) = 0.9772498680518208, Phi(-1) = 0.15865525393145707
    np.testing.assert_allclose(oracle.gelu(np.array([1.0, 2.0, -1.0])),
                               [0.8413447460685429, 2 * 0.9772498680518208, -0.15865525393145707],
                               rtol=2e-15, atol=0)
    x = np.random.default_rng(3).normal(0.0, 3.0, 200)
    np.testing.assert_allclose(oracle.gelu(x) - oracle.gelu(-x), x, rtol=0, atol=1e-14)
    assert oracle.gelu(np.array([10.0]))[0] == 10.0
    assert abs(oracle.gelu(np.array([-10.0]))[0]) < 1e-20
    # the far negative tail, relatively: Phi(-5) = 2.866515718791939e-07,
    # Phi(-8) = 6.220960574271784e-16, Phi(-10) = 7.619853024160470e-24
    np.testing.assert_allclose(oracle.gelu(np.array([-5.0, -8.0, -10.0])),
                               [-5 * 2.866515718791939e-07, -8 * 6.220960574271784e-16,
                                -10 * 7.619853024160470e-24], rtol=1e-12, atol=0)
    pdf = lambda t: np.exp(-0.5 * t * t) / np.sqrt(2 * np.pi)
    for v in (-2.5, -0.3, 0.7, 1.9):
        phi = 0.5 + scipy.integrate.quad(pdf, 0.0, v, epsabs=1e-15, epsrel=1e-14)[0]
        assert abs(oracle.gelu(np.array([v]))[0] - v * phi) < 1e-13


def _dense_layer(blob, lay, n_seg, x_f64):
    """y = (x H) (W_hat + U V_seg)^T from the numpy decode of the packed bytes and
    scipy's Sylvester matrix (block = K), in original output order."""
    idx, What, U, V = _decode_blob_numpy(blob, lay.N, lay.K, lay.r, n_seg)
    seg = idx // (lay.N // n_seg)
    low = np.stack([U[p] @ V[seg[p] * lay.r:(seg[p] + 1) * lay.r] for p in range(lay.N)])
    H = scipy.linalg.hadamard(lay.K) / np.sqrt(lay.K)
    y = np.zeros((x_f64.shape[0], lay.N))
    y[:, idx] = (x_f64 @ H) @ (What + low).T
    return y


@pytest.fixture(scope="module")
def mlp_case():
    I, Hd = 128, 128
    gu = synth.Layer("mlp_gu", N=2 * I, K=Hd, block=Hd, r=4, n_seg=2, n_outlier=2, outlier_tag="mlp")
    dn = synth.Layer("mlp_dn", N=Hd, K=I, block=I, r=4)
    bg = oracle.quantize(synth.weights_bf16(0, gu), gu.r, gu.block, n_seg=2, full_svd=True)
    bd = oracle.quantize(synth.weights_bf16(1, dn), dn.r, dn.block, full_svd=True)
    return gu, dn, bg, bd


def test_mlp_chain_dense_brute_force(mlp_case):
    """The chained oracle against a dense route: decoded matrices, scipy's
    Hadamard matrix, GELU through scipy.stats' normal CDF, bf16 rounding by exact
    rational arithmetic between the projections."""
    import scipy.stats
    gu, dn, bg, bd = mlp_case
    x = synth.activations_bf16(0, "mlp", 3, gu.K)
    y = oracle.mlp_forward(bg, (gu.N, gu.K, gu.r, gu.block), bd, (dn.N, dn.K, dn.r, dn.block), x)
    rb = np.vectorize(lambda v: synth.bf16_bits_to_f64(np.array([exact_bf16(float(v))], dtype=np.uint16))[0])
    ygu = _dense_layer(bg, gu, 2, synth.bf16_bits_to_f64(x))
    I = gu.N // 2
    g, u = rb(ygu[:, :I]), rb(ygu[:, I:])
    h = rb(g * scipy.stats.norm.cdf(g) * u)
    ref = _dense_layer(bd, dn, 1, h)
    assert np.abs(y - ref).max() <= 1e-10 * np.abs(ref).max()
    # planted mistakes (in the dense route): gate and up swapped, GELU dropped
    for bad in (rb(u * scipy.stats.norm.cdf(u) * g), rb(g * u)):
        assert np.abs(y - _dense_layer(bd, dn, 1, bad)).max() > 1e-3 * np.abs(ref).max()


def test_mlp_chain_columns_and_zero(mlp_case):
    gu, dn, bg, bd = mlp_case
    x = synth.activations_bf16(1, "mlp", 2, gu.K)
    a, b = (gu.N, gu.K, gu.r, gu.block), (dn.N, dn.K, dn.r, dn.block)
    y = oracle.mlp_forward(bg, a, bd, b, x)
    cols = np.array([0, 77, 127, 3])
    np.testing.assert_array_equal(oracle.mlp_forward_cols(bg, a, bd, b, x, cols), y[:, cols])
    z = oracle.mlp_forward(bg, a, bd, b, np.zeros_like(x))
    assert np.all(z == 0.0)


# ------------------------------------------------------------------ dense materialization

def test_materialize_reproduces_forward(tiny_case):
    """x W^T with the materialized weight equals the layer's forward (which
    rotates x instead), and matches a dense route from the numpy decode and
    scipy's Hadamard matrix."""
    lay, W, blob, _ = tiny_case
    Wm = oracle.materialize(blob, lay.N, lay.K, lay.r, lay.block)
    x = synth.activations_bf16(2, "tiny", 5, lay.K)
    y = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, 1, x)
    yd = synth.bf16_bits_to_f64(x) @ Wm.T
    assert np.abs(y - yd).max() <= 1e-12 * np.abs(y).max()
    idx, What, U, V = _decode_blob_numpy(blob, lay.N, lay.K, lay.r, 1)
    H = scipy.linalg.hadamard(lay.K) / np.sqrt(lay.K)
    ref = np.zeros_like(Wm)
    ref[idx] = (What + U @ V) @ H
    assert np.abs(Wm - ref).max() <= 1e-12 * np.abs(ref).max()
    # and it approximates the weight the layer was quantized from
    Wt = synth.bf16_bits_to_f64(W)
    assert np.linalg.norm(Wm - Wt) <= 0.1 * np.linalg.norm(Wt)     # INT4 grid of Gaussian rows: ~7 %


def test_materialize_two_segments():
    lay = synth.Layer("seg2m", N=2 * 128, K=128, block=64, r=3, n_seg=2, n_outlier=2, outlier_tag="seg2m")
    blob = oracle.quantize(synth.weights_bf16(4, lay), lay.r, lay.block, n_seg=2, full_svd=True)
    Wm = oracle.materialize(blob, lay.N, lay.K, lay.r, lay.block, 2)
    x = synth.activations_bf16(4, "seg2m", 3, lay.K)
    y = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, 2, x)
    assert np.abs(y - synth.bf16_bits_to_f64(x) @ Wm.T).max() <= 1e-12 * np.abs(y).max()


# ------------------------------------------------------------------ randomized SVD inside the quantizer

@pytest.mark.parametrize("power_iters", [2, 6])
def test_quantizer_randomized_svd_two_segments(power_iters):
    """The quantizer's randomized-SVD branch (the one every full-size layer
    takes: subspace iteration on a per-segment sketch, then Jacobi) on a
    two-segment layer of 1024 rows per segment, r = 8.  For each segment s,
    with R_s = W_rot - W_hat rebuilt here from the weights and the unpacked codes:
    * the quantizer's ||R_s|| is that residual's norm;
    * its stored factors are those of svd_lowrank(R_s, sketch of segment s),
      placed at the segment's packed rows (the wiring of segment, sketch and rows);
    * the residual shrinks strictly, with fp64 and with the stored bf16 factors;
    * it is never below the optimum sqrt(sum_{i>r} sigma_i^2) (numpy's SVD), and
      the energy the factors remove is at least half of the optimum's."""
    lay = synth.Layer("svd_pin", N=2 * 1024, K=512, block=256, r=8, n_seg=2, n_outlier=5, outlier_tag="svd_pin")
    W = synth.weights_bf16(0, lay)
    l = lay.r + 8
    omega = np.stack([synth.sketch(0, lay, s, l) for s in range(2)])
    blob, diag = oracle.quantize(W, lay.r, lay.block, 2, omega=omega, power_iters=power_iters, want_diag=True)
    idx, What, U, V = oracle.unpack(blob, lay.N, lay.K, lay.r, 2)
    Wrot = oracle.fwht_rows(synth.bf16_bits_to_f64(W), lay.block)
    Ns = lay.N // 2
    for s in range(2):
        rows = np.nonzero(idx // Ns == s)[0]            # packed rows of segment s, in packed order
        order = np.argsort(idx[rows])                   # -> original row order of the segment
        prow = rows[order]
        R = Wrot[idx[prow]] - What[prow]
        fr = np.linalg.norm(R)
        assert abs(diag[s, 0] - fr) <= 1e-12 * fr
        A, B, _ = oracle.svd_lowrank(R, lay.r, omega[s], power_iters)
        np.testing.assert_array_equal(U[prow], synth.bf16_bits_to_f64(oracle.bf16_round_bits(A)))
        np.testing.assert_array_equal(V[s * lay.r:(s + 1) * lay.r], synth.bf16_bits_to_f64(oracle.bf16_round_bits(B)))
        f64, fbf = diag[s, 1], diag[s, 2]
        assert f64 < fr and fbf < fr
        assert abs(np.linalg.norm(R - U[prow] @ V[s * lay.r:(s + 1) * lay.r]) - fbf) <= 1e-9 * fr
        sv = np.linalg.svd(R, compute_uv=False)
        opt = np.sqrt((sv[lay.r:] ** 2).sum())
        assert f64 >= opt * (1 - 1e-12)
        assert fr ** 2 - f64 ** 2 >= 0.5 * (fr ** 2 - opt ** 2)
