"""GPU quantizer parity: dvssq_quantize (through the C ABI) against the fp64
oracle's quantizer on the same bf16 weights and the same Gaussian sketches.

Bar: idx, INT4 codes and scales, INT8 codes and scales and every padding byte
bit-exact; U and V (bf16 rank-r factors, whose fp64 sums run in another order)
within one bf16 unit, with at most 1e-3 of their entries off at all; and the
layer's forward on the GPU-quantized blob within the parity tolerance of the
oracle's forward on the oracle's blob.
"""
import functools

import numpy as np
import pytest

import cases
import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bit_linear_amd as dv  # noqa: E402

DEV = "cuda:0"


def sketches(lay, l, seed=0):
    return np.stack([synth.sketch(seed, lay, s, l) for s in range(lay.n_seg)])


@functools.lru_cache(maxsize=None)
def weights(name, variant=""):
    lay = cases.LAYERS[name]
    W = synth.weights_bf16(0, lay).copy()
    if variant == "pairs":
        # every row repeated once: each salience value appears twice, and with
        # an odd INT8 count per segment one tied pair straddles the tier cut
        W[1::2] = W[0::2]
        W[7] = 0          # an all-zero row (zero scales, zero codes)
    elif variant == "zero":
        W[:] = 0
    return W


@functools.lru_cache(maxsize=None)
def oracle_blob(name, l, p, variant=""):
    lay = cases.LAYERS[name]
    return oracle.quantize(weights(name, variant), lay.r, lay.block, lay.n_seg,
                           omega=sketches(lay, l), power_iters=p)


def gpu_quantize(lay, W, om, l, p, blob=None, ws=None):
    L = dv.pack_info(lay.N, lay.K, lay.r, lay.block, lay.n_seg)
    Wd = torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).to(DEV)
    od = torch.from_numpy(np.ascontiguousarray(om, dtype=np.float64)).to(DEV)
    if blob is None:
        blob = dv.device_buffer(L.blob_bytes, DEV)
        blob.fill_(0xA5)            # every byte must be overwritten
    if ws is None:
        ws = dv.device_buffer(dv.quantize_ws_bytes(L, l), DEV)
        ws.fill_(0xFF)              # no initialization expected
    dv.quantize(L, Wd, od, l, p, blob, ws)
    torch.cuda.synchronize()
    return blob.cpu().numpy(), blob, ws


def bf16_key(bits):
    """Monotone integer key of bf16 bit patterns (one step = one unit)."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def compare(lay, got, ref):
    L = oracle.layout(lay.N, lay.K, lay.r, lay.n_seg)
    oU, oV = L["off_U"], L["off_V"]
    nU, nV = 2 * lay.N * lay.r, 2 * lay.n_seg * lay.r * lay.K
    assert got.size == ref.size
    # idx, q4, s4, q8, s8 and the padding up to U: bit for bit
    bad = np.flatnonzero(got[:oU] != ref[:oU])
    assert bad.size == 0, f"{bad.size} code/scale bytes differ, first at {bad[:8]}"
    # padding after U and after V
    np.testing.assert_array_equal(got[oU + nU:oV], ref[oU + nU:oV])
    np.testing.assert_array_equal(got[oV + nV:], ref[oV + nV:])
    for name, a, n in (("U", oU, nU), ("V", oV, nV)):
        g = bf16_key(got[a:a + n].view(np.uint16))
        r = bf16_key(ref[a:a + n].view(np.uint16))
        d = np.abs(g - r)
        assert d.max() <= 1, f"{name}: {d.max()} bf16 units apart"
        assert (d > 0).mean() <= 1e-3, f"{name}: {(d > 0).mean():.2e} of entries differ"


QZ_CASES = [
    # name, l - r, power_iters
    ("tiny", 8, 2),
    ("tiny", 0, 2),
    ("tiny", 8, 0),
    ("tiny", 8, 4),
    ("seg2_small", 8, 2),
    ("ragged_b64_r1", 8, 2),
    ("k192_b64", 8, 2),
    ("b128_r64", 8, 2),
    ("b128_r64", 32, 1),          # l = min(N, K) = 96
    ("seg2_b512_r32", 8, 2),
    ("b1024_tail", 8, 2),
    ("b2048_ragged", 8, 2),
    ("mlp_tiny_gu", 8, 2),
    ("spark_up", 8, 2),
    ("spark_down", 8, 2),         # K = 10240: the rotation row needs > 64 KB of LDS
    ("spark_gateup", 8, 2),       # two segments of 10240 rows, r = 24
    ("minicpm_gate", 8, 2),       # blocks of 2048
    ("minicpm_down", 8, 2),       # K = 6144, three blocks of 2048
    ("minicpm_gate_r32", 8, 2),   # r = 32
]


@pytest.mark.parametrize("name,extra,p", QZ_CASES)
def test_quantize_parity(name, extra, p):
    lay = cases.LAYERS[name]
    l = lay.r + extra
    print(f"quantize {name} l={l} p={p}", flush=True)
    ref = oracle_blob(name, l, p)
    got, _, _ = gpu_quantize(lay, weights(name), sketches(lay, l), l, p)
    compare(lay, got, ref)


def test_quantize_ties_and_zero_rows():
    # N = 8 * 67: 67 INT8 rows, so one pair of equal saliences is split by the cut
    lay = synth.Layer("pairs_536", N=536, K=256, block=256, r=4, n_outlier=3, outlier_tag="pairs")
    cases.LAYERS.setdefault(lay.name, lay)
    l = lay.r + 8
    ref = oracle_blob(lay.name, l, 2, "pairs")
    got, _, _ = gpu_quantize(lay, weights(lay.name, "pairs"), sketches(lay, l), l, 2)
    compare(lay, got, ref)
    L = oracle.layout(lay.N, lay.K, lay.r, lay.n_seg)
    idx = got[L["off_idx"]:L["off_idx"] + 4 * lay.N].view(np.int32)
    assert sorted(idx.tolist()) == list(range(lay.N))


def test_quantize_zero_weight():
    name = "tiny"
    lay = cases.LAYERS[name]
    l = lay.r + 8
    ref = oracle_blob(name, l, 2, "zero")
    got, _, _ = gpu_quantize(lay, weights(name, "zero"), sketches(lay, l), l, 2)
    compare(lay, got, ref)
    L = oracle.layout(lay.N, lay.K, lay.r, lay.n_seg)
    assert not got[L["off_U"]:].any()            # zero residual: zero factors
    assert np.all(got[L["off_q4"]:L["off_q4"] + L["N4"] * lay.K // 2] == 0x88)


def test_quantize_repeat_and_reuse():
    # a second call into the same blob and workspace (left dirty by a larger
    # layer's call) gives the same bytes
    big, small = cases.LAYERS["seg2_small"], cases.LAYERS["tiny"]
    lb, ls = big.r + 8, small.r + 8
    Lb = dv.pack_info(big.N, big.K, big.r, big.block, big.n_seg)
    Ls = dv.pack_info(small.N, small.K, small.r, small.block, small.n_seg)
    ws = dv.device_buffer(max(dv.quantize_ws_bytes(Lb, lb), dv.quantize_ws_bytes(Ls, ls)), DEV)
    blob = dv.device_buffer(max(Lb.blob_bytes, Ls.blob_bytes), DEV)
    gpu_quantize(big, weights("seg2_small"), sketches(big, lb), lb, 2, blob=blob, ws=ws)
    a, _, _ = gpu_quantize(small, weights("tiny"), sketches(small, ls), ls, 2, blob=blob, ws=ws)
    b, _, _ = gpu_quantize(small, weights("tiny"), sketches(small, ls), ls, 2, blob=blob, ws=ws)
    n = Ls.blob_bytes
    np.testing.assert_array_equal(a[:n], b[:n])
    compare(small, a[:n], oracle_blob("tiny", ls, 2))


@pytest.mark.parametrize("name,M", [("tiny", 1), ("tiny", 40), ("seg2_small", 3)])
def test_quantize_then_forward(name, M):
    # the whole path on the GPU: quantize, then the layer's forward on that blob
    lay = cases.LAYERS[name]
    l = lay.r + 8
    got, blob_d, _ = gpu_quantize(lay, weights(name), sketches(lay, l), l, 2)
    x_bits = cases.activations(name, M)
    y_ref = oracle.forward(oracle_blob(name, l, 2), lay.N, lay.K, lay.r, lay.block, lay.n_seg, x_bits)
    lin = dv.Linear(got, lay.N, lay.K, lay.r, lay.block, lay.n_seg, M_max=max(M, 32), device=DEV)
    y = lin.forward(cases.to_device_bf16(x_bits, DEV))
    torch.cuda.synchronize()
    assert cases.rel_err(cases.from_device_bf16(y), y_ref) <= cases.TOL
