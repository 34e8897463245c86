"""GPU parity: every call goes through the C ABI (libdvssq.so) and is compared
with the fp64 oracle on the same seeded inputs and the same packed blob.

Bar: max|y_gpu - y_ref| / max|y_ref| <= 5e-3 (bf16 activations, fp32
accumulation); bit-exact for the blob round trip and for repeated calls.
"""
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


def gpu_layer(name, M_max):
    lay, blob = cases.quantized(name)
    return lay, blob, dv.Linear(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, M_max=M_max, device=DEV)


def run(lin, x_bits, path, flags=0):
    x = cases.to_device_bf16(x_bits, DEV)
    y = lin.forward(x, flags=flags, path=path)
    torch.cuda.synchronize()
    return cases.from_device_bf16(y)


# ------------------------------------------------------------------ rotation

@pytest.mark.parametrize("b", [64, 128, 256, 512, 1024, 2048])
@pytest.mark.parametrize("M", [1, 5, 37])
def test_fwht_parity(b, M):
    K = b * (3 if b <= 512 else 2)
    x_bits = synth.activations_bf16(7, f"fwht{b}", M, K)
    ref = oracle.rotate_x(x_bits, b)
    x = cases.to_device_bf16(x_bits, DEV)
    out = torch.empty_like(x)
    dv.fwht(x, out, M, K, b)
    torch.cuda.synchronize()
    got = cases.from_device_bf16(out)
    err = np.abs(got - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max())
    same = got == synth.bf16_bits_to_f64(synth.to_bf16_bits(ref))
    assert same.mean() >= 0.99
    # in place
    dv.fwht(x, x, M, K, b)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cases.from_device_bf16(x), got)


def test_fwht_exact_special_cases():
    b, K = 256, 512
    x = np.zeros((3, K))
    x[0, 3] = 1.0                 # one-hot -> +-1/16 everywhere in its block
    x[1, 256:] = 1.0              # constant block -> 16 e_0
    x[2, 100] = -2.0
    bits = synth.to_bf16_bits(x)
    d = cases.to_device_bf16(bits, DEV)
    out = torch.empty_like(d)
    dv.fwht(d, out, 3, K, b)
    torch.cuda.synchronize()
    got = cases.from_device_bf16(out)
    np.testing.assert_array_equal(got, oracle.rotate_x(bits, b))
    np.testing.assert_array_equal(np.abs(got[0, :256]), np.full(256, 1 / 16))
    assert got[1, 256] == 16 and not got[1, 257:].any() and not got[1, :256].any()


# ------------------------------------------------------------------ decode

DECODE_CASES = [
    ("tiny", 1), ("tiny", 4), ("tiny", 3), ("tiny", 8), ("tiny", 9), ("tiny", 16), ("tiny", 17),
    ("tiny", 32),
    ("spark_up", 1), ("spark_up", 4), ("spark_up", 16), ("spark_up", 32),
    ("spark_down", 1), ("spark_down", 8), ("spark_down", 32),
    ("minicpm_gate", 1), ("minicpm_up", 1), ("minicpm_down", 1),
    ("minicpm_gate_r32", 1), ("minicpm_down_r32", 1),
    ("spark_gateup", 1), ("spark_gateup", 4),
    ("ragged_b64_r1", 1), ("ragged_b64_r1", 7), ("b128_r64", 32), ("seg2_b512_r32", 5),
    ("b1024_tail", 3), ("b2048_ragged", 17), ("b2048_ragged", 32), ("seg2_small", 2),
    # K not a multiple of 256, and blocks of 2048 at M = 32: the decode call's prefill route
    ("k192_b64", 1), ("k192_b64", 7), ("minicpm_down", 32),
]


@pytest.mark.parametrize("name,M", DECODE_CASES, ids=[f"{n}-M{m}" for n, m in DECODE_CASES])
def test_decode_parity(name, M):
    lay, blob, lin = gpu_layer(name, 32)
    x_bits = cases.activations(name, 32)[:M]
    y = run(lin, x_bits, "decode")
    ref = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, x_bits)
    err = cases.rel_err(y, ref)
    print(f"{name} M={M} decode rel_err={err:.3e}")
    assert err <= cases.TOL


# ------------------------------------------------------------------ prefill

PREFILL_CASES = [
    ("tiny", 1), ("tiny", 4), ("tiny", 33), ("tiny", 130), ("tiny", 257),
    ("ragged_b64_r1", 45), ("k192_b64", 19), ("b128_r64", 200), ("seg2_b512_r32", 129), ("b1024_tail", 64),
    ("b2048_ragged", 100), ("seg2_small", 77), ("spark_up", 40),
    # 120 GEMM tiles (K split in two) and 160 tiles (no split), element by element
    ("spark_up", 384), ("spark_up", 512),
]


@pytest.mark.parametrize("name,M", PREFILL_CASES, ids=[f"{n}-M{m}" for n, m in PREFILL_CASES])
def test_prefill_parity(name, M):
    lay, blob, lin = gpu_layer(name, M)
    x_bits = cases.activations(name, M)
    y = run(lin, x_bits, "prefill")
    ref = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, x_bits)
    err = cases.rel_err(y, ref)
    print(f"{name} M={M} prefill rel_err={err:.3e}")
    assert err <= cases.TOL


def test_prefill_full_size_gateup_m512_every_element():
    """The fused gate+up layer (two segments, N = 20480) at M = 512, the
    benchmark's shape and launch, compared on every output element."""
    lay, blob, lin = gpu_layer("spark_gateup", 512)
    x_bits = cases.activations("spark_gateup", 512)
    y = run(lin, x_bits, "prefill")
    ref = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, x_bits)
    err = cases.rel_err(y, ref)
    print(f"spark_gateup M=512 prefill (every element) rel_err={err:.3e}")
    assert err <= cases.TOL


FULL_PREFILL = [("spark_gateup", 2048), ("minicpm_gate", 4096),
                ("minicpm_up", 4096), ("minicpm_down", 4096), ("minicpm_down_r32", 4096)]


@pytest.mark.parametrize("name,M", FULL_PREFILL, ids=[f"{n}-M{m}" for n, m in FULL_PREFILL])
def test_prefill_full_size_sampled(name, M):
    """Full-size prefill, checked on sampled output columns (all tokens)."""
    lay, blob, lin = gpu_layer(name, M)
    x_bits = cases.activations(name, M)
    y = run(lin, x_bits, "prefill")
    cols = cases.sample_columns(lay, blob)
    ref = oracle.forward_cols(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, x_bits, cols)
    err = cases.rel_err(y[:, cols], ref)
    print(f"{name} M={M} prefill sampled({cols.size} cols) rel_err={err:.3e}")
    assert err <= cases.TOL


# ------------------------------------------------------------------ special inputs and properties

@pytest.mark.parametrize("path,M", [("decode", 5), ("prefill", 70)])
def test_zero_input_gives_zero(path, M):
    lay, blob, lin = gpu_layer("tiny", max(M, 32))
    y = run(lin, np.zeros((M, lay.K), dtype=np.uint16), path)
    assert not y.any()


@pytest.mark.parametrize("path,M", [("decode", 6), ("prefill", 40)])
def test_prerotated_input_flag(path, M):
    lay, blob, lin = gpu_layer("spark_down" if path == "decode" else "tiny", max(M, 32))
    x_bits = cases.activations(lay.name, M)
    xr_bits = synth.to_bf16_bits(oracle.rotate_x(x_bits, lay.block))
    y = run(lin, xr_bits, path, flags=dv.DVSSQ_X_ROTATED)
    idx, What, U, V = oracle.unpack(blob, lay.N, lay.K, lay.r, lay.n_seg)
    xr = synth.bf16_bits_to_f64(xr_bits)
    ref = np.zeros((M, lay.N))
    Ns = lay.N // lay.n_seg
    t = xr @ V.T
    for s in range(lay.n_seg):
        rows = np.nonzero(idx // Ns == s)[0]
        ref[:, idx[rows]] = xr @ What[rows].T + t[:, s * lay.r:(s + 1) * lay.r] @ U[rows].T
    assert cases.rel_err(y, ref) <= cases.TOL


def test_blob_roundtrip_bit_exact():
    lay, blob, lin = gpu_layer("spark_up", 32)
    back = lin.blob.cpu().numpy()
    np.testing.assert_array_equal(back, blob)


@pytest.mark.parametrize("path,name,M", [("decode", "spark_down", 8), ("prefill", "tiny", 130)])
def test_repeat_calls_are_bit_identical(path, name, M):
    lay, blob, lin = gpu_layer(name, max(M, 32))
    x = cases.to_device_bf16(cases.activations(name, M), DEV)
    first = lin.forward(x, path=path).clone()
    for _ in range(20):
        again = lin.forward(x, path=path)
        assert torch.equal(again.view(torch.int16), first.view(torch.int16))


def test_decode_and_prefill_share_workspace():
    lay, blob, lin = gpu_layer("tiny", 64)
    x_bits = cases.activations("tiny", 64)
    ref = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, x_bits)
    x = cases.to_device_bf16(x_bits, DEV)
    yd = lin.forward(x[:3], path="decode")
    yp = lin.forward(x, path="prefill")
    yd2 = lin.forward(x[:32], path="decode")
    torch.cuda.synchronize()
    assert cases.rel_err(cases.from_device_bf16(yd), ref[:3]) <= cases.TOL
    assert cases.rel_err(cases.from_device_bf16(yp), ref) <= cases.TOL
    assert cases.rel_err(cases.from_device_bf16(yd2), ref[:32]) <= cases.TOL


def test_decode_matches_prefill():
    lay, blob, lin = gpu_layer("spark_up", 32)
    x = cases.to_device_bf16(cases.activations("spark_up", 16), DEV)
    yd = cases.from_device_bf16(lin.forward(x, path="decode"))
    yp = cases.from_device_bf16(lin.forward(x, path="prefill"))
    assert cases.rel_err(yd, yp) <= cases.TOL


# ------------------------------------------------------------------ gated MLP block (decode)

MLP_CASES = [("mlp_tiny_gu", "mlp_tiny_dn", 1), ("mlp_tiny_gu", "mlp_tiny_dn", 3), ("mlp_tiny_gu", "mlp_tiny_dn", 32),
             ("spark_gateup", "spark_down", 1), ("spark_gateup", "spark_down", 4)]


def gpu_mlp(gname, dname):
    g, gb, lg = gpu_layer(gname, 32)
    d, db, ld = gpu_layer(dname, 32)
    return g, gb, d, db, dv.MLP(lg, ld)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """One unit in the last place of bf16 at |v| (normal range)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def check_mlp_stages(mlp, g, gb, d, db, x_bits, y_gpu, rows=None):
    """Each stage of the block on its own, at the layer tolerance:
    (1) the fused gate+up output (from the block's workspace) against the
        oracle's fused layer on the same x;
    (2) the intermediate h against bf16(gelu(g) u) computed in fp64 from the
        GPU's own bf16 g and u: within one bf16 unit;
    (3) the block's output against the oracle's down projection of the GPU's
        own h.
    The end-to-end error against the chained oracle is printed, not asserted:
    a tie of a bf16 rounding in g, u or h that falls the other way moves an
    element of h by one unit, which the down projection carries on.
    rows: token rows to check (default all)."""
    M = x_bits.shape[0]
    rows = np.arange(M) if rows is None else np.asarray(rows)
    off_ygu, off_h = dv.mlp_ws_offsets(mlp.gu.layout, mlp.down.layout)
    ws = mlp.ws
    ygu_bits = ws[off_ygu:off_ygu + 2 * M * g.N].view(torch.int16).view(M, g.N).cpu().numpy().view(np.uint16)
    h_bits = ws[off_h:off_h + 2 * M * d.K].view(torch.int16).view(M, d.K).cpu().numpy().view(np.uint16)
    ygu_bits, h_bits = ygu_bits[rows], h_bits[rows]
    xr = x_bits[rows]
    ygu = synth.bf16_bits_to_f64(ygu_bits)
    ref_gu = oracle.forward(gb, g.N, g.K, g.r, g.block, 2, xr)
    e1 = cases.rel_err(ygu, ref_gu)
    I = g.N // 2
    h = synth.bf16_bits_to_f64(h_bits)
    h_ref = oracle.gelu(ygu[:, :I]) * ygu[:, I:]
    e2 = float((np.abs(h - h_ref) / bf16_ulp(h_ref)).max())
    ref_y = oracle.forward(db, d.N, d.K, d.r, d.block, 1, h_bits)
    e3 = cases.rel_err(y_gpu[rows], ref_y)
    e2e = cases.rel_err(y_gpu[rows], oracle.mlp_forward(gb, (g.N, g.K, g.r, g.block), db,
                                                        (d.N, d.K, d.r, d.block), xr))
    print(f"mlp stages: gate+up rel_err={e1:.3e}  h worst/ulp={e2:.3f}  down rel_err={e3:.3e}  "
          f"(end to end {e2e:.3e})")
    assert e1 <= cases.TOL
    assert e2 <= 1.0
    assert e3 <= cases.TOL


@pytest.mark.parametrize("gname,dname,M", MLP_CASES, ids=[f"{g}-M{m}" for g, _, m in MLP_CASES])
def test_mlp_decode_parity(gname, dname, M):
    """y = down(gelu(gate(x)) * up(x)) through dvssq_mlp_decode, stage by stage."""
    g, gb, d, db, mlp = gpu_mlp(gname, dname)
    x_bits = cases.activations(gname, M)
    y = mlp.forward(cases.to_device_bf16(x_bits, DEV))
    torch.cuda.synchronize()
    check_mlp_stages(mlp, g, gb, d, db, x_bits, cases.from_device_bf16(y))


MLP_PREFILL_CASES = [("mlp_tiny_gu", "mlp_tiny_dn", 40), ("mlp_tiny_gu", "mlp_tiny_dn", 130),
                     ("spark_gateup", "spark_down", 48)]


@pytest.mark.parametrize("gname,dname,M", MLP_PREFILL_CASES, ids=[f"{g}-M{m}" for g, _, m in MLP_PREFILL_CASES])
def test_mlp_prefill_parity(gname, dname, M):
    """The prefill form of the block (dvssq_mlp_prefill), stage by stage."""
    g, gb, lg = gpu_layer(gname, 256)
    d, db, ld = gpu_layer(dname, 256)
    mlp = dv.MLP(lg, ld)
    x_bits = cases.activations(gname, M)
    y = mlp.forward(cases.to_device_bf16(x_bits, DEV), path="prefill")
    torch.cuda.synchronize()
    check_mlp_stages(mlp, g, gb, d, db, x_bits, cases.from_device_bf16(y))


def test_mlp_prefill_full_size_sampled():
    """The Spark block at M=2048 tokens (the shape and launch the benchmark times),
    stage by stage on sampled tokens: each token's output depends on its own row
    of x only.  The rows cover the first and last 128-token tiles, a tile
    boundary and the middle."""
    M = 2048
    g, gb, lg = gpu_layer("spark_gateup", M)
    d, db, ld = gpu_layer("spark_down", M)
    mlp = dv.MLP(lg, ld)
    x_bits = cases.activations("spark_gateup", M)
    y = cases.from_device_bf16(mlp.forward(cases.to_device_bf16(x_bits, DEV), path="prefill"))
    torch.cuda.synchronize()
    check_mlp_stages(mlp, g, gb, d, db, x_bits, y, rows=[0, 1, 127, 128, 1000, 1919, 2047])


def test_mlp_decode_matches_its_parts():
    """The block equals its three steps run separately: the fused decode, the
    GELU product on the host (fp32, one bf16 rounding) and the down decode."""
    g, gb, d, db, mlp = gpu_mlp("mlp_tiny_gu", "mlp_tiny_dn")
    M = 5
    x = cases.to_device_bf16(cases.activations("mlp_tiny_gu", M), DEV)
    y = mlp.forward(x)
    ygu = mlp.gu.forward(x, path="decode").float()
    I = g.N // 2
    h = (torch.nn.functional.gelu(ygu[:, :I]) * ygu[:, I:]).to(torch.bfloat16)
    y2 = mlp.down.forward(h, path="decode")
    torch.cuda.synchronize()
    assert cases.rel_err(cases.from_device_bf16(y), cases.from_device_bf16(y2)) <= 0.2 * cases.TOL


def test_mlp_decode_rejects_mismatched_pair():
    g, gb, lg = gpu_layer("mlp_tiny_gu", 32)
    d, db, ld = gpu_layer("tiny", 32)
    with pytest.raises(dv.DvssqError):
        dv.MLP(lg, ld)


# ------------------------------------------------------------------ dense materialization

DENSE_CASES = ["tiny", "ragged_b64_r1", "b128_r64", "seg2_b512_r32", "b1024_tail", "b2048_ragged", "seg2_small",
               "spark_up"]


@pytest.mark.parametrize("name", DENSE_CASES)
def test_materialize_parity(name):
    """dvssq_materialize against the oracle's (W_hat + U V_seg) H, element by
    element: one bf16 rounding of an fp32 value."""
    lay, blob, lin = gpu_layer(name, 8)
    w = torch.empty((lay.N, lay.K), dtype=torch.bfloat16, device=DEV)
    dv.materialize(lin.layout, lin.blob, w)
    torch.cuda.synchronize()
    got = cases.from_device_bf16(w)
    ref = oracle.materialize(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max()
    worst = float((np.abs(got - ref) / bound).max())
    print(f"{name} materialize worst/bound={worst:.3f}")
    assert worst <= 1.0


def test_materialized_dense_gemm_matches_layer():
    """x W^T on the materialized weights (a plain bf16 GEMM, fp32 accumulation)
    reproduces the layer's forward."""
    lay, blob, lin = gpu_layer("spark_up", 8)
    w = torch.empty((lay.N, lay.K), dtype=torch.bfloat16, device=DEV)
    dv.materialize(lin.layout, lin.blob, w)
    x_bits = cases.activations("spark_up", 8)
    x = cases.to_device_bf16(x_bits, DEV)
    y = torch.matmul(x.float(), w.float().t())
    torch.cuda.synchronize()
    ref = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, 1, x_bits)
    assert cases.rel_err(y.cpu().double().numpy(), ref) <= cases.TOL
