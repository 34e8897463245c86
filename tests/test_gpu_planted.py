"""GPU parity on planted packed layers (tests/planted.py), element by element
against the fp64 oracle on the same blob, through the C ABI.

* Low-rank only: the output is t U^T alone, so the low-rank term is held to
  5e-3 of its own scale (in the quantized layers it is ~1 % of max|y|, too
  small for the layer tolerance to see a wrong term).
* Edge codes: codes -8 and -128, whole rows and groups at the extremes, zero
  groups and zero INT8 rows.
* Scale range: INT4 group scales in [2^-20, 2^-14) and (63, 256], INT8 row
  scales over [2^-30, 2^10]; each class of rows is checked against its own
  largest output.
Every case runs on the decode kernel, the prefill path and, for shapes that
the single-launch decode does not take (blocks of 2048 at M = 32, K not a
multiple of 256), the decode call's prefill route.
"""
import numpy as np
import pytest

import cases
import oracle
import planted

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bit_linear_amd as dv  # noqa: E402

DEV = "cuda:0"


def run_blob(lay, blob, M, path, flags=0, M_max=None):
    lin = dv.Linear(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, M_max=M_max or max(M, 32), device=DEV)
    x_bits = cases.activations(lay.name, M)
    y = lin.forward(cases.to_device_bf16(x_bits, DEV), flags=flags, path=path)
    torch.cuda.synchronize()
    return x_bits, cases.from_device_bf16(y), lin


LOWRANK = [
    ("decode", "spark_up", 1), ("decode", "spark_up", 4), ("decode", "spark_up", 16), ("decode", "spark_up", 32),
    ("decode", "spark_down", 1), ("decode", "spark_down", 32), ("decode", "spark_gateup", 1),
    ("decode", "minicpm_down", 1), ("decode", "minicpm_gate_r32", 1), ("decode", "tiny", 5),
    ("decode", "seg2_b512_r32", 7), ("decode", "b2048_ragged", 32), ("decode", "k192_b64", 3),
    ("prefill", "spark_gateup", 512), ("prefill", "minicpm_down", 4096), ("prefill", "tiny", 130),
    ("prefill", "seg2_b512_r32", 129), ("prefill", "spark_down", 512),
]


@pytest.mark.parametrize("path,name,M", LOWRANK, ids=[f"{p}-{n}-M{m}" for p, n, m in LOWRANK])
def test_lowrank_term_alone(path, name, M):
    lay, blob, _ = cases.planted_blob(name, "lowrank")
    x_bits, y, _ = run_blob(lay, blob, M, path)
    ref = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, x_bits)
    err = cases.rel_err(y, ref)
    print(f"lowrank {path} {name} M={M} rel_err={err:.3e}")
    assert np.abs(ref).max() > 0
    assert err <= cases.TOL


EDGE = [
    ("decode", "tiny", 1), ("decode", "tiny", 5), ("decode", "tiny", 32), ("decode", "spark_up", 4),
    ("decode", "spark_down", 8), ("decode", "spark_gateup", 1), ("decode", "minicpm_down", 1),
    ("decode", "k192_b64", 7), ("decode", "b2048_ragged", 32),
    ("prefill", "tiny", 130), ("prefill", "spark_up", 384), ("prefill", "seg2_small", 77),
    ("prefill", "b1024_tail", 64), ("prefill", "spark_down", 200),
]


@pytest.mark.parametrize("path,name,M", EDGE, ids=[f"{p}-{n}-M{m}" for p, n, m in EDGE])
def test_edge_codes(path, name, M):
    lay, blob, _ = cases.planted_blob(name, "edge")
    x_bits, y, _ = run_blob(lay, blob, M, path)
    ref = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, x_bits)
    err = cases.rel_err(y, ref)
    print(f"edge {path} {name} M={M} rel_err={err:.3e}")
    assert err <= cases.TOL


SCALES = [
    ("decode", "tiny", 1), ("decode", "tiny", 9), ("decode", "spark_up", 1), ("decode", "spark_down", 32),
    ("decode", "b2048_ragged", 32), ("decode", "k192_b64", 5),
    ("prefill", "tiny", 130), ("prefill", "spark_up", 384), ("prefill", "spark_down", 200),
    ("prefill", "minicpm_gate", 256), ("prefill", "ragged_b64_r1", 45),
]


@pytest.mark.parametrize("path,name,M", SCALES, ids=[f"{p}-{n}-M{m}" for p, n, m in SCALES])
def test_scales_across_the_bf16_range(path, name, M):
    lay, blob, cls = cases.planted_blob(name, "scales")
    x_bits, y, _ = run_blob(lay, blob, M, path)
    ref = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, x_bits)
    labels = list(planted.SCALE_CLASSES) + ["INT8 rows"]
    for label, cols in zip(labels, planted.class_columns(blob, lay, cls)):
        if cols.size == 0:
            continue
        err = cases.rel_err(y[:, cols], ref[:, cols])
        print(f"scales {path} {name} M={M} {label}: rel_err={err:.3e}")
        assert np.abs(ref[:, cols]).max() > 0
        assert err <= cases.TOL, label


# ------------------------------------------------------------------ bounded waits

TIMEOUT_CASES = [("tiny", 1), ("tiny", 5), ("spark_down", 8)]


@pytest.mark.parametrize("name,M", TIMEOUT_CASES, ids=[f"{n}-M{m}" for n, m in TIMEOUT_CASES])
def test_wait_timeout_poisons_outputs(name, M):
    """DVSSQ_TEST_NO_PUBLISH keeps the producers from publishing, so every
    consumer's bounded wait gives up after a few polls: every output is NaN
    and the workspace's status word reads DVSSQ_STATUS_WAIT_TIMEOUT.  Every
    kernel exits normally; the next ordinary call is correct again."""
    lay, blob = cases.quantized(name)
    lin = dv.Linear(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, M_max=32, device=DEV)
    lin.ws[:dv.DVSSQ_WS_STATUS_BYTES].zero_()
    x_bits = cases.activations(name, M)
    x = cases.to_device_bf16(x_bits, DEV)
    y = lin.forward(x, flags=dv.DVSSQ_TEST_NO_PUBLISH, path="decode")
    torch.cuda.synchronize()
    assert torch.isnan(y.float()).all()
    status = int(lin.ws[:4].view(torch.int32).item())
    assert status == dv.DVSSQ_STATUS_WAIT_TIMEOUT
    y2 = cases.from_device_bf16(lin.forward(x, path="decode"))
    ref = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, x_bits)
    assert cases.rel_err(y2, ref) <= cases.TOL


def test_status_word_stays_clear_on_success():
    lay, blob = cases.quantized("spark_up")
    lin = dv.Linear(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, M_max=32, device=DEV)
    lin.ws[:dv.DVSSQ_WS_STATUS_BYTES].zero_()
    x = cases.to_device_bf16(cases.activations("spark_up", 16), DEV)
    for M in (1, 4, 16):
        lin.forward(x[:M], path="decode")
    torch.cuda.synchronize()
    assert int(lin.ws[:4].view(torch.int32).item()) == 0
