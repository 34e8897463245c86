"""dvssq_linear_decode_noalloc (the decode call without a workspace, for
callers that cannot allocate) against dvssq_linear_decode through the C ABI:
the same outputs bit for bit, and within 5e-3 of the oracle, on calls in a row
that share the library's scratch array, each later call on a smaller input
(fewer rows, then a smaller layer)."""
import numpy as np
import pytest

import cases
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bit_linear_amd as dv  # noqa: E402

DEV = "cuda:0"

# split-K plan, then fewer rows of a wider layer, then the small layer, then a
# shape that takes the prefill route (K not a multiple of 256)
SEQUENCE = [("spark_down", 32), ("spark_up", 4), ("spark_up", 1), ("tiny", 3), ("k192_b64", 5), ("tiny", 1)]


def test_noalloc_matches_decode_on_calls_in_a_row():
    for name, M in SEQUENCE:
        lay, blob = cases.quantized(name)
        lin = dv.Linear(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, M_max=32, device=DEV)
        x_bits = cases.activations(name, M)
        x = cases.to_device_bf16(x_bits, DEV)
        y_ws = lin.forward(x, path="decode")
        y_na = torch.full_like(y_ws, float("nan"))
        dv.linear_decode_noalloc(lin.layout, lin.blob, x, y_na, M)
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), (name, M)
        ref = oracle.forward(blob, lay.N, lay.K, lay.r, lay.block, lay.n_seg, x_bits)
        err = cases.rel_err(cases.from_device_bf16(y_na), ref)
        print(f"noalloc {name} M={M}: bit-identical to the workspace call, rel_err={err:.3e}")
        assert err <= cases.TOL


def test_noalloc_rejects_a_call_beyond_the_scratch_array():
    """A call that needs more than the array holds (K = 262208, not a multiple of
    256, takes the prefill route, whose f16 x_rot tiles alone are 2 x 128 x K =
    67 MB): a clear error, nothing launched."""
    K = 262144 + 64
    L = dv.pack_info(8, K, 1, 64, 1, M_max=32)
    blob = torch.zeros(L.blob_bytes, dtype=torch.uint8, device=DEV)
    x = torch.zeros((32, K), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros((32, 8), dtype=torch.bfloat16, device=DEV)
    rc = dv.lib().dvssq_linear_decode_noalloc(dv.C.byref(L), blob.data_ptr(), x.data_ptr(), y.data_ptr(), 32, 0,
                                              torch.cuda.current_stream().cuda_stream)
    assert rc == dv.DVSSQ_EUNSUPPORTED
