"""CPU pins of the planted blobs (tests/planted.py) that the GPU parity tests
use: each planted blob decodes to what it claims, independently of the
oracle's forward."""
import numpy as np
import pytest

import cases
import oracle
import planted
import synth


@pytest.fixture(scope="module")
def tiny():
    return cases.quantized("tiny")


def test_parts_pack_roundtrip(tiny):
    lay, blob = tiny
    np.testing.assert_array_equal(planted.pack(planted.parts(blob, lay), lay), blob)


def test_lowrank_only_is_the_lowrank_term(tiny):
    """With every code 0 the layer is x H V^T U^T: the unpacked weights are zero
    and the oracle's forward equals that product, computed here from the
    unpacked factors and the dense Sylvester matrix (scipy)."""
    import scipy.linalg
    lay, blob = tiny
    b = planted.lowrank_only(blob, lay)
    idx, What, U, V = oracle.unpack(b, lay.N, lay.K, lay.r, lay.n_seg)
    assert not What.any()
    x_bits = cases.activations("tiny", 4)
    x = synth.bf16_bits_to_f64(x_bits)
    H = scipy.linalg.hadamard(lay.block) / np.sqrt(lay.block)
    xr = np.concatenate([x[:, i:i + lay.block] @ H for i in range(0, lay.K, lay.block)], axis=1)
    ref = np.zeros((4, lay.N))
    ref[:, idx] = (xr @ V.T) @ U.T
    y = oracle.forward(b, lay.N, lay.K, lay.r, lay.block, lay.n_seg, x_bits)
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()
    assert np.abs(ref).max() > 0


def test_edge_codes_are_present(tiny):
    lay, blob = tiny
    b = planted.edge_codes(blob, lay)
    p = planted.parts(b, lay)
    nib = np.concatenate([p["q4"] & 0xF, p["q4"] >> 4], axis=1)
    assert (nib == 0).any() and (nib == 15).any()                 # codes -8 and +7
    assert (p["q8"] == -128).any() and (p["q8"] == 127).any()
    assert (p["s4"] == 0).any()                                   # zero groups
    zero_rows = np.nonzero((p["s8"] == 0) & ~p["q8"].any(axis=1))[0]
    assert zero_rows.size > 0                                     # all-zero INT8 rows
    idx, What, U, V = oracle.unpack(b, lay.N, lay.K, lay.r, lay.n_seg)
    n4 = p["q4"].shape[0]
    s = synth.bf16_bits_to_f64(p["s4"])
    # a row planted at code -8 dequantizes to -8 s in every group with a nonzero scale
    for row in range(0, n4, 5):
        g = np.nonzero(s[row] > 0)[0]
        if g.size and not (p["q4"][row] != 0).any():
            np.testing.assert_array_equal(What[row, 64 * g[0]:64 * g[0] + 64], -8 * s[row, g[0]])
    # an all-zero INT8 row is zero
    assert not What[n4 + zero_rows].any()


def test_scale_classes_cover_the_ranges(tiny):
    lay, blob = tiny
    b, cls, e8 = planted.scale_range(blob, lay)
    s = synth.bf16_bits_to_f64(planted.parts(b, lay)["s4"])
    assert (s[cls == 1] >= 2.0 ** -20).all() and (s[cls == 1] < 2.0 ** -14).all()
    assert (s[cls == 2] > 63).all() and (s[cls == 2] <= 256).all()
    assert s[cls == 1].min() < 2.0 ** -17      # below the f16-exact window of an unshifted scale
    assert not planted.parts(b, lay)["U"].any()
    cols = planted.class_columns(b, lay, cls)
    assert sorted(np.concatenate(cols).tolist()) == list(range(lay.N))
