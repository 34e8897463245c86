"""GPU parity of dvssq_kvbss_attention (through the C ABI) against the fp64
oracle (oracle.kvbss_attention) on the same seeded bf16 q, k, v.

Bar: max|o_gpu - o_ref| <= 5e-3 max|v|, element by element.  Derivation: the
GPU rounds each weight exp(s - m) to bf16 before the product with v (relative
error <= 2^-9, so the weighted mean moves by <= 2^-9 max|v|) and rounds the
output to bf16 (<= 2^-9 |o| <= 2^-9 max|v|); fp32 logits (bf16 products
summed in fp32 over <= 256 dims, |s| < 40) and exp2 add below 2^-12 max|v|;
a key within fp32 rounding of the haze threshold that one side keeps and the
other drops weighs about e^-12 of the row's largest.  Total < 2^-8 + 2^-12
< 5e-3.  Cases with exactly representable logits compare exactly.
"""
import math

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
TOL_ATTN = 5e-3


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def run(q, k, v, window=0, haze=oracle.KVBSS_HAZE, scale=None):
    B, Mq, Hq, D = q.shape
    _, Nk, Hkv, _ = k.shape
    if scale is None:
        scale = float(np.float32(oracle.KVBSS_TAU / math.sqrt(D)))
    sh = dv.AttnShape(B=B, Mq=Mq, Nk=Nk, Hq=Hq, Hkv=Hkv, D=D, window=window, scale=scale, haze=haze)
    o = torch.empty((B, Mq, Hq, D), dtype=torch.int16, device=DEV)
    nws = dv.kvbss_attention_ws_bytes(sh)
    ws = dv.device_buffer(nws, DEV).fill_(0x7F) if nws else None     # no initialization expected
    dv.kvbss_attention(sh, dev(q), dev(k), dev(v), o, ws)
    torch.cuda.synchronize()
    return synth.bf16_bits_to_f64(o.cpu().numpy().view(np.uint16)), scale


def check(q, k, v, window=0, haze=oracle.KVBSS_HAZE, rows=None):
    got, scale = run(q, k, v, window, haze)
    D = q.shape[-1]
    ref = oracle.kvbss_attention(q, k, v, scale, haze, window=window, rows=rows)
    g = got.reshape(-1, D) if rows is None else got.reshape(-1, D)[rows]
    r = ref.reshape(-1, D)
    err = np.abs(g - r).max() / np.abs(synth.bf16_bits_to_f64(v)).max()
    print(f"attention rel err {err:.3e}", flush=True)
    assert err <= TOL_ATTN
    return got


ATTN_CASES = [
    # B, Mq, Nk, Hq, Hkv, D, window
    (2, 5, 37, 8, 2, 64, 0),
    (1, 70, 70, 4, 4, 128, 0),       # prefill, a ragged second tile
    (1, 9, 130, 8, 1, 64, 7),        # sliding window
    (2, 1, 300, 16, 4, 256, 0),      # decode, Spark heads
    (1, 33, 200, 16, 4, 256, 64),    # Spark heads, window
    (1, 1, 1, 4, 2, 128, 0),         # a single token
    (3, 17, 65, 2, 2, 256, 0),       # keys one past a block of 64
    (1, 512, 512, 16, 4, 256, 0),    # Spark prefill
]


@pytest.mark.parametrize("B,Mq,Nk,Hq,Hkv,D,window", ATTN_CASES)
def test_attention_parity(B, Mq, Nk, Hq, Hkv, D, window):
    print(f"attention B={B} Mq={Mq} Nk={Nk} Hq={Hq} Hkv={Hkv} D={D} window={window}", flush=True)
    q, k, v = synth.attention_qkv(11, f"gpu{Mq}x{Nk}", B, Mq, Nk, Hq, Hkv, D)
    check(q, k, v, window)


def test_attention_haze_off():
    q, k, v = synth.attention_qkv(12, "off", 1, 40, 150, 8, 2, 128)
    check(q, k, v, haze=math.inf)


def test_attention_single_token_is_v():
    q, k, v = synth.attention_qkv(13, "one", 2, 1, 1, 4, 2, 64)
    got, _ = run(q, k, v)
    # one visible key: weight exactly 1, the output is v (rounded to bf16: exact)
    want = np.repeat(synth.bf16_bits_to_f64(v), 2, axis=2)
    np.testing.assert_array_equal(got, want)


def test_attention_exact_haze_boundary():
    """Logits exactly representable on both sides (q = 16 e_0, k_j = l_j e_0,
    scale 1/16): the kept set is decided exactly, dropped keys add exactly
    nothing, and a single dominant key gives exactly its v."""
    logits = [0.0, -12.0, -12.0625, -11.9375, -30.0, -1.0, 20.0]
    D, n = 64, len(logits)
    q = np.zeros((1, 2, 1, D))
    q[0, :, 0, 0] = 16.0
    k = np.zeros((1, n, 1, D))
    k[0, :, 0, 0] = logits
    v = np.zeros((1, n, 1, D))
    for j in range(n):
        v[0, j, 0, j] = j + 1
    qb, kb, vb = (synth.to_bf16_bits(a) for a in (q, k, v))
    got, _ = run(qb, kb, vb, scale=1.0 / 16.0)
    ref = oracle.kvbss_attention(qb, kb, vb, 1.0 / 16.0, oracle.KVBSS_HAZE)
    row0, row1 = got[0, 0, 0], got[0, 1, 0]
    assert row0[2] == 0.0 and row0[4] == 0.0 and row0[6] == 0.0     # dropped / not visible
    assert all(row0[j] > 0 for j in (0, 1, 3, 5))
    np.testing.assert_allclose(row0, ref[0, 0, 0], rtol=2 ** -7, atol=0)
    assert row1[6] == 7.0 and not np.delete(row1, 6).any()


def test_attention_repeat_is_bit_identical():
    q, k, v = synth.attention_qkv(14, "rep", 1, 64, 256, 16, 4, 256)
    a, _ = run(q, k, v)
    b, _ = run(q, k, v)
    np.testing.assert_array_equal(a, b)


# the split-key form: at most 16 (query, head) rows per KV head and more than 512 keys
SPLIT_CASES = [
    # B, Mq, Nk, Hq, Hkv, D, window
    (2, 1, 3000, 16, 4, 256, 0),     # decode, Spark heads, ragged last range
    (1, 4, 1537, 16, 4, 256, 0),     # 16 rows: four queries of a group of four heads
    (3, 1, 2048, 8, 1, 128, 0),      # 8 heads sharing one KV head
    (1, 2, 1100, 4, 2, 64, 300),     # window: most ranges see no key of the rows
    (1, 1, 513, 2, 2, 256, 0),       # one key past a range
]


@pytest.mark.parametrize("B,Mq,Nk,Hq,Hkv,D,window", SPLIT_CASES)
def test_attention_split_parity(B, Mq, Nk, Hq, Hkv, D, window):
    sh = dv.AttnShape(B=B, Mq=Mq, Nk=Nk, Hq=Hq, Hkv=Hkv, D=D, window=window, scale=0.1, haze=12.0)
    assert dv.kvbss_attention_ws_bytes(sh) > 0           # the two-launch form
    print(f"attention split B={B} Mq={Mq} Nk={Nk} Hq={Hq} Hkv={Hkv} D={D} window={window}", flush=True)
    q, k, v = synth.attention_qkv(15, f"split{Mq}x{Nk}", B, Mq, Nk, Hq, Hkv, D)
    check(q, k, v, window)


def test_attention_split_repeat_is_bit_identical():
    q, k, v = synth.attention_qkv(16, "srep", 2, 1, 2600, 16, 4, 256)
    a, _ = run(q, k, v)
    b, _ = run(q, k, v)
    np.testing.assert_array_equal(a, b)


def spark_rows(B, Mq, Hq, n=96, seed=2):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(B * Mq * Hq, size=n, replace=False).tolist())
    for i in (0, 1, 15, 16, Mq // 2, Mq - 17, Mq - 16, Mq - 1):    # tile edges (16 queries per tile)
        for h in (0, 3, 4, 15):
            rows.add(i * Hq + h)
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("window", [0, 512])
def test_attention_spark_prefill_2048_sampled(window):
    """The Spark full (window 0) and sliding (window 512) attention layers on a
    2048-token prefill, the shape the benchmark times; sampled query rows."""
    B, Mq, Nk, Hq, Hkv, D = 1, 2048, 2048, 16, 4, 256
    q, k, v = synth.attention_qkv(0, "spark_prefill", B, Mq, Nk, Hq, Hkv, D)
    check(q, k, v, window, rows=spark_rows(B, Mq, Hq))


def test_attention_spark_decode_32k():
    """One new token over a 32768-token context, every head (Spark full layer):
    the split-key form the benchmark times."""
    B, Mq, Nk, Hq, Hkv, D = 1, 1, 32768, 16, 4, 256
    q, k, v = synth.attention_qkv(0, "spark_decode", B, Mq, Nk, Hq, Hkv, D)
    check(q, k, v)
