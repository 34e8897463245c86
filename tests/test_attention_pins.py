"""Pins of the KV-BSS attention oracle (oracle.kvbss_attention) against what the
pages and the mathematics fix, independently of the oracle's own code:

- with the haze mask off, it is causal grouped-query softmax attention with the
  focus-scaled logits: torch's scaled_dot_product_attention (fp64, CPU) with an
  explicit causal / sliding-window mask and the KV heads repeated per query
  group is that library routine;
- logits built to land exactly on, just above and just below max - 12 show the
  boundary (a logit exactly 12 below the maximum is kept, anything lower is
  dropped), that the test is made on the scaled logits, and that dropped keys
  contribute exactly nothing (closed form);
- the maximum is per query row over that row's visible keys (a key only a
  later query sees does not move an earlier row's threshold);
- evaluating a subset of rows gives the same values as the full evaluation.

Pages: Spark-X2.5-4B-Hadamard-GSQ model card, section 2 (KV-BSS: focus factor
scaling, attention haze truncation); Spark-X2.5-4B discussion 14, Mathematical
Formulation 1-2 and the eager attention change; Spark-X2.5-4B GGUF page, "The
model" (grouped-query heads, sliding window).
"""
import math

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")


def sdpa_reference(q_bits, k_bits, v_bits, scale, window):
    q = torch.from_numpy(synth.bf16_bits_to_f64(q_bits))      # [B][Mq][Hq][D]
    k = torch.from_numpy(synth.bf16_bits_to_f64(k_bits))      # [B][Nk][Hkv][D]
    v = torch.from_numpy(synth.bf16_bits_to_f64(v_bits))
    B, Mq, Hq, D = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    rep = Hq // Hkv
    qh = q.permute(0, 2, 1, 3)                                  # [B][Hq][Mq][D]
    kh = k.permute(0, 2, 1, 3).repeat_interleave(rep, dim=1)    # [B][Hq][Nk][D]
    vh = v.permute(0, 2, 1, 3).repeat_interleave(rep, dim=1)
    pos = torch.arange(Nk - Mq, Nk).unsqueeze(1)
    j = torch.arange(Nk).unsqueeze(0)
    mask = j <= pos
    if window > 0:
        mask &= j > pos - window
    o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("B,Mq,Nk,Hq,Hkv,D,window", [
    (2, 5, 37, 8, 2, 64, 0),
    (1, 37, 37, 4, 4, 32, 0),      # prefill: every query of the sequence
    (1, 9, 40, 8, 1, 64, 7),       # sliding window
    (2, 1, 50, 4, 2, 128, 0),      # decode
])
def test_haze_off_is_causal_gqa_softmax_attention(B, Mq, Nk, Hq, Hkv, D, window):
    q, k, v = synth.attention_qkv(3, "pin", B, Mq, Nk, Hq, Hkv, D)
    scale = oracle.KVBSS_TAU / math.sqrt(D)
    got = oracle.kvbss_attention(q, k, v, scale, math.inf, window=window)
    ref = sdpa_reference(q, k, v, scale, window)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def _one_dim_case(logits, values_scale=1.0):
    """One query and len(logits) keys along dimension 0 so that, with scale
    1/16 and q = 16 e_0, the scaled logit of key j is exactly logits[j]; v_j is
    (j + 1) e_j (distinct directions, exact in bf16)."""
    n = len(logits)
    D = 64
    q = np.zeros((1, 1, 1, D))
    q[0, 0, 0, 0] = 16.0
    k = np.zeros((1, n, 1, D))
    k[0, :, 0, 0] = logits
    v = np.zeros((1, n, 1, D))
    for j in range(n):
        v[0, j, 0, j] = (j + 1) * values_scale
    bits = [synth.to_bf16_bits(a) for a in (q, k, v)]
    for a, b in zip((q, k, v), bits):
        assert np.array_equal(synth.bf16_bits_to_f64(b), a)    # every value exact in bf16
    return bits


def test_haze_boundary_closed_form():
    logits = [0.0, -12.0, -12.0625, -11.9375, -30.0, -1.0]
    q, k, v = _one_dim_case(logits)
    o = oracle.kvbss_attention(q, k, v, 1.0 / 16.0, 12.0)[0, 0, 0]
    kept = [j for j, s in enumerate(logits) if s >= -12.0]
    assert kept == [0, 1, 3, 5]
    z = sum(math.exp(logits[j]) for j in kept)
    for j, s in enumerate(logits):
        want = (j + 1) * math.exp(s) / z if j in kept else 0.0
        assert o[j] == pytest.approx(want, rel=1e-14, abs=0.0)
    assert o[2] == 0.0 and o[4] == 0.0          # dropped keys: exactly nothing
    assert not o[len(logits):].any()
    # without the mask every key contributes
    o_all = oracle.kvbss_attention(q, k, v, 1.0 / 16.0, math.inf)[0, 0, 0]
    z_all = sum(math.exp(s) for s in logits)
    assert o_all[2] == pytest.approx(3 * math.exp(-12.0625) / z_all, rel=1e-14)


def test_haze_is_tested_on_scaled_logits():
    # raw dot products 16x the logits: a mask on unscaled values would drop keys 1 and 3
    logits = [0.0, -0.75, -12.5, -0.5]
    q, k, v = _one_dim_case(logits)
    o = oracle.kvbss_attention(q, k, v, 1.0 / 16.0, 12.0)[0, 0, 0]
    assert o[1] > 0 and o[3] > 0 and o[2] == 0.0


def test_maximum_is_per_row_over_visible_keys():
    # two queries: row 0 (position Nk - 2) does not see the last key, whose
    # logit (+20) would put every other key more than 12 below it
    logits = [0.0, -12.0, -12.0625, -11.9375, -30.0, -1.0, 20.0]
    _, k, v = _one_dim_case(logits)
    D = 64
    q = np.zeros((1, 2, 1, D))
    q[0, :, 0, 0] = 16.0
    qb = synth.to_bf16_bits(q)
    o = oracle.kvbss_attention(qb, k, v, 1.0 / 16.0, 12.0)
    row0, row1 = o[0, 0, 0], o[0, 1, 0]
    assert row0[6] == 0.0 and row0[0] > 0 and row0[1] > 0 and row0[2] == 0.0
    # row 1: only the +20 key survives, so the output is exactly v_6 = 7 e_6
    assert row1[6] == 7.0 and not np.delete(row1, 6).any()


def test_row_subset_matches_full():
    B, Mq, Nk, Hq, Hkv, D = 2, 6, 30, 8, 2, 64
    q, k, v = synth.attention_qkv(5, "rows", B, Mq, Nk, Hq, Hkv, D)
    scale = oracle.KVBSS_TAU / math.sqrt(D)
    full = oracle.kvbss_attention(q, k, v, scale, oracle.KVBSS_HAZE).reshape(-1, D)
    rows = np.array([0, 7, 13, B * Mq * Hq - 1, 40])
    part = oracle.kvbss_attention(q, k, v, scale, oracle.KVBSS_HAZE, rows=rows)
    np.testing.assert_array_equal(part, full[rows])


def test_haze_drops_keys_on_the_wide_heads():
    """The synthetic inputs exercise the mask: on the heads with the largest
    query gain most visible keys fall more than 12 nats below the row maximum,
    on the smallest none do (checked on the exact logits)."""
    B, Mq, Nk, Hq, Hkv, D = 1, 4, 2048, 4, 1, 256
    q, k, _ = synth.attention_qkv(0, "spread", B, Mq, Nk, Hq, Hkv, D)
    qf, kf = synth.bf16_bits_to_f64(q)[0, -1], synth.bf16_bits_to_f64(k)[0, :, 0]
    s = (qf @ kf.T) * (oracle.KVBSS_TAU / math.sqrt(D))      # [Hq][Nk], last query sees every key
    dropped = (s < s.max(axis=1, keepdims=True) - oracle.KVBSS_HAZE).mean(axis=1)
    assert dropped[0] == 0.0 and dropped[3] > 0.5
