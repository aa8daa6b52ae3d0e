"""Pins of the oracle's FP8 KV-cache writer and decode attention reference.

The pages ("NVIDIA NeMo RL ...", section "Ganancias de rendimiento en el mundo real") say only
that FP8 is extended to the KV cache and attention; the cache reading (1x128 blocks = one scale
per head vector, section "El avance técnico") and the attention definition (softmax of scaled
dot products, grouped-query head mapping) are pinned here against closed forms, invariants and
a pure-Python brute force, independently of the oracle's own NumPy path:

* one cached token: the output is that token's dequantized value row, exactly;
* identical keys: uniform weights, the output is the mean of the value rows;
* a dominant key (logit gap > 60): the output is that token's value row to 1e-20;
* grouped-query mapping: a KV head whose values are all c gives c for exactly its query heads;
* tokens past the sequence length (filled with NaN codes) do not change the result;
* q -> 2q with sm_scale -> sm_scale / 2 leaves the result unchanged;
* brute force: math.exp and plain loops on tiny shapes, 1e-12 relative;
* the cache writer stores exactly the blockwise 1x128 quantization of each head vector and
  leaves other slots untouched.
"""
import math

import numpy as np
import pytest

import oracle

E4M3, E5M2 = oracle.E4M3, oracle.E5M2


def bf16_bits(a):
    f = np.asarray(a, dtype=np.float32)
    b = f.view(np.uint32)
    # round to nearest even to bf16
    r = ((b >> 16) & 1) + 0x7FFF
    return ((b + r) >> 16).astype(np.uint16)


def bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def finite_codes(g, shape, fmt, lo=0, hi=0x70):
    # small positive and negative finite codes (no NaN / inf)
    c = g.integers(lo, hi, size=shape, dtype=np.uint8)
    sign = g.integers(0, 2, size=shape, dtype=np.uint8) << 7
    return (c | sign).astype(np.uint8)


def make_cache(g, b, t, kvh, fmt):
    kc = finite_codes(g, (b, t, kvh, 128), fmt)
    vc = finite_codes(g, (b, t, kvh, 128), fmt)
    ks = (g.random((b, t, kvh)) * 0.02 + 0.001).astype(np.float32)
    vs = (g.random((b, t, kvh)) * 0.02 + 0.001).astype(np.float32)
    return kc, ks, vc, vs


def dequant_rows(codes, si, fmt):
    return oracle.decode(fmt, codes).astype(np.float64) * si[..., None].astype(np.float64)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_single_token_returns_its_value_row(fmt):
    g = np.random.default_rng(1)
    kc, ks, vc, vs = make_cache(g, 2, 4, 2, fmt)
    q = bf16_bits(g.normal(size=(2, 4, 128)))
    out = oracle.attention_decode(q, kc, ks, vc, vs, [1, 1], 0.1, fmt)
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(out[b, h], dequant_rows(vc[b, 0, h // 2], vs[b, 0, h // 2], fmt))


def test_identical_keys_give_the_mean_value():
    g = np.random.default_rng(2)
    kc, ks, vc, vs = make_cache(g, 1, 9, 1, E4M3)
    kc[0, :] = kc[0, 0]
    ks[0, :] = ks[0, 0]
    q = bf16_bits(g.normal(size=(1, 2, 128)))
    out = oracle.attention_decode(q, kc, ks, vc, vs, [7], 0.088, E4M3)
    mean = dequant_rows(vc[0, :7, 0], vs[0, :7, 0], E4M3).mean(axis=0)
    for h in range(2):
        np.testing.assert_allclose(out[0, h], mean, rtol=1e-13, atol=1e-16)


def test_dominant_key_selects_its_value_row():
    g = np.random.default_rng(3)
    kc, ks, vc, vs = make_cache(g, 1, 6, 1, E4M3)
    q = bf16_bits(np.ones((1, 1, 128)))
    kc[0, :, 0] = 0x00                     # zero keys ...
    kc[0, 4, 0] = 0x7E                     # ... except token 4: all 448
    ks[0, :, 0] = 1.0
    out = oracle.attention_decode(q, kc, ks, vc, vs, [6], 1.0 / 128, E4M3)   # logit gap 448
    np.testing.assert_allclose(out[0, 0], dequant_rows(vc[0, 4, 0], vs[0, 4, 0], E4M3), rtol=0,
                               atol=1e-20)


def test_grouped_query_head_mapping():
    g = np.random.default_rng(4)
    kvh, group = 4, 3
    kc, ks, vc, vs = make_cache(g, 1, 5, kvh, E4M3)
    vc[0, :, 2] = 0x38                     # 1.0 in E4M3
    vs[0, :, 2] = 0.5
    q = bf16_bits(g.normal(size=(1, kvh * group, 128)))
    out = oracle.attention_decode(q, kc, ks, vc, vs, [5], 0.1, E4M3)
    for h in range(kvh * group):
        if h // group == 2:
            np.testing.assert_allclose(out[0, h], 0.5, rtol=1e-14)
        else:
            assert not np.allclose(out[0, h], 0.5)


def test_tokens_past_the_length_are_ignored():
    g = np.random.default_rng(5)
    kc, ks, vc, vs = make_cache(g, 2, 8, 2, E4M3)
    q = bf16_bits(g.normal(size=(2, 4, 128)))
    ref = oracle.attention_decode(q, kc, ks, vc, vs, [3, 8], 0.1, E4M3)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[0, 3:] = 0x7F                       # NaN codes past the length of sequence 0
    vc2[0, 3:] = 0xFF
    ks2 = ks.copy()
    ks2[0, 3:] = np.inf
    out = oracle.attention_decode(q, kc2, ks2, vc2, vs, [3, 8], 0.1, E4M3)
    np.testing.assert_array_equal(out, ref)
    # lengths outside [0, T] are clamped; an empty sequence gives zeros
    out = oracle.attention_decode(q, kc, ks, vc, vs, [0, 99], 0.1, E4M3)
    np.testing.assert_array_equal(out[0], 0.0)
    np.testing.assert_array_equal(out[1], ref[1])


def test_query_scale_invariance():
    g = np.random.default_rng(6)
    kc, ks, vc, vs = make_cache(g, 1, 10, 1, E5M2)
    x = g.normal(size=(1, 2, 128))
    q1 = bf16_bits(x)
    q2 = bf16_bits(bits_to_f64(q1) * 2.0)   # exact doubling
    a = oracle.attention_decode(q1, kc, ks, vc, vs, [10], 0.125, E5M2)
    b = oracle.attention_decode(q2, kc, ks, vc, vs, [10], 0.0625, E5M2)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-18)


def brute_force(q_bits, kc, ks, vc, vs, lens, sm_scale, fmt):
    table = [float(v) for v in oracle.decode_table(fmt)]
    nb, nh, d = q_bits.shape
    kvh = kc.shape[2]
    group = nh // kvh
    out = [[[0.0] * d for _ in range(nh)] for _ in range(nb)]
    for b in range(nb):
        n = lens[b]
        for h in range(nh):
            kv = h // group
            q = [float(np.uint32(int(q_bits[b, h, i]) << 16).view(np.float32)) for i in range(d)]
            s = []
            for t in range(n):
                acc = 0.0
                for i in range(d):
                    acc += q[i] * table[kc[b, t, kv, i]] * float(ks[b, t, kv])
                s.append(acc * sm_scale)
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            tot = sum(w)
            for i in range(d):
                out[b][h][i] = sum(w[t] / tot * table[vc[b, t, kv, i]] * float(vs[b, t, kv])
                                   for t in range(n))
    return np.array(out)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_brute_force_tiny(fmt):
    g = np.random.default_rng(7)
    kc, ks, vc, vs = make_cache(g, 2, 5, 2, fmt)
    q = bf16_bits(g.normal(size=(2, 4, 128)))
    lens = [5, 3]
    ref = brute_force(q, kc, ks, vc, vs, lens, 0.09, fmt)
    out = oracle.attention_decode(q, kc, ks, vc, vs, lens, 0.09, fmt)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("mode", [oracle.SCALE_FP32, oracle.SCALE_POW2])
def test_cache_append_is_blockwise_quantization(mode):
    g = np.random.default_rng(8)
    b, t, kvh = 3, 6, 4
    codes = np.full((b, t, kvh, 128), 0xA5, dtype=np.uint8)
    si = np.full((b, t, kvh), 7.0, dtype=np.float32)
    new = bf16_bits(g.standard_t(3.0, size=(b, kvh, 128)))
    oracle.kv_cache_append(codes, si, new, [2, -1, 5], E4M3, mode)
    for bb, pos in ((0, 2), (2, 5)):
        q, s = oracle.quantize_blockwise(new[bb], E4M3, oracle.BLOCK_1x128, mode)
        np.testing.assert_array_equal(codes[bb, pos], q)
        np.testing.assert_array_equal(si[bb, pos], s[:, 0])
        # each head vector's factor: amax / 448 up to the scale's own rounding
        amax = np.abs(bits_to_f64(new[bb])).max(axis=1)
        if mode == oracle.SCALE_FP32:
            np.testing.assert_allclose(si[bb, pos], amax / 448.0, rtol=2e-7)
    untouched = np.ones((b, t), dtype=bool)
    untouched[0, 2] = untouched[2, 5] = False
    assert np.all(codes[untouched] == 0xA5) and np.all(si[untouched] == 7.0)
