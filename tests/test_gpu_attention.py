"""GPU parity of the FP8 KV cache ("NVIDIA NeMo RL ...", section "Ganancias de rendimiento en
el mundo real": FP8 KV cache and attention) against the oracle.

* fp8_kv_cache_append: bit-exact codes and factors (the 1x128 rule per head vector), other
  slots untouched, slots outside the cache skipped.
* fp8_attention_decode: fp32 arithmetic on the dequantized cache, bf16 output, against the fp64
  reference.  Tolerance, from the arithmetic: the output is rounded to bf16 (relative 2^-9);
  fp32 dot products, exponentials and sums over at most a few thousand tokens add relative
  errors of order 1e-5 of the row's value scale.  Bound used, per element:
  |gpu - ref| <= 2^-8 |ref| + 1e-3 max|ref[b, h, :]|, and a relative Frobenius norm <= 4e-3.
"""
import math

import numpy as np
import pytest
import torch

import block_scaled_quantize_amd as bsq
import oracle
import synth
from helpers import assert_bytes_equal, bits, f32_bits

pytestmark = pytest.mark.gpu

E4, E5 = bsq.E4M3, bsq.E5M2


def make_cache(B, T, KVH, fmt, seed, name, std=1.0):
    """K/V codes and factors quantized by the oracle from seeded normal values."""
    k = synth.normal((B * T * KVH, 128), std, seed, f"{name}/K")
    v = synth.normal((B * T * KVH, 128), std, seed, f"{name}/V")
    kc, ks = oracle.quantize_blockwise(bits(k), fmt, oracle.BLOCK_1x128, oracle.SCALE_FP32)
    vc, vs = oracle.quantize_blockwise(bits(v), fmt, oracle.BLOCK_1x128, oracle.SCALE_FP32)
    return (kc.reshape(B, T, KVH, 128), ks.reshape(B, T, KVH),
            vc.reshape(B, T, KVH, 128), vs.reshape(B, T, KVH))


def run_decode(q_bits, kc, ks, vc, vs, lens, sm_scale, fmt, split=None):
    dev = "cuda"
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = bsq.attention_decode(q, t(kc), t(ks), t(vc), t(vs),
                               torch.tensor(lens, dtype=torch.int32, device=dev), sm_scale, fmt,
                               split_tokens=split)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def check_close(out, ref, what):
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    err = np.abs(out - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * scale
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements out of bound, worst "
                           f"{np.max(err - bound):.3g} at {np.argwhere(bad)[0]}")
    assert oracle.rel_frobenius(out, ref) <= 4e-3, what


def q_bits_of(B, H, seed, name):
    return bits(synth.normal((B, H, 128), 1.0, seed, name)).reshape(B, H, 128)


@pytest.mark.parametrize("H,KVH", [(8, 8), (8, 4), (32, 8), (32, 4)])
@pytest.mark.parametrize("fmt", [E4, E5])
def test_decode_parity_ragged(gpu, H, KVH, fmt):
    B, T = 5, 300
    kc, ks, vc, vs = make_cache(B, T, KVH, fmt, 1, f"attn/{H}/{KVH}")
    q = q_bits_of(B, H, 1, f"attn/q/{H}/{KVH}")
    lens = [0, 1, 300, 137, 33]          # empty, one token, full, mid-step tails
    sm = 1.0 / math.sqrt(128)
    out = run_decode(q, kc, ks, vc, vs, lens, sm, fmt)
    ref = oracle.attention_decode(q, kc, ks, vc, vs, lens, sm, fmt)
    check_close(out, ref, f"H={H} KVH={KVH} fmt={fmt}")
    assert np.all(out[0] == 0.0)


@pytest.mark.parametrize("H,KVH", [(8, 8), (8, 4), (32, 8), (32, 4)])
@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("split", [32, 96, 256])
def test_decode_split_parity_ragged(gpu, H, KVH, fmt, split):
    """fp8_attention_decode_split: chunks of 32, 96 and 256 tokens over sequences of 0, 1,
    300, 137 and 33 tokens (empty chunks, one-token chunks, chunks ending mid-batch), against
    the oracle, and against the unsplit entry point."""
    B, T = 5, 300
    kc, ks, vc, vs = make_cache(B, T, KVH, fmt, 1, f"attn/{H}/{KVH}")
    q = q_bits_of(B, H, 1, f"attn/q/{H}/{KVH}")
    lens = [0, 1, 300, 137, 33]
    sm = 1.0 / math.sqrt(128)
    out = run_decode(q, kc, ks, vc, vs, lens, sm, fmt, split=split)
    ref = oracle.attention_decode(q, kc, ks, vc, vs, lens, sm, fmt)
    check_close(out, ref, f"split {split} H={H} KVH={KVH} fmt={fmt}")
    assert np.all(out[0] == 0.0)
    whole = run_decode(q, kc, ks, vc, vs, lens, sm, fmt)
    assert np.max(np.abs(out - whole)) <= 2.0 ** -7 * np.max(np.abs(whole))


def test_decode_split_long_sequences(gpu):
    """Split decode at the benchmark's chunk size, sequences up to 2100 tokens."""
    B, T, H, KVH = 3, 2100, 32, 8
    kc, ks, vc, vs = make_cache(B, T, KVH, E4, 4, "attn/split-long")
    q = q_bits_of(B, H, 4, "attn/q/split-long")
    lens = [2100, 1025, 1023]
    sm = 1.0 / math.sqrt(128)
    out = run_decode(q, kc, ks, vc, vs, lens, sm, E4, split=1024)
    ref = oracle.attention_decode(q, kc, ks, vc, vs, lens, sm, E4)
    check_close(out, ref, "split 1024, long sequences")


def test_decode_sharp_and_flat_softmax(gpu):
    B, T, H, KVH = 2, 200, 16, 4
    kc, ks, vc, vs = make_cache(B, T, KVH, E4, 2, "attn/sharp")
    q = q_bits_of(B, H, 2, "attn/q/sharp")
    for sm in (2.0, 1e-4):               # near one-hot and near uniform weights
        out = run_decode(q, kc, ks, vc, vs, [200, 150], sm, E4)
        ref = oracle.attention_decode(q, kc, ks, vc, vs, [200, 150], sm, E4)
        check_close(out, ref, f"sm_scale={sm}")


def test_tokens_past_the_length_are_never_read(gpu):
    B, T, H, KVH = 3, 64, 8, 2
    kc, ks, vc, vs = make_cache(B, T, KVH, E4, 3, "attn/past")
    q = q_bits_of(B, H, 3, "attn/q/past")
    lens = [10, 64, 17]
    clean = run_decode(q, kc, ks, vc, vs, lens, 0.1, E4)
    kc2, vc2, ks2, vs2 = kc.copy(), vc.copy(), ks.copy(), vs.copy()
    for b, n in enumerate(lens):
        kc2[b, n:] = 0x7F
        vc2[b, n:] = 0xFF
        ks2[b, n:] = np.inf
        vs2[b, n:] = np.nan
    dirty = run_decode(q, kc2, ks2, vc2, vs2, lens, 0.1, E4)
    np.testing.assert_array_equal(dirty, clean)
    # lengths are clamped to [0, T]
    out = run_decode(q, kc, ks, vc, vs, [-5, 1000, 17], 0.1, E4)
    ref = oracle.attention_decode(q, kc, ks, vc, vs, [-5, 1000, 17], 0.1, E4)
    check_close(out, ref, "clamped lengths")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("mode", [bsq.SCALE_FP32, bsq.SCALE_POW2])
def test_append_bit_exact(gpu, fmt, mode):
    B, T, KVH = 5, 10, 8
    codes0 = np.full((B, T, KVH, 128), 0xA5, dtype=np.uint8)
    si0 = np.full((B, T, KVH), 12345.0, dtype=np.float32)
    kn = synth.student_t((B * KVH, 128), 3.0, 4, "attn/append/k")
    vn = synth.student_t((B * KVH, 128), 3.0, 4, "attn/append/v")
    pos = [0, 9, -1, 3, 10]
    kc, ks, vc, vs = to_dev(codes0), to_dev(si0), to_dev(codes0), to_dev(si0)
    bsq.kv_cache_append(kn.reshape(B, KVH, 128).cuda(), vn.reshape(B, KVH, 128).cuda(),
                        torch.tensor(pos, dtype=torch.int32, device="cuda"), kc, ks, vc, vs,
                        fmt, mode)
    torch.cuda.synchronize()
    for new, c_dev, s_dev, what in ((kn, kc, ks, "K"), (vn, vc, vs, "V")):
        c_ref, s_ref = codes0.copy(), si0.copy()
        oracle.kv_cache_append(c_ref, s_ref, bits(new).reshape(B, KVH, 128), pos, fmt, mode)
        assert_bytes_equal(c_dev.cpu().numpy(), c_ref, f"{what} codes")
        assert_bytes_equal(f32_bits(s_dev.cpu().numpy()), f32_bits(s_ref), f"{what} factors")


def test_append_special_head_vectors(gpu):
    B, T, KVH = 2, 4, 8
    x = synth.normal((B * KVH, 128), 1.0, 5, "attn/append/special").float()
    x[0] = 0.0                      # all-zero head vector: factor 1
    x[1, 5] = float("nan")
    x[2, 7] = float("inf")
    x[3, :] = 1e-40                 # bf16 subnormals
    x[4, :] = 3e38
    x[5, 9] = float("-inf")
    xb = x.to(torch.bfloat16)
    codes0 = np.zeros((B, T, KVH, 128), dtype=np.uint8)
    si0 = np.zeros((B, T, KVH), dtype=np.float32)
    for fmt in (E4, E5):
        kc, ks, vc, vs = to_dev(codes0), to_dev(si0), to_dev(codes0), to_dev(si0)
        pos = [1, 3]
        dev = xb.reshape(B, KVH, 128).cuda()
        bsq.kv_cache_append(dev, dev, torch.tensor(pos, dtype=torch.int32, device="cuda"), kc, ks,
                            vc, vs, fmt, bsq.SCALE_FP32)
        torch.cuda.synchronize()
        c_ref, s_ref = codes0.copy(), si0.copy()
        oracle.kv_cache_append(c_ref, s_ref, bits(xb).reshape(B, KVH, 128), pos, fmt,
                               bsq.SCALE_FP32)
        assert_bytes_equal(kc.cpu().numpy(), c_ref, f"codes fmt {fmt}")
        assert_bytes_equal(vc.cpu().numpy(), c_ref, f"codes fmt {fmt}")
        assert_bytes_equal(f32_bits(ks.cpu().numpy()), f32_bits(s_ref), f"factors fmt {fmt}")


def test_append_then_decode(gpu):
    """A cache filled token by token on the GPU equals the oracle's, and decoding it matches."""
    B, T, H, KVH = 3, 24, 16, 4
    codes0 = np.zeros((B, T, KVH, 128), dtype=np.uint8)
    si0 = np.ones((B, T, KVH), dtype=np.float32)
    kc, ks, vc, vs = to_dev(codes0), to_dev(si0), to_dev(codes0), to_dev(si0)
    c_k, s_k, c_v, s_v = codes0.copy(), si0.copy(), codes0.copy(), si0.copy()
    for t in range(T):
        kn = synth.normal((B * KVH, 128), 1.0, 6 + t, "attn/e2e/k")
        vn = synth.normal((B * KVH, 128), 1.0, 6 + t, "attn/e2e/v")
        pos = [t, t if t < 20 else -1, t if t < 7 else T]
        bsq.kv_cache_append(kn.reshape(B, KVH, 128).cuda(), vn.reshape(B, KVH, 128).cuda(),
                            torch.tensor(pos, dtype=torch.int32, device="cuda"), kc, ks, vc, vs)
        oracle.kv_cache_append(c_k, s_k, bits(kn).reshape(B, KVH, 128), pos, E4, bsq.SCALE_FP32)
        oracle.kv_cache_append(c_v, s_v, bits(vn).reshape(B, KVH, 128), pos, E4, bsq.SCALE_FP32)
    torch.cuda.synchronize()
    assert_bytes_equal(kc.cpu().numpy(), c_k, "K cache")
    assert_bytes_equal(vc.cpu().numpy(), c_v, "V cache")
    q = q_bits_of(B, H, 7, "attn/e2e/q")
    lens = [24, 20, 7]
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    out = bsq.attention_decode(qd, kc, ks, vc, vs, torch.tensor(lens, dtype=torch.int32,
                                                                  device="cuda"), 0.0884, E4)
    torch.cuda.synchronize()
    ref = oracle.attention_decode(q, c_k, s_k, c_v, s_v, lens, 0.0884, E4)
    check_close(out.float().cpu().numpy().astype(np.float64), ref, "append then decode")


def test_decode_llama8b_shape_sampled(gpu):
    """32 query heads, 8 KV heads, 4096-token cache, 16 sequences of mixed lengths; four
    sequences checked against the oracle."""
    B, T, H, KVH = 16, 4096, 32, 8
    g = np.random.default_rng(8)
    lens = g.integers(1, T + 1, size=B).astype(np.int32)
    lens[0], lens[1] = T, 1
    kc, ks, vc, vs = make_cache(B, T, KVH, E4, 8, "attn/full")
    q = q_bits_of(B, H, 8, "attn/q/full")
    out = run_decode(q, kc, ks, vc, vs, lens.tolist(), 1.0 / math.sqrt(128), E4)
    for b in (0, 1, 7, 15):
        ref = oracle.attention_decode(q[b:b + 1], kc[b:b + 1], ks[b:b + 1], vc[b:b + 1],
                                      vs[b:b + 1], [int(lens[b])], 1.0 / math.sqrt(128), E4)
        check_close(out[b:b + 1], ref, f"sequence {b} (length {lens[b]})")
