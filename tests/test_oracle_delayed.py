"""Pins of the oracle's per-tensor delayed scaling.

The recipe is the one shown in "Infraestructura de Entrenamiento FP8: Precisión Numérica de
Nueva Generación", section "Transformer Engine: la base de software": margin 0, history of 16
amax values reduced with "max", HYBRID formats (E4M3 forward, E5M2 for gradients), and the
scale of a step taken from the magnitudes seen in earlier steps.  The expected scales below
are closed forms over scripted amax sequences (powers of two, so every quotient is exact),
not re-computations through the oracle's code path.
"""
import numpy as np
import pytest
import torch

import oracle

E4M3, E5M2 = oracle.E4M3, oracle.E5M2
FP32, POW2 = oracle.SCALE_FP32, oracle.SCALE_POW2


def bits_of(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def tensor_with_amax(a: float, step: int, n: int = 1000) -> torch.Tensor:
    """bf16 tensor whose largest magnitude is exactly a (a power of two)."""
    g = np.random.Generator(np.random.PCG64(100 + step))
    v = g.uniform(-0.49, 0.49, size=n).astype(np.float32) * np.float32(a)
    v[g.integers(0, n)] = a if step % 2 == 0 else -a
    return torch.from_numpy(v).to(torch.bfloat16)


def run(seq, fmt=E4M3, mode=FP32, margin=0, hist_len=16):
    st = oracle.DelayedState(hist_len)
    out = []
    for t, a in enumerate(seq):
        x = tensor_with_amax(a, t)
        q, siu = oracle.delayed_step(bits_of(x), fmt, mode, margin, st)
        out.append((x, q, siu, st.history.copy(), st.scale[0]))
    return out


def expected_scale_used(seq, t, fmax, hist_len=16, margin=0):
    if t == 0:
        return 1.0
    window = seq[max(0, t - hist_len):t]
    return fmax / max(window) / 2.0 ** margin


@pytest.mark.parametrize("steps", [10, 40])
def test_periodic_sequence_closed_form(oracle_lib, steps):
    seq = [2.0 ** (t % 5) for t in range(steps)]
    res = run(seq)
    for t, (x, q, siu, hist, s_next) in enumerate(res):
        s_used = expected_scale_used(seq, t, 448.0)
        assert siu == np.float32(1.0) / np.float32(s_used)
        # codes: each element x*s_used (exact here) encoded to the nearest E4M3 value
        y = x.float().numpy() * np.float32(s_used)
        assert np.array_equal(q, oracle.encode(E4M3, y))
        # history newest first, unfilled slots zero
        want = [seq[t - i] if t - i >= 0 else 0.0 for i in range(16)]
        assert hist.tolist() == want
        assert s_next == np.float32(expected_scale_used(seq, t + 1, 448.0))


def test_decay_rolls_out_after_history_length(oracle_lib):
    seq = [2.0 ** -t for t in range(40)]
    res = run(seq, fmt=E5M2)
    for t, (_, _, siu, _, s_next) in enumerate(res):
        s_used = expected_scale_used(seq, t, 57344.0)
        assert siu == np.float32(1.0 / s_used)
        # once t >= 16 the largest value in the window is the one 16 steps back
        if t >= 16:
            assert s_next == np.float32(57344.0 / seq[t - 15])


def test_margin_and_pow2(oracle_lib):
    seq = [3.0, 5.0, 0.75, 12.0]                     # not powers of two
    st = oracle.DelayedState()
    st_p = oracle.DelayedState()
    for t, a in enumerate(seq):
        x = torch.full((64,), a, dtype=torch.bfloat16)
        oracle.delayed_step(bits_of(x), E4M3, FP32, 2, st)
        oracle.delayed_step(bits_of(x), E4M3, POW2, 0, st_p)
        ref = max(seq[: t + 1])
        # margin 2: s = fl32(448/ref) / 4
        assert st.scale[0] == np.float32(np.float32(448.0) / np.float32(ref)) / np.float32(4)
        # pow2: largest power of two not above 448/ref
        p = 2.0 ** np.floor(np.log2(448.0 / ref))
        assert st_p.scale[0] == np.float32(p)


def test_non_finite_and_zero_keep_scale(oracle_lib):
    st = oracle.DelayedState(4)
    x1 = torch.full((8,), 2.0, dtype=torch.bfloat16)
    oracle.delayed_step(bits_of(x1), E4M3, FP32, 0, st)
    assert st.scale[0] == 224.0
    xnan = x1.clone()
    xnan[3] = float("nan")
    q, siu = oracle.delayed_step(bits_of(xnan), E4M3, FP32, 0, st)
    assert siu == np.float32(1 / 224.0)
    assert q[3] == 0x7F and np.isnan(st.history[0])
    assert st.scale[0] == 224.0                       # NaN in the window: scale kept
    zero = torch.zeros(8, dtype=torch.bfloat16)
    for _ in range(3):
        oracle.delayed_step(bits_of(zero), E4M3, FP32, 0, st)
        assert st.scale[0] == 224.0                   # NaN still in the window of 4
    oracle.delayed_step(bits_of(zero), E4M3, FP32, 0, st)
    assert st.history.tolist() == [0.0, 0.0, 0.0, 0.0]
    assert st.scale[0] == 224.0                       # all-zero window: scale kept
    xinf = x1.clone()
    xinf[0] = float("inf")
    q, _ = oracle.delayed_step(bits_of(xinf), E4M3, FP32, 0, st)
    assert q[0] == 0x7E and st.history[0] == np.inf and st.scale[0] == 224.0


def test_stale_scale_saturates(oracle_lib):
    st = oracle.DelayedState()
    x = torch.full((16,), 1.0, dtype=torch.bfloat16)
    oracle.delayed_step(bits_of(x), E4M3, FP32, 0, st)          # s becomes 448
    q, _ = oracle.delayed_step(bits_of(x * 1000), E4M3, FP32, 0, st)
    assert np.all(q == 0x7E)                                     # 1000 * 448 saturates
    q5, _ = oracle.delayed_step(bits_of(-x * 1e6), E5M2, FP32, 0, oracle.DelayedState())
    assert np.all(q5 == 0xFB)                                    # E5M2 saturates too (s = 1)


def test_checkpoint_resume_is_identical(oracle_lib):
    seq = [2.0 ** ((3 * t) % 7 - 3) for t in range(10)]
    straight = run(seq)
    st = oracle.DelayedState()
    for t in range(5):
        oracle.delayed_step(bits_of(tensor_with_amax(seq[t], t)), E4M3, FP32, 0, st)
    saved = (st.history.tobytes(), st.scale.tobytes())
    st2 = oracle.DelayedState(16, np.frombuffer(saved[0], dtype=np.float32).copy(),
                              np.frombuffer(saved[1], dtype=np.float32).copy())
    for t in range(5, 10):
        q, siu = oracle.delayed_step(bits_of(tensor_with_amax(seq[t], t)), E4M3, FP32, 0, st2)
        assert np.array_equal(q, straight[t][1]) and siu == straight[t][2]
    assert np.array_equal(st2.history, straight[-1][3]) and st2.scale[0] == straight[-1][4]
