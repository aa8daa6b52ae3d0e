"""fp8_quantize_delayed_noalloc (the delayed quantizer for callers that cannot allocate: its
amax partials live in the library's own per-device scratch array) gives bit for bit what
fp8_quantize_delayed gives with a caller workspace -- codes, scale_inv_used, amax history and
scale -- over consecutive calls, the second on a smaller tensor, and over a multi-step sequence
with both formats.  Calls go through the C ABI."""
import numpy as np
import pytest
import torch

import block_scaled_quantize_amd as bsq
import synth

pytestmark = pytest.mark.gpu


def _state_bits(st):
    return (st.history.cpu().numpy().view(np.uint32).copy(), st.scale.cpu().numpy().view(np.uint32).copy())


def _step(x, fmt, st, noalloc, mode=bsq.SCALE_FP32):
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    siu = torch.empty(1, dtype=torch.float32, device="cuda")
    bsq.quantize_delayed(x, fmt, st, mode=mode, q=q, scale_inv_used=siu, noalloc=noalloc)
    return q, siu


@pytest.mark.parametrize("fmt,mode", [(bsq.E4M3, bsq.SCALE_FP32), (bsq.E5M2, bsq.SCALE_POW2)])
def test_noalloc_matches_workspace_entry(gpu, fmt, mode):
    # large first (a full 2048-workgroup grid), then smaller (fewer partials): the second call
    # must not see the first call's partials
    sizes = [(8192, 4096), (300, 129), (4096, 4096), (1, 16), (2048, 14336), (7, 5)]
    ref, new = bsq.DelayedState(16), bsq.DelayedState(16)
    for i, shape in enumerate(sizes):
        scale = 1e-3 if i % 2 else 4.0
        x = synth.normal(shape, scale, i, f"noalloc/x{i}").cuda()
        q0, s0 = _step(x, fmt, ref, False, mode)
        q1, s1 = _step(x, fmt, new, True, mode)
        torch.cuda.synchronize()
        assert torch.equal(q0, q1), f"codes differ at call {i} {shape}"
        assert s0.cpu().numpy().view(np.uint32)[0] == s1.cpu().numpy().view(np.uint32)[0]
        h0, c0 = _state_bits(ref)
        h1, c1 = _state_bits(new)
        assert np.array_equal(h0, h1) and np.array_equal(c0, c1), f"state differs at call {i}"


def test_noalloc_second_call_smaller_with_larger_amax(gpu):
    """The partials the first (large) call leaves behind hold a larger amax than the second
    (small) tensor has; the second call's history entry must be its own amax."""
    big = synth.normal((8192, 4096), 100.0, 0, "noalloc/big").cuda()
    small = synth.normal((64, 64), 0.01, 1, "noalloc/small").cuda()
    ref, new = bsq.DelayedState(4), bsq.DelayedState(4)
    for x in (big, small):
        q0, s0 = _step(x, bsq.E4M3, ref, False)
        q1, s1 = _step(x, bsq.E4M3, new, True)
        torch.cuda.synchronize()
        assert torch.equal(q0, q1)
        assert np.array_equal(_state_bits(ref)[0], _state_bits(new)[0])
    assert float(new.history[0]) == float(small.float().abs().max())


def test_noalloc_argument_errors(gpu):
    lib = bsq.load()
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    st = bsq.DelayedState(16)
    q = torch.empty(16, dtype=torch.uint8, device="cuda")
    s = torch.empty(1, device="cuda")
    args = [x.data_ptr(), 16, bsq.E4M3, bsq.SCALE_FP32, 0, 16, st.history.data_ptr(),
            st.scale.data_ptr(), q.data_ptr(), s.data_ptr(), None]
    bad = list(args); bad[5] = 0
    assert lib.fp8_quantize_delayed_noalloc(*bad) == bsq.ERR_ARG
    bad = list(args); bad[1] = -1
    assert lib.fp8_quantize_delayed_noalloc(*bad) == bsq.ERR_SHAPE
    bad = list(args); bad[6] = None
    assert lib.fp8_quantize_delayed_noalloc(*bad) == bsq.ERR_NULL
    assert lib.fp8_quantize_delayed_noalloc(*args) == bsq.OK
    torch.cuda.synchronize()
