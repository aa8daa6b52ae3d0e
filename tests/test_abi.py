"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* the shared library loads and exports every function include/fp8bs.h declares;
* invalid arguments are rejected by host-side validation with the documented status codes,
  before anything is enqueued (null device pointers never get dereferenced here).
"""
import ctypes
import functools

import pytest

import block_scaled_quantize_amd as bsq

FAKE = 1 << 40          # a 16-byte aligned non-null address that is never dereferenced
FAKE_ODD = FAKE + 1


def test_library_exports_every_declared_symbol():
    lib = bsq.load()
    names = bsq.declared_functions()
    assert set(names) >= {"fp8_quantize_blockwise", "fp8_quantize_delayed",
                          "fp8_quantize_delayed_workspace_size", "fp8_gemm_blockscaled",
                          "fp8_grouped_gemm", "fp8_cast_fp32", "fp8bs_status_string",
                          "fp8_gemm_blockscaled_pow2", "fp8_grouped_gemm_pow2"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6, -7, 99):
        assert isinstance(bsq.status_string(s), str) and bsq.status_string(s)


def test_workspace_size_constant():
    assert bsq.delayed_workspace_size() > 0
    assert bsq.delayed_workspace_size() == bsq.delayed_workspace_size()


def q_blockwise(**kw):
    a = dict(x=FAKE, rows=4, cols=256, ld_x=256, fmt=0, gran=0, mode=0, q=FAKE, ld_q=256,
             s=FAKE, stream=None)
    a.update(kw)
    return bsq.load().fp8_quantize_blockwise(a["x"], a["rows"], a["cols"], a["ld_x"], a["fmt"],
                                             a["gran"], a["mode"], a["q"], a["ld_q"], a["s"],
                                             a["stream"])


def test_quantize_blockwise_validation():
    assert q_blockwise(fmt=2) == bsq.ERR_ARG
    assert q_blockwise(gran=2) == bsq.ERR_ARG        # per-tensor is the delayed entry point
    assert q_blockwise(mode=5) == bsq.ERR_ARG
    assert q_blockwise(rows=-1) == bsq.ERR_SHAPE
    assert q_blockwise(ld_x=100) == bsq.ERR_SHAPE
    assert q_blockwise(ld_q=100) == bsq.ERR_SHAPE
    assert q_blockwise(x=None) == bsq.ERR_NULL
    assert q_blockwise(q=None) == bsq.ERR_NULL
    assert q_blockwise(s=None) == bsq.ERR_NULL
    assert q_blockwise(s=FAKE + 2) == bsq.ERR_ALIGN
    assert q_blockwise(rows=0) == bsq.OK                # empty: no-op, nothing launched
    assert q_blockwise(cols=0, x=None) == bsq.OK


def q_delayed(**kw):
    a = dict(x=FAKE, n=1024, fmt=0, mode=0, margin=0, hist=16, h=FAKE, s=FAKE, q=FAKE, siu=FAKE,
             ws=FAKE, wsb=bsq.delayed_workspace_size())
    a.update(kw)
    return bsq.load().fp8_quantize_delayed(a["x"], a["n"], a["fmt"], a["mode"], a["margin"],
                                           a["hist"], a["h"], a["s"], a["q"], a["siu"], a["ws"],
                                           a["wsb"], None)


def test_quantize_delayed_validation():
    assert q_delayed(hist=0) == bsq.ERR_ARG
    assert q_delayed(hist=1025) == bsq.ERR_ARG
    assert q_delayed(margin=-1) == bsq.ERR_ARG
    assert q_delayed(margin=65) == bsq.ERR_ARG
    assert q_delayed(fmt=7) == bsq.ERR_ARG
    assert q_delayed(n=-5) == bsq.ERR_SHAPE
    assert q_delayed(h=None) == bsq.ERR_NULL
    assert q_delayed(x=None) == bsq.ERR_NULL
    assert q_delayed(ws=None) == bsq.ERR_WORKSPACE
    assert q_delayed(wsb=4) == bsq.ERR_WORKSPACE
    assert q_delayed(s=FAKE_ODD) == bsq.ERR_ALIGN


def gemm(entry="fp8_gemm_blockscaled", **kw):
    a = dict(layout=0, M=256, N=256, K=256, A=FAKE, lda=256, fa=0, ga=0, sa=FAKE, B=FAKE,
             ldb=256, fb=0, gb=1, sb=FAKE, C=FAKE, ldc=256)
    a.update(kw)
    return getattr(bsq.load(), entry)(a["layout"], a["M"], a["N"], a["K"], a["A"], a["lda"],
                                      a["fa"], a["ga"], a["sa"], a["B"], a["ldb"], a["fb"],
                                      a["gb"], a["sb"], a["C"], a["ldc"], None)


@pytest.mark.parametrize("entry", ["fp8_gemm_blockscaled", "fp8_gemm_blockscaled_pow2"])
def test_gemm_validation(entry):
    gemm = functools.partial(globals()["gemm"], entry)
    assert gemm(layout=3) == bsq.ERR_ARG
    assert gemm(fa=2) == bsq.ERR_ARG
    assert gemm(gb=3) == bsq.ERR_ARG
    assert gemm(M=-1) == bsq.ERR_SHAPE
    assert gemm(lda=128) == bsq.ERR_SHAPE
    assert gemm(ldc=100) == bsq.ERR_SHAPE
    assert gemm(A=None) == bsq.ERR_NULL
    assert gemm(C=None) == bsq.ERR_NULL
    assert gemm(A=FAKE_ODD) == bsq.ERR_ALIGN
    assert gemm(lda=264) == bsq.ERR_ALIGN
    assert gemm(ldc=257) == bsq.ERR_ALIGN
    # 1x128 scales only on a K-major operand (fprop takes them on both sides)
    assert gemm(layout=2, ga=0, gb=1) == bsq.ERR_UNSUPPORTED   # wgrad: A is MN-major
    assert gemm(layout=2, ga=1, gb=0) == bsq.ERR_UNSUPPORTED   # wgrad: B is MN-major
    assert gemm(layout=1, ga=0, gb=0) == bsq.ERR_UNSUPPORTED   # dgrad: B is MN-major
    assert gemm(M=0) == bsq.OK and gemm(N=0, C=None) == bsq.OK
    # scale arrays of 4 GiB or more (1x128 scales of 2^30 rows x 4 K blocks): rejected before
    # any launch
    assert gemm(M=1 << 30, K=512, lda=512) == bsq.ERR_SHAPE


def grouped(entry="fp8_grouped_gemm", **kw):
    a = dict(G=4, off=FAKE, M=512, N=256, K=256, A=FAKE, lda=256, fa=0, sa=FAKE, B=FAKE,
             ldb=256, fb=0, sb=FAKE, C=FAKE, ldc=256)
    a.update(kw)
    return getattr(bsq.load(), entry)(a["G"], a["off"], a["M"], a["N"], a["K"], a["A"], a["lda"],
                                      a["fa"], a["sa"], a["B"], a["ldb"], a["fb"], a["sb"], a["C"],
                                      a["ldc"], None)


@pytest.mark.parametrize("entry", ["fp8_grouped_gemm", "fp8_grouped_gemm_pow2"])
def test_grouped_validation(entry):
    grouped = functools.partial(globals()["grouped"], entry)
    assert grouped(G=-1) == bsq.ERR_ARG
    assert grouped(G=5000) == bsq.ERR_ARG
    assert grouped(fb=9) == bsq.ERR_ARG
    assert grouped(K=0) == bsq.ERR_SHAPE
    assert grouped(off=None) == bsq.ERR_NULL
    assert grouped(lda=64) == bsq.ERR_SHAPE
    assert grouped(off=FAKE + 4) == bsq.ERR_ALIGN
    assert grouped(M=0) == bsq.OK and grouped(G=0) == bsq.OK
    assert grouped(M=1 << 30, K=512, lda=512) == bsq.ERR_SHAPE   # activation scales >= 4 GiB


def qcol(**kw):
    a = dict(x=FAKE, rows=256, cols=128, ldx=128, fmt=0, mode=0, qt=FAKE, ldqt=256, s=FAKE)
    a.update(kw)
    return bsq.load().fp8_quantize_columnwise_t(a["x"], a["rows"], a["cols"], a["ldx"], a["fmt"],
                                                a["mode"], a["qt"], a["ldqt"], a["s"], None)


def test_quantize_rows_and_columnwise_validation():
    f = bsq.load().fp8_quantize_1x128_and_columnwise_t
    def call(**kw):
        a = dict(x=FAKE, rows=256, cols=128, ldx=128, fmt=0, mode=0, q=FAKE, ldq=128, s=FAKE,
                 qt=FAKE, ldqt=256, st=FAKE)
        a.update(kw)
        return f(a["x"], a["rows"], a["cols"], a["ldx"], a["fmt"], a["mode"], a["q"], a["ldq"],
                 a["s"], a["qt"], a["ldqt"], a["st"], None)
    assert call(fmt=2) == bsq.ERR_ARG
    assert call(mode=5) == bsq.ERR_ARG
    assert call(ldq=100) == bsq.ERR_SHAPE
    assert call(ldqt=255) == bsq.ERR_SHAPE
    assert call(q=None) == bsq.ERR_NULL
    assert call(st=None) == bsq.ERR_NULL
    assert call(s=FAKE_ODD) == bsq.ERR_ALIGN
    assert call(st=FAKE_ODD) == bsq.ERR_ALIGN
    assert call(rows=0) == bsq.OK and call(cols=0, x=None) == bsq.OK


def test_quantize_columnwise_validation():
    assert qcol(fmt=2) == bsq.ERR_ARG
    assert qcol(mode=5) == bsq.ERR_ARG
    assert qcol(rows=-1) == bsq.ERR_SHAPE
    assert qcol(ldx=100) == bsq.ERR_SHAPE
    assert qcol(ldqt=255) == bsq.ERR_SHAPE          # the transposed rows hold `rows` codes
    assert qcol(x=None) == bsq.ERR_NULL
    assert qcol(s=None) == bsq.ERR_NULL
    assert qcol(s=FAKE_ODD) == bsq.ERR_ALIGN
    assert qcol(rows=0) == bsq.OK and qcol(cols=0, x=None) == bsq.OK


def qout(**kw):
    a = dict(M=256, N=256, K=256, A=FAKE, lda=256, ga=0, sa=FAKE, B=FAKE, ldb=256, gb=1, sb=FAKE,
             p2=0, C=FAKE, ldc=256, mode=0, Cq=FAKE, ldcq=256, cqs=FAKE)
    a.update(kw)
    return bsq.load().fp8_gemm_blockscaled_qout(a["M"], a["N"], a["K"], a["A"], a["lda"], a["ga"],
                                                a["sa"], a["B"], a["ldb"], a["gb"], a["sb"],
                                                a["p2"], a["C"], a["ldc"], a["mode"], a["Cq"],
                                                a["ldcq"], a["cqs"], None)


def test_gemm_qout_validation():
    assert qout(mode=2) == bsq.ERR_ARG
    assert qout(p2=3) == bsq.ERR_ARG
    assert qout(ga=5) == bsq.ERR_ARG
    assert qout(Cq=None) == bsq.ERR_NULL
    assert qout(cqs=None) == bsq.ERR_NULL
    assert qout(A=None) == bsq.ERR_NULL
    assert qout(ldcq=100) == bsq.ERR_SHAPE
    assert qout(cqs=FAKE_ODD) == bsq.ERR_ALIGN
    assert qout(gb=0) == bsq.ERR_UNSUPPORTED                 # 1x128 weight scales: not here
    assert qout(M=0) == bsq.OK and qout(N=0, C=None) == bsq.OK


def test_tiled_entry_validation():
    """The entry points with an explicit tile configuration reject tile and pow2 values out of
    range, and otherwise validate exactly as the plain entry points do."""
    lib = bsq.load()
    g = dict(layout=0, M=256, N=256, K=256, A=FAKE, lda=256, fa=0, ga=0, sa=FAKE, B=FAKE,
             ldb=256, fb=0, gb=1, sb=FAKE, C=FAKE, ldc=256)

    def tiled(tile, pow2, **kw):
        a = dict(g, **kw)
        return lib.fp8_gemm_blockscaled_tiled(tile, pow2, *a.values(), None)

    for tile in (-1, 5, 99):
        assert tiled(tile, 0) == bsq.ERR_ARG
    assert tiled(bsq.TILE_256x256_W8, 2) == bsq.ERR_ARG
    for tile in range(5):
        for p2 in (0, 1):
            assert tiled(tile, p2, layout=3) == bsq.ERR_ARG
            assert tiled(tile, p2, M=-1) == bsq.ERR_SHAPE
            assert tiled(tile, p2, A=None) == bsq.ERR_NULL
            assert tiled(tile, p2, layout=2, ga=0) == bsq.ERR_UNSUPPORTED
            assert tiled(tile, p2, M=0) == bsq.OK
    gr = dict(G=4, off=FAKE, M=512, N=256, K=256, A=FAKE, lda=256, fa=0, sa=FAKE, B=FAKE,
              ldb=256, fb=0, sb=FAKE, C=FAKE, ldc=256)

    def gtiled(tile, pow2, **kw):
        a = dict(gr, **kw)
        return lib.fp8_grouped_gemm_tiled(tile, pow2, *a.values(), None)

    for tile in (-1, bsq.TILE_256x128_W4, 5):               # 256x128 with 4 waves: dense only
        assert gtiled(tile, 0) == bsq.ERR_ARG
    assert gtiled(bsq.TILE_AUTO, 3) == bsq.ERR_ARG
    for tile in (bsq.TILE_AUTO, bsq.TILE_256x128_W8, bsq.TILE_256x256_W8, bsq.TILE_128x128_W4):
        assert gtiled(tile, 1, K=0) == bsq.ERR_SHAPE
        assert gtiled(tile, 0, off=None) == bsq.ERR_NULL
        assert gtiled(tile, 0, G=0) == bsq.OK
    q = dict(M=256, N=256, K=256, A=FAKE, lda=256, ga=0, sa=FAKE, B=FAKE, ldb=256, gb=1, sb=FAKE,
             p2=0, C=FAKE, ldc=256, mode=0, Cq=FAKE, ldcq=256, cqs=FAKE)

    def qtiled(tile, **kw):
        a = dict(q, **kw)
        return lib.fp8_gemm_blockscaled_qout_tiled(tile, *a.values(), None)

    assert qtiled(7) == bsq.ERR_ARG and qtiled(-2) == bsq.ERR_ARG
    for tile in range(5):
        assert qtiled(tile, Cq=None) == bsq.ERR_NULL
        assert qtiled(tile, gb=0) == bsq.ERR_UNSUPPORTED
        assert qtiled(tile, M=0) == bsq.OK


def test_quantize_batched_validation():
    """fp8_quantize_blockwise_batched checks every tensor before launching anything."""
    import ctypes
    lib = bsq.load()
    P, I64, I32 = ctypes.c_void_p * 2, ctypes.c_int64 * 2, ctypes.c_int * 2

    def call(n=2, x=(FAKE, FAKE), rows=(4, 8), cols=(256, 128), ldx=(256, 128), gran=(0, 1),
             fmt=0, mode=0, q=(FAKE, FAKE), ldq=(256, 128), s=(FAKE, FAKE)):
        return lib.fp8_quantize_blockwise_batched(n, P(*x), I64(*rows), I64(*cols), I64(*ldx),
                                                  I32(*gran), fmt, mode, P(*q), I64(*ldq), P(*s),
                                                  None)

    assert call(n=-1) == bsq.ERR_ARG and call(n=17) == bsq.ERR_ARG
    assert call(fmt=2) == bsq.ERR_ARG and call(mode=2) == bsq.ERR_ARG
    assert call(gran=(0, 2)) == bsq.ERR_ARG            # per tensor: the delayed entry point
    assert call(rows=(4, -1)) == bsq.ERR_SHAPE
    assert call(ldx=(256, 100)) == bsq.ERR_SHAPE
    assert call(ldq=(255, 128)) == bsq.ERR_SHAPE
    assert call(x=(FAKE, None)) == bsq.ERR_NULL
    assert call(s=(FAKE, FAKE + 2)) == bsq.ERR_ALIGN
    assert call(n=0) == bsq.OK
    assert call(rows=(0, 0), x=(None, None)) == bsq.OK   # empty tensors: nothing to launch
    assert lib.fp8_quantize_blockwise_batched(1, None, None, None, None, None, 0, 0, None, None,
                                              None, None) == bsq.ERR_NULL


def test_delayed_noalloc_validation():
    """fp8_quantize_delayed_noalloc validates like fp8_quantize_delayed (no workspace argument);
    invalid calls return before any device is touched."""
    lib = bsq.load()
    a = [FAKE, 1024, 0, 0, 0, 16, FAKE, FAKE, FAKE, FAKE, None]

    def call(**kw):
        b = list(a)
        for k, v in kw.items():
            b[int(k[1:])] = v
        return lib.fp8_quantize_delayed_noalloc(*b)

    assert call(a2=2) == bsq.ERR_ARG          # format
    assert call(a3=3) == bsq.ERR_ARG          # scale mode
    assert call(a4=-1) == bsq.ERR_ARG         # margin
    assert call(a5=0) == bsq.ERR_ARG          # history length
    assert call(a5=1025) == bsq.ERR_ARG
    assert call(a1=-1) == bsq.ERR_SHAPE
    assert call(a6=None) == bsq.ERR_NULL      # history
    assert call(a0=None) == bsq.ERR_NULL      # input with numel > 0
    assert call(a7=FAKE + 2) == bsq.ERR_ALIGN  # scale


def test_cast_validation():
    lib = bsq.load()
    assert lib.fp8_cast_fp32(FAKE, 16, 3, FAKE, None) == bsq.ERR_ARG
    assert lib.fp8_cast_fp32(FAKE, -1, 0, FAKE, None) == bsq.ERR_SHAPE
    assert lib.fp8_cast_fp32(None, 16, 0, FAKE, None) == bsq.ERR_NULL
    assert lib.fp8_cast_fp32(FAKE + 2, 16, 0, FAKE, None) == bsq.ERR_ALIGN
    assert lib.fp8_cast_fp32(None, 0, 0, None, None) == bsq.OK


def kv_append(**kw):
    a = dict(B=2, KVH=8, T=16, kn=FAKE, vn=FAKE, pos=FAKE, fmt=0, mode=0, kc=FAKE, ks=FAKE,
             vc=FAKE, vs=FAKE)
    a.update(kw)
    return bsq.load().fp8_kv_cache_append(a["B"], a["KVH"], a["T"], a["kn"], a["vn"], a["pos"],
                                          a["fmt"], a["mode"], a["kc"], a["ks"], a["vc"], a["vs"],
                                          None)


def test_kv_cache_append_validation():
    assert kv_append(fmt=3) == bsq.ERR_ARG
    assert kv_append(mode=2) == bsq.ERR_ARG
    assert kv_append(B=-1) == bsq.ERR_SHAPE
    assert kv_append(T=-1) == bsq.ERR_SHAPE
    assert kv_append(B=70000) == bsq.ERR_SHAPE
    assert kv_append(B=1 << 40, T=1 << 20) == bsq.ERR_SHAPE   # cache bytes overflow
    assert kv_append(kn=None) == bsq.ERR_NULL
    assert kv_append(pos=None) == bsq.ERR_NULL
    assert kv_append(vs=None) == bsq.ERR_NULL
    assert kv_append(kn=FAKE + 8) == bsq.ERR_ALIGN
    assert kv_append(kc=FAKE + 4) == bsq.ERR_ALIGN
    assert kv_append(ks=FAKE + 2) == bsq.ERR_ALIGN
    assert kv_append(B=0, kn=None) == bsq.OK        # empty: nothing launched
    assert kv_append(T=0, kn=None) == bsq.OK


def attn(**kw):
    a = dict(B=2, H=32, KVH=8, T=16, q=FAKE, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE, lens=FAKE,
             sm=0.088, fmt=0, out=FAKE)
    a.update(kw)
    return bsq.load().fp8_attention_decode(a["B"], a["H"], a["KVH"], a["T"], a["q"], a["kc"],
                                           a["ks"], a["vc"], a["vs"], a["lens"], a["sm"],
                                           a["fmt"], a["out"], None)


def test_attention_decode_validation():
    assert attn(fmt=2) == bsq.ERR_ARG
    assert attn(sm=float("inf")) == bsq.ERR_ARG
    assert attn(sm=float("nan")) == bsq.ERR_ARG
    assert attn(H=-1) == bsq.ERR_SHAPE
    assert attn(KVH=0) == bsq.ERR_SHAPE
    assert attn(H=30, KVH=8) == bsq.ERR_SHAPE            # not a multiple
    assert attn(H=48, KVH=3) == bsq.ERR_UNSUPPORTED      # 16 query heads per KV head
    assert attn(H=24, KVH=8) == bsq.ERR_UNSUPPORTED      # 3
    assert attn(q=None) == bsq.ERR_NULL
    assert attn(lens=None) == bsq.ERR_NULL
    assert attn(kc=None) == bsq.ERR_NULL
    assert attn(out=None) == bsq.ERR_NULL
    assert attn(q=FAKE + 8) == bsq.ERR_ALIGN
    assert attn(vc=FAKE + 4) == bsq.ERR_ALIGN
    assert attn(out=FAKE + 2) == bsq.ERR_ALIGN
    assert attn(B=0, q=None) == bsq.OK                   # empty: nothing launched
    assert attn(H=0, q=None) == bsq.OK


def attn_split(**kw):
    a = dict(B=2, H=32, KVH=8, T=100, q=FAKE, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE, lens=FAKE,
             sm=0.088, fmt=0, chunk=32, ws=FAKE, wsb=1 << 20, out=FAKE)
    a.update(kw)
    return bsq.load().fp8_attention_decode_split(a["B"], a["H"], a["KVH"], a["T"], a["q"],
                                                 a["kc"], a["ks"], a["vc"], a["vs"], a["lens"],
                                                 a["sm"], a["fmt"], a["chunk"], a["ws"],
                                                 a["wsb"], a["out"], None)


def test_attention_decode_workspace_size():
    # B * KVH * ceil(T / chunk) * (H / KVH) * 130 floats
    assert bsq.attention_decode_workspace_size(2, 32, 8, 100, 32) == 2 * 8 * 4 * 4 * 130 * 4
    assert bsq.attention_decode_workspace_size(64, 32, 8, 4096, 1024) == 64 * 8 * 4 * 4 * 130 * 4
    assert bsq.attention_decode_workspace_size(1, 8, 8, 33, 32) == 8 * 2 * 1 * 130 * 4
    assert bsq.attention_decode_workspace_size(0, 32, 8, 100, 32) == 0
    assert bsq.attention_decode_workspace_size(2, 30, 8, 100, 32) == 0
    assert bsq.attention_decode_workspace_size(2, 32, 8, 100, 0) == 0
    assert bsq.attention_decode_workspace_size(1 << 40, 32, 8, 1 << 20, 32) == 0   # overflow


def test_attention_decode_split_validation():
    need = bsq.attention_decode_workspace_size(2, 32, 8, 100, 32)
    assert attn_split(fmt=2) == bsq.ERR_ARG
    assert attn_split(sm=float("nan")) == bsq.ERR_ARG
    assert attn_split(chunk=0) == bsq.ERR_SHAPE
    assert attn_split(chunk=48) == bsq.ERR_SHAPE             # not a multiple of 32
    assert attn_split(chunk=-32) == bsq.ERR_SHAPE
    assert attn_split(KVH=0) == bsq.ERR_SHAPE
    assert attn_split(H=30, KVH=8) == bsq.ERR_SHAPE
    assert attn_split(H=128, KVH=8) == bsq.ERR_UNSUPPORTED   # 16 query heads per KV head
    assert attn_split(wsb=need - 4) == bsq.ERR_SHAPE         # workspace too small
    assert attn_split(ws=None) == bsq.ERR_NULL
    assert attn_split(q=None) == bsq.ERR_NULL
    assert attn_split(kc=None) == bsq.ERR_NULL
    assert attn_split(ws=FAKE + 2) == bsq.ERR_ALIGN
    assert attn_split(q=FAKE + 8) == bsq.ERR_ALIGN
    assert attn_split(B=0, q=None, ws=None) == bsq.OK        # empty: nothing launched
    assert attn_split(H=0, q=None, ws=None) == bsq.OK


def test_decode_split_tokens_choice():
    # 64 sequences x 8 KV heads already give every CU two workgroups: unsplit
    assert bsq.decode_split_tokens(64, 8, 4096) is None
    assert bsq.decode_split_tokens(16, 8, 4096) == 1024     # 128 groups x 4 chunks
    assert bsq.decode_split_tokens(4, 8, 4096) == 256       # 32 groups x 16 chunks
    assert bsq.decode_split_tokens(1, 1, 100) == 256        # at least 256 tokens per chunk
    for B, KVH, T in ((3, 8, 5000), (1, 4, 32768), (7, 2, 999)):
        c = bsq.decode_split_tokens(B, KVH, T)
        assert c % 256 == 0 and c >= 256
        assert B * KVH * -(-T // c) <= 512 + B * KVH        # about the target, not far above


def test_attention_decode_offset_limit():
    # the matrix-core kernels (1, 2 or 4 query heads per KV head) address one sequence and KV
    # head's rows with 32-bit offsets
    big = (1 << 32) // (8 * 128)          # T with (T + 32) * 8 * 128 >= 2^32
    assert attn(T=big, KVH=8, H=32) == bsq.ERR_UNSUPPORTED
    assert attn_split(T=big, KVH=8, H=32, wsb=1 << 40) == bsq.ERR_UNSUPPORTED
    assert attn(T=big - 64, KVH=8, H=32, q=None) == bsq.ERR_NULL   # within the limit: validated on


def test_bench_library_probes_reject_invalid_arguments():
    """libfp8bs_bench.so (the benchmark's streaming and matrix-core probes, not the C ABI) loads,
    exports both probes, and rejects invalid arguments before launching anything."""
    import os
    path = os.path.join(os.path.dirname(bsq.__file__), "libfp8bs_bench.so")
    blib = ctypes.CDLL(path)
    blib.fp8bs_bench_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    blib.fp8bs_bench_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_void_p]
    mfma = blib.fp8bs_bench_mfma
    assert mfma(None, FAKE, 0, 10, 256, 0, None) == -1          # no codes
    assert mfma(FAKE, None, 0, 10, 256, 0, None) == -1          # no output
    assert mfma(FAKE_ODD, FAKE, 0, 10, 256, 0, None) == -1      # misaligned codes
    assert mfma(FAKE, FAKE, 2, 10, 256, 0, None) == -1          # no such shape
    assert mfma(FAKE, FAKE, 0, 0, 256, 0, None) == -1           # no steps
    assert mfma(FAKE, FAKE, 0, 10, 0, 0, None) == -1            # no workgroups
    assert mfma(FAKE, FAKE, 0, 10, 256, 161 * 1024, None) == -1  # more LDS than a CU has
    assert blib.fp8bs_bench_stream(None, 16, FAKE, 0, None) == -1
    assert blib.fp8bs_bench_stream(FAKE, 15, FAKE, 0, None) == -1
    assert blib.fp8bs_bench_stream(FAKE, 16, FAKE, 9, None) == -1      # no such variant
    assert blib.fp8bs_bench_stream(FAKE, 4096, FAKE, 8, None) == -1    # not whole 32-row tiles


def test_mx_validation():
    lib = bsq.load()
    # quantizer: format, pitches, null pointers, scale alignment; empty is a no-op
    assert lib.fp8_quantize_mx(FAKE, 4, 64, 64, 2, FAKE, 64, FAKE, None) == bsq.ERR_ARG
    assert lib.fp8_quantize_mx(FAKE, 4, 64, 32, 0, FAKE, 64, FAKE, None) == bsq.ERR_SHAPE
    assert lib.fp8_quantize_mx(FAKE, 4, 64, 64, 0, FAKE, 63, FAKE, None) == bsq.ERR_SHAPE
    assert lib.fp8_quantize_mx(None, 4, 64, 64, 0, FAKE, 64, FAKE, None) == bsq.ERR_NULL
    assert lib.fp8_quantize_mx(FAKE, 4, 64, 64, 0, FAKE, 64, FAKE_ODD, None) == bsq.ERR_ALIGN
    assert lib.fp8_quantize_mx(None, 0, 64, 64, 0, None, 64, None, None) == bsq.OK
    # columnwise form: the transposed codes' rows hold `rows` codes
    qmt = lib.fp8_quantize_mx_columnwise_t
    assert qmt(FAKE, 256, 64, 64, 2, FAKE, 256, FAKE, None) == bsq.ERR_ARG
    assert qmt(FAKE, 256, 64, 63, 0, FAKE, 256, FAKE, None) == bsq.ERR_SHAPE
    assert qmt(FAKE, 256, 64, 64, 0, FAKE, 255, FAKE, None) == bsq.ERR_SHAPE
    assert qmt(FAKE, 256, 64, 64, 0, None, 256, FAKE, None) == bsq.ERR_NULL
    assert qmt(FAKE, 256, 64, 64, 0, FAKE, 256, FAKE_ODD, None) == bsq.ERR_ALIGN
    assert qmt(None, 0, 64, 64, 0, None, 0, None, None) == bsq.OK
    # rows and columns in one pass
    qmr = lib.fp8_quantize_mx_and_columnwise_t
    assert qmr(FAKE, 256, 64, 64, 2, FAKE, 64, FAKE, FAKE, 256, FAKE, None) == bsq.ERR_ARG
    assert qmr(FAKE, 256, 64, 64, 0, FAKE, 63, FAKE, FAKE, 256, FAKE, None) == bsq.ERR_SHAPE
    assert qmr(FAKE, 256, 64, 64, 0, FAKE, 64, FAKE, FAKE, 255, FAKE, None) == bsq.ERR_SHAPE
    assert qmr(FAKE, 256, 64, 64, 0, FAKE, 64, FAKE, None, 256, FAKE, None) == bsq.ERR_NULL
    assert qmr(FAKE, 256, 64, 64, 0, FAKE, 64, FAKE_ODD, FAKE, 256, FAKE, None) == bsq.ERR_ALIGN
    assert qmr(FAKE, 256, 64, 64, 0, FAKE, 64, FAKE, FAKE, 256, FAKE_ODD, None) == bsq.ERR_ALIGN
    assert qmr(None, 0, 64, 64, 0, None, 64, None, None, 0, None, None) == bsq.OK
    # grouped form
    gmx = lib.fp8_grouped_gemm_mx
    def grouped(**kw):
        v = dict(G=4, off=FAKE, M=512, N=256, K=256, lda=256, fa=0, sa=FAKE, ldb=256, fb=0, sb=FAKE,
                 C=FAKE, ldc=256)
        v.update(kw)
        return gmx(v["G"], v["off"], v["M"], v["N"], v["K"], FAKE, v["lda"], v["fa"], v["sa"], FAKE,
                   v["ldb"], v["fb"], v["sb"], v["C"], v["ldc"], None)
    assert grouped(G=-1) == bsq.ERR_ARG
    assert grouped(fb=9) == bsq.ERR_ARG
    assert grouped(K=0) == bsq.ERR_SHAPE
    assert grouped(off=None) == bsq.ERR_NULL
    assert grouped(sb=None) == bsq.ERR_NULL
    assert grouped(sa=FAKE + 2) == bsq.ERR_ALIGN
    assert grouped(sb=FAKE + 1) == bsq.ERR_ALIGN
    assert grouped(M=0) == bsq.OK and grouped(G=0) == bsq.OK
    # GEMM: formats, misaligned scales, null scales, pitches; empty is a no-op
    def gemm(**kw):
        v = dict(M=64, N=64, K=128, lda=128, fa=0, sa=FAKE, ldb=128, fb=0, sb=FAKE, C=FAKE, ldc=64)
        v.update(kw)
        return lib.fp8_gemm_mx(v["M"], v["N"], v["K"], FAKE, v["lda"], v["fa"], v["sa"], FAKE,
                               v["ldb"], v["fb"], v["sb"], v["C"], v["ldc"], None)
    assert gemm(fb=5) == bsq.ERR_ARG
    assert gemm(sb=FAKE + 2) == bsq.ERR_ALIGN
    assert gemm(sa=None) == bsq.ERR_NULL
    assert gemm(ldb=100) == bsq.ERR_SHAPE
    assert gemm(M=0) == bsq.OK


def test_binding_rejects_bad_tensors_before_any_call():
    """The Python wrappers of the microscaling and one-pass entry points validate dtype, rank and
    device before marshalling anything (CPU tensors here: nothing reaches the library)."""
    import torch
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bsq.quantize_mx(x.float(), bsq.E4M3)                        # not bf16
    with pytest.raises(ValueError):
        bsq.quantize_mx_columnwise_t(x[:, ::2], bsq.E4M3)           # column stride 2
    with pytest.raises(ValueError):
        bsq.quantize_mx_and_columnwise_t(x.reshape(-1), bsq.E4M3)   # not 2-D
    with pytest.raises(ValueError):
        bsq.quantize_1x128_and_columnwise_t(x, bsq.E4M3)            # host tensors
    a = torch.zeros((4, 128), dtype=torch.uint8)
    with pytest.raises(ValueError):
        bsq.gemm_mx(a, torch.zeros((1, 4, 4), dtype=torch.uint8), a[:, :64],
                    torch.zeros((1, 4, 4), dtype=torch.uint8))      # K mismatch
    with pytest.raises(ValueError):
        bsq.grouped_gemm_mx(torch.zeros(2, dtype=torch.int64), a, torch.zeros((1, 4, 4), dtype=torch.uint8),
                            a, torch.zeros((1, 4, 4), dtype=torch.uint8))   # b not [G, N, K]
