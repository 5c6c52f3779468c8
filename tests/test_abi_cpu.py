"""C-ABI checks that need no GPU: the library loads, exports every function
``include/swiglu.h`` declares, and rejects invalid arguments before any HIP
call (so nothing is launched).  Fake device addresses are used: validation
fails before they could be dereferenced or passed to HIP."""
import ctypes
import os

import pytest

from gated_mlp_gemm_amd import swiglu as sw

ERR_NULL, ERR_SHAPE, ERR_ALIGN = sw.SWIGLU_ERR_NULL, sw.SWIGLU_ERR_SHAPE, sw.SWIGLU_ERR_ALIGN
ERR_UNSUP, ERR_ALIAS = sw.SWIGLU_ERR_UNSUPPORTED, sw.SWIGLU_ERR_ALIAS

# fake, 16-byte aligned, far apart "device" addresses (never dereferenced)
A_, W1_, W2_, WF_, Y_, G_, U_, WS_ = (0x10_0000_0000 * (i + 1) for i in range(8))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sw.LIBRARY):
        pytest.fail("libswiglu.so is not built (python -m gated_mlp_gemm_amd.build)")
    return sw.load_library()


def test_exports_every_declared_function(lib):
    names = sw.header_functions()
    assert set(names) >= {"swiglu_pack_weights", "swiglu_fused_gemm",
                          "swiglu_unfused_ablation", "swiglu_select_variant",
                          "swiglu_status_string"}
    raw = ctypes.CDLL(sw.LIBRARY)
    for n in names:
        assert hasattr(raw, n), f"{n} declared in swiglu.h but not exported"


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert sw.swiglu_status_string(code) != "unknown status"
    assert sw.swiglu_status_string(17) == "unknown status"


def test_dispatcher_thresholds(lib, monkeypatch):
    # built-in: variant I at every M (measured faster than S on MI355X)
    monkeypatch.delenv("SWIGLU_M_SWITCH", raising=False)
    assert sw.swiglu_m_switch() == 2 ** 31 - 1
    for M in (0, 1, 128, 2048, 2049, 8192, 2 ** 31 - 1):
        assert sw.swiglu_select_variant(M, 8960, 1536) == sw.SWIGLU_VARIANT_I
    assert lib.swiglu_select_variant(-1, 8, 8) == ERR_SHAPE
    # the pages' small/large-batch split, set through the environment
    monkeypatch.setenv("SWIGLU_M_SWITCH", "2048")
    assert sw.swiglu_m_switch() == 2048
    assert sw.swiglu_select_variant(2048) == sw.SWIGLU_VARIANT_I
    assert sw.swiglu_select_variant(2049) == sw.SWIGLU_VARIANT_S
    monkeypatch.setenv("SWIGLU_M_SWITCH", "100")
    assert sw.swiglu_select_variant(100) == sw.SWIGLU_VARIANT_I
    assert sw.swiglu_select_variant(101) == sw.SWIGLU_VARIANT_S
    monkeypatch.setenv("SWIGLU_M_SWITCH", "not-a-number")
    assert sw.swiglu_m_switch() == 2 ** 31 - 1


def fused(lib, A=A_, WF=WF_, Y=Y_, M=256, N=256, K=256, v=2, ws=None, wsb=0):
    return lib.swiglu_fused_gemm(A, WF, Y, M, N, K, v, ws, wsb, None)


def test_fused_validation(lib):
    # shapes
    assert fused(lib, M=-1) == ERR_SHAPE
    assert fused(lib, N=-8) == ERR_SHAPE
    assert fused(lib, K=0) == ERR_SHAPE
    assert fused(lib, K=4) == ERR_SHAPE
    assert fused(lib, K=20) == ERR_SHAPE          # not a multiple of 8
    assert fused(lib, N=12) == ERR_SHAPE
    assert fused(lib, K=(1 << 21) + 8) == ERR_SHAPE
    assert fused(lib, N=(1 << 22) + 8) == ERR_SHAPE
    assert fused(lib, M=1 << 31) == ERR_SHAPE
    # variant
    assert fused(lib, v=3) == ERR_UNSUP
    assert fused(lib, v=-1) == ERR_UNSUP
    # null pointers, every variant
    for v in (0, 1, 2):
        assert fused(lib, A=None, v=v) == ERR_NULL
        assert fused(lib, Y=None, v=v) == ERR_NULL
        assert fused(lib, WF=None, v=v) == ERR_NULL
    # alignment
    assert fused(lib, A=A_ + 2) == ERR_ALIGN
    assert fused(lib, Y=Y_ + 8) == ERR_ALIGN
    assert fused(lib, WF=WF_ + 4, v=1) == ERR_ALIGN
    # aliasing: Y inside A, Y inside W_fused (whose extent is 2*N*K elements)
    assert fused(lib, Y=A_ + 1024) == ERR_ALIAS
    assert fused(lib, Y=WF_ + 4096, v=2) == ERR_ALIAS
    assert fused(lib, Y=WF_ + 2 * 256 * 256 * 2 - 16, v=1) == ERR_ALIAS
    # workspace: 256-byte aligned, disjoint from the operands
    assert fused(lib, ws=WS_ + 16, wsb=1 << 20) == ERR_ALIGN
    assert fused(lib, ws=Y_ + 256, wsb=1 << 20) == ERR_ALIAS
    assert fused(lib, ws=A_, wsb=1 << 20) == ERR_ALIAS
    assert "overlaps" in sw.swiglu_last_error()


def test_empty_problems_succeed_without_pointers(lib):
    assert lib.swiglu_fused_gemm(None, None, None, 0, 256, 64, 0, None, 0, None) == 0
    assert lib.swiglu_fused_gemm(None, None, None, 64, 0, 64, 0, None, 0, None) == 0
    assert lib.swiglu_unfused_ablation(None, None, None, None, None, 0, 64, 64, None, 0,
                                       None) == 0
    assert lib.swiglu_pack_weights(None, None, None, 0, 64, None) == 0
    assert lib.swiglu_pack_weights(None, None, None, 64, 0, None) == 0
    assert lib.swiglu_silu_mul(None, None, None, 0, None) == 0
    assert sw.swiglu_last_error() == ""


def test_pack_validation(lib):
    P = lib.swiglu_pack_weights
    assert P(W1_, W2_, WF_, -1, 8, None) == ERR_SHAPE
    assert P(W1_, W2_, WF_, 8, 12, None) == ERR_SHAPE
    assert P(W1_, W2_, WF_, 12, 8, None) == ERR_SHAPE     # K is the packed row length
    assert P(W1_, W2_, WF_, 1, 8, None) == ERR_SHAPE
    assert P(None, W2_, WF_, 8, 8, None) == ERR_NULL
    assert P(W1_, W2_, None, 8, 8, None) == ERR_NULL
    assert P(W1_ + 2, W2_, WF_, 8, 8, None) == ERR_ALIGN
    assert P(W1_, W2_, W1_ + 64, 8, 8, None) == ERR_ALIAS


def test_ablation_validation(lib):
    F = lib.swiglu_unfused_ablation
    ok = dict(A=A_, WF=WF_, G=G_, U=U_, Y=Y_)

    def call(**kw):
        a = {**ok, **kw}
        return F(a["A"], a["WF"], a["G"], a["U"], a["Y"], 256, 256, 256, a.get("WS"),
                 a.get("WSB", 0), None)

    assert call(G=None) == ERR_NULL
    assert call(U=None) == ERR_NULL
    assert call(WF=None) == ERR_NULL
    assert call(G=G_ + 2) == ERR_ALIGN
    assert call(U=G_ + 1024) == ERR_ALIAS        # two outputs overlap
    assert call(Y=U_ + 16) == ERR_ALIAS
    assert call(G=WF_ + 64) == ERR_ALIAS         # output inside an input
    assert call(G=A_ + 64) == ERR_ALIAS
    assert call(WS=U_ + 512, WSB=1 << 20) == ERR_ALIAS
    assert call(WS=WS_ + 8, WSB=1 << 20) == ERR_ALIGN
    assert F(A_, WF_, G_, U_, Y_, 256, 20, 256, None, 0, None) == ERR_SHAPE


def test_workspace_size_validation(lib):
    import ctypes
    out = ctypes.c_uint64(7)
    assert lib.swiglu_workspace_size(256, 256, 256, 2, None) == ERR_NULL
    assert lib.swiglu_workspace_size(256, 20, 256, 2, ctypes.byref(out)) == ERR_SHAPE
    assert out.value == 0
    assert lib.swiglu_workspace_size(256, 256, 256, 5, ctypes.byref(out)) == ERR_UNSUP
    assert lib.swiglu_workspace_size(0, 256, 256, 2, ctypes.byref(out)) == 0 and out.value == 0


def test_describe_launch_validation(lib):
    import ctypes
    buf = ctypes.create_string_buffer(128)
    assert lib.swiglu_describe_launch(256, 256, 256, 2, 0, None, 0) == ERR_NULL
    assert lib.swiglu_describe_launch(256, 256, 256, 5, 0, buf, len(buf)) == ERR_UNSUP
    assert lib.swiglu_describe_launch(256, 20, 256, 2, 0, buf, len(buf)) == ERR_SHAPE
    assert lib.swiglu_describe_launch(0, 256, 256, 2, 0, buf, len(buf)) == 0
    assert buf.value == b"nothing (empty problem)"
    tiny = ctypes.create_string_buffer(8)                 # truncates, stays terminated
    assert lib.swiglu_describe_launch(0, 256, 256, -1, 0, tiny, len(tiny)) == 0
    assert tiny.value == b"nothing"


def test_silu_mul_validation(lib):
    F = lib.swiglu_silu_mul
    assert F(G_, U_, Y_, 12, None) == ERR_SHAPE
    assert F(G_, U_, Y_, -8, None) == ERR_SHAPE
    assert F(None, U_, Y_, 8, None) == ERR_NULL
    assert F(G_, U_ + 2, Y_, 8, None) == ERR_ALIGN
    assert F(G_, U_, G_ + 16, 64, None) == ERR_ALIAS


def test_pack_nk_validation(lib):
    P = lib.swiglu_pack_weights_nk
    assert P(W1_, W2_, WF_, -8, 8, None) == ERR_SHAPE
    assert P(W1_, W2_, WF_, 12, 8, None) == ERR_SHAPE     # K is every row's length
    assert P(W1_, W2_, WF_, 1 << 22, 8, None) == ERR_SHAPE
    assert P(None, None, None, 0, 8, None) == 0           # empty
    assert P(None, None, None, 8, 0, None) == 0
    assert P(None, W2_, WF_, 8, 8, None) == ERR_NULL
    assert P(W1_, W2_ + 8, WF_, 8, 8, None) == ERR_ALIGN
    assert P(W1_, W2_, W2_ + 64, 8, 8, None) == ERR_ALIAS


H_, W3_, O_ = A_ + 0x1_0000_0000, W1_ + 0x1_0000_0000, Y_ + 0x1_0000_0000


def test_down_proj_validation(lib):
    F = lib.swiglu_down_proj

    def call(H=H_, W3=W3_, O=O_, M=256, N=256, D=256, WS=None, WSB=0):
        return F(H, W3, O, M, N, D, WS, WSB, None)

    assert call(M=-1) == ERR_SHAPE
    assert call(N=0) == ERR_SHAPE                        # N is the reduction length
    assert call(N=12) == ERR_SHAPE
    assert call(D=20) == ERR_SHAPE
    assert call(N=1 << 22) == ERR_SHAPE
    assert call(M=0, H=None, W3=None, O=None) == 0      # empty
    assert call(D=0, H=None, W3=None, O=None) == 0
    assert call(W3=None) == ERR_NULL
    assert call(O=O_ + 2) == ERR_ALIGN
    assert call(O=H_ + 64) == ERR_ALIAS
    assert call(O=W3_ + 64) == ERR_ALIAS
    assert call(WS=O_ + 256, WSB=1 << 20) == ERR_ALIAS
    assert call(WS=WS_ + 16, WSB=1 << 20) == ERR_ALIGN


def test_gated_mlp_validation(lib):
    F = lib.swiglu_gated_mlp

    def call(A=A_, WF=WF_, W3=W3_, H=H_, O=O_, M=256, N=256, K=256, v=2, WS=None, WSB=0):
        return F(A, WF, W3, H, O, M, N, K, v, WS, WSB, None)

    assert call(v=7) == ERR_UNSUP
    assert call(K=4) == ERR_SHAPE
    assert call(N=0) == ERR_SHAPE                        # the down projection reduces over N
    assert call(N=20) == ERR_SHAPE
    assert call(M=0, A=None, WF=None, W3=None, H=None, O=None) == 0
    for name in ("A", "WF", "W3", "H", "O"):
        assert call(**{name: None}) == ERR_NULL, name
    assert call(H=H_ + 8) == ERR_ALIGN
    assert call(H=A_ + 64) == ERR_ALIAS                  # intermediate inside an input
    assert call(O=W3_ + 64) == ERR_ALIAS
    assert call(O=H_ + 64) == ERR_ALIAS                  # output overlaps the intermediate
    assert call(WS=H_ + 256, WSB=1 << 20) == ERR_ALIAS
    assert call(WS=WS_ + 16, WSB=1 << 20) == ERR_ALIGN


def test_describe_down_proj_validation(lib):
    import ctypes
    buf = ctypes.create_string_buffer(128)
    assert lib.swiglu_describe_launch(256, 256, 256, -4, 0, buf, len(buf)) == ERR_UNSUP
    assert lib.swiglu_describe_launch(256, 4, 256, -2, 0, buf, len(buf)) == ERR_SHAPE
    assert lib.swiglu_describe_launch(0, 256, 256, -2, 0, buf, len(buf)) == 0
    assert buf.value == b"nothing (empty problem)"


def test_fp8_scale_exp(lib):
    f = sw.swiglu_fp8_scale_exp
    assert f(448.0) == 0 and f(448.1) == 1 and f(224.0) == -1 and f(896.0) == 1
    assert f(5.0) == -6                      # 5 * 64 = 320 <= 448, 5 * 128 > 448
    for amax in (1e-30, 0.37, 3.0, 1000.0, 3e38):
        e = f(amax)
        assert amax * 2.0 ** -e <= 448.0 < amax * 2.0 ** -(e - 1)
    assert f(0.0) == 0 and f(-1.0) == 0 and f(float("nan")) == 0


A8_, W8_ = A_ + 0x2_0000_0000, WF_ + 0x2_0000_0000


def test_fp8_validation(lib):
    Qz = lib.swiglu_quantize_fp8
    assert Qz(G_, U_, 24, 0, None) == ERR_SHAPE          # count % 16
    assert Qz(G_, U_, 32, 127, None) == ERR_SHAPE
    assert Qz(None, None, 0, 0, None) == 0
    assert Qz(None, U_, 32, 0, None) == ERR_NULL
    assert Qz(G_ + 8, U_, 32, 0, None) == ERR_ALIGN
    assert Qz(G_, G_ + 32, 32, 0, None) == ERR_ALIAS
    F = lib.swiglu_fused_gemm_fp8

    def call(A=A8_, W=W8_, Y=Y_, M=256, N=256, K=256, ea=-6, ew=-8, v=2, WS=None, WSB=0):
        return F(A, W, Y, M, N, K, ea, ew, v, WS, WSB, None)

    assert call(v=5) == ERR_UNSUP

    assert call(K=24) == ERR_SHAPE                         # FP8 rows are 16-byte multiples
    assert call(N=12) == ERR_SHAPE
    assert call(ea=100, ew=100) == ERR_SHAPE
    assert call(ea=-127) == ERR_SHAPE
    assert call(M=0, A=None, W=None, Y=None) == 0
    assert call(W=None) == ERR_NULL
    assert call(Y=Y_ + 4) == ERR_ALIGN
    assert call(Y=W8_ + 64) == ERR_ALIAS
    assert call(WS=Y_ + 256, WSB=1 << 20) == ERR_ALIAS
    import ctypes
    buf = ctypes.create_string_buffer(64)
    assert lib.swiglu_describe_launch(0, 256, 256, -3, 0, buf, len(buf)) == 0
    assert lib.swiglu_describe_launch(256, 256, 256, -4, 0, buf, len(buf)) == ERR_UNSUP


def test_strided_validation(lib):
    F = lib.swiglu_fused_gemm_strided

    def call(A=A_, lda=256, W=WF_, Y=Y_, ldy=256, M=256, N=256, K=256, v=2):
        return F(A, lda, W, Y, ldy, M, N, K, v, None, 0, None)

    assert call(lda=248) == ERR_SHAPE                     # lda < K
    assert call(lda=260) == ERR_SHAPE                     # rows not 16-byte aligned
    assert call(lda=1 << 22) == ERR_SHAPE
    assert call(ldy=200) == ERR_SHAPE                     # ldy < N
    assert call(ldy=(1 << 22) + 8) == ERR_SHAPE
    assert call(M=0, A=None, W=None, Y=None) == 0
    assert call(Y=None) == ERR_NULL
    # Y inside A's strided span (rows of A are 4096 elements apart)
    assert call(lda=4096, Y=A_ + 2 * 304) == ERR_ALIAS
    # contiguous call = strided with lda = K, ldy = N: same errors
    assert lib.swiglu_fused_gemm(A_, WF_, A_ + 64, 256, 256, 256, 2, None, 0, None) == ERR_ALIAS


def test_plain_c_client(tmp_path, lib):
    """The header compiles as C11 and a C program links the library and gets
    the documented statuses back (host-only and validation paths: no GPU)."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(sw.LIBRARY)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(root, "include"), os.path.join(root, "tests", "c", "abi_check.c"),
                    "-o", str(exe), "-L", libdir, "-lswiglu", f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stderr


def test_noalloc_validation(lib):
    def f(A=A_, WF=WF_, Y=Y_, M=256, N=256, K=256, v=2):
        return lib.swiglu_fused_gemm_noalloc(A, WF, Y, M, N, K, v, None)

    assert f(M=-1) == ERR_SHAPE
    assert f(K=20) == ERR_SHAPE
    assert f(N=(1 << 22) + 8) == ERR_SHAPE
    assert f(v=3) == ERR_UNSUP
    for v in (0, 1, 2):
        assert f(A=None, v=v) == ERR_NULL
        assert f(WF=None, v=v) == ERR_NULL
        assert f(Y=None, v=v) == ERR_NULL
    assert f(A=A_ + 2) == ERR_ALIGN
    assert f(Y=Y_ + 8) == ERR_ALIGN
    assert f(Y=A_ + 1024) == ERR_ALIAS
    assert f(Y=WF_ + 4096) == ERR_ALIAS
    assert lib.swiglu_fused_gemm_noalloc(None, None, None, 0, 256, 64, 0, None) == 0
    assert lib.swiglu_fused_gemm_noalloc(None, None, None, 64, 0, 64, 2, None) == 0
