"""CPU oracle for Y = SiLU(A.W1) (.) (A.W2) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never links, loads or
calls it, and it uses nothing from the HIP library: the only thing the two
share is the seeded input generator, which holds none of the method's
arithmetic.

The arithmetic lives in ``swiglu_oracle.c`` (plain C, double precision, k
ascending, one final round-to-nearest-even to bf16); its header states the
definition it follows and cites the pages.  This module builds that file with
gcc and exposes it over ctypes for numpy ``uint16`` arrays holding bf16 bit
patterns.

``build(defines=...)`` can also compile planted-mistake variants (``PLANT_*``
macros) so the tests can show that every pin catches a plausible slip.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Iterable, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "swiglu_oracle.c")
LIBRARY = os.path.join(_HERE, "libswiglu_oracle.so")

_U16P = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_F64P = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_I64P = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")


def build(out: str = LIBRARY, defines: Iterable[str] = ()) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-std=c11", "-O3", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off"]
    cmd += [f"-D{d}" for d in defines]
    tmp = out + ".tmp"
    cmd += [SOURCE, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _nullable(ptr_type):
    """ctypes argtype that accepts a numpy array or None (NULL)."""
    class _Nullable:
        @classmethod
        def from_param(cls, obj):
            if obj is None:
                return ctypes.c_void_p(None)
            return ptr_type.from_param(obj)
    return _Nullable


class Oracle:
    """Thin typed wrapper over one build of ``swiglu_oracle.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64 = ctypes.c_int64
        nf64 = _nullable(_F64P)
        nu16 = _nullable(_U16P)
        lib.swo_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.swo_bf16_to_double.restype = ctypes.c_double
        lib.swo_double_to_bf16.argtypes = [ctypes.c_double]
        lib.swo_double_to_bf16.restype = ctypes.c_uint16
        lib.swo_silu.argtypes = [ctypes.c_double]
        lib.swo_silu.restype = ctypes.c_double
        lib.swo_matmul.argtypes = [_U16P, _U16P, i64, i64, i64, _F64P]
        lib.swo_swiglu_rows.argtypes = [_U16P, _U16P, _U16P, i64, i64,
                                        _nullable(_I64P), i64, nf64, nu16]
        lib.swo_swiglu_separate.argtypes = [_U16P, _U16P, _U16P, i64, i64,
                                            i64, nf64, nu16]
        lib.swo_swiglu_interleaved.argtypes = [_U16P, _U16P, i64, i64, i64,
                                               nf64, nu16]
        lib.swo_swiglu_block.argtypes = [_U16P, _U16P, _U16P, i64, i64, _I64P, i64,
                                         i64, i64, nf64, nu16]
        lib.swo_swiglu_points.argtypes = [_U16P, _U16P, _U16P, i64, i64,
                                          _I64P, _I64P, i64, nf64, nu16]
        lib.swo_pack.argtypes = [_U16P, _U16P, _U16P, i64, i64]
        lib.swo_swiglu_materialised.argtypes = [_U16P, _U16P, _U16P, i64,
                                                i64, i64, nu16, nu16, nu16]
        lib.swo_silu_mul.argtypes = [_U16P, _U16P, i64, _U16P]
        lib.swo_pack_nk.argtypes = [_U16P, _U16P, _U16P, i64, i64]
        lib.swo_down_proj.argtypes = [_U16P, _U16P, i64, i64, i64, nf64, _U16P]
        lib.swo_gated_mlp.argtypes = [_U16P, _U16P, _U16P, _U16P, i64, i64,
                                      i64, _U16P, _U16P]
        _U8P = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
        lib.swo_fp8_to_double.argtypes = [ctypes.c_uint8]
        lib.swo_fp8_to_double.restype = ctypes.c_double
        lib.swo_double_to_fp8.argtypes = [ctypes.c_double]
        lib.swo_double_to_fp8.restype = ctypes.c_uint8
        lib.swo_quantize_fp8.argtypes = [_U16P, i64, ctypes.c_int, _U8P]
        lib.swo_swiglu_fp8_rows.argtypes = [_U8P, _U8P, i64, i64, _nullable(_I64P), i64,
                                            ctypes.c_int, ctypes.c_int, nf64, nu16]
        lib.swo_num_threads.restype = ctypes.c_int
        self._lib = lib
        self.path = path

    # -- scalars ---------------------------------------------------------
    def bf16_to_double(self, bits: int) -> float:
        return self._lib.swo_bf16_to_double(int(bits))

    def double_to_bf16(self, x: float) -> int:
        return int(self._lib.swo_double_to_bf16(float(x)))

    def silu(self, x: float) -> float:
        return self._lib.swo_silu(float(x))

    def num_threads(self) -> int:
        return int(self._lib.swo_num_threads())

    # -- arrays (bf16 bit patterns as uint16) -----------------------------
    @staticmethod
    def _u16(x):
        x = np.ascontiguousarray(x)
        if x.dtype != np.uint16:
            raise TypeError(f"expected uint16 bf16 bit patterns, got {x.dtype}")
        return x

    def matmul(self, A, B):
        """D = A.B in double (k ascending); A [M,K], B [K,C] bf16 patterns."""
        A, B = self._u16(A), self._u16(B)
        M, K = A.shape
        K2, C = B.shape
        assert K == K2
        D = np.empty((M, C), dtype=np.float64)
        self._lib.swo_matmul(A, B, M, K, C, D)
        return D

    def swiglu(self, A, W1, W2, want_f64: bool = False):
        """Separate formulation; returns Y bf16 patterns [M,N] (and y64)."""
        A, W1, W2 = self._u16(A), self._u16(W1), self._u16(W2)
        M, K = A.shape
        N = W1.shape[1]
        assert W1.shape == (K, N) and W2.shape == (K, N)
        y = np.empty((M, N), dtype=np.uint16)
        y64 = np.empty((M, N), dtype=np.float64) if want_f64 else None
        self._lib.swo_swiglu_separate(A, W1, W2, M, N, K, y64, y)
        return (y, y64) if want_f64 else y

    def swiglu_rows(self, A, W1, W2, rows, want_f64: bool = False):
        """Full output rows for a subset of row indices."""
        A, W1, W2 = self._u16(A), self._u16(W1), self._u16(W2)
        K = A.shape[1]
        N = W1.shape[1]
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < A.shape[0])
        y = np.empty((rows.size, N), dtype=np.uint16)
        y64 = np.empty((rows.size, N), dtype=np.float64) if want_f64 else None
        self._lib.swo_swiglu_rows(A, W1, W2, N, K, rows, rows.size, y64, y)
        return (y, y64) if want_f64 else y

    def swiglu_block(self, A, W1, W2, rows, c0: int, c1: int, want_f64: bool = False):
        """Outputs Y[rows, c0:c1] (a column window of whole rows)."""
        A, W1, W2 = self._u16(A), self._u16(W1), self._u16(W2)
        K = A.shape[1]
        N = W1.shape[1]
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < A.shape[0])
        assert 0 <= c0 <= c1 <= N
        y = np.empty((rows.size, c1 - c0), dtype=np.uint16)
        y64 = np.empty((rows.size, c1 - c0), dtype=np.float64) if want_f64 else None
        if rows.size and c1 > c0:
            self._lib.swo_swiglu_block(A, W1, W2, N, K, rows, rows.size, c0, c1, y64, y)
        return (y, y64) if want_f64 else y

    def swiglu_interleaved(self, A, Wf, want_f64: bool = False):
        """Interleaved formulation over W_fused [K, 2N]."""
        A, Wf = self._u16(A), self._u16(Wf)
        M, K = A.shape
        assert Wf.shape[0] == K and Wf.shape[1] % 2 == 0
        N = Wf.shape[1] // 2
        y = np.empty((M, N), dtype=np.uint16)
        y64 = np.empty((M, N), dtype=np.float64) if want_f64 else None
        self._lib.swo_swiglu_interleaved(A, Wf, M, N, K, y64, y)
        return (y, y64) if want_f64 else y

    def swiglu_points(self, A, W1, W2, rows, cols, want_f64: bool = False):
        """Single outputs Y[rows[i], cols[i]], each computed on its own."""
        A, W1, W2 = self._u16(A), self._u16(W1), self._u16(W2)
        K = A.shape[1]
        N = W1.shape[1]
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        assert rows.shape == cols.shape
        if rows.size:
            assert rows.min() >= 0 and rows.max() < A.shape[0]
            assert cols.min() >= 0 and cols.max() < N
        y = np.empty(rows.size, dtype=np.uint16)
        y64 = np.empty(rows.size, dtype=np.float64) if want_f64 else None
        self._lib.swo_swiglu_points(A, W1, W2, N, K, rows, cols, rows.size,
                                    y64, y)
        return (y, y64) if want_f64 else y

    def pack(self, W1, W2):
        W1, W2 = self._u16(W1), self._u16(W2)
        K, N = W1.shape
        assert W2.shape == (K, N)
        Wf = np.empty((K, 2 * N), dtype=np.uint16)
        self._lib.swo_pack(W1, W2, Wf, K, N)
        return Wf

    def pack_nk(self, W1t, W2t):
        """W_fused [K, 2N] from linear-layer weights W1t, W2t [N, K]."""
        W1t, W2t = self._u16(W1t), self._u16(W2t)
        N, K = W1t.shape
        assert W2t.shape == (N, K)
        Wf = np.empty((K, 2 * N), dtype=np.uint16)
        self._lib.swo_pack_nk(W1t, W2t, Wf, K, N)
        return Wf

    def down_proj(self, H, W3, want_f64: bool = False):
        """Out = bf16(H . W3); H [M, N], W3 [N, D]; returns [M, D] (and o64)."""
        H, W3 = self._u16(H), self._u16(W3)
        M, N = H.shape
        N2, D = W3.shape
        assert N == N2
        out = np.empty((M, D), dtype=np.uint16)
        o64 = np.empty((M, D), dtype=np.float64) if want_f64 else None
        self._lib.swo_down_proj(H, W3, M, N, D, o64, out)
        return (out, o64) if want_f64 else out

    def gated_mlp(self, A, W1, W2, W3):
        """MLP block: returns (H [M, N], Out [M, K]) bf16 patterns."""
        A, W1, W2, W3 = (self._u16(x) for x in (A, W1, W2, W3))
        M, K = A.shape
        N = W1.shape[1]
        assert W1.shape == (K, N) and W2.shape == (K, N) and W3.shape == (N, K)
        h = np.empty((M, N), dtype=np.uint16)
        out = np.empty((M, K), dtype=np.uint16)
        self._lib.swo_gated_mlp(A, W1, W2, W3, M, N, K, h, out)
        return h, out

    # -- FP8 (E4M3) inputs ------------------------------------------------
    def fp8_to_double(self, code: int) -> float:
        return self._lib.swo_fp8_to_double(int(code))

    def double_to_fp8(self, x: float) -> int:
        return int(self._lib.swo_double_to_fp8(float(x)))

    def quantize_fp8(self, x, scale_exp: int):
        """fp8(x * 2^-scale_exp) codes (uint8) for bf16 patterns x."""
        x = self._u16(x)
        q = np.empty(x.shape, dtype=np.uint8)
        self._lib.swo_quantize_fp8(x.reshape(-1), x.size, int(scale_exp), q.reshape(-1))
        return q

    def swiglu_fp8(self, A8, WfT8, a_exp: int, w_exp: int, rows=None,
                   want_f64: bool = False):
        """Fused SwiGLU on FP8 codes: A8 [M,K] uint8, WfT8 [2N,K] uint8
        (W_fused stored by columns); all rows, or the listed ones."""
        A8 = np.ascontiguousarray(A8, dtype=np.uint8)
        WfT8 = np.ascontiguousarray(WfT8, dtype=np.uint8)
        M, K = A8.shape
        assert WfT8.shape[1] == K and WfT8.shape[0] % 2 == 0
        N = WfT8.shape[0] // 2
        if rows is None:
            rws, n = None, M
        else:
            rws = np.ascontiguousarray(rows, dtype=np.int64)
            assert rws.size == 0 or (rws.min() >= 0 and rws.max() < M)
            n = rws.size
        y = np.empty((n, N), dtype=np.uint16)
        y64 = np.empty((n, N), dtype=np.float64) if want_f64 else None
        self._lib.swo_swiglu_fp8_rows(A8, WfT8, N, K, rws, n, int(a_exp), int(w_exp), y64, y)
        return (y, y64) if want_f64 else y

    def swiglu_materialised(self, A, W1, W2):
        """Unfused pipeline: returns (gate_bf16, up_bf16, y_bf16)."""
        A, W1, W2 = self._u16(A), self._u16(W1), self._u16(W2)
        M, K = A.shape
        N = W1.shape[1]
        g = np.empty((M, N), dtype=np.uint16)
        u = np.empty((M, N), dtype=np.uint16)
        y = np.empty((M, N), dtype=np.uint16)
        self._lib.swo_swiglu_materialised(A, W1, W2, M, N, K, g, u, y)
        return g, u, y

    def silu_mul(self, g, u):
        g, u = self._u16(g), self._u16(u)
        assert g.shape == u.shape
        y = np.empty(g.shape, dtype=np.uint16)
        self._lib.swo_silu_mul(g.reshape(-1), u.reshape(-1), g.size,
                               y.reshape(-1))
        return y


_default: Optional[Oracle] = None


def load(path: Optional[str] = None) -> Oracle:
    """Load the oracle library, compiling it first if it is not built."""
    global _default
    if path is not None:
        return Oracle(path)
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default


# ---------------------------------------------------------------------------
# Comparison predicate (pure host logic, no method arithmetic).
# An element mismatches iff |y - ref| > max(atol, rtol * |ref|): the pages'
# criterion is "relative error above 1 % against an FP32 reference"
# [gist: Core contributions; abstract: zero mismatches]; the absolute floor
# 1e-3 covers outputs near zero, where a relative bound is meaningless.
# ---------------------------------------------------------------------------
RTOL = 1e-2
ATOL = 1e-3


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 patterns (uint16) to float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def mismatches(y_bits, ref_bits, rtol: float = RTOL, atol: float = ATOL):
    """Boolean mask of elements outside max(atol, rtol*|ref|).

    NaN in either operand counts as a mismatch; -0 equals +0.
    """
    y = bf16_bits_to_f64(y_bits)
    r = bf16_bits_to_f64(ref_bits)
    err = np.abs(y - r)
    bound = np.maximum(atol, rtol * np.abs(r))
    bad = ~(err <= bound)
    return bad


def parity_report(y_bits, ref_bits, rtol: float = RTOL, atol: float = ATOL):
    """Mismatch count, max relative error where |ref| > 0.1, max abs error."""
    bad = mismatches(y_bits, ref_bits, rtol, atol)
    y = bf16_bits_to_f64(y_bits)
    r = bf16_bits_to_f64(ref_bits)
    err = np.abs(y - r)
    big = np.abs(r) > 0.1
    max_rel = float((err[big] / np.abs(r[big])).max()) if big.any() else 0.0
    return {
        "count": int(np.asarray(y_bits).size),
        "mismatches": int(bad.sum()),
        "max_rel_err": max_rel,
        "max_abs_err": float(err.max()) if err.size else 0.0,
    }
