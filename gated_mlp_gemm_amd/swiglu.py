"""Python binding of the C ABI in ``include/swiglu.h`` (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libswiglu.so``.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is not built, or a call fails,
an exception is raised.

The functions carry the C names.  Tensors are ``torch.bfloat16``, contiguous,
on one ROCm device; outputs are allocated with torch when not given.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re
from typing import Optional, Tuple

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libswiglu.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "swiglu.h")

SWIGLU_OK = 0
SWIGLU_ERR_NULL = -1
SWIGLU_ERR_SHAPE = -2
SWIGLU_ERR_ALIGN = -3
SWIGLU_ERR_UNSUPPORTED = -4
SWIGLU_ERR_HIP = -5
SWIGLU_ERR_ALIAS = -6

SWIGLU_AUTO = 0
SWIGLU_VARIANT_S = 1
SWIGLU_VARIANT_I = 2
VARIANTS = {"auto": SWIGLU_AUTO, "s": SWIGLU_VARIANT_S, "i": SWIGLU_VARIANT_I}


class SwigluError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {detail} (status {status})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load ``libswiglu.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m gated_mlp_gemm_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.swiglu_pack_weights.argtypes = [P, P, P, I64, I64, P]
    U64 = ctypes.c_uint64
    lib.swiglu_fused_gemm.argtypes = [P, P, P, I64, I64, I64, I32, P, U64, P]
    lib.swiglu_fused_gemm_noalloc.argtypes = [P, P, P, I64, I64, I64, I32, P]
    lib.swiglu_unfused_ablation.argtypes = [P, P, P, P, P, I64, I64, I64, P, U64, P]
    lib.swiglu_fused_gemm_strided.argtypes = [P, I64, P, P, I64, I64, I64, I64, I32, P, U64, P]
    lib.swiglu_workspace_size.argtypes = [I64, I64, I64, I32, ctypes.POINTER(U64)]
    lib.swiglu_describe_launch.argtypes = [I64, I64, I64, I32, U64, ctypes.c_char_p, U64]
    lib.swiglu_silu_mul.argtypes = [P, P, P, I64, P]
    lib.swiglu_pack_weights_nk.argtypes = [P, P, P, I64, I64, P]
    lib.swiglu_down_proj.argtypes = [P, P, P, I64, I64, I64, P, U64, P]
    lib.swiglu_gated_mlp.argtypes = [P, P, P, P, P, I64, I64, I64, I32, P, U64, P]
    lib.swiglu_fp8_scale_exp.argtypes = [ctypes.c_double]
    lib.swiglu_quantize_fp8.argtypes = [P, P, I64, I32, P]
    lib.swiglu_fused_gemm_fp8.argtypes = [P, P, P, I64, I64, I64, I32, I32, I32, P, U64, P]
    lib.swiglu_select_variant.argtypes = [I64, I64, I64]
    lib.swiglu_m_switch.argtypes = []
    lib.swiglu_m_switch.restype = I64
    lib.swiglu_status_string.argtypes = [I32]
    lib.swiglu_status_string.restype = ctypes.c_char_p
    lib.swiglu_last_error.argtypes = []
    lib.swiglu_last_error.restype = ctypes.c_char_p
    for name in ("swiglu_pack_weights", "swiglu_fused_gemm", "swiglu_unfused_ablation",
                 "swiglu_silu_mul", "swiglu_select_variant", "swiglu_workspace_size",
                 "swiglu_describe_launch", "swiglu_pack_weights_nk", "swiglu_down_proj",
                 "swiglu_gated_mlp", "swiglu_fp8_scale_exp", "swiglu_quantize_fp8",
                 "swiglu_fused_gemm_fp8", "swiglu_fused_gemm_strided",
                 "swiglu_fused_gemm_noalloc"):
        getattr(lib, name).restype = I32
    _lib = lib
    return lib


def header_functions(header: str = HEADER):
    """Names of the functions ``include/swiglu.h`` declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swiglu_[a-z_0-9]+)\s*\(", text)))


def _check(status: int, where: str):
    if status != SWIGLU_OK:
        lib = load_library()
        detail = lib.swiglu_last_error().decode() or lib.swiglu_status_string(status).decode()
        raise SwigluError(status, where, detail)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev_tensor(t: torch.Tensor, name: str, shape) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a ROCm device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.shape != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _dev_bytes(t: torch.Tensor, name: str, shape) -> torch.Tensor:
    """A contiguous uint8 device tensor (FP8 E4M3 codes) of the given shape."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must hold FP8 codes as uint8, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a ROCm device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.shape != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


# torch's raw-handle accessor skips building a Stream object on every call
# (about 1.5 us of the host cost of a small call); older builds lack it.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_NO_SWITCH = contextlib.nullcontext()


def _on_device(device):
    """Make `device` current for the call; a no-op when it already is."""
    if device.index is None or device.index == torch.cuda.current_device():
        return _NO_SWITCH
    return torch.cuda.device(device)


def _stream(device) -> int:
    """The handle of torch's current stream on `device`."""
    if _raw_stream is not None:
        idx = torch.cuda.current_device() if device.index is None else device.index
        return _raw_stream(idx)
    return torch.cuda.current_stream(device).cuda_stream


# ---------------------------------------------------------------------------
# C-named entry points
# ---------------------------------------------------------------------------
def swiglu_pack_weights(W1: torch.Tensor, W2: torch.Tensor,
                        W_fused: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Pack W1, W2 [K, N] into W_fused, returned as its [2N, K] storage.

    Row c of the result is column c of the interleaved K x 2N matrix:
    rows 0, 2, 4, ... are the columns of W1 (Gate), rows 1, 3, ... those of W2.
    """
    lib = load_library()
    K, N = W1.shape
    _dev_tensor(W1, "W1", (K, N))
    _dev_tensor(W2, "W2", (K, N))
    if W_fused is None:
        W_fused = torch.empty((2 * N, K), dtype=torch.bfloat16, device=W1.device)
    _dev_tensor(W_fused, "W_fused", (2 * N, K))
    with _on_device(W1.device):
        _check(lib.swiglu_pack_weights(_ptr(W1), _ptr(W2), _ptr(W_fused), K, N,
                                       _stream(W1.device)), "swiglu_pack_weights")
    return W_fused


def swiglu_pack_weights_nk(W1t: torch.Tensor, W2t: torch.Tensor,
                           W_fused: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Pack linear-layer-layout weights W1t, W2t [N, K] (W1, W2 transposed)
    into the same [2N, K] W_fused storage as swiglu_pack_weights."""
    lib = load_library()
    N, K = W1t.shape
    _dev_tensor(W1t, "W1t", (N, K))
    _dev_tensor(W2t, "W2t", (N, K))
    if W_fused is None:
        W_fused = torch.empty((2 * N, K), dtype=torch.bfloat16, device=W1t.device)
    _dev_tensor(W_fused, "W_fused", (2 * N, K))
    with _on_device(W1t.device):
        _check(lib.swiglu_pack_weights_nk(_ptr(W1t), _ptr(W2t), _ptr(W_fused), K, N,
                                          _stream(W1t.device)), "swiglu_pack_weights_nk")
    return W_fused


def _ws(workspace: Optional[torch.Tensor]):
    if workspace is None:
        return None, 0
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


# swiglu_describe_launch / swiglu_workspace_size codes beyond the variants
_CALL_CODES = {"ablation": -1, "down_proj": -2, "fp8": -3}


def _call_code(variant) -> int:
    if isinstance(variant, str):
        v = variant.lower()
        return _CALL_CODES[v] if v in _CALL_CODES else VARIANTS[v]
    return int(variant)


def swiglu_workspace_size(M: int, N: int, K: int, variant="auto") -> int:
    """Bytes of scratch that let a call split the tail round ('ablation' for the
    ablation; the down projection and the gated MLP use the ablation's size)."""
    v = _call_code(variant)
    if v == -2:
        v = -1
    elif v == -3:
        v = SWIGLU_VARIANT_I   # the FP8 call uses variant I's workspace
    out = ctypes.c_uint64(0)
    _check(load_library().swiglu_workspace_size(M, N, K, v, ctypes.byref(out)),
           "swiglu_workspace_size")
    return int(out.value)


def swiglu_describe_launch(M: int, N: int, K: int, variant="auto",
                           workspace_bytes: int = 0) -> str:
    """The kernels a call would launch ('ablation' for the unfused pipeline,
    'down_proj' for the gated MLP's down projection over (M, N, K))."""
    v = _call_code(variant)
    buf = ctypes.create_string_buffer(512)
    _check(load_library().swiglu_describe_launch(M, N, K, v, workspace_bytes, buf, len(buf)),
           "swiglu_describe_launch")
    return buf.value.decode()


def make_workspace(M: int, N: int, K: int, variant="auto", device="cuda") -> Optional[torch.Tensor]:
    """A device scratch tensor of swiglu_workspace_size() bytes (None if 0);
    needs no initialisation and may be reused by later stream-ordered calls."""
    n = swiglu_workspace_size(M, N, K, variant)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def swiglu_fused_gemm(A: torch.Tensor, W_fused: torch.Tensor,
                      Y: Optional[torch.Tensor] = None, variant="auto",
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = bf16(SiLU(A.W1) * (A.W2)) from the packed weight; variant 'auto' | 's' | 'i'."""
    lib = load_library()
    v = VARIANTS[variant.lower()] if isinstance(variant, str) else int(variant)
    M, K = A.shape
    _dev_tensor(A, "A", (M, K))
    N = W_fused.shape[0] // 2
    _dev_tensor(W_fused, "W_fused", (2 * N, K))
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _dev_tensor(Y, "Y", (M, N))
    with _on_device(A.device):
        ws, wsb = _ws(workspace)
        _check(lib.swiglu_fused_gemm(_ptr(A), _ptr(W_fused), _ptr(Y), M, N, K, v, ws, wsb,
                                     _stream(A.device)), "swiglu_fused_gemm")
    return Y


def swiglu_fused_gemm_noalloc(A: torch.Tensor, W_fused: torch.Tensor, Y: torch.Tensor,
                              variant="auto") -> torch.Tensor:
    """swiglu_fused_gemm with the library's static split-tail scratch: the C
    call allocates nothing (Y must be given, so the binding allocates nothing
    either).  Calls that may overlap on one device race on that scratch."""
    lib = load_library()
    v = VARIANTS[variant.lower()] if isinstance(variant, str) else int(variant)
    M, K = A.shape
    _dev_tensor(A, "A", (M, K))
    N = W_fused.shape[0] // 2
    _dev_tensor(W_fused, "W_fused", (2 * N, K))
    _dev_tensor(Y, "Y", (M, N))
    with _on_device(A.device):
        _check(lib.swiglu_fused_gemm_noalloc(_ptr(A), _ptr(W_fused), _ptr(Y), M, N, K, v,
                                             _stream(A.device)), "swiglu_fused_gemm_noalloc")
    return Y


def _dev_rows(t: torch.Tensor, name: str, shape) -> int:
    """A bf16 device matrix whose rows are contiguous (stride 1 along a row);
    returns the row pitch in elements."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a ROCm device, got {t.device}")
    if t.dim() != 2 or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name} must have contiguous rows")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def swiglu_fused_gemm_strided(A: torch.Tensor, W_fused: torch.Tensor, Y: torch.Tensor,
                              variant="auto",
                              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """swiglu_fused_gemm on row-strided views: A [M, K] and Y [M, N] may be
    column slices of wider tensors (their row strides are passed as lda / ldy)."""
    lib = load_library()
    v = VARIANTS[variant.lower()] if isinstance(variant, str) else int(variant)
    M, K = A.shape
    N = W_fused.shape[0] // 2
    lda = _dev_rows(A, "A", (M, K))
    ldy = _dev_rows(Y, "Y", (M, N))
    _dev_tensor(W_fused, "W_fused", (2 * N, K))
    with _on_device(A.device):
        ws, wsb = _ws(workspace)
        _check(lib.swiglu_fused_gemm_strided(_ptr(A), lda, _ptr(W_fused), _ptr(Y), ldy, M, N, K,
                                             v, ws, wsb, _stream(A.device)),
               "swiglu_fused_gemm_strided")
    return Y


def swiglu_unfused_ablation(A: torch.Tensor, W_fused: torch.Tensor,
                            gate_ws: Optional[torch.Tensor] = None,
                            up_ws: Optional[torch.Tensor] = None,
                            Y: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None
                            ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Two GEMMs + SiLU-mul from the packed weight; returns (Y, gate_ws, up_ws)."""
    lib = load_library()
    M, K = A.shape
    N = W_fused.shape[0] // 2
    _dev_tensor(A, "A", (M, K))
    _dev_tensor(W_fused, "W_fused", (2 * N, K))
    outs = []
    for name, t in (("gate_ws", gate_ws), ("up_ws", up_ws), ("Y", Y)):
        if t is None:
            t = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
        outs.append(_dev_tensor(t, name, (M, N)))
    gate_ws, up_ws, Y = outs
    with _on_device(A.device):
        ws, wsb = _ws(workspace)
        _check(lib.swiglu_unfused_ablation(_ptr(A), _ptr(W_fused), _ptr(gate_ws), _ptr(up_ws),
                                           _ptr(Y), M, N, K, ws, wsb, _stream(A.device)),
               "swiglu_unfused_ablation")
    return Y, gate_ws, up_ws


def swiglu_down_proj(H: torch.Tensor, W3t: torch.Tensor, Out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Out [M, D] = bf16(H . W3) for H [M, N] and W3t = W3^T stored [D, N]."""
    lib = load_library()
    M, N = H.shape
    D = W3t.shape[0]
    _dev_tensor(H, "H", (M, N))
    _dev_tensor(W3t, "W3t", (D, N))
    if Out is None:
        Out = torch.empty((M, D), dtype=torch.bfloat16, device=H.device)
    _dev_tensor(Out, "Out", (M, D))
    with _on_device(H.device):
        ws, wsb = _ws(workspace)
        _check(lib.swiglu_down_proj(_ptr(H), _ptr(W3t), _ptr(Out), M, N, D, ws, wsb,
                                    _stream(H.device)), "swiglu_down_proj")
    return Out


def swiglu_gated_mlp(A: torch.Tensor, W_fused: torch.Tensor, W3t: torch.Tensor,
                     H: Optional[torch.Tensor] = None, Out: Optional[torch.Tensor] = None,
                     variant="auto", workspace: Optional[torch.Tensor] = None
                     ) -> Tuple[torch.Tensor, torch.Tensor]:
    """The gated MLP block: H = fused SwiGLU GEMM, Out = bf16(H . W3); returns (Out, H)."""
    lib = load_library()
    v = VARIANTS[variant.lower()] if isinstance(variant, str) else int(variant)
    M, K = A.shape
    N = W_fused.shape[0] // 2
    _dev_tensor(A, "A", (M, K))
    _dev_tensor(W_fused, "W_fused", (2 * N, K))
    _dev_tensor(W3t, "W3t", (K, N))
    if H is None:
        H = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    if Out is None:
        Out = torch.empty((M, K), dtype=torch.bfloat16, device=A.device)
    _dev_tensor(H, "H", (M, N))
    _dev_tensor(Out, "Out", (M, K))
    with _on_device(A.device):
        ws, wsb = _ws(workspace)
        _check(lib.swiglu_gated_mlp(_ptr(A), _ptr(W_fused), _ptr(W3t), _ptr(H), _ptr(Out),
                                    M, N, K, v, ws, wsb, _stream(A.device)), "swiglu_gated_mlp")
    return Out, H


def swiglu_silu_mul(gate: torch.Tensor, up: torch.Tensor,
                    Y: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = load_library()
    _dev_tensor(gate, "gate", gate.shape)
    _dev_tensor(up, "up", gate.shape)
    if Y is None:
        Y = torch.empty_like(gate)
    _dev_tensor(Y, "Y", gate.shape)
    with _on_device(gate.device):
        _check(lib.swiglu_silu_mul(_ptr(gate), _ptr(up), _ptr(Y), gate.numel(),
                                   _stream(gate.device)), "swiglu_silu_mul")
    return Y


def swiglu_fp8_scale_exp(amax: float) -> int:
    """Smallest e with amax * 2^-e <= 448 (the largest E4M3 value)."""
    return int(load_library().swiglu_fp8_scale_exp(float(amax)))


def swiglu_quantize_fp8(X: torch.Tensor, scale_exp: int,
                        Q: Optional[torch.Tensor] = None) -> torch.Tensor:
    """E4M3 codes of X * 2^-scale_exp (uint8, the shape of X)."""
    lib = load_library()
    _dev_tensor(X, "X", X.shape)
    if Q is None:
        Q = torch.empty(X.shape, dtype=torch.uint8, device=X.device)
    _dev_bytes(Q, "Q", X.shape)
    with _on_device(X.device):
        _check(lib.swiglu_quantize_fp8(_ptr(X), _ptr(Q), X.numel(), int(scale_exp),
                                       _stream(X.device)), "swiglu_quantize_fp8")
    return Q


def swiglu_fused_gemm_fp8(A8: torch.Tensor, W_fused8: torch.Tensor, a_exp: int, w_exp: int,
                          Y: Optional[torch.Tensor] = None, variant="auto",
                          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = bf16(SiLU(2^(a+w) A8.W1_8) * (2^(a+w) A8.W2_8)) on FP8 codes (A8 [M, K],
    W_fused8 [2N, K], both uint8); variant 'auto' | 's' | 'i'."""
    lib = load_library()
    v = VARIANTS[variant.lower()] if isinstance(variant, str) else int(variant)
    M, K = A8.shape
    N = W_fused8.shape[0] // 2
    _dev_bytes(A8, "A8", (M, K))
    _dev_bytes(W_fused8, "W_fused8", (2 * N, K))
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=A8.device)
    _dev_tensor(Y, "Y", (M, N))
    with _on_device(A8.device):
        ws, wsb = _ws(workspace)
        _check(lib.swiglu_fused_gemm_fp8(_ptr(A8), _ptr(W_fused8), _ptr(Y), M, N, K, int(a_exp),
                                         int(w_exp), v, ws, wsb, _stream(A8.device)),
               "swiglu_fused_gemm_fp8")
    return Y


def swiglu_select_variant(M: int, N: int = 0, K: int = 0) -> int:
    v = load_library().swiglu_select_variant(M, N, K)
    if v < 0:
        _check(v, "swiglu_select_variant")
    return v


def swiglu_m_switch() -> int:
    return int(load_library().swiglu_m_switch())


def swiglu_status_string(status: int) -> str:
    return load_library().swiglu_status_string(status).decode()


def swiglu_last_error() -> str:
    return load_library().swiglu_last_error().decode()
