"""EQ-Linear (group-circulant linear layer over the cyclic group C_T) on MI355X.

The layer's weight is one set of shared parameters w[D', C', T] replicated under
cyclic shifts, W[d*T+g, c*T+h] = w[d, c, (g-h) mod T] ("Insight Central" in
"Resumo Tecnico: Flash EQ-Linear"); it is evaluated exactly by a group-axis DFT,
per-frequency channel GEMMs on the half spectrum and the inverse DFT, all in
hand-written HIP kernels for gfx950 behind the C ABI in include/eqlinear.h.

This module is the thin ctypes binding of that ABI: one Python function per C
entry point, with the same name and argument order.  Buffers may be given as
torch tensors on a ROCm device or as raw device addresses (int); `stream` as a
torch.cuda.Stream, a raw hipStream_t (int) or None for torch's current stream.
A non-zero status raises EqlError.  No computation happens in Python, and there
is no fallback: if libeqlinear.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "EQL_F32", "EQL_F16", "EQL_PACK_FWD", "EQL_PACK_BWDX", "EQL_ACT_NONE", "EQL_ACT_GELU", "EQL_MAX_T",
    "EqlError",
    "lib", "library_path", "eqlinear_abi_version", "eqlinear_status_string",
    "eqlinear_packed_weight_bytes", "eqlinear_pack_weight", "eqlinear_pack_weight_both", "eqlinear_fwd", "eqlinear_fwd_fused", "eqlinear_bwd_x",
    "eqlinear_fused_epilogue_bwd_workspace_bytes", "eqlinear_fused_epilogue_bwd",
    "eqlinear_fused_epilogue_bwd_noalloc", "EQL_NOALLOC_SCRATCH_BYTES",
    "eqlinear_bwd_w_workspace_bytes", "eqlinear_bwd_w",
    "eqlinear_fwd_train", "eqlinear_fwd_fused_train", "eqlinear_bwd_x_train", "eqlinear_bwd_w_train",
    "eqlinear_p4m_expand_weight", "eqlinear_p4m_fold_weight_grad",
]

EQL_F32, EQL_F16 = 0, 1
EQL_PACK_FWD, EQL_PACK_BWDX = 0, 1
EQL_ACT_NONE, EQL_ACT_GELU = 0, 1
EQL_MAX_T = 16
EQL_OK, EQL_EINVAL, EQL_EALIGN, EQL_EUNSUPPORTED, EQL_EHIP, EQL_ESCRATCH = 0, 1, 2, 3, 4, 5
EQL_NOALLOC_SCRATCH_BYTES = 16 << 20

_PKG = os.path.dirname(os.path.abspath(__file__))
# EQL_LIBRARY names another build of the same library (for instance the NaN-poisoned
# debug build, libeqlinear_poison.so); by default the in-tree libeqlinear.so.
_LIB_PATH = os.environ.get("EQL_LIBRARY") or os.path.join(_PKG, "libeqlinear.so")
_lib = None


class EqlError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, eqlinear_status_string(status), status))


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libeqlinear.so (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libeqlinear.so is not built (run `python -m group_circulant_linear_p4_amd.build`); "
                              "there is no fallback implementation")
        L = ctypes.CDLL(_LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        L.eqlinear_abi_version.argtypes, L.eqlinear_abi_version.restype = [], i32
        L.eqlinear_status_string.argtypes, L.eqlinear_status_string.restype = [i32], ctypes.c_char_p
        L.eqlinear_packed_weight_bytes.argtypes = [i64, i64, i32, i32]
        L.eqlinear_packed_weight_bytes.restype = sz
        L.eqlinear_pack_weight.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp]
        L.eqlinear_pack_weight.restype = i32
        L.eqlinear_pack_weight_both.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp]
        L.eqlinear_pack_weight_both.restype = i32
        L.eqlinear_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i32, i32, vp]
        L.eqlinear_fwd.restype = i32
        L.eqlinear_fwd_fused.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp]
        L.eqlinear_fwd_fused.restype = i32
        L.eqlinear_fused_epilogue_bwd_workspace_bytes.argtypes = [i64, i64, i32, i32]
        L.eqlinear_fused_epilogue_bwd_workspace_bytes.restype = sz
        L.eqlinear_fused_epilogue_bwd.argtypes = [vp, vp, vp, vp, vp, sz, i64, i64, i32, i32, i32, vp]
        L.eqlinear_fused_epilogue_bwd.restype = i32
        L.eqlinear_fused_epilogue_bwd_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, vp]
        L.eqlinear_fused_epilogue_bwd_noalloc.restype = i32
        for name in ("eqlinear_p4m_expand_weight", "eqlinear_p4m_fold_weight_grad"):
            getattr(L, name).argtypes = [vp, vp, i64, i64, i32, vp]
            getattr(L, name).restype = i32
        L.eqlinear_bwd_x.argtypes = [vp, vp, vp, i64, i64, i64, i32, i32, vp]
        L.eqlinear_bwd_x.restype = i32
        L.eqlinear_bwd_w_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
        L.eqlinear_bwd_w_workspace_bytes.restype = sz
        L.eqlinear_bwd_w.argtypes = [vp, vp, vp, vp, sz, i64, i64, i64, i32, i32, vp]
        L.eqlinear_bwd_w.restype = i32
        for name in ("eqlinear_fwd_train", "eqlinear_bwd_x_train"):
            getattr(L, name).argtypes = [vp, vp, vp, vp, sz, i64, i64, i64, i32, i32, vp]
            getattr(L, name).restype = i32
        L.eqlinear_fwd_fused_train.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i32, i32, i32, vp]
        L.eqlinear_fwd_fused_train.restype = i32
        L.eqlinear_bwd_w_train.argtypes = [vp, vp, vp, sz, i64, i64, i64, i32, i32, vp]
        L.eqlinear_bwd_w_train.restype = i32
        _lib = L
    return _lib


def _ptr(buf):
    if buf is None:
        return None
    if isinstance(buf, int):
        return buf or None
    data_ptr = getattr(buf, "data_ptr", None)
    if data_ptr is None:
        raise TypeError("expected a device tensor or an int address, got %r" % type(buf))
    if not buf.is_cuda:
        raise ValueError("EQ-Linear buffers must live in GPU memory (got a %s tensor)" % buf.device)
    if not buf.is_contiguous():
        raise ValueError("EQ-Linear buffers must be contiguous")
    return data_ptr() or None


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return getattr(stream, "cuda_stream", stream) or None


def _dtype(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    import torch
    if dtype == torch.float16:
        return EQL_F16
    if dtype == torch.float32:
        return EQL_F32
    raise ValueError("unsupported dtype %r (fp16 or fp32)" % (dtype,))


def _check(status: int, where: str) -> None:
    if status != EQL_OK:
        raise EqlError(status, where)


def eqlinear_abi_version() -> int:
    return lib().eqlinear_abi_version()


def eqlinear_status_string(status: int) -> str:
    return lib().eqlinear_status_string(int(status)).decode()


def eqlinear_packed_weight_bytes(out_ch: int, in_ch: int, T: int, dtype) -> int:
    return lib().eqlinear_packed_weight_bytes(out_ch, in_ch, T, _dtype(dtype))


def eqlinear_pack_weight(w, w_packed, Dp: int, Cp: int, T: int, dtype, mode: int, stream=None) -> None:
    _check(lib().eqlinear_pack_weight(_ptr(w), _ptr(w_packed), Dp, Cp, T, _dtype(dtype), mode, _stream(stream)),
           "eqlinear_pack_weight")


def eqlinear_pack_weight_both(w, w_packed, w_packed_bwdx, Dp: int, Cp: int, T: int, dtype, stream=None) -> None:
    """Both packings (forward and input-gradient) in one launch."""
    _check(lib().eqlinear_pack_weight_both(_ptr(w), _ptr(w_packed), _ptr(w_packed_bwdx), Dp, Cp, T, _dtype(dtype),
                                           _stream(stream)), "eqlinear_pack_weight_both")


def eqlinear_fwd(x, w_packed, y, N: int, Cp: int, Dp: int, T: int, dtype, stream=None) -> None:
    _check(lib().eqlinear_fwd(_ptr(x), _ptr(w_packed), _ptr(y), N, Cp, Dp, T, _dtype(dtype), _stream(stream)),
           "eqlinear_fwd")


def eqlinear_fwd_fused(x, w_packed, bias, residual, y, pre_out, N: int, Cp: int, Dp: int, T: int, dtype,
                       act: int, stream=None) -> None:
    """bias / residual / pre_out may be None; residual may be y itself."""
    _check(lib().eqlinear_fwd_fused(_ptr(x), _ptr(w_packed), _ptr(bias), _ptr(residual), _ptr(y), _ptr(pre_out),
                                    N, Cp, Dp, T, _dtype(dtype), int(act), _stream(stream)), "eqlinear_fwd_fused")


def eqlinear_fused_epilogue_bwd_workspace_bytes(N: int, Dp: int, T: int, dtype) -> int:
    return lib().eqlinear_fused_epilogue_bwd_workspace_bytes(N, Dp, T, _dtype(dtype))


def eqlinear_fused_epilogue_bwd(dy, pre, dpre, dbias, workspace, ws_bytes: int, N: int, Dp: int, T: int, dtype,
                                act: int, stream=None) -> None:
    """pre may be None without an activation, dbias may be None, dpre may be dy."""
    _check(lib().eqlinear_fused_epilogue_bwd(_ptr(dy), _ptr(pre), _ptr(dpre), _ptr(dbias), _ptr(workspace),
                                             int(ws_bytes), N, Dp, T, _dtype(dtype), int(act), _stream(stream)),
           "eqlinear_fused_epilogue_bwd")


def eqlinear_fused_epilogue_bwd_noalloc(dy, pre, dpre, dbias, N: int, Dp: int, T: int, dtype, act: int,
                                        stream=None) -> None:
    """eqlinear_fused_epilogue_bwd with the library's static per-device scratch in place of a
    workspace (no allocation; overlapping calls on one device race)."""
    _check(lib().eqlinear_fused_epilogue_bwd_noalloc(_ptr(dy), _ptr(pre), _ptr(dpre), _ptr(dbias), N, Dp, T,
                                                     _dtype(dtype), int(act), _stream(stream)),
           "eqlinear_fused_epilogue_bwd_noalloc")


def eqlinear_bwd_x(dy, w_packed_bwdx, dx, N: int, Cp: int, Dp: int, T: int, dtype, stream=None) -> None:
    _check(lib().eqlinear_bwd_x(_ptr(dy), _ptr(w_packed_bwdx), _ptr(dx), N, Cp, Dp, T, _dtype(dtype),
                                _stream(stream)), "eqlinear_bwd_x")


def eqlinear_bwd_w_workspace_bytes(N: int, Cp: int, Dp: int, T: int, dtype) -> int:
    return lib().eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, _dtype(dtype))


def eqlinear_bwd_w(x, dy, dw, workspace, ws_bytes: int, N: int, Cp: int, Dp: int, T: int, dtype,
                   stream=None) -> None:
    _check(lib().eqlinear_bwd_w(_ptr(x), _ptr(dy), _ptr(dw), _ptr(workspace), ws_bytes, N, Cp, Dp, T,
                                _dtype(dtype), _stream(stream)), "eqlinear_bwd_w")


def eqlinear_fwd_train(x, w_packed, y, workspace, ws_bytes: int, N: int, Cp: int, Dp: int, T: int, dtype,
                       stream=None) -> None:
    """eqlinear_fwd that also leaves x's half spectrum in the weight-gradient workspace."""
    _check(lib().eqlinear_fwd_train(_ptr(x), _ptr(w_packed), _ptr(y), _ptr(workspace), ws_bytes, N, Cp, Dp, T,
                                    _dtype(dtype), _stream(stream)), "eqlinear_fwd_train")


def eqlinear_fwd_fused_train(x, w_packed, bias, residual, y, pre_out, workspace, ws_bytes: int, N: int, Cp: int,
                             Dp: int, T: int, dtype, act: int, stream=None) -> None:
    """eqlinear_fwd_fused that also leaves x's half spectrum in the weight-gradient workspace."""
    _check(lib().eqlinear_fwd_fused_train(_ptr(x), _ptr(w_packed), _ptr(bias), _ptr(residual), _ptr(y), _ptr(pre_out),
                                          _ptr(workspace), ws_bytes, N, Cp, Dp, T, _dtype(dtype), int(act),
                                          _stream(stream)), "eqlinear_fwd_fused_train")


def eqlinear_bwd_x_train(dy, w_packed_bwdx, dx, workspace, ws_bytes: int, N: int, Cp: int, Dp: int, T: int, dtype,
                         stream=None) -> None:
    """eqlinear_bwd_x that also leaves dy's half spectrum in the workspace (separate path)."""
    _check(lib().eqlinear_bwd_x_train(_ptr(dy), _ptr(w_packed_bwdx), _ptr(dx), _ptr(workspace), ws_bytes, N, Cp,
                                      Dp, T, _dtype(dtype), _stream(stream)), "eqlinear_bwd_x_train")


def eqlinear_bwd_w_train(dy, dw, workspace, ws_bytes: int, N: int, Cp: int, Dp: int, T: int, dtype,
                         stream=None) -> None:
    """Weight gradient from the spectra the two calls above left in the workspace."""
    _check(lib().eqlinear_bwd_w_train(_ptr(dy), _ptr(dw), _ptr(workspace), ws_bytes, N, Cp, Dp, T, _dtype(dtype),
                                      _stream(stream)), "eqlinear_bwd_w_train")


def eqlinear_p4m_expand_weight(w, w_c4, Dp: int, Cp: int, dtype, stream=None) -> None:
    """p4m parameters w [Dp][Cp][8] -> the tied C_4 weight [2Dp][2Cp][4]."""
    _check(lib().eqlinear_p4m_expand_weight(_ptr(w), _ptr(w_c4), Dp, Cp, _dtype(dtype), _stream(stream)),
           "eqlinear_p4m_expand_weight")


def eqlinear_p4m_fold_weight_grad(dw_c4, dw, Dp: int, Cp: int, dtype, stream=None) -> None:
    """C_4 weight gradient [2Dp][2Cp][4] -> the p4m weight gradient [Dp][Cp][8]."""
    _check(lib().eqlinear_p4m_fold_weight_grad(_ptr(dw_c4), _ptr(dw), Dp, Cp, _dtype(dtype), _stream(stream)),
           "eqlinear_p4m_fold_weight_grad")
