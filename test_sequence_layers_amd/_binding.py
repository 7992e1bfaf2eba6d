"""ctypes binding of libttt.so.

Argument marshalling only: every step of the forward pass runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  There is no CPU
fallback; if the library is missing every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libttt.so")

TTT_OK, TTT_E_INVALID, TTT_E_UNSUPPORTED, TTT_E_HIP, TTT_E_NONFINITE = 0, -1, -2, -3, -4
TTT_F32, TTT_BF16 = 0, 1

_lib = None
_lock = threading.Lock()

_vp = ctypes.c_void_p
_i = ctypes.c_int
_ll = ctypes.c_longlong
_f = ctypes.c_float

# name -> (restype, argtypes); mirrors include/ttt.h
SIGNATURES = {
    "ttt_linear_fwd": (_i, [_vp, _vp, _vp, _vp, _ll, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _i,
                            _i, _i, _vp]),
    "ttt_mlp_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _ll, _vp, _vp, _vp,
                         _i, _i, _i, _i, _i, _i, _i, _f, _vp, _i, _i, _i, _vp]),
    "ttt_linear_ln_fwd": (_i, [_vp, _vp, _vp, _vp, _ll, _vp, _vp, _f, _vp, _vp, _i, _i, _i, _i, _i,
                               _i, _f, _vp, _i, _i, _i, _vp]),
    "ttt_mlp_ln_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _ll, _vp, _vp, _f, _vp, _vp, _vp,
                            _i, _i, _i, _i, _i, _i, _i, _f, _vp, _i, _i, _i, _vp]),
    "ttt_mlp_fwd_workspace_size": (ctypes.c_size_t, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "ttt_mlp_fwd_ws": (_i, [_vp, _vp, _vp, _vp, _vp, _ll, _vp, _vp, _vp,
                            _i, _i, _i, _i, _i, _i, _i, _f, _vp, _i, _i, _i,
                            _vp, ctypes.c_size_t, _vp]),
    "ttt_mlp_ln_fwd_ws": (_i, [_vp, _vp, _vp, _vp, _vp, _ll, _vp, _vp, _f, _vp, _vp, _vp,
                               _i, _i, _i, _i, _i, _i, _i, _f, _vp, _i, _i, _i,
                               _vp, ctypes.c_size_t, _vp]),
    "delta_rule_fwd": (_i, [_vp, _vp, _vp, _vp, _ll, _vp, _vp, _i, _i, _i, _i, _f, _vp, _i, _vp]),
    "ttt_linear_bwd": (_i, [_vp, _vp, _vp, _vp, _ll, _vp, _vp, _vp, _vp, _vp, _vp,
                            _i, _i, _i, _i, _i, _f, _vp, _vp, _i, _i, _vp]),
    "ttt_linear_bwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _ll, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _i, _i, _i, _i, _i, _f, _vp, _vp, _i, _i, _vp]),
    "ttt_mlp_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _ll, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                         _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _i, _i, _vp]),
    "ttt_linear_ln_bwd": (_i, [_vp, _vp, _vp, _vp, _ll, _vp, _vp, _f, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _vp, _i, _i, _vp]),
    "ttt_mlp_ln_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _ll, _vp, _vp, _f, _vp, _vp, _vp, _vp, _vp, _vp,
                            _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _i, _i, _vp]),
    "ttt_linear_nc_bwd": (_i, [_vp, _vp, _vp, _vp, _ll, _vp, _vp, _vp, _vp, _vp, _vp,
                               _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _i, _i, _vp]),
    "ttt_mlp_nc_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _ll, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                            _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _i, _i, _vp]),
    "ttt_last_error": (ctypes.c_char_p, []),
    "ttt_abi_version": (_i, []),
    "ttt_set_check_finite": (_i, [_i]),
    "ttt_get_check_finite": (_i, []),
    "ttt_set_split_debug": (_i, [_i]),
}


class TTTError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"libttt error {code}: {message}")
        self.code = code


def load_library(path: str = LIB_PATH):
    """Load libttt.so once (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m test_sequence_layers_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def last_error() -> str:
    return load_library().ttt_last_error().decode()


def set_check_finite(on: bool) -> bool:
    """Switch the library's finite check of every call's outputs on or off (debugging; calls
    then wait for their stream and fail with TTT_E_NONFINITE on a NaN or an infinity).
    Returns the previous setting."""
    return bool(load_library().ttt_set_check_finite(1 if on else 0))


def set_split_debug(flags: int) -> int:
    """Debug switches of the two-workgroup MLP kernel (TTT_SPLIT_FORMAL = 1,
    TTT_SPLIT_TEST_ABORT = 2); returns the previous flags."""
    return int(load_library().ttt_set_split_debug(int(flags)))


def get_check_finite() -> bool:
    return bool(load_library().ttt_get_check_finite())


def _check(rc):
    if rc != TTT_OK:
        raise TTTError(rc, last_error())


# --------------------------------------------------------------------------- torch wrappers

def _torch():
    import torch
    return torch


def _io_dtype(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return TTT_F32
    if t.dtype == torch.bfloat16:
        return TTT_BF16
    raise TypeError(f"token tensors must be float32 or bfloat16, got {t.dtype}")


def _tokens(q, k, v):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a [B, H, T, d] tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k and v must have the same shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must have the same dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on the same device")
    return tuple(q.shape)


def _state(w, B, H, shape, name, device):
    """Return (tensor, batch_stride_in_floats) for an initial state [H,...] or [B,H,...]."""
    torch = _torch()
    if not isinstance(w, torch.Tensor) or w.dtype != torch.float32 or not w.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor")
    if w.device != device:
        raise ValueError(f"{name} must be on {device}")
    per = 1
    for s in shape:
        per *= s
    if tuple(w.shape) == (H, *shape):
        return w, 0
    if tuple(w.shape) == (B, H, *shape):
        return w, H * per
    raise ValueError(f"{name} must have shape [H, {shape}] or [B, H, {shape}], got {tuple(w.shape)}")


def _rates(eta_tok, B, H, T, device):
    """Device pointer of optional per-token rate factors [B, H, T] float32 (None -> NULL)."""
    torch = _torch()
    if eta_tok is None:
        return None
    if (not isinstance(eta_tok, torch.Tensor) or eta_tok.dtype != torch.float32
            or not eta_tok.is_contiguous() or tuple(eta_tok.shape) != (B, H, T)
            or eta_tok.device != device):
        raise ValueError(f"eta_tok must be a contiguous float32 tensor of shape {(B, H, T)} on {device}")
    return eta_tok.data_ptr()


_LOSSES = {"mse": 0, "dot": 1}


def _loss(loss):
    if loss not in _LOSSES:
        raise ValueError(f"loss must be one of {sorted(_LOSSES)}, got {loss!r}")
    return _LOSSES[loss]


def _stream(device, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _out(t, shape, dtype, device, name):
    torch = _torch()
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")
    return t


def _ln(ln_weight, ln_bias, ln_eps, H, d, device):
    """Pointers of the per-head layer-norm gain and bias ([H, d] float32 each)."""
    torch = _torch()
    for name, t in (("ln_weight", ln_weight), ("ln_bias", ln_bias)):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_contiguous()
                or tuple(t.shape) != (H, d) or t.device != device):
            raise ValueError(f"{name} must be a contiguous float32 tensor [H, d] = [{H}, {d}] on {device}")
    return ln_weight.data_ptr(), ln_bias.data_ptr(), float(ln_eps)


def _linear(q, k, v, w0, eta, chunk, causal, ln, eta_tok, loss, epochs, z, w_out, return_state,
            stream):
    torch = _torch()
    lib = load_library()
    B, H, T, d = _tokens(q, k, v)
    w0, stride = _state(w0, B, H, (d, d), "w0", q.device)
    z = _out(z, (B, H, T, d), q.dtype, q.device, "z")
    if return_state or w_out is not None:
        w_out = _out(w_out, (B, H, d, d), torch.float32, q.device, "w_out")
    tail = (z.data_ptr(), w_out.data_ptr() if w_out is not None else None,
            B, H, T, d, int(chunk), int(bool(causal)), float(eta),
            _rates(eta_tok, B, H, T, q.device), _loss(loss), int(epochs),
            _io_dtype(q), _stream(q.device, stream))
    with torch.cuda.device(q.device):
        if ln is None:
            rc = lib.ttt_linear_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), w0.data_ptr(), stride,
                                    *tail)
        else:
            rc = lib.ttt_linear_ln_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), w0.data_ptr(),
                                       stride, *_ln(*ln, H, d, q.device), *tail)
    _check(rc)
    return (z, w_out) if w_out is not None else z


def ttt_linear_fwd(q, k, v, w0, eta, chunk, causal=True, *, eta_tok=None, loss="mse", epochs=1,
                   z=None, w_out=None, return_state=False, stream=None):
    """TTT-Linear forward.  q, k, v [B,H,T,d] (float32 or bfloat16, same device);
    w0 float32 [H,d,d] (shared over the batch) or [B,H,d,d]; eta_tok optional float32
    [B,H,T] per-token rate factors (token t learns at eta * eta_tok[t]); loss "mse"
    (reconstruction) or "dot" (negative dot product); epochs: passes over the chunks
    before the queries are read (non-causal only).  Returns z (and the final state
    [B,H,d,d] when return_state or w_out is given)."""
    return _linear(q, k, v, w0, eta, chunk, causal, None, eta_tok, loss, epochs, z, w_out,
                   return_state, stream)


def ttt_linear_ln_fwd(q, k, v, w0, ln_weight, ln_bias, eta, chunk, causal=True, *, ln_eps=1e-6,
                      eta_tok=None, loss="mse", epochs=1, z=None, w_out=None,
                      return_state=False, stream=None):
    """The paper's TTT-Linear, f(x) = x + LN(W x) with per-head ln_weight, ln_bias float32
    [H, d]; every other argument as ttt_linear_fwd."""
    return _linear(q, k, v, w0, eta, chunk, causal, (ln_weight, ln_bias, ln_eps), eta_tok, loss,
                   epochs, z, w_out, return_state, stream)


def ttt_linear_bwd(q, k, v, w0, eta, chunk, dz, dw_out=None, *, eta_tok=None, loss="mse",
                   stream=None):
    """Gradients of the causal TTT-Linear layer (reconstruction loss) for the upstream
    gradients dz [B,H,T,d] (dtype of q) and dw_out [B,H,d,d] float32 (or None).  Returns
    (dq, dk, dv, dw0) with dw0 [B,H,d,d] per sequence (sum it over the batch when w0 is
    shared); with per-token rate factors eta_tok [B,H,T] float32 (as in ttt_linear_fwd) also
    their gradient, (dq, dk, dv, dw0, deta_tok).  loss: "mse" or "dot", as in the forward."""
    return _linear_bwd("ttt_linear_bwd", q, k, v, w0, eta, chunk, dz, dw_out, eta_tok, loss,
                       stream, None)


def ttt_linear_bwd_noalloc(q, k, v, w0, eta, chunk, dz, dw_out=None, *, eta_tok=None,
                           loss="mse", stream=None, out=None):
    """ttt_linear_bwd through the library's allocation-free entry point: the state history
    lives in the library's fixed 64 MiB scratch array (calls that need more raise).  out:
    optional preallocated (dq, dk, dv, dw0[, deta_tok]) to write into."""
    return _linear_bwd("ttt_linear_bwd_noalloc", q, k, v, w0, eta, chunk, dz, dw_out, eta_tok,
                       loss, stream, out)


def _linear_bwd(fn, q, k, v, w0, eta, chunk, dz, dw_out, eta_tok, loss, stream, out):
    torch = _torch()
    lib = load_library()
    B, H, T, d = _tokens(q, k, v)
    w0, stride = _state(w0, B, H, (d, d), "w0", q.device)
    if (not isinstance(dz, torch.Tensor) or tuple(dz.shape) != (B, H, T, d) or dz.dtype != q.dtype
            or dz.device != q.device or not dz.is_contiguous()):
        raise ValueError(f"dz must be a contiguous {q.dtype} tensor of shape {(B, H, T, d)}")
    if dw_out is not None:
        dw_out = _out(dw_out, (B, H, d, d), torch.float32, q.device, "dw_out")
    et = _rates(eta_tok, B, H, T, q.device)
    if out is not None:
        dq = _out(out[0], (B, H, T, d), q.dtype, q.device, "dq")
        dk = _out(out[1], (B, H, T, d), q.dtype, q.device, "dk")
        dv = _out(out[2], (B, H, T, d), q.dtype, q.device, "dv")
        dw0 = _out(out[3], (B, H, d, d), torch.float32, q.device, "dw0")
        deta = (_out(out[4], (B, H, T), torch.float32, q.device, "deta_tok")
                if et is not None else None)
    else:
        dq = torch.empty_like(q)
        dk = torch.empty_like(q)
        dv = torch.empty_like(q)
        dw0 = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
        deta = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if et is not None else None
    with torch.cuda.device(q.device):
        rc = getattr(lib, fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), w0.data_ptr(), stride,
                              dz.data_ptr(), dw_out.data_ptr() if dw_out is not None else None,
                              dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dw0.data_ptr(),
                              B, H, T, d, int(chunk), float(eta), et,
                              deta.data_ptr() if deta is not None else None, _loss(loss),
                              _io_dtype(q), _stream(q.device, stream))
    _check(rc)
    return (dq, dk, dv, dw0) if deta is None else (dq, dk, dv, dw0, deta)


def ttt_mlp_bwd(q, k, v, w1, w2, eta, chunk, dz, dw1_out=None, dw2_out=None, *, eta_tok=None,
                loss="mse", stream=None):
    """Gradients of the causal TTT-MLP layer (SiLU; loss "mse" or "dot") for the upstream
    gradients dz [B,H,T,d] (dtype of q) and dw1_out [B,H,dh,d], dw2_out [B,H,d,dh] float32 (or
    None).  Returns (dq, dk, dv, dw1, dw2) with the state gradients per sequence (sum them over
    the batch when the states are shared); with per-token rate factors eta_tok [B,H,T] (as in
    ttt_mlp_fwd) also their gradient, (dq, dk, dv, dw1, dw2, deta_tok)."""
    torch = _torch()
    lib = load_library()
    B, H, T, d = _tokens(q, k, v)
    if w1.dim() < 2:
        raise ValueError("w1 must be [H, dh, d] or [B, H, dh, d]")
    dh = int(w1.shape[-2])
    w1, s1 = _state(w1, B, H, (dh, d), "w1", q.device)
    w2, s2 = _state(w2, B, H, (d, dh), "w2", q.device)
    if s1 != s2:
        raise ValueError("w1 and w2 must both be shared over the batch or both per batch")
    if (not isinstance(dz, torch.Tensor) or tuple(dz.shape) != (B, H, T, d) or dz.dtype != q.dtype
            or dz.device != q.device or not dz.is_contiguous()):
        raise ValueError(f"dz must be a contiguous {q.dtype} tensor of shape {(B, H, T, d)}")
    if (dw1_out is None) != (dw2_out is None):
        raise ValueError("give both dw1_out and dw2_out, or neither")
    if dw1_out is not None:
        dw1_out = _out(dw1_out, (B, H, dh, d), torch.float32, q.device, "dw1_out")
        dw2_out = _out(dw2_out, (B, H, d, dh), torch.float32, q.device, "dw2_out")
    et = _rates(eta_tok, B, H, T, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dw1 = torch.empty((B, H, dh, d), dtype=torch.float32, device=q.device)
    dw2 = torch.empty((B, H, d, dh), dtype=torch.float32, device=q.device)
    deta = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if et is not None else None
    ptr = lambda t: t.data_ptr() if t is not None else None
    with torch.cuda.device(q.device):
        rc = lib.ttt_mlp_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), w1.data_ptr(), w2.data_ptr(),
                             s1, dz.data_ptr(), ptr(dw1_out), ptr(dw2_out), dq.data_ptr(),
                             dk.data_ptr(), dv.data_ptr(), dw1.data_ptr(), dw2.data_ptr(),
                             B, H, T, d, dh, int(chunk), float(eta), et, ptr(deta), _loss(loss),
                             _io_dtype(q), _stream(q.device, stream))
    _check(rc)
    return (dq, dk, dv, dw1, dw2) if deta is None else (dq, dk, dv, dw1, dw2, deta)


def _dz(dz, q, B, H, T, d):
    torch = _torch()
    if (not isinstance(dz, torch.Tensor) or tuple(dz.shape) != (B, H, T, d) or dz.dtype != q.dtype
            or dz.device != q.device or not dz.is_contiguous()):
        raise ValueError(f"dz must be a contiguous {q.dtype} tensor of shape {(B, H, T, d)}")
    return dz


def ttt_linear_ln_bwd(q, k, v, w0, ln_weight, ln_bias, eta, chunk, dz, dw_out=None, *,
                      ln_eps=1e-6, eta_tok=None, loss="mse", stream=None):
    """Gradients of the paper's causal TTT-Linear layer x + LN(W x) (ttt_linear_ln_fwd with
    the same arguments) for the upstream gradients dz and dw_out.  Returns (dq, dk, dv, dw0,
    dln_weight, dln_bias), plus deta_tok [B,H,T] with eta_tok; dw0 [B,H,d,d] and the layer-norm
    gradients [B,H,d] per sequence."""
    torch = _torch()
    lib = load_library()
    B, H, T, d = _tokens(q, k, v)
    w0, stride = _state(w0, B, H, (d, d), "w0", q.device)
    lw, lb, eps = _ln(ln_weight, ln_bias, ln_eps, H, d, q.device)
    dz = _dz(dz, q, B, H, T, d)
    if dw_out is not None:
        dw_out = _out(dw_out, (B, H, d, d), torch.float32, q.device, "dw_out")
    et = _rates(eta_tok, B, H, T, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dw0 = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    dlw = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    dlb = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    deta = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if et is not None else None
    ptr = lambda t: t.data_ptr() if t is not None else None
    with torch.cuda.device(q.device):
        rc = lib.ttt_linear_ln_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), w0.data_ptr(), stride,
                                   lw, lb, eps, dz.data_ptr(),
                                   ptr(dw_out), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                   dw0.data_ptr(), dlw.data_ptr(), dlb.data_ptr(), B, H, T, d,
                                   int(chunk), float(eta), et, ptr(deta), _loss(loss), _io_dtype(q),
                                   _stream(q.device, stream))
    _check(rc)
    res = (dq, dk, dv, dw0, dlw, dlb)
    return res if deta is None else res + (deta,)


def ttt_mlp_ln_bwd(q, k, v, w1, w2, ln_weight, ln_bias, eta, chunk, dz, dw1_out=None,
                   dw2_out=None, *, ln_eps=1e-6, eta_tok=None, loss="mse", stream=None):
    """Gradients of the paper's causal TTT-MLP layer x + LN(W2 GELU(W1 x)) (ttt_mlp_ln_fwd
    with the same arguments).  Returns (dq, dk, dv, dw1, dw2, dln_weight, dln_bias), plus
    deta_tok [B,H,T] with eta_tok; state and layer-norm gradients per sequence."""
    torch = _torch()
    lib = load_library()
    B, H, T, d = _tokens(q, k, v)
    if w1.dim() < 2:
        raise ValueError("w1 must be [H, dh, d] or [B, H, dh, d]")
    dh = int(w1.shape[-2])
    w1, s1 = _state(w1, B, H, (dh, d), "w1", q.device)
    w2, s2 = _state(w2, B, H, (d, dh), "w2", q.device)
    if s1 != s2:
        raise ValueError("w1 and w2 must both be shared over the batch or both per batch")
    lw, lb, eps = _ln(ln_weight, ln_bias, ln_eps, H, d, q.device)
    dz = _dz(dz, q, B, H, T, d)
    if (dw1_out is None) != (dw2_out is None):
        raise ValueError("give both dw1_out and dw2_out, or neither")
    if dw1_out is not None:
        dw1_out = _out(dw1_out, (B, H, dh, d), torch.float32, q.device, "dw1_out")
        dw2_out = _out(dw2_out, (B, H, d, dh), torch.float32, q.device, "dw2_out")
    et = _rates(eta_tok, B, H, T, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dw1 = torch.empty((B, H, dh, d), dtype=torch.float32, device=q.device)
    dw2 = torch.empty((B, H, d, dh), dtype=torch.float32, device=q.device)
    dlw = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    dlb = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    deta = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if et is not None else None
    ptr = lambda t: t.data_ptr() if t is not None else None
    with torch.cuda.device(q.device):
        rc = lib.ttt_mlp_ln_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), w1.data_ptr(),
                                w2.data_ptr(), s1, lw, lb, eps, dz.data_ptr(), ptr(dw1_out),
                                ptr(dw2_out), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                dw1.data_ptr(), dw2.data_ptr(), dlw.data_ptr(), dlb.data_ptr(),
                                B, H, T, d, dh, int(chunk), float(eta), et, ptr(deta), _loss(loss),
                                _io_dtype(q), _stream(q.device, stream))
    _check(rc)
    res = (dq, dk, dv, dw1, dw2, dlw, dlb)
    return res if deta is None else res + (deta,)


def ttt_linear_nc_bwd(q, k, v, w0, eta, chunk, dz, dw_out=None, *, epochs=1, eta_tok=None,
                      loss="mse", stream=None):
    """Gradients of the non-causal TTT-Linear layer (ttt_linear_fwd with causal=False, the
    same chunk, epochs, eta_tok and loss) for the upstream gradients dz [B,H,T,d] (dtype of q)
    and dw_out [B,H,d,d] float32 (or None).  Returns (dq, dk, dv, dw0), plus deta_tok
    [B,H,T] with eta_tok; dw0 per sequence."""
    torch = _torch()
    lib = load_library()
    B, H, T, d = _tokens(q, k, v)
    w0, stride = _state(w0, B, H, (d, d), "w0", q.device)
    dz = _dz(dz, q, B, H, T, d)
    if dw_out is not None:
        dw_out = _out(dw_out, (B, H, d, d), torch.float32, q.device, "dw_out")
    et = _rates(eta_tok, B, H, T, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dw0 = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    deta = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if et is not None else None
    ptr = lambda t: t.data_ptr() if t is not None else None
    with torch.cuda.device(q.device):
        rc = lib.ttt_linear_nc_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), w0.data_ptr(), stride,
                                   dz.data_ptr(), ptr(dw_out), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), dw0.data_ptr(), B, H, T, d, int(chunk),
                                   int(epochs), float(eta), et, ptr(deta), _loss(loss),
                                   _io_dtype(q), _stream(q.device, stream))
    _check(rc)
    return (dq, dk, dv, dw0) if deta is None else (dq, dk, dv, dw0, deta)


def ttt_mlp_nc_bwd(q, k, v, w1, w2, eta, chunk, dz, dw1_out=None, dw2_out=None, *, epochs=1,
                   eta_tok=None, loss="mse", stream=None):
    """Gradients of the non-causal TTT-MLP layer (ttt_mlp_fwd with causal=False; SiLU) for
    the upstream gradients dz and dw1_out [B,H,dh,d], dw2_out [B,H,d,dh] (or None).  Returns
    (dq, dk, dv, dw1, dw2), plus deta_tok [B,H,T] with eta_tok; state gradients per
    sequence."""
    torch = _torch()
    lib = load_library()
    B, H, T, d = _tokens(q, k, v)
    if w1.dim() < 2:
        raise ValueError("w1 must be [H, dh, d] or [B, H, dh, d]")
    dh = int(w1.shape[-2])
    w1, s1 = _state(w1, B, H, (dh, d), "w1", q.device)
    w2, s2 = _state(w2, B, H, (d, dh), "w2", q.device)
    if s1 != s2:
        raise ValueError("w1 and w2 must both be shared over the batch or both per batch")
    dz = _dz(dz, q, B, H, T, d)
    if (dw1_out is None) != (dw2_out is None):
        raise ValueError("give both dw1_out and dw2_out, or neither")
    if dw1_out is not None:
        dw1_out = _out(dw1_out, (B, H, dh, d), torch.float32, q.device, "dw1_out")
        dw2_out = _out(dw2_out, (B, H, d, dh), torch.float32, q.device, "dw2_out")
    et = _rates(eta_tok, B, H, T, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dw1 = torch.empty((B, H, dh, d), dtype=torch.float32, device=q.device)
    dw2 = torch.empty((B, H, d, dh), dtype=torch.float32, device=q.device)
    deta = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if et is not None else None
    ptr = lambda t: t.data_ptr() if t is not None else None
    with torch.cuda.device(q.device):
        rc = lib.ttt_mlp_nc_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), w1.data_ptr(),
                                w2.data_ptr(), s1, dz.data_ptr(), ptr(dw1_out), ptr(dw2_out),
                                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dw1.data_ptr(),
                                dw2.data_ptr(), B, H, T, d, dh, int(chunk), int(epochs),
                                float(eta), et, ptr(deta), _loss(loss), _io_dtype(q),
                                _stream(q.device, stream))
    _check(rc)
    return (dq, dk, dv, dw1, dw2) if deta is None else (dq, dk, dv, dw1, dw2, deta)


def delta_rule_fwd(q, k, v, w0, eta, *, eta_tok=None, z=None, w_out=None, return_state=False,
                   stream=None):
    """Delta-rule forward (one token per update, causal).  Arguments as ttt_linear_fwd."""
    torch = _torch()
    lib = load_library()
    B, H, T, d = _tokens(q, k, v)
    w0, stride = _state(w0, B, H, (d, d), "w0", q.device)
    z = _out(z, (B, H, T, d), q.dtype, q.device, "z")
    if return_state or w_out is not None:
        w_out = _out(w_out, (B, H, d, d), torch.float32, q.device, "w_out")
    with torch.cuda.device(q.device):
        rc = lib.delta_rule_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), w0.data_ptr(), stride,
                                z.data_ptr(), w_out.data_ptr() if w_out is not None else None,
                                B, H, T, d, float(eta), _rates(eta_tok, B, H, T, q.device),
                                _io_dtype(q), _stream(q.device, stream))
    _check(rc)
    return (z, w_out) if w_out is not None else z


def _mlp(q, k, v, w1, w2, eta, chunk, causal, ln, eta_tok, loss, epochs, z, w1_out, w2_out,
         return_state, stream, workspace=False):
    torch = _torch()
    lib = load_library()
    B, H, T, d = _tokens(q, k, v)
    if w1.dim() < 2:
        raise ValueError("w1 must be [H, dh, d] or [B, H, dh, d]")
    dh = int(w1.shape[-2])
    w1, s1 = _state(w1, B, H, (dh, d), "w1", q.device)
    w2, s2 = _state(w2, B, H, (d, dh), "w2", q.device)
    if s1 != s2:
        raise ValueError("w1 and w2 must both be shared over the batch or both per batch")
    z = _out(z, (B, H, T, d), q.dtype, q.device, "z")
    want = return_state or w1_out is not None or w2_out is not None
    if want:
        w1_out = _out(w1_out, (B, H, dh, d), torch.float32, q.device, "w1_out")
        w2_out = _out(w2_out, (B, H, d, dh), torch.float32, q.device, "w2_out")
    tail = (z.data_ptr(), w1_out.data_ptr() if want else None, w2_out.data_ptr() if want else None,
            B, H, T, d, dh, int(chunk), int(bool(causal)), float(eta),
            _rates(eta_tok, B, H, T, q.device), _loss(loss), int(epochs),
            _io_dtype(q), _stream(q.device, stream))
    with torch.cuda.device(q.device):
        if workspace is not False:
            # the _ws entry points: tail without the stream, then workspace, size, stream
            need = lib.ttt_mlp_fwd_workspace_size(B, H, T, d, dh, int(chunk), int(bool(causal)),
                                                  _io_dtype(q))
            if workspace is None:
                workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
            if not (workspace.is_cuda and workspace.device == q.device and workspace.is_contiguous()):
                raise ValueError("workspace must be a contiguous tensor on the device of q")
            ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size())
            if ln is None:
                rc = lib.ttt_mlp_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), w1.data_ptr(),
                                        w2.data_ptr(), s1, *tail[:-1], *ws, tail[-1])
            else:
                rc = lib.ttt_mlp_ln_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           w1.data_ptr(), w2.data_ptr(), s1,
                                           *_ln(*ln, H, d, q.device), *tail[:-1], *ws, tail[-1])
        elif ln is None:
            rc = lib.ttt_mlp_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), w1.data_ptr(),
                                 w2.data_ptr(), s1, *tail)
        else:
            rc = lib.ttt_mlp_ln_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), w1.data_ptr(),
                                    w2.data_ptr(), s1, *_ln(*ln, H, d, q.device), *tail)
    _check(rc)
    return (z, w1_out, w2_out) if want else z


def ttt_mlp_fwd(q, k, v, w1, w2, eta, chunk, causal=True, *, eta_tok=None, loss="mse", epochs=1,
                z=None, w1_out=None, w2_out=None, return_state=False, stream=None):
    """TTT-MLP forward, f(k) = W2 SiLU(W1 k).  w1 float32 [H,dh,d] or [B,H,dh,d], w2 float32
    [H,d,dh] or [B,H,d,dh] (both shared or both per batch); eta_tok, loss and epochs as in
    ttt_linear_fwd.
    Returns z (and the final states when return_state or an output state is given)."""
    return _mlp(q, k, v, w1, w2, eta, chunk, causal, None, eta_tok, loss, epochs, z, w1_out,
                w2_out, return_state, stream)


def ttt_mlp_fwd_workspace_size(B, H, T, d, dh, chunk, causal=True, io_dtype="bf16"):
    """Bytes of workspace ttt_mlp_fwd_ws / ttt_mlp_ln_fwd_ws need for this shape (0: none,
    the call then runs as ttt_mlp_fwd / ttt_mlp_ln_fwd)."""
    lib = load_library()
    code = {"bf16": 1, "f32": 0, "float32": 0, "bfloat16": 1}[str(io_dtype).replace("torch.", "")]
    return int(lib.ttt_mlp_fwd_workspace_size(int(B), int(H), int(T), int(d), int(dh), int(chunk),
                                              int(bool(causal)), code))


def ttt_mlp_fwd_ws(q, k, v, w1, w2, eta, chunk, causal=True, *, workspace=None, eta_tok=None,
                   loss="mse", epochs=1, z=None, w1_out=None, w2_out=None, return_state=False,
                   stream=None):
    """ttt_mlp_fwd on the two-workgroup kernel, with a caller workspace: a contiguous device
    tensor of at least ttt_mlp_fwd_workspace_size(...) bytes (None: one is allocated with
    torch for this call)."""
    return _mlp(q, k, v, w1, w2, eta, chunk, causal, None, eta_tok, loss, epochs, z, w1_out,
                w2_out, return_state, stream, workspace)


def ttt_mlp_ln_fwd_ws(q, k, v, w1, w2, ln_weight, ln_bias, eta, chunk, causal=True, *,
                      workspace=None, ln_eps=1e-6, eta_tok=None, loss="mse", epochs=1, z=None,
                      w1_out=None, w2_out=None, return_state=False, stream=None):
    """ttt_mlp_ln_fwd on the two-workgroup kernel; workspace as in ttt_mlp_fwd_ws."""
    return _mlp(q, k, v, w1, w2, eta, chunk, causal, (ln_weight, ln_bias, ln_eps), eta_tok, loss,
                epochs, z, w1_out, w2_out, return_state, stream, workspace)


def ttt_mlp_ln_fwd(q, k, v, w1, w2, ln_weight, ln_bias, eta, chunk, causal=True, *, ln_eps=1e-6,
                   eta_tok=None, loss="mse", epochs=1, z=None, w1_out=None, w2_out=None,
                   return_state=False, stream=None):
    """The paper's TTT-MLP, f(x) = x + LN(W2 GELU(W1 x)) with per-head ln_weight, ln_bias
    float32 [H, d]; every other argument as ttt_mlp_fwd."""
    return _mlp(q, k, v, w1, w2, eta, chunk, causal, (ln_weight, ln_bias, ln_eps), eta_tok, loss,
                epochs, z, w1_out, w2_out, return_state, stream)
