"""ctypes binding of libhaste.so (the C ABI in include/haste.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory and the current HIP stream.  There is
no fallback: when libhaste.so is missing or a call fails, a HasteError is
raised.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhaste.so")

HASTE_OK = 0
STATUS = {
    0: "HASTE_OK", -1: "HASTE_ERR_NULL", -2: "HASTE_ERR_DIM", -3: "HASTE_ERR_UNSUPPORTED",
    -4: "HASTE_ERR_ALIGN", -5: "HASTE_ERR_WORKSPACE", -6: "HASTE_ERR_INDEX", -7: "HASTE_ERR_HIP",
}
OP = {"fwd": 0, "bwd_w": 1, "bwd_h": 2, "fwd_bce": 3, "step": 4, "fixed_fwd": 5, "fixed_bwd_w": 6,
      "fixed_bwd_h": 7, "fwd_bce_bwd": 8}
DH_MODE = {"atomic": 0, "det": 1, "deterministic": 1, 0: 0, 1: 1}

# name -> (restype, argtypes); P = pointer, I = int64, S = size_t, F = float, M = int
_P, _I, _S, _F, _M = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_int
SIGNATURES = {
    "haste_workspace_size": (_S, [_M, _I, _I, _I, _I, _I, _M]),
    "haste_fwd": (_M, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _S, _P]),
    "haste_bwd_w": (_M, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _S, _P]),
    "haste_bwd_h": (_M, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _M, _P, _S, _P]),
    "haste_fwd_bce": (_M, [_P, _P, _P, _P, _P, _F, _P, _P, _P, _I, _I, _I, _I, _I, _P, _S, _P]),
    "haste_step": (_M, [_P, _P, _P, _P, _P, _F, _P, _P, _P, _P, _I, _I, _I, _I, _I, _M, _P, _S, _P]),
    "haste_step_timed": (_M, [_P, _P, _P, _P, _P, _F, _P, _P, _P, _P, _I, _I, _I, _I, _I, _M, _P, _S, _P, _P]),
    "haste_step_bf16dw": (_M, [_P, _P, _P, _P, _P, _F, _P, _P, _P, _I, _I, _I, _I, _I, _M, _P, _S, _P, _P]),
    "haste_bwd_h_workspace_size": (_S, [_I, _I, _I, _I, _I, _M]),
    "haste_step_noalloc": (_M, [_P, _P, _P, _P, _P, _F, _P, _P, _P, _P, _I, _I, _I, _I, _I, _M, _P]),
    "haste_fwd_bce_bwd": (_M, [_P, _P, _P, _P, _P, _F, _P, _P, _P, _M, _P, _S, _I, _I, _I, _I, _I, _P]),
    "haste_fixed_fwd": (_M, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _S, _P]),
    "haste_fixed_bwd_w": (_M, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _S, _P]),
    "haste_fixed_bwd_h": (_M, [_P, _P, _P, _P, _I, _I, _I, _I, _M, _P, _S, _P]),
    "haste_head_workspace_size": (_S, [_I, _I, _I]),
    "haste_head_step": (_M, [_P, _P, _P, _P, _F, _P, _P, _P, _P, _I, _I, _I, _P, _S, _P]),
    "haste_joint_workspace_size": (_S, [_I, _I, _I, _I, _I, _I, _M]),
    "haste_joint_step": (_M, [_P, _P, _P, _P, _P, _P, _P, _P, _F, _F, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _M,
                              _P, _S, _P]),
    "haste_quantize_w8": (_M, [_P, _P, _P, _I, _I, _I, _P]),
    "haste_fwd_w8": (_M, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _S, _P]),
    "haste_step_w8": (_M, [_P, _P, _P, _P, _P, _P, _F, _P, _P, _P, _P, _I, _I, _I, _I, _I, _M, _P, _S, _P]),
    "haste_step_w8_timed": (_M, [_P, _P, _P, _P, _P, _P, _F, _P, _P, _P, _P, _I, _I, _I, _I, _I, _M, _P, _S, _P,
                                 _P]),
    "haste_kmeans_assign_workspace_size": (_S, [_I, _I, _I, _M]),
    "haste_kmeans_assign": (_M, [_P, _P, _I, _I, _P, _I, _I, _P, _P, _P, _S, _P]),
    "haste_kmeans_init": (_M, [_P, _P, _I, _I, _I, _P, _P, _P, _P]),
    "haste_kmeans_update_workspace_size": (_S, [_I, _I]),
    "haste_kmeans_update": (_M, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _S, _P]),
    "haste_group_workspace_size": (_S, [_I, _I]),
    "haste_group_greedy": (_M, [_P, _P, _I, _I, _I, _I, _P, _P, _S, _P]),
    "haste_label_emb_workspace_size": (_S, [_I]),
    "haste_label_emb_accumulate": (_M, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _S, _P]),
    "haste_label_emb_finalize": (_M, [_P, _P, _I, _I, _P, _P]),
    "haste_rewire_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "haste_rewire": (_M, [_P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _S, _P]),
    "haste_rewire_timed": (_M, [_P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _S, _P, _P]),
    "haste_order_slots": (_M, [_P, _P, _P, _I, _I, _I, _P]),
    "haste_validate_idx": (_M, [_P, _I, _I, _I, _P, _P]),
    "haste_validate_labels": (_M, [_P, _P, _I, _I, _P, _P]),
    "haste_workspace_status": (_M, [_P, _P, _P]),
    "haste_test_set_turn_spins": (None, [_M]),
    "haste_status_string": (ctypes.c_char_p, [_M]),
    "haste_version": (ctypes.c_char_p, []),
}

_lib = None


class HasteError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} returned {code} ({STATUS.get(code, '?')})")


class HandoffError(RuntimeError):
    """A feature-gradient call reported a bounded turn wait that gave up (its dh is invalid)."""


# When true, every call that runs the grouped feature gradient reads its
# workspace status word afterwards (a stream synchronisation) and raises
# HandoffError if it is set.  The tests turn this on; timing code leaves it off.
CHECK_DH_STATUS = False


def lib(path: str | None = None):
    """Load libhaste.so; raises if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise HasteError("load", -7) from FileNotFoundError(
            f"{p} is missing: build it with group_shared_fixed_amd/build.py (hipcc, gfx950)")
    L = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = L
    return L


def _check(fn, code):
    if code != HASTE_OK:
        raise HasteError(fn, code)


# ---------------------------------------------------------------- torch glue

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t, stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _bits(t):
    """bf16 tensor (or its int16/uint16 bit view) as a bf16-bit tensor."""
    torch = _torch()
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"expected bfloat16 (or its 16-bit patterns), got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t


def _i32(t):
    torch = _torch()
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError("index tensors must be contiguous int32")
    return t


def workspace_status(workspace, stream=None) -> int:
    """The status word of the last feature-gradient call on `workspace`
    (0 = ok, 1 = a turn wait gave up); synchronises the stream."""
    out = ctypes.c_int32(-1)
    _check("haste_workspace_status", lib().haste_workspace_status(_ptr(workspace), ctypes.byref(out),
                                                                   _stream(workspace, stream)))
    return int(out.value)


def _check_dh(fn, workspace, stream):
    if CHECK_DH_STATUS and workspace is not None:
        st = workspace_status(workspace, stream)
        if st != 0:
            raise HandoffError(f"{fn}: status word {st}: a feature-gradient turn wait gave up")


def test_set_turn_spins(spins: int) -> None:
    """Test hook: bound of the feature-gradient turn waits (negative: default)."""
    lib().haste_test_set_turn_spins(int(spins))


def workspace_size(op: str, B, H, K, G, F, dh_mode="atomic") -> int:
    return int(lib().haste_workspace_size(OP[op], B, H, K, G, F, DH_MODE[dh_mode]))


def _workspace(op, B, H, K, G, F, dh_mode, device, workspace):
    torch = _torch()
    n = workspace_size(op, B, H, K, G, F, dh_mode)
    if workspace is not None:
        return workspace, n
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def fwd(h, idx, W, G, Z=None, workspace=None, stream=None):
    """Z = forward logits (B x L fp32)."""
    torch = _torch()
    _bits(h); _bits(W); _i32(idx)
    B, H = h.shape
    K, F = idx.shape
    if Z is None:
        Z = torch.empty(B, K * G, dtype=torch.float32, device=h.device)
    ws, n = _workspace("fwd", B, H, K, G, F, 0, h.device, workspace)
    _check("haste_fwd", lib().haste_fwd(_ptr(h), _ptr(idx), _ptr(W), _ptr(Z), B, H, K, G, F,
                                         _ptr(ws), ws.numel() if ws is not None else 0, _stream(h, stream)))
    return Z


def bwd_w(h, idx, dZ, G, dW=None, workspace=None, stream=None):
    """dW (L x F fp32) from bf16 dZ."""
    torch = _torch()
    _bits(h); _bits(dZ); _i32(idx)
    B, H = h.shape
    K, F = idx.shape
    if dW is None:
        dW = torch.empty(K * G, F, dtype=torch.float32, device=h.device)
    ws, n = _workspace("bwd_w", B, H, K, G, F, 0, h.device, workspace)
    _check("haste_bwd_w", lib().haste_bwd_w(_ptr(h), _ptr(idx), _ptr(dZ), _ptr(dW), B, H, K, G, F,
                                             _ptr(ws), ws.numel() if ws is not None else 0, _stream(h, stream)))
    return dW


def bwd_h(dZ, idx, W, G, H, mode="atomic", dh=None, workspace=None, stream=None):
    """dh (B x H fp32) from bf16 dZ."""
    torch = _torch()
    _bits(dZ); _bits(W); _i32(idx)
    B = dZ.shape[0]
    K, F = idx.shape
    if dh is None:
        dh = torch.empty(B, H, dtype=torch.float32, device=dZ.device)
    m = DH_MODE[mode]
    ws, n = _workspace("bwd_h", B, H, K, G, F, m, dZ.device, workspace)
    _check("haste_bwd_h", lib().haste_bwd_h(_ptr(dZ), _ptr(idx), _ptr(W), _ptr(dh), B, H, K, G, F, m,
                                             _ptr(ws), ws.numel() if ws is not None else 0, _stream(dZ, stream)))
    _check_dh("haste_bwd_h", ws, stream)
    return dh


def fwd_bce(h, idx, W, y_rowptr, y_col, scale, G, want_Z=False, want_loss=False, workspace=None, stream=None):
    """(dZ bf16 B x L, Z fp32 or None, loss double tensor or None)."""
    torch = _torch()
    _bits(h); _bits(W); _i32(idx); _i32(y_rowptr); _i32(y_col)
    B, H = h.shape
    K, F = idx.shape
    dZ = torch.empty(B, K * G, dtype=torch.bfloat16, device=h.device)
    Z = torch.empty(B, K * G, dtype=torch.float32, device=h.device) if want_Z else None
    loss = torch.empty(2, dtype=torch.float64, device=h.device) if want_loss else None
    ws, n = _workspace("fwd_bce", B, H, K, G, F, 0, h.device, workspace)
    _check("haste_fwd_bce", lib().haste_fwd_bce(
        _ptr(h), _ptr(idx), _ptr(W), _ptr(y_rowptr), _ptr(y_col), float(scale), _ptr(dZ), _ptr(Z), _ptr(loss),
        B, H, K, G, F, _ptr(ws), ws.numel() if ws is not None else 0, _stream(h, stream)))
    return dZ, Z, (loss[:1] if loss is not None else None)


def step(h, idx, W, y_rowptr, y_col, scale, G, mode="atomic", want_Z=False, want_loss=False, out=None,
         workspace=None, stream=None, events=None, dw_bf16=False):
    """Fused forward + BCE + dW + dh.  Returns dict(dW, dh, Z, loss).

    events: optional ctypes array of 5 hipEvent_t handles (haste_step_timed).
    dw_bf16: store dW as bf16 (haste_step_bf16dw; no Z output)."""
    torch = _torch()
    _bits(h); _bits(W); _i32(idx); _i32(y_rowptr); _i32(y_col)
    B, H = h.shape
    K, F = idx.shape
    if dw_bf16 and (want_Z or (out is not None and out.get("Z") is not None)):
        raise ValueError("the bf16-dW pass has no logits output")
    if out is None:
        out = {
            "dW": torch.empty(K * G, F, dtype=torch.bfloat16 if dw_bf16 else torch.float32, device=h.device),
            "dh": torch.empty(B, H, dtype=torch.float32, device=h.device),
            "Z": torch.empty(B, K * G, dtype=torch.float32, device=h.device) if want_Z else None,
            "loss": torch.empty(2, dtype=torch.float64, device=h.device) if want_loss else None,
        }
    m = DH_MODE[mode]
    ws, n = _workspace("step", B, H, K, G, F, m, h.device, workspace)
    if dw_bf16:
        _bits(out["dW"])
        ev = None if events is None else ctypes.cast(events, ctypes.c_void_p)
        _check("haste_step_bf16dw", lib().haste_step_bf16dw(
            _ptr(h), _ptr(idx), _ptr(W), _ptr(y_rowptr), _ptr(y_col), float(scale), _ptr(out["dW"]), _ptr(out["dh"]),
            _ptr(out.get("loss")), B, H, K, G, F, m, _ptr(ws), ws.numel() if ws is not None else 0,
            _stream(h, stream), ev))
        _check_dh("haste_step_bf16dw", ws, stream)
        return out
    args = (_ptr(h), _ptr(idx), _ptr(W), _ptr(y_rowptr), _ptr(y_col), float(scale), _ptr(out["dW"]),
            _ptr(out["dh"]), _ptr(out.get("Z")), _ptr(out.get("loss")), B, H, K, G, F, m, _ptr(ws),
            ws.numel() if ws is not None else 0, _stream(h, stream))
    if events is None:
        _check("haste_step", lib().haste_step(*args))
    else:
        _check("haste_step_timed", lib().haste_step_timed(*args, ctypes.cast(events, ctypes.c_void_p)))
    _check_dh("haste_step", ws, stream)
    return out


def bwd_h_workspace_size(B, H, K, G, F, mode="atomic") -> int:
    return int(lib().haste_bwd_h_workspace_size(B, H, K, G, F, DH_MODE[mode]))


def fwd_bce_bwd(h, idx, W, y_rowptr, y_col, scale, G, mode="atomic", want_loss=False, out=None, workspace=None,
                stream=None):
    """Fused forward + BCE + dW + dh (haste_fwd_bce_bwd, fp32 loss).
    Returns dict(dW, dh, loss)."""
    torch = _torch()
    _bits(h); _bits(W); _i32(idx); _i32(y_rowptr); _i32(y_col)
    B, H = h.shape
    K, F = idx.shape
    if out is None:
        out = {
            "dW": torch.empty(K * G, F, dtype=torch.float32, device=h.device),
            "dh": torch.empty(B, H, dtype=torch.float32, device=h.device),
            "loss": torch.empty(4, dtype=torch.float32, device=h.device) if want_loss else None,
        }
    m = DH_MODE[mode]
    ws, n = _workspace("fwd_bce_bwd", B, H, K, G, F, m, h.device, workspace)
    _check("haste_fwd_bce_bwd", lib().haste_fwd_bce_bwd(
        _ptr(h), _ptr(idx), _ptr(W), _ptr(y_rowptr), _ptr(y_col), float(scale), _ptr(out["dW"]), _ptr(out["dh"]),
        _ptr(out.get("loss")), m, _ptr(ws), ws.numel() if ws is not None else 0, B, H, K, G, F, _stream(h, stream)))
    _check_dh("haste_fwd_bce_bwd", ws, stream)
    return out


def step_noalloc(h, idx, W, y_rowptr, y_col, scale, G, mode="atomic", want_Z=False, want_loss=False, out=None,
                 stream=None):
    """haste_step without a workspace (the library's per-GPU scratch array).
    Returns dict(dW, dh, Z, loss)."""
    torch = _torch()
    _bits(h); _bits(W); _i32(idx); _i32(y_rowptr); _i32(y_col)
    B, H = h.shape
    K, F = idx.shape
    if out is None:
        out = {
            "dW": torch.empty(K * G, F, dtype=torch.float32, device=h.device),
            "dh": torch.empty(B, H, dtype=torch.float32, device=h.device),
            "Z": torch.empty(B, K * G, dtype=torch.float32, device=h.device) if want_Z else None,
            "loss": torch.empty(2, dtype=torch.float64, device=h.device) if want_loss else None,
        }
    _check("haste_step_noalloc", lib().haste_step_noalloc(
        _ptr(h), _ptr(idx), _ptr(W), _ptr(y_rowptr), _ptr(y_col), float(scale), _ptr(out["dW"]), _ptr(out["dh"]),
        _ptr(out.get("Z")), _ptr(out.get("loss")), B, H, K, G, F, DH_MODE[mode], _stream(h, stream)))
    return out


def fixed_fwd(h, idx1, W, Z=None, workspace=None, stream=None):
    torch = _torch()
    _bits(h); _bits(W); _i32(idx1)
    B, H = h.shape
    L, F = idx1.shape
    if Z is None:
        Z = torch.empty(B, L, dtype=torch.float32, device=h.device)
    ws, n = _workspace("fixed_fwd", B, H, L, 1, F, 0, h.device, workspace)
    _check("haste_fixed_fwd", lib().haste_fixed_fwd(_ptr(h), _ptr(idx1), _ptr(W), _ptr(Z), B, H, L, F,
                                                     _ptr(ws), ws.numel() if ws is not None else 0,
                                                     _stream(h, stream)))
    return Z


def fixed_bwd_w(h, idx1, dZ, dW=None, workspace=None, stream=None):
    torch = _torch()
    _bits(h); _bits(dZ); _i32(idx1)
    B, H = h.shape
    L, F = idx1.shape
    if dW is None:
        dW = torch.empty(L, F, dtype=torch.float32, device=h.device)
    ws, n = _workspace("fixed_bwd_w", B, H, L, 1, F, 0, h.device, workspace)
    _check("haste_fixed_bwd_w", lib().haste_fixed_bwd_w(_ptr(h), _ptr(idx1), _ptr(dZ), _ptr(dW), B, H, L, F,
                                                         _ptr(ws), ws.numel() if ws is not None else 0,
                                                         _stream(h, stream)))
    return dW


def fixed_bwd_h(dZ, idx1, W, H, mode="atomic", dh=None, workspace=None, stream=None):
    torch = _torch()
    _bits(dZ); _bits(W); _i32(idx1)
    B = dZ.shape[0]
    L, F = idx1.shape
    if dh is None:
        dh = torch.empty(B, H, dtype=torch.float32, device=dZ.device)
    m = DH_MODE[mode]
    ws, n = _workspace("fixed_bwd_h", B, H, L, 1, F, m, dZ.device, workspace)
    _check("haste_fixed_bwd_h", lib().haste_fixed_bwd_h(_ptr(dZ), _ptr(idx1), _ptr(W), _ptr(dh), B, H, L, F, m,
                                                         _ptr(ws), ws.numel() if ws is not None else 0,
                                                         _stream(dZ, stream)))
    return dh


def head_workspace_size(B, H, L_head) -> int:
    return int(lib().haste_head_workspace_size(B, H, L_head))


def head_step(h, W_head, y_rowptr, y_col, scale, want_Z=False, want_loss=False, out=None, workspace=None,
              stream=None):
    """Dense head pass: Z = h W^T, BCE gradient, dW, dh.  Returns dict(dW, dh, Z, loss)."""
    torch = _torch()
    _bits(h); _bits(W_head); _i32(y_rowptr); _i32(y_col)
    B, H = h.shape
    L = W_head.shape[0]
    if W_head.shape[1] != H:
        raise ValueError("W_head must be L_head x H")
    if out is None:
        out = {
            "dW": torch.empty(L, H, dtype=torch.float32, device=h.device),
            "dh": torch.empty(B, H, dtype=torch.float32, device=h.device),
            "Z": torch.empty(B, L, dtype=torch.float32, device=h.device) if want_Z else None,
            "loss": torch.empty(2, dtype=torch.float64, device=h.device) if want_loss else None,
        }
    n = head_workspace_size(B, H, L)
    ws = workspace if workspace is not None else torch.empty(n, dtype=torch.uint8, device=h.device)
    _check("haste_head_step", lib().haste_head_step(
        _ptr(h), _ptr(W_head), _ptr(y_rowptr), _ptr(y_col), float(scale), _ptr(out["dW"]), _ptr(out["dh"]),
        _ptr(out.get("Z")), _ptr(out.get("loss")), B, H, L, _ptr(ws), ws.numel(), _stream(h, stream)))
    return out


def joint_workspace_size(B, H, K, G, F, L_head, dh_mode="atomic") -> int:
    return int(lib().haste_joint_workspace_size(B, H, K, G, F, L_head, DH_MODE[dh_mode]))


def joint_step(h, idx, W_tail, yt_rowptr, yt_col, W_head, yh_rowptr, yh_col, scale_tail, scale_head, G,
               mode="atomic", want_loss=False, out=None, workspace=None, stream=None):
    """Head + tail pass on shared features.  Returns dict(dW_tail, dW_head, dh, loss)."""
    torch = _torch()
    _bits(h); _bits(W_tail); _bits(W_head); _i32(idx)
    _i32(yt_rowptr); _i32(yt_col); _i32(yh_rowptr); _i32(yh_col)
    B, H = h.shape
    K, F = idx.shape
    L = W_head.shape[0]
    if W_head.shape[1] != H:
        raise ValueError("W_head must be L_head x H")
    if out is None:
        out = {
            "dW_tail": torch.empty(K * G, F, dtype=torch.float32, device=h.device),
            "dW_head": torch.empty(L, H, dtype=torch.float32, device=h.device),
            "dh": torch.empty(B, H, dtype=torch.float32, device=h.device),
            "loss": torch.empty(2, dtype=torch.float64, device=h.device) if want_loss else None,
        }
    m = DH_MODE[mode]
    n = joint_workspace_size(B, H, K, G, F, L, m)
    ws = workspace if workspace is not None else torch.empty(n, dtype=torch.uint8, device=h.device)
    _check("haste_joint_step", lib().haste_joint_step(
        _ptr(h), _ptr(idx), _ptr(W_tail), _ptr(yt_rowptr), _ptr(yt_col), _ptr(W_head), _ptr(yh_rowptr),
        _ptr(yh_col), float(scale_tail), float(scale_head), _ptr(out["dW_tail"]), _ptr(out["dW_head"]),
        _ptr(out["dh"]), _ptr(out.get("loss")), B, H, K, G, F, L, m, _ptr(ws), ws.numel(), _stream(h, stream)))
    _check_dh("haste_joint_step", ws, stream)
    return out


def _u8(t):
    torch = _torch()
    if t.dtype != torch.uint8 or not t.is_contiguous():
        raise TypeError("FP8 codes must be a contiguous uint8 tensor")
    return t


def quantize_w8(W, G, W8=None, wexp=None, stream=None):
    """bf16 W (L x F) -> (W8 uint8 E4M3 codes L x F, wexp int32 K)."""
    torch = _torch()
    _bits(W)
    L, F = W.shape
    K = L // G
    if W8 is None:
        W8 = torch.empty(L, F, dtype=torch.uint8, device=W.device)
    if wexp is None:
        wexp = torch.empty(K, dtype=torch.int32, device=W.device)
    _check("haste_quantize_w8", lib().haste_quantize_w8(_ptr(W), _ptr(W8), _ptr(wexp), K, G, F, _stream(W, stream)))
    return W8, wexp


def fwd_w8(h, idx, W8, wexp, G, Z=None, workspace=None, stream=None):
    """Z (B x L fp32) from FP8 weights."""
    torch = _torch()
    _bits(h); _u8(W8); _i32(idx); _i32(wexp)
    B, H = h.shape
    K, F = idx.shape
    if Z is None:
        Z = torch.empty(B, K * G, dtype=torch.float32, device=h.device)
    ws, n = _workspace("fwd", B, H, K, G, F, 0, h.device, workspace)
    _check("haste_fwd_w8", lib().haste_fwd_w8(_ptr(h), _ptr(idx), _ptr(W8), _ptr(wexp), _ptr(Z), B, H, K, G, F,
                                               _ptr(ws), ws.numel() if ws is not None else 0, _stream(h, stream)))
    return Z


def step_w8(h, idx, W8, wexp, y_rowptr, y_col, scale, G, mode="atomic", want_Z=False, want_loss=False, out=None,
            workspace=None, stream=None, events=None):
    """Fused step from FP8 weights.  Returns dict(dW, dh, Z, loss)."""
    torch = _torch()
    _bits(h); _u8(W8); _i32(idx); _i32(wexp); _i32(y_rowptr); _i32(y_col)
    B, H = h.shape
    K, F = idx.shape
    if out is None:
        out = {
            "dW": torch.empty(K * G, F, dtype=torch.float32, device=h.device),
            "dh": torch.empty(B, H, dtype=torch.float32, device=h.device),
            "Z": torch.empty(B, K * G, dtype=torch.float32, device=h.device) if want_Z else None,
            "loss": torch.empty(2, dtype=torch.float64, device=h.device) if want_loss else None,
        }
    m = DH_MODE[mode]
    ws, n = _workspace("step", B, H, K, G, F, m, h.device, workspace)
    args = (_ptr(h), _ptr(idx), _ptr(W8), _ptr(wexp), _ptr(y_rowptr), _ptr(y_col), float(scale), _ptr(out["dW"]),
            _ptr(out["dh"]), _ptr(out.get("Z")), _ptr(out.get("loss")), B, H, K, G, F, m, _ptr(ws),
            ws.numel() if ws is not None else 0, _stream(h, stream))
    if events is None:
        _check("haste_step_w8", lib().haste_step_w8(*args))
    else:
        _check("haste_step_w8_timed", lib().haste_step_w8_timed(*args, ctypes.cast(events, ctypes.c_void_p)))
    _check_dh("haste_step_w8", ws, stream)
    return out


def _ws(n, dev, workspace):
    torch = _torch()
    return workspace if workspace is not None else torch.empty(max(n, 256), dtype=torch.uint8, device=dev)


def kmeans_assign(E, M, rows=None, want_score=False, workspace=None, stream=None):
    """Nearest centre (largest dot product, lowest index on ties) of E rows
    (all, or E[rows]).  Returns (assign int32, score fp32 or None)."""
    torch = _torch()
    _bits(E); _bits(M)
    L, H = E.shape
    C = M.shape[0]
    n = L if rows is None else _i32(rows).numel()
    a = torch.empty(n, dtype=torch.int32, device=E.device)
    sc = torch.empty(n, dtype=torch.float32, device=E.device) if want_score else None
    ws = _ws(int(lib().haste_kmeans_assign_workspace_size(n, C, H, int(rows is not None))), E.device, workspace)
    _check("haste_kmeans_assign", lib().haste_kmeans_assign(_ptr(E), _ptr(rows), n, L, _ptr(M), C, H, _ptr(a),
                                                             _ptr(sc), _ptr(ws), ws.numel(), _stream(E, stream)))
    return a, sc


def kmeans_init(E, init, stream=None):
    """Centres from labels init: (Mc fp32 C x H, Mb bf16 C x H, counts int32 C)."""
    torch = _torch()
    _bits(E); _i32(init)
    L, H = E.shape
    C = init.numel()
    Mc = torch.empty(C, H, dtype=torch.float32, device=E.device)
    Mb = torch.empty(C, H, dtype=torch.bfloat16, device=E.device)
    v = torch.empty(C, dtype=torch.int32, device=E.device)
    _check("haste_kmeans_init", lib().haste_kmeans_init(_ptr(E), _ptr(init), L, C, H, _ptr(Mc), _ptr(Mb), _ptr(v),
                                                         _stream(E, stream)))
    return Mc, Mb, v


def kmeans_update(E, batch, assign, Mc, Mb, counts, workspace=None, stream=None):
    """One mini-batch step, in place on (Mc, Mb, counts)."""
    _bits(E); _bits(Mb); _i32(batch); _i32(assign); _i32(counts)
    L, H = E.shape
    C = Mc.shape[0]
    n = batch.numel()
    ws = _ws(int(lib().haste_kmeans_update_workspace_size(n, C)), E.device, workspace)
    _check("haste_kmeans_update", lib().haste_kmeans_update(_ptr(E), _ptr(batch), _ptr(assign), n, L, C, H, _ptr(Mc),
                                                             _ptr(Mb), _ptr(counts), _ptr(ws), ws.numel(),
                                                             _stream(E, stream)))
    return Mc, Mb, counts


def group_greedy(E, assign, C, G, workspace=None, stream=None):
    """Label permutation whose consecutive G-blocks are the groups."""
    torch = _torch()
    _bits(E); _i32(assign)
    L, H = E.shape
    perm = torch.empty(L, dtype=torch.int32, device=E.device)
    ws = _ws(int(lib().haste_group_workspace_size(L, C)), E.device, workspace)
    _check("haste_group_greedy", lib().haste_group_greedy(_ptr(E), _ptr(assign), L, C, H, G, _ptr(perm), _ptr(ws),
                                                           ws.numel(), _stream(E, stream)))
    return perm


def label_emb_accumulate(h, y_rowptr, y_col, S, counts, nnz=None, workspace=None, stream=None):
    """Adds one batch into the per-label feature sums S (L x H fp32) and
    positive counts (L int32), in place.  nnz defaults to y_col.numel()."""
    _bits(h); _i32(y_rowptr); _i32(y_col); _i32(counts)
    B, H = h.shape
    L = S.shape[0]
    n = int(y_col.numel() if nnz is None else nnz)
    ws = _ws(int(lib().haste_label_emb_workspace_size(n)), h.device, workspace)
    _check("haste_label_emb_accumulate", lib().haste_label_emb_accumulate(
        _ptr(h), _ptr(y_rowptr), _ptr(y_col), n, B, H, L, _ptr(S), _ptr(counts), _ptr(ws), ws.numel(),
        _stream(h, stream)))
    return S, counts


def label_emb_finalize(S, counts, E=None, stream=None):
    """E (L x H bf16) = the directions of the per-label sums (0 without positives)."""
    torch = _torch()
    _i32(counts)
    L, H = S.shape
    if E is None:
        E = torch.empty(L, H, dtype=torch.bfloat16, device=S.device)
    _check("haste_label_emb_finalize", lib().haste_label_emb_finalize(_ptr(S), _ptr(counts), L, H, _ptr(E),
                                                                       _stream(S, stream)))
    return E


def rewire_workspace_size(B, H, K, G, F) -> int:
    return int(lib().haste_rewire_workspace_size(B, H, K, G, F))


def rewire(h, dZ, idx, W, G, n_swap, idx_out=None, W_out=None, want_scores=False, workspace=None, stream=None,
           events=None):
    """Group-level rewiring.  Returns dict(idx, W, grow, prune); idx_out /
    W_out may be idx / W (in place).  events: optional ctypes array of 4
    hipEvent_t handles (haste_rewire_timed)."""
    torch = _torch()
    _bits(h); _bits(dZ); _bits(W); _i32(idx)
    B, H = h.shape
    K, F = idx.shape
    if idx_out is None:
        idx_out = torch.empty_like(idx)
    if W_out is None:
        W_out = torch.empty_like(W)
    grow = torch.empty(K, H, dtype=torch.float32, device=h.device) if want_scores else None
    prune = torch.empty(K, F, dtype=torch.float32, device=h.device) if want_scores else None
    n = rewire_workspace_size(B, H, K, G, F)
    ws = workspace if workspace is not None else torch.empty(n, dtype=torch.uint8, device=h.device)
    args = (_ptr(h), _ptr(dZ), _ptr(idx), _ptr(W), int(n_swap), _ptr(idx_out), _ptr(W_out), _ptr(grow), _ptr(prune),
            B, H, K, G, F, _ptr(ws), ws.numel(), _stream(h, stream))
    if events is None:
        _check("haste_rewire", lib().haste_rewire(*args))
    else:
        _check("haste_rewire_timed", lib().haste_rewire_timed(*args, ctypes.cast(events, ctypes.c_void_p)))
    return {"idx": idx_out, "W": W_out, "grow": grow, "prune": prune}


def order_slots(idx, W=None, G=None, perm=False, stream=None):
    """Bank-balanced slot order of every group, in place on idx (K x F int32)
    and, if given, the columns of W (K G x F bf16).  Returns the K x F uint8
    tensor perm (perm[k, s] = old slot now at s) when perm is True, else None."""
    torch = _torch()
    _i32(idx)
    K, F = idx.shape
    if W is not None:
        _bits(W)
        if G is None or W.shape != (K * G, F):
            raise ValueError("W must be K*G x F with G given")
    Gv = G if G is not None else 32
    p = torch.empty(K, F, dtype=torch.uint8, device=idx.device) if perm else None
    _check("haste_order_slots", lib().haste_order_slots(_ptr(idx), _ptr(W), _ptr(p), K, Gv, F, _stream(idx, stream)))
    return p


def validate_idx(idx, H, stream=None) -> int:
    """Number of index rows with an entry outside [0, H) or an entry twice."""
    torch = _torch()
    _i32(idx)
    bad = torch.empty(4, dtype=torch.int32, device=idx.device)
    rows, F = idx.shape
    _check("haste_validate_idx", lib().haste_validate_idx(_ptr(idx), rows, F, H, _ptr(bad), _stream(idx, stream)))
    return int(bad[0].item())


def validate_labels(y_rowptr, y_col, L, stream=None) -> int:
    torch = _torch()
    _i32(y_rowptr); _i32(y_col)
    bad = torch.empty(4, dtype=torch.int32, device=y_rowptr.device)
    B = y_rowptr.numel() - 1
    _check("haste_validate_labels", lib().haste_validate_labels(_ptr(y_rowptr), _ptr(y_col), B, L, _ptr(bad),
                                                                 _stream(y_rowptr, stream)))
    return int(bad[0].item())


def status_string(code: int) -> str:
    return lib().haste_status_string(code).decode()


def version() -> str:
    return lib().haste_version().decode()
