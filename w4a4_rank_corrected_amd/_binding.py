"""ctypes binding of the C ABI in include/svdq.h (argument marshalling only).

Every computation runs in ``libsvdq.so``: the host entry points in its C++
preparation code, the device entry points in its HIP kernels.  PyTorch is used
only to own device memory and to name the current HIP stream.  If the library
has not been built, every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

SVDQ_OK = 0
SVDQ_ERR_INVALID_ARG = 1
SVDQ_ERR_UNSUPPORTED = 2
SVDQ_ERR_ALIGNMENT = 3
SVDQ_ERR_NONFINITE = 4
SVDQ_ERR_NO_CONVERGENCE = 5
SVDQ_ERR_WORKSPACE = 6
SVDQ_ERR_HIP = 7
SVDQ_ERR_IO = 8
SVDQ_OUT_BF16 = 0
SVDQ_OUT_F32 = 1
SVDQ_GROUP = 64
SVDQ_MAX_RANK = 256
SVDQ_MAX_DIM = 1 << 22
SVDQ_W8A8_MAX_M = 131072

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsvdq.so")

_c_int = ctypes.c_int
_vp = ctypes.c_void_p
_size = ctypes.c_size_t


class svdq_layer(ctypes.Structure):
    """Mirror of ``struct svdq_layer`` (all pointers are device addresses)."""
    _fields_ = [("m", ctypes.c_int32), ("n", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("group", ctypes.c_int32), ("smooth_inv", _vp), ("qw", _vp), ("wscale", _vp),
                ("l1", _vp), ("l2", _vp), ("bias", _vp)]


class svdq_host_layer(ctypes.Structure):
    """Mirror of ``struct svdq_host_layer`` (all pointers are host addresses)."""
    _fields_ = [("m", ctypes.c_int32), ("n", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("group", ctypes.c_int32), ("alpha", ctypes.c_float), ("lambda_", _vp), ("smooth_inv", _vp),
                ("qw", _vp), ("wscale", _vp), ("l1", _vp), ("l2", _vp), ("bias", _vp)]


class svdq_w8a8_layer(ctypes.Structure):
    """Mirror of ``struct svdq_w8a8_layer`` (all pointers are device addresses)."""
    _fields_ = [("m", ctypes.c_int32), ("n", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("smooth_inv", _vp), ("qw", _vp), ("wscale", _vp), ("l1", _vp), ("l2", _vp), ("bias", _vp)]


class svdq_fp4_layer(ctypes.Structure):
    """Mirror of ``struct svdq_fp4_layer`` (all pointers are device addresses)."""
    _fields_ = [("m", ctypes.c_int32), ("n", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("t_x", ctypes.c_float), ("t_w", ctypes.c_float), ("smooth_inv", _vp), ("qw", _vp),
                ("wscale", _vp), ("l1", _vp), ("l2", _vp), ("bias", _vp)]


# (name, restype, argtypes) for every exported symbol of include/svdq.h
SIGNATURES = [
    ("svdq_prepare_weights", _c_int,
     [_vp, _vp, _c_int, _c_int, _c_int, _c_int, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    ("svdq_prepare_weights_refined", _c_int,
     [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp,
      _vp, _vp, _vp, _vp, _vp]),
    ("svdq_quantize_residual", _c_int, [_vp, _c_int, _c_int, _c_int, _vp, _vp]),
    ("svdq_save_layer", _c_int, [ctypes.c_char_p, ctypes.POINTER(svdq_host_layer)]),
    ("svdq_load_layer_info", _c_int, [ctypes.c_char_p, _vp, _vp, _vp, _vp, _vp]),
    ("svdq_load_layer", _c_int, [ctypes.c_char_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    ("svdq_append_lora", _c_int,
     [_vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _c_int, ctypes.c_float, _vp, _vp]),
    ("svdq_calibrate_act_amax", _c_int, [_vp, _c_int, _c_int, _vp, _c_int, _vp]),
    ("svdq_act_workspace_size", _size, [_c_int, _c_int, _c_int]),
    ("svdq_quantize_act_lowrank_down", _c_int,
     [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _size, _vp]),
    ("svdq_gemm_workspace_size", _size, [_c_int, _c_int, _c_int]),
    ("svdq_gemm_schedule", _c_int, [_c_int, _c_int, _c_int, _c_int, ctypes.POINTER(_c_int)]),
    ("svdq_gemm_w4a4_lowrank_up", _c_int,
     [_vp, _vp, _vp, ctypes.POINTER(svdq_layer), _c_int, _vp, _c_int, _vp, _size, _vp]),
    ("svdq_linear_workspace_size", _size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    ("svdq_linear", _c_int,
     [_vp, ctypes.POINTER(svdq_layer), _c_int, _vp, _c_int, _vp, _size, _vp]),
    ("svdq_linear_noalloc", _c_int, [_vp, ctypes.POINTER(svdq_layer), _c_int, _vp, _c_int, _vp]),
    ("svdq_linear_noalloc_max_workspace", _size, []),
    ("svdq_linear_unfused_workspace_size", _size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    ("svdq_linear_unfused", _c_int,
     [_vp, ctypes.POINTER(svdq_layer), _c_int, _vp, _c_int, _vp, _size, _vp]),
    ("svdq_status_string", ctypes.c_char_p, [_c_int]),
    ("svdq_last_error", ctypes.c_char_p, []),
    ("svdq_abi_version", _c_int, []),
    ("svdq_test_set_svd_iteration_limit", _c_int, [_c_int]),
    ("svdq_w8a8_prepare_weights", _c_int,
     [_vp, _vp, _c_int, _c_int, _c_int, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    ("svdq_w8a8_act_workspace_size", _size, [_c_int, _c_int, _c_int]),
    ("svdq_w8a8_quantize_act_lowrank_down", _c_int,
     [_vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _size, _vp]),
    ("svdq_w8a8_gemm_workspace_size", _size, [_c_int, _c_int, _c_int]),
    ("svdq_w8a8_gemm_lowrank_up", _c_int,
     [_vp, _vp, _vp, ctypes.POINTER(svdq_w8a8_layer), _c_int, _vp, _c_int, _vp, _size, _vp]),
    ("svdq_w8a8_linear_workspace_size", _size, [_c_int, _c_int, _c_int, _c_int]),
    ("svdq_w8a8_linear", _c_int,
     [_vp, ctypes.POINTER(svdq_w8a8_layer), _c_int, _vp, _c_int, _vp, _size, _vp]),
    ("svdq_fp4_prepare_weights", _c_int,
     [_vp, _vp, _c_int, _c_int, _c_int, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    ("svdq_fp4_act_workspace_size", _size, [_c_int, _c_int, _c_int]),
    ("svdq_fp4_quantize_act_lowrank_down", _c_int,
     [_vp, _c_int, _c_int, _c_int, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _size, _vp]),
    ("svdq_fp4_gemm_workspace_size", _size, [_c_int, _c_int, _c_int]),
    ("svdq_fp4_gemm_lowrank_up", _c_int,
     [_vp, _vp, _vp, ctypes.POINTER(svdq_fp4_layer), _c_int, _vp, _c_int, _vp, _size, _vp]),
    ("svdq_fp4_linear_workspace_size", _size, [_c_int, _c_int, _c_int, _c_int]),
    ("svdq_fp4_linear", _c_int,
     [_vp, ctypes.POINTER(svdq_fp4_layer), _c_int, _vp, _c_int, _vp, _size, _vp]),
]

_lib = None


class SvdqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"svdq status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != SVDQ_OK:
        L = lib()
        msg = L.svdq_last_error().decode() or L.svdq_status_string(status).decode()
        raise SvdqError(status, msg)


def _ptr(a) -> Optional[int]:
    """Address of a numpy array / torch tensor (None passes through as NULL)."""
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("host arrays must be C-contiguous")
        return a.ctypes.data
    if not a.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return a.data_ptr()


# The device entry points take raw addresses, so a tensor of the wrong device,
# dtype or shape would make a kernel read or write out of bounds.  Every tensor
# a device call receives is checked here first (None passes where the C ABI
# allows NULL).
def _dev(t, name: str, dtype=None, shape=None, device=None) -> None:
    if t is None:
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _input(x, name: str = "x"):
    """A bf16 GPU activation matrix [b][m]; returns (b, m)."""
    import torch
    _dev(x, name, torch.bfloat16)
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D [b][m], got shape {tuple(x.shape)}")
    return x.shape


def _out_code(out_dtype) -> int:
    import torch
    if out_dtype is None or out_dtype == torch.bfloat16:
        return SVDQ_OUT_BF16
    if out_dtype == torch.float32:
        return SVDQ_OUT_F32
    raise ValueError(f"out_dtype must be torch.bfloat16 or torch.float32, not {out_dtype}")


def _output(y, b: int, n: int, out_dtype, device):
    """The output tensor [b][n] (allocated if None) and its C-ABI dtype code."""
    import torch
    code = _out_code(out_dtype)
    dt = torch.bfloat16 if code == SVDQ_OUT_BF16 else torch.float32
    if y is None:
        return torch.empty((b, n), dtype=dt, device=device), code
    _dev(y, "y", dt, (b, n), device)
    return y, code


def _workspace(ws, need: int, device):
    """The workspace (allocated if None; at least one byte) and its size in bytes."""
    import torch
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _dev(ws, "workspace", device=device)
    return ws, ws.numel() * ws.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# host entry points (offline preparation)
# ---------------------------------------------------------------------------

def svdq_prepare_weights(W: np.ndarray, act_amax: Optional[np.ndarray], rank: int,
                         group: int = SVDQ_GROUP, alpha: float = 0.5,
                         want_residual: bool = False) -> dict:
    """Host preparation of one layer; returns the host arrays of the layer bundle.

    Keys: qw uint8 [m/64][n][32], wscale uint16 (fp16 bits) [m/64][n],
    l1 uint16 (bf16 bits) [rank][m], l2 uint16 [n][rank], lambda / smooth_inv
    float32 [m], residual float32 [m][n] (if requested), m, n, rank.
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    m, n = W.shape
    a = None if act_amax is None else np.ascontiguousarray(act_amax, dtype=np.float32)
    G = max(m // SVDQ_GROUP, 0)
    out = {
        "qw": np.zeros((G, n, 32), np.uint8),
        "wscale": np.zeros((G, n), np.uint16),
        "l1": np.zeros((rank, m), np.uint16),
        "l2": np.zeros((n, rank), np.uint16),
        "lambda": np.zeros(m, np.float32),
        "smooth_inv": np.zeros(m, np.float32),
        "m": m, "n": n, "rank": rank,
    }
    res = np.zeros((m, n), np.float32) if want_residual else None
    _check(lib().svdq_prepare_weights(
        _ptr(W), _ptr(a), m, n, rank, group, alpha, _ptr(out["qw"]), _ptr(out["wscale"]),
        _ptr(out["l1"]) if rank else None, _ptr(out["l2"]) if rank else None,
        _ptr(out["lambda"]), _ptr(out["smooth_inv"]), _ptr(res)))
    if want_residual:
        out["residual"] = res
    return out


def svdq_prepare_weights_refined(W: np.ndarray, act_amax: Optional[np.ndarray], x_cal_bits: np.ndarray,
                                 rank: int, alphas=(0.2, 0.3, 0.4, 0.5, 0.6, 0.7, 0.8, 0.9, 1.0), iters: int = 2,
                                 group: int = SVDQ_GROUP, want_residual: bool = False) -> dict:
    """Preparation with a search over migration strengths and factor refinement,
    scored by layer-output error on calibration rows (bf16 bits [b_cal][m]).

    Returns the keys of ``svdq_prepare_weights`` plus alpha, iteration, rel_err.
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    m, n = W.shape
    a = None if act_amax is None else np.ascontiguousarray(act_amax, dtype=np.float32)
    xc = np.ascontiguousarray(x_cal_bits, dtype=np.uint16)
    al = np.ascontiguousarray(np.asarray(alphas, dtype=np.float32).ravel())
    G = max(m // SVDQ_GROUP, 0)
    out = {
        "qw": np.zeros((G, n, 32), np.uint8),
        "wscale": np.zeros((G, n), np.uint16),
        "l1": np.zeros((rank, m), np.uint16),
        "l2": np.zeros((n, rank), np.uint16),
        "lambda": np.zeros(m, np.float32),
        "smooth_inv": np.zeros(m, np.float32),
        "m": m, "n": n, "rank": rank,
    }
    res = np.zeros((m, n), np.float32) if want_residual else None
    alpha_out = np.zeros(1, np.float32)
    iter_out = np.zeros(1, np.int32)
    err_out = np.zeros(1, np.float64)
    _check(lib().svdq_prepare_weights_refined(
        _ptr(W), _ptr(a), _ptr(xc), xc.shape[0] if xc.ndim == 2 else 0, m, n, rank, group, _ptr(al), al.size,
        iters, _ptr(out["qw"]), _ptr(out["wscale"]), _ptr(out["l1"]) if rank else None,
        _ptr(out["l2"]) if rank else None, _ptr(out["lambda"]), _ptr(out["smooth_inv"]), _ptr(res),
        _ptr(alpha_out), _ptr(iter_out), _ptr(err_out)))
    if want_residual:
        out["residual"] = res
    out.update(alpha=float(alpha_out[0]), iteration=int(iter_out[0]), rel_err=float(err_out[0]))
    return out


def svdq_save_layer(path: str, host: dict, alpha: float = 0.5, bias: Optional[np.ndarray] = None) -> None:
    """Write a prepared layer (the host dict of ``svdq_prepare_weights``, with
    ``l1``/``l2`` possibly widened by ``svdq_append_lora``) to a layer file."""
    m, n, rank = int(host["m"]), int(host["n"]), int(host["rank"])
    arr = lambda a, dt: None if a is None else np.ascontiguousarray(a, dtype=dt)
    lam, inv = arr(host["lambda"], np.float32), arr(host["smooth_inv"], np.float32)
    qw, ws = arr(host["qw"], np.uint8), arr(host["wscale"], np.uint16)
    l1 = arr(host["l1"], np.uint16) if rank else None
    l2 = arr(host["l2"], np.uint16) if rank else None
    bb = arr(bias, np.uint16)
    G = m // SVDQ_GROUP
    expect = {"lambda": (lam, (m,)), "smooth_inv": (inv, (m,)), "qw": (qw, (G, n, 32)), "wscale": (ws, (G, n)),
              "l1": (l1, (rank, m)), "l2": (l2, (n, rank)), "bias": (bb, (n,))}
    for name, (a, shape) in expect.items():
        if a is not None and a.shape != shape:
            raise ValueError(f"{name} has shape {a.shape}, expected {shape}")
    L = svdq_host_layer(m, n, rank, SVDQ_GROUP, float(alpha), _ptr(lam), _ptr(inv), _ptr(qw), _ptr(ws),
                        _ptr(l1), _ptr(l2), _ptr(bb))
    _check(lib().svdq_save_layer(os.fsencode(path), ctypes.byref(L)))


def svdq_load_layer(path: str) -> dict:
    """Read a layer file; returns the host dict (keys of ``svdq_prepare_weights``
    plus ``alpha`` and ``bias``, None when the file stores none)."""
    m, n, rank, hb = (ctypes.c_int32() for _ in range(4))
    alpha = ctypes.c_float()
    _check(lib().svdq_load_layer_info(os.fsencode(path), ctypes.byref(m), ctypes.byref(n), ctypes.byref(rank),
                                      ctypes.byref(hb), ctypes.byref(alpha)))
    m, n, rank = m.value, n.value, rank.value
    G = m // SVDQ_GROUP
    out = {"m": m, "n": n, "rank": rank, "alpha": float(alpha.value),
           "lambda": np.zeros(m, np.float32), "smooth_inv": np.zeros(m, np.float32),
           "qw": np.zeros((G, n, 32), np.uint8), "wscale": np.zeros((G, n), np.uint16),
           "l1": np.zeros((rank, m), np.uint16), "l2": np.zeros((n, rank), np.uint16),
           "bias": np.zeros(n, np.uint16) if hb.value else None}
    _check(lib().svdq_load_layer(os.fsencode(path), _ptr(out["lambda"]), _ptr(out["smooth_inv"]), _ptr(out["qw"]),
                                 _ptr(out["wscale"]), _ptr(out["l1"]) if rank else None,
                                 _ptr(out["l2"]) if rank else None, _ptr(out["bias"])))
    return out


def svdq_quantize_residual(R: np.ndarray, group: int = SVDQ_GROUP):
    R = np.ascontiguousarray(R, dtype=np.float32)
    m, n = R.shape
    qw = np.zeros((max(m // SVDQ_GROUP, 0), n, 32), np.uint8)
    ws = np.zeros((max(m // SVDQ_GROUP, 0), n), np.uint16)
    _check(lib().svdq_quantize_residual(_ptr(R), m, n, group, _ptr(qw), _ptr(ws)))
    return qw, ws


def svdq_append_lora(l1: Optional[np.ndarray], l2: Optional[np.ndarray], m: int, n: int, rank: int,
                     lam: Optional[np.ndarray], A: np.ndarray, B: np.ndarray, scale: float):
    A = np.ascontiguousarray(A, dtype=np.float32)
    B = np.ascontiguousarray(B, dtype=np.float32)
    k = A.shape[1]
    l1o = np.zeros((rank + k, m), np.uint16)
    l2o = np.zeros((n, rank + k), np.uint16)
    lam = None if lam is None else np.ascontiguousarray(lam, dtype=np.float32)
    l1 = None if (l1 is None or rank == 0) else np.ascontiguousarray(l1, dtype=np.uint16)
    l2 = None if (l2 is None or rank == 0) else np.ascontiguousarray(l2, dtype=np.uint16)
    _check(lib().svdq_append_lora(_ptr(l1), _ptr(l2), m, n, rank, _ptr(lam), _ptr(A), _ptr(B), k,
                                  float(scale), _ptr(l1o), _ptr(l2o)))
    return l1o, l2o


# ---------------------------------------------------------------------------
# device entry points
# ---------------------------------------------------------------------------

def svdq_calibrate_act_amax(x, amax=None, accumulate: bool = False, stream=None):
    """x: bf16 CUDA tensor [b][m]; returns fp32 amax [m] (allocated if None)."""
    import torch
    b, m = _input(x)
    if amax is None:
        amax = torch.empty(m, dtype=torch.float32, device=x.device)
    _dev(amax, "amax", torch.float32, (m,), x.device)
    _check(lib().svdq_calibrate_act_amax(_ptr(x), b, m, _ptr(amax), int(accumulate), _stream(stream)))
    return amax


def svdq_act_workspace_size(b: int, m: int, rank: int) -> int:
    return int(lib().svdq_act_workspace_size(b, m, rank))


def svdq_quantize_act_lowrank_down(x, smooth_inv, l1, rank: int, group: int = SVDQ_GROUP,
                                   qx=None, ascale=None, z=None, workspace=None, stream=None):
    """Returns (qx uint8 [m/64][b][32], ascale fp16 [m/64][b], z fp32 [b][rank] or None)."""
    import torch
    b, m = _input(x)
    dev = x.device
    G = m // SVDQ_GROUP
    if qx is None:
        qx = torch.empty((G, b, 32), dtype=torch.uint8, device=dev)
    if ascale is None:
        ascale = torch.empty((G, b), dtype=torch.float16, device=dev)
    if z is None and rank > 0:
        z = torch.empty((b, rank), dtype=torch.float32, device=dev)
    _act_operands(dev, m, rank, smooth_inv, l1, qx, (G, b, 32), torch.uint8, ascale, (G, b), torch.float16, z, b)
    need = svdq_act_workspace_size(b, m, rank)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().svdq_quantize_act_lowrank_down(
        _ptr(x), b, m, rank, group, _ptr(smooth_inv), _ptr(l1), _ptr(qx), _ptr(ascale), _ptr(z),
        _ptr(workspace), wsb, _stream(stream)))
    return qx, ascale, z


def _act_operands(dev, m, rank, smooth_inv, l1, qx, qx_shape, qx_dtype, ascale, as_shape, as_dtype, z, b):
    import torch
    _dev(smooth_inv, "smooth_inv", torch.float32, (m,), dev)
    _dev(l1, "l1", torch.bfloat16, (rank, m), dev)
    _dev(qx, "qx", qx_dtype, qx_shape, dev)
    _dev(ascale, "ascale", as_dtype, as_shape, dev)
    _dev(z, "z", torch.float32, (b, rank), dev)


def _gemm_operands(qx, ascale, z, layer, b, per_group_scales: bool, record: int, qx_dtype, as_dtype,
                   as_tail=()):
    """Checks the GEMM's activation-side inputs against the layer; returns b."""
    import torch
    G = layer.m // SVDQ_GROUP
    _dev(qx, "qx", qx_dtype)
    if b is None:
        if qx.dim() != 3:
            raise ValueError(f"qx must be 3-D [m/64][b][{record}], got shape {tuple(qx.shape)}")
        b = qx.shape[1]
    dev = layer.qw.device
    _dev(qx, "qx", qx_dtype, (G, b, record), dev)
    _dev(ascale, "ascale", as_dtype, ((G, b) if per_group_scales else (b,)) + tuple(as_tail), dev)
    _dev(z, "z", torch.float32, (b, layer.rank), dev)
    return b


class DeviceLayer:
    """A prepared layer resident in device memory plus its ``svdq_layer`` struct."""

    def __init__(self, host: dict, device="cuda", bias: Optional[np.ndarray] = None,
                 smoothing: bool = True):
        import torch
        self.m, self.n, self.rank = int(host["m"]), int(host["n"]), int(host["rank"])
        t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(device=device).view(dt)
        self.qw = t(host["qw"], torch.uint8)
        self.wscale = t(host["wscale"].view(np.int16), torch.float16)
        self.smooth_inv = t(host["smooth_inv"], torch.float32) if smoothing else None
        self.l1 = t(host["l1"].view(np.int16), torch.bfloat16) if self.rank else None
        self.l2 = t(host["l2"].view(np.int16), torch.bfloat16) if self.rank else None
        self.bias = None if bias is None else t(np.asarray(bias, np.uint16).view(np.int16), torch.bfloat16)
        self.struct = svdq_layer(self.m, self.n, self.rank, SVDQ_GROUP, _ptr(self.smooth_inv),
                                 _ptr(self.qw), _ptr(self.wscale), _ptr(self.l1), _ptr(self.l2),
                                 _ptr(self.bias))

    @classmethod
    def from_tensors(cls, m, n, rank, qw, wscale, l1=None, l2=None, smooth_inv=None, bias=None):
        import torch
        dev = qw.device
        G = m // SVDQ_GROUP
        _dev(qw, "qw", torch.uint8, (G, n, 32), dev)
        _dev(wscale, "wscale", torch.float16, (G, n), dev)
        _dev(l1, "l1", torch.bfloat16, (rank, m), dev)
        _dev(l2, "l2", torch.bfloat16, (n, rank), dev)
        _dev(smooth_inv, "smooth_inv", torch.float32, (m,), dev)
        _dev(bias, "bias", torch.bfloat16, (n,), dev)
        self = cls.__new__(cls)
        self.m, self.n, self.rank = m, n, rank
        self.qw, self.wscale, self.l1, self.l2 = qw, wscale, l1, l2
        self.smooth_inv, self.bias = smooth_inv, bias
        self.struct = svdq_layer(m, n, rank, SVDQ_GROUP, _ptr(smooth_inv), _ptr(qw), _ptr(wscale),
                                 _ptr(l1), _ptr(l2), _ptr(bias))
        return self


def svdq_gemm_workspace_size(b: int, n: int, m: int) -> int:
    return int(lib().svdq_gemm_workspace_size(b, n, m))


GEMM_SETTINGS = {"int4": 0, "w8a8": 1, "fp4": 2}  # SVDQ_GEMM_INT4, _W8A8, _FP4


def svdq_gemm_schedule(b: int, n: int, m: int, setting: str = "int4") -> dict:
    """The GEMM kernel's schedule for a b x n output with m input channels on
    the current device: tiles, workgroups launched, the split workgroups and
    the tiles they split (both 0 when each workgroup computes one whole tile),
    and the resident workgroups per CU of the kernel chosen."""
    info = (_c_int * 5)()
    _check(lib().svdq_gemm_schedule(b, n, m, GEMM_SETTINGS[setting], info))
    return {"tiles": info[0], "grid": info[1], "split_workgroups": info[2], "split_tiles": info[3],
            "workgroups_per_cu": info[4]}


def svdq_gemm_w4a4_lowrank_up(qx, ascale, z, layer: DeviceLayer, b: Optional[int] = None,
                              out_dtype=None, y=None, workspace=None, stream=None):
    import torch
    b = _gemm_operands(qx, ascale, z, layer, b, True, 32, torch.uint8, torch.float16)
    y, code = _output(y, b, layer.n, out_dtype, qx.device)
    workspace, wsb = _workspace(workspace, svdq_gemm_workspace_size(b, layer.n, layer.m), qx.device)
    _check(lib().svdq_gemm_w4a4_lowrank_up(_ptr(qx), _ptr(ascale), _ptr(z), ctypes.byref(layer.struct),
                                           b, _ptr(y), code, _ptr(workspace), wsb, _stream(stream)))
    return y


def svdq_linear_workspace_size(b: int, m: int, n: int, rank: int, group: int = SVDQ_GROUP) -> int:
    return int(lib().svdq_linear_workspace_size(b, m, n, rank, group))


def svdq_linear(x, layer: DeviceLayer, out_dtype=None, y=None, workspace=None, stream=None):
    b, m = _input(x)
    _dev(x, "x", device=layer.qw.device)
    if m != layer.m:
        raise ValueError(f"x has {m} channels, the layer {layer.m}")
    y, code = _output(y, b, layer.n, out_dtype, x.device)
    workspace, wsb = _workspace(workspace, svdq_linear_workspace_size(b, m, layer.n, layer.rank), x.device)
    _check(lib().svdq_linear(_ptr(x), ctypes.byref(layer.struct), b, _ptr(y), code, _ptr(workspace),
                             wsb, _stream(stream)))
    return y


def svdq_linear_noalloc(x, layer: DeviceLayer, out_dtype=None, y=None, stream=None):
    """svdq_linear on the library's device scratch (no workspace argument; y is
    allocated here when None, so callers that must not allocate pass y)."""
    b, m = _input(x)
    _dev(x, "x", device=layer.qw.device)
    if m != layer.m:
        raise ValueError(f"x has {m} channels, the layer {layer.m}")
    y, code = _output(y, b, layer.n, out_dtype, x.device)
    _check(lib().svdq_linear_noalloc(_ptr(x), ctypes.byref(layer.struct), b, _ptr(y), code, _stream(stream)))
    return y


def svdq_linear_noalloc_max_workspace() -> int:
    return int(lib().svdq_linear_noalloc_max_workspace())


def svdq_linear_unfused_workspace_size(b: int, m: int, n: int, rank: int, group: int = SVDQ_GROUP) -> int:
    return int(lib().svdq_linear_unfused_workspace_size(b, m, n, rank, group))


def svdq_linear_unfused(x, layer: DeviceLayer, out_dtype=None, y=None, workspace=None, stream=None):
    """The layer without the kernel fusion (five launches), for A/B timing."""
    b, m = _input(x)
    _dev(x, "x", device=layer.qw.device)
    if m != layer.m:
        raise ValueError(f"x has {m} channels, the layer {layer.m}")
    y, code = _output(y, b, layer.n, out_dtype, x.device)
    workspace, wsb = _workspace(workspace, svdq_linear_unfused_workspace_size(b, m, layer.n, layer.rank), x.device)
    _check(lib().svdq_linear_unfused(_ptr(x), ctypes.byref(layer.struct), b, _ptr(y), code,
                                     _ptr(workspace), wsb, _stream(stream)))
    return y


# ---------------------------------------------------------------------------
# the 8-bit setting (per-token / per-channel INT8 with the low-rank branch)
# ---------------------------------------------------------------------------

def svdq_w8a8_prepare_weights(W: np.ndarray, act_amax: Optional[np.ndarray], rank: int, alpha: float = 0.5,
                              want_residual: bool = False) -> dict:
    """Host preparation of an 8-bit layer.  Keys: qw int8 [m/64][n][64],
    wscale uint16 (fp16 bits) [n], l1, l2, lambda, smooth_inv, residual (if
    requested), m, n, rank."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    m, n = W.shape
    a = None if act_amax is None else np.ascontiguousarray(act_amax, dtype=np.float32)
    out = {
        "qw": np.zeros((max(m // SVDQ_GROUP, 0), n, 64), np.int8),
        "wscale": np.zeros(n, np.uint16),
        "l1": np.zeros((rank, m), np.uint16),
        "l2": np.zeros((n, rank), np.uint16),
        "lambda": np.zeros(m, np.float32),
        "smooth_inv": np.zeros(m, np.float32),
        "m": m, "n": n, "rank": rank,
    }
    res = np.zeros((m, n), np.float32) if want_residual else None
    _check(lib().svdq_w8a8_prepare_weights(
        _ptr(W), _ptr(a), m, n, rank, alpha, _ptr(out["qw"]), _ptr(out["wscale"]),
        _ptr(out["l1"]) if rank else None, _ptr(out["l2"]) if rank else None,
        _ptr(out["lambda"]), _ptr(out["smooth_inv"]), _ptr(res)))
    if want_residual:
        out["residual"] = res
    return out


class DeviceLayer8:
    """A prepared 8-bit layer resident in device memory plus its ``svdq_w8a8_layer`` struct."""

    def __init__(self, host: dict, device="cuda", bias: Optional[np.ndarray] = None, smoothing: bool = True):
        import torch
        self.m, self.n, self.rank = int(host["m"]), int(host["n"]), int(host["rank"])
        t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(device=device).view(dt)
        self.qw = t(host["qw"], torch.int8)
        self.wscale = t(host["wscale"].view(np.int16), torch.float16)
        self.smooth_inv = t(host["smooth_inv"], torch.float32) if smoothing else None
        self.l1 = t(host["l1"].view(np.int16), torch.bfloat16) if self.rank else None
        self.l2 = t(host["l2"].view(np.int16), torch.bfloat16) if self.rank else None
        self.bias = None if bias is None else t(np.asarray(bias, np.uint16).view(np.int16), torch.bfloat16)
        self.struct = svdq_w8a8_layer(self.m, self.n, self.rank, _ptr(self.smooth_inv), _ptr(self.qw),
                                      _ptr(self.wscale), _ptr(self.l1), _ptr(self.l2), _ptr(self.bias))


def svdq_w8a8_act_workspace_size(b: int, m: int, rank: int) -> int:
    return int(lib().svdq_w8a8_act_workspace_size(b, m, rank))


def svdq_w8a8_quantize_act_lowrank_down(x, smooth_inv, l1, rank: int, qx=None, ascale=None, z=None,
                                        workspace=None, stream=None):
    """Returns (qx int8 [m/64][b][64], ascale fp16 [b], z fp32 [b][rank] or None)."""
    import torch
    b, m = _input(x)
    dev = x.device
    G = m // SVDQ_GROUP
    if qx is None:
        qx = torch.empty((G, b, 64), dtype=torch.int8, device=dev)
    if ascale is None:
        ascale = torch.empty(b, dtype=torch.float16, device=dev)
    if z is None and rank > 0:
        z = torch.empty((b, rank), dtype=torch.float32, device=dev)
    _act_operands(dev, m, rank, smooth_inv, l1, qx, (G, b, 64), torch.int8, ascale, (b,), torch.float16, z, b)
    need = svdq_w8a8_act_workspace_size(b, m, rank)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().svdq_w8a8_quantize_act_lowrank_down(
        _ptr(x), b, m, rank, _ptr(smooth_inv), _ptr(l1), _ptr(qx), _ptr(ascale), _ptr(z),
        _ptr(workspace), wsb, _stream(stream)))
    return qx, ascale, z


def svdq_w8a8_gemm_workspace_size(b: int, n: int, m: int) -> int:
    return int(lib().svdq_w8a8_gemm_workspace_size(b, n, m))


def svdq_w8a8_gemm_lowrank_up(qx, ascale, z, layer: DeviceLayer8, b: Optional[int] = None, out_dtype=None,
                              y=None, workspace=None, stream=None):
    import torch
    b = _gemm_operands(qx, ascale, z, layer, b, False, 64, torch.int8, torch.float16)
    y, code = _output(y, b, layer.n, out_dtype, qx.device)
    workspace, wsb = _workspace(workspace, svdq_w8a8_gemm_workspace_size(b, layer.n, layer.m), qx.device)
    _check(lib().svdq_w8a8_gemm_lowrank_up(_ptr(qx), _ptr(ascale), _ptr(z), ctypes.byref(layer.struct), b,
                                           _ptr(y), code, _ptr(workspace), wsb, _stream(stream)))
    return y


def svdq_w8a8_linear_workspace_size(b: int, m: int, n: int, rank: int) -> int:
    return int(lib().svdq_w8a8_linear_workspace_size(b, m, n, rank))


def svdq_w8a8_linear(x, layer: DeviceLayer8, out_dtype=None, y=None, workspace=None, stream=None):
    b, m = _input(x)
    _dev(x, "x", device=layer.qw.device)
    if m != layer.m:
        raise ValueError(f"x has {m} channels, the layer {layer.m}")
    y, code = _output(y, b, layer.n, out_dtype, x.device)
    workspace, wsb = _workspace(workspace, svdq_w8a8_linear_workspace_size(b, m, layer.n, layer.rank), x.device)
    _check(lib().svdq_w8a8_linear(_ptr(x), ctypes.byref(layer.struct), b, _ptr(y), code, _ptr(workspace),
                                  wsb, _stream(stream)))
    return y


# ---------------------------------------------------------------------------
# the NVFP4 setting (FP4 E2M1 codes, E4M3 scales per 16 channels, tensor scales)
# ---------------------------------------------------------------------------

def svdq_fp4_prepare_weights(W: np.ndarray, act_amax: Optional[np.ndarray], rank: int, alpha: float = 0.5,
                             want_residual: bool = False) -> dict:
    """Host preparation of an NVFP4 layer.  Keys: qw uint8 [m/64][n][32] (E2M1
    codes), wscale uint8 [m/64][n][4] (E4M3 block scales), l1, l2, lambda,
    smooth_inv, residual (if requested), t_x, t_w, m, n, rank."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    m, n = W.shape
    a = None if act_amax is None else np.ascontiguousarray(act_amax, dtype=np.float32)
    G = max(m // SVDQ_GROUP, 0)
    out = {
        "qw": np.zeros((G, n, 32), np.uint8),
        "wscale": np.zeros((G, n, 4), np.uint8),
        "l1": np.zeros((rank, m), np.uint16),
        "l2": np.zeros((n, rank), np.uint16),
        "lambda": np.zeros(m, np.float32),
        "smooth_inv": np.zeros(m, np.float32),
        "m": m, "n": n, "rank": rank,
    }
    res = np.zeros((m, n), np.float32) if want_residual else None
    tx = np.zeros(1, np.float32)
    tw = np.zeros(1, np.float32)
    _check(lib().svdq_fp4_prepare_weights(
        _ptr(W), _ptr(a), m, n, rank, alpha, _ptr(out["qw"]), _ptr(out["wscale"]),
        _ptr(out["l1"]) if rank else None, _ptr(out["l2"]) if rank else None,
        _ptr(out["lambda"]), _ptr(out["smooth_inv"]), _ptr(res), _ptr(tx), _ptr(tw)))
    if want_residual:
        out["residual"] = res
    out.update(t_x=float(tx[0]), t_w=float(tw[0]))
    return out


class DeviceLayerFp4:
    """A prepared NVFP4 layer resident in device memory plus its ``svdq_fp4_layer`` struct."""

    def __init__(self, host: dict, device="cuda", bias: Optional[np.ndarray] = None, smoothing: bool = True):
        import torch
        self.m, self.n, self.rank = int(host["m"]), int(host["n"]), int(host["rank"])
        self.t_x, self.t_w = float(host["t_x"]), float(host["t_w"])
        t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(device=device).view(dt)
        self.qw = t(host["qw"], torch.uint8)
        self.wscale = t(host["wscale"], torch.uint8)
        self.smooth_inv = t(host["smooth_inv"], torch.float32) if smoothing else None
        self.l1 = t(host["l1"].view(np.int16), torch.bfloat16) if self.rank else None
        self.l2 = t(host["l2"].view(np.int16), torch.bfloat16) if self.rank else None
        self.bias = None if bias is None else t(np.asarray(bias, np.uint16).view(np.int16), torch.bfloat16)
        self.struct = svdq_fp4_layer(self.m, self.n, self.rank, self.t_x, self.t_w, _ptr(self.smooth_inv),
                                     _ptr(self.qw), _ptr(self.wscale), _ptr(self.l1), _ptr(self.l2),
                                     _ptr(self.bias))


def svdq_fp4_act_workspace_size(b: int, m: int, rank: int) -> int:
    return int(lib().svdq_fp4_act_workspace_size(b, m, rank))


def svdq_fp4_quantize_act_lowrank_down(x, smooth_inv, l1, rank: int, t_x: float, qx=None, ascale=None, z=None,
                                       workspace=None, stream=None):
    """Returns (qx uint8 [m/64][b][32], ascale uint8 [m/64][b][4], z fp32 [b][rank] or None)."""
    import torch
    b, m = _input(x)
    dev = x.device
    G = m // SVDQ_GROUP
    if qx is None:
        qx = torch.empty((G, b, 32), dtype=torch.uint8, device=dev)
    if ascale is None:
        ascale = torch.empty((G, b, 4), dtype=torch.uint8, device=dev)
    if z is None and rank > 0:
        z = torch.empty((b, rank), dtype=torch.float32, device=dev)
    _act_operands(dev, m, rank, smooth_inv, l1, qx, (G, b, 32), torch.uint8, ascale, (G, b, 4), torch.uint8, z, b)
    need = svdq_fp4_act_workspace_size(b, m, rank)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().svdq_fp4_quantize_act_lowrank_down(
        _ptr(x), b, m, rank, _ptr(smooth_inv), _ptr(l1), float(t_x), _ptr(qx), _ptr(ascale), _ptr(z),
        _ptr(workspace), wsb, _stream(stream)))
    return qx, ascale, z


def svdq_fp4_gemm_workspace_size(b: int, n: int, m: int) -> int:
    return int(lib().svdq_fp4_gemm_workspace_size(b, n, m))


def svdq_fp4_gemm_lowrank_up(qx, ascale, z, layer: DeviceLayerFp4, b: Optional[int] = None, out_dtype=None,
                             y=None, workspace=None, stream=None):
    import torch
    b = _gemm_operands(qx, ascale, z, layer, b, True, 32, torch.uint8, torch.uint8, (4,))
    y, code = _output(y, b, layer.n, out_dtype, qx.device)
    workspace, wsb = _workspace(workspace, svdq_fp4_gemm_workspace_size(b, layer.n, layer.m), qx.device)
    _check(lib().svdq_fp4_gemm_lowrank_up(_ptr(qx), _ptr(ascale), _ptr(z), ctypes.byref(layer.struct), b,
                                          _ptr(y), code, _ptr(workspace), wsb, _stream(stream)))
    return y


def svdq_fp4_linear_workspace_size(b: int, m: int, n: int, rank: int) -> int:
    return int(lib().svdq_fp4_linear_workspace_size(b, m, n, rank))


def svdq_fp4_linear(x, layer: DeviceLayerFp4, out_dtype=None, y=None, workspace=None, stream=None):
    b, m = _input(x)
    _dev(x, "x", device=layer.qw.device)
    if m != layer.m:
        raise ValueError(f"x has {m} channels, the layer {layer.m}")
    y, code = _output(y, b, layer.n, out_dtype, x.device)
    workspace, wsb = _workspace(workspace, svdq_fp4_linear_workspace_size(b, m, layer.n, layer.rank), x.device)
    _check(lib().svdq_fp4_linear(_ptr(x), ctypes.byref(layer.struct), b, _ptr(y), code, _ptr(workspace),
                                 wsb, _stream(stream)))
    return y
