"""Python binding of libssmscan.so, the gfx950 selective-scan library.

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity) and their device pointers, sizes and torch's current HIP stream
are passed to the C ABI declared in include/ssm_scan.h.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
library is missing the import of this module still works, but every call
raises -- build it with ``python -m mamba_selective_scan_ssm_amd.build``.

Non-contiguous inputs are rejected rather than copied: strided x/z views of
a packed in-projection were a source of wrong results in the llama.cpp Mamba
GPU port ("ggml : add GPU support for Mamba models", the ggml_cont fixes).
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssmscan.so")

SSM_F32, SSM_BF16 = 0, 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "hip error"}


class SSMError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: status {code} ({STATUS.get(code, '?')})")
        self.code = code


class Tuning(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("chunk_len", ctypes.c_int32),
                ("states_per_lane", ctypes.c_int32), ("reserved", ctypes.c_int32 * 5)]


class DeltaOpts(ctypes.Structure):
    """ssm_delta_opts: step size delta + bias, then softplus (optional)."""
    _fields_ = [("bias", ctypes.c_void_p), ("softplus", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 3)]


def _dopts(bias, softplus):
    if bias is None and not softplus:
        return None
    return ctypes.byref(DeltaOpts(None if bias is None else bias.data_ptr(), 1 if softplus else 0))


_lib = None


def lib():
    """Load libssmscan.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: the HIP library has not been built")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        L.ssm_scan_fwd.argtypes = [i64, i64, i64, i64, ctypes.c_int] + [vp] * 10 + [vp, sz, vp, vp]
        L.ssm_scan_fwd.restype = ctypes.c_int
        L.ssm_scan_fwd_workspace_size.argtypes = [i64, i64, i64, i64, vp]
        L.ssm_scan_fwd_workspace_size.restype = sz
        L.ssm_state_update.argtypes = [i64, i64, i64, ctypes.c_int] + [vp] * 9 + [vp]
        L.ssm_state_update.restype = ctypes.c_int
        L.ssm_ssd_fwd.argtypes = [i64] * 7 + [ctypes.c_int] + [vp] * 10 + [vp, sz, vp]
        L.ssm_ssd_fwd.restype = ctypes.c_int
        L.ssm_ssd_fwd_workspace_size.argtypes = [i64] * 7
        L.ssm_ssd_fwd_workspace_size.restype = sz
        L.ssm_scan_fwd_ex.argtypes = [i64, i64, i64, i64, ctypes.c_int] + [vp] * 10 + [vp, sz, vp, vp, vp]
        L.ssm_scan_fwd_ex.restype = ctypes.c_int
        L.ssm_scan_fwd_noalloc.argtypes = [i64, i64, i64, i64, ctypes.c_int] + [vp] * 10 + [vp, vp, vp]
        L.ssm_scan_fwd_noalloc.restype = ctypes.c_int
        L.ssm_state_update_ex.argtypes = [i64, i64, i64, ctypes.c_int] + [vp] * 9 + [vp, vp]
        L.ssm_state_update_ex.restype = ctypes.c_int
        L.ssm_ssd_fwd_ex.argtypes = [i64] * 7 + [ctypes.c_int] + [vp] * 10 + [vp, sz, vp, vp]
        L.ssm_ssd_fwd_ex.restype = ctypes.c_int
        L.ssm_scan_bwd.argtypes = [i64] * 4 + [ctypes.c_int] + [vp] * 21 + [vp, sz, vp]
        L.ssm_scan_fwd_train.argtypes = [i64] * 4 + [ctypes.c_int] + [vp] * 12 + [vp]
        L.ssm_scan_fwd_train.restype = ctypes.c_int
        L.ssm_scan_bwd.restype = ctypes.c_int
        L.ssm_scan_bwd_workspace_size.argtypes = [i64] * 4
        L.ssm_scan_bwd_workspace_size.restype = ctypes.c_size_t
        L.ssm_scan_bwd_workspace_size_ex.argtypes = [i64] * 4 + [ctypes.c_int32]
        L.ssm_scan_bwd_workspace_size_ex.restype = ctypes.c_size_t
        L.ssm_decode_steps.argtypes = [i64] * 4 + [ctypes.c_int, vp, i64, vp] + [vp] * 8 + [vp, vp]
        L.ssm_decode_steps.restype = ctypes.c_int
        L.ssm_conv1d_fwd.argtypes = [i64] * 4 + [ctypes.c_int] + [vp] * 4 + [ctypes.c_int32, vp, vp, vp]
        L.ssm_conv1d_fwd.restype = ctypes.c_int
        L.ssm_conv1d_update.argtypes = [i64] * 3 + [ctypes.c_int] + [vp] * 4 + [ctypes.c_int32, vp, vp]
        L.ssm_conv1d_update.restype = ctypes.c_int
        L.ssm_status_string.argtypes = [ctypes.c_int]
        L.ssm_status_string.restype = ctypes.c_char_p
        L.ssm_version.argtypes = []
        L.ssm_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: expected float32 or bfloat16")


def _check(name, t, shape, dtype, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _call(fn_name, *args):
    rc = getattr(lib(), fn_name)(*args)
    if rc != 0:
        raise SSMError(fn_name, rc)


def scan_fwd(x, delta, A, Bm, Cm, D_skip=None, z=None, h0=None, *, y=None, h_final=None,
             return_final=True, variant=0, chunk_len=0, states_per_lane=0, workspace=None,
             delta_bias=None, delta_softplus=False):
    """Mamba-1 selective scan (ssm_scan_fwd).

    x, delta, z: (B, L, D); Bm, Cm: (B, L, N), all float32 or all bfloat16;
    A: (D, N) float32; D_skip: (D,) float32; h0: (B, D, N) float32.
    delta_bias: (D,) float32 added to delta, then softplus if delta_softplus.
    Returns (y, h_final); y has the input dtype, h_final is float32.
    """
    if x.dim() != 3 or Bm.dim() != 3:
        raise ValueError("x must be (B, L, D) and Bm (B, L, N)")
    B, L, D = x.shape
    N = Bm.shape[2]
    dev, dt = x.device, x.dtype
    code = _dtype_code(x)
    _check("x", x, (B, L, D), dt, dev)
    _check("delta", delta, (B, L, D), dt, dev)
    _check("z", z, (B, L, D), dt, dev)
    _check("Bm", Bm, (B, L, N), dt, dev)
    _check("Cm", Cm, (B, L, N), dt, dev)
    _check("A", A, (D, N), torch.float32, dev)
    _check("D_skip", D_skip, (D,), torch.float32, dev)
    _check("h0", h0, (B, D, N), torch.float32, dev)
    _check("delta_bias", delta_bias, (D,), torch.float32, dev)
    if y is None:
        y = torch.empty((B, L, D), dtype=dt, device=dev)
    _check("y", y, (B, L, D), dt, dev)
    if h_final is None and return_final:
        h_final = torch.empty((B, D, N), dtype=torch.float32, device=dev)
    _check("h_final", h_final, (B, D, N), torch.float32, dev)
    tun = Tuning(variant, chunk_len, states_per_lane)
    ws_bytes = lib().ssm_scan_fwd_workspace_size(B, L, D, N, ctypes.byref(tun))
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("ssm_scan_fwd_ex", B, L, D, N, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
          _ptr(D_skip), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_final), _ptr(workspace), ws_len,
          ctypes.byref(tun), _dopts(delta_bias, delta_softplus), _stream(dev))
    return y, h_final


def scan_fwd_noalloc(x, delta, A, Bm, Cm, D_skip=None, z=None, h0=None, *, y, h_final=None,
                     variant=0, chunk_len=0, states_per_lane=0, delta_bias=None, delta_softplus=False):
    """scan_fwd through ssm_scan_fwd_noalloc: the outputs are the caller's
    (y required, h_final optional) and the library's device scratch stands in
    for the workspace, so the call allocates nothing.  Returns (y, h_final)."""
    if x.dim() != 3 or Bm.dim() != 3:
        raise ValueError("x must be (B, L, D) and Bm (B, L, N)")
    B, L, D = x.shape
    N = Bm.shape[2]
    dev, dt = x.device, x.dtype
    code = _dtype_code(x)
    for name, t, shp, tdt in (("x", x, (B, L, D), dt), ("delta", delta, (B, L, D), dt),
                              ("z", z, (B, L, D), dt), ("Bm", Bm, (B, L, N), dt), ("Cm", Cm, (B, L, N), dt),
                              ("A", A, (D, N), torch.float32), ("D_skip", D_skip, (D,), torch.float32),
                              ("h0", h0, (B, D, N), torch.float32), ("delta_bias", delta_bias, (D,), torch.float32),
                              ("y", y, (B, L, D), dt), ("h_final", h_final, (B, D, N), torch.float32)):
        _check(name, t, shp, tdt, dev)
    tun = Tuning(variant, chunk_len, states_per_lane)
    _call("ssm_scan_fwd_noalloc", B, L, D, N, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
          _ptr(D_skip), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_final), ctypes.byref(tun),
          _dopts(delta_bias, delta_softplus), _stream(dev))
    return y, h_final


def scan_fwd_workspace_size(B, L, D, N, variant=0, chunk_len=0, states_per_lane=0) -> int:
    t = Tuning(variant, chunk_len, states_per_lane)
    return int(lib().ssm_scan_fwd_workspace_size(B, L, D, N, ctypes.byref(t)))


def state_update(state, x, delta, A, Bm, Cm, D_skip=None, z=None, *, y=None, delta_bias=None,
                 delta_softplus=False):
    """One decode step (ssm_state_update); `state` (S, D, N) float32 is updated in place.

    x, delta, z: (S, D); Bm, Cm: (S, N) float32 or bfloat16.  Returns y (S, D).
    """
    S, D, N = state.shape
    dev, dt = x.device, x.dtype
    code = _dtype_code(x)
    _check("state", state, (S, D, N), torch.float32, dev)
    for nm, t in (("x", x), ("delta", delta), ("z", z)):
        _check(nm, t, (S, D), dt, dev)
    _check("Bm", Bm, (S, N), dt, dev)
    _check("Cm", Cm, (S, N), dt, dev)
    _check("A", A, (D, N), torch.float32, dev)
    _check("D_skip", D_skip, (D,), torch.float32, dev)
    _check("delta_bias", delta_bias, (D,), torch.float32, dev)
    if y is None:
        y = torch.empty((S, D), dtype=dt, device=dev)
    _check("y", y, (S, D), dt, dev)
    _call("ssm_state_update_ex", S, D, N, code, _ptr(state), _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm),
          _ptr(Cm), _ptr(D_skip), _ptr(z), _ptr(y), _dopts(delta_bias, delta_softplus), _stream(dev))
    return y


def ssd_fwd(x, dt, A, Bm, Cm, D_skip=None, z=None, h0=None, *, chunk=256, y=None, h_final=None,
            return_final=True, workspace=None, dt_bias=None, dt_softplus=False):
    """Mamba-2 SSD chunked scan (ssm_ssd_fwd).

    x, z: (B, L, H, P); dt: (B, L, H); Bm, Cm: (B, L, G, N), all bfloat16 or all float32;
    A, D_skip: (H,) float32; h0: (B, H, P, N) float32.  dt_bias: (H,)
    float32 added to dt, then softplus if dt_softplus.  Returns (y, h_final).
    """
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    dev, typ = x.device, x.dtype
    code = _dtype_code(x)
    _check("x", x, (B, L, H, P), typ, dev)
    _check("dt", dt, (B, L, H), typ, dev)
    _check("z", z, (B, L, H, P), typ, dev)
    _check("Bm", Bm, (B, L, G, N), typ, dev)
    _check("Cm", Cm, (B, L, G, N), typ, dev)
    _check("A", A, (H,), torch.float32, dev)
    _check("D_skip", D_skip, (H,), torch.float32, dev)
    _check("h0", h0, (B, H, P, N), torch.float32, dev)
    _check("dt_bias", dt_bias, (H,), torch.float32, dev)
    if y is None:
        y = torch.empty((B, L, H, P), dtype=typ, device=dev)
    _check("y", y, (B, L, H, P), typ, dev)
    if h_final is None and return_final:
        h_final = torch.empty((B, H, P, N), dtype=torch.float32, device=dev)
    _check("h_final", h_final, (B, H, P, N), torch.float32, dev)
    ws_bytes = lib().ssm_ssd_fwd_workspace_size(B, L, H, P, G, N, chunk)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("ssm_ssd_fwd_ex", B, L, H, P, G, N, chunk, code, _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm),
          _ptr(Cm), _ptr(D_skip), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_final), _ptr(workspace),
          ws_len, _dopts(dt_bias, dt_softplus), _stream(dev))
    return y, h_final


def ssd_fwd_workspace_size(B, L, H, P, G, N, chunk) -> int:
    return int(lib().ssm_ssd_fwd_workspace_size(B, L, H, P, G, N, chunk))


def version() -> int:
    return int(lib().ssm_version())


def _act_code(activation) -> int:
    if activation in (None, "none", "identity"):
        return 0
    if activation == "silu":
        return 1
    raise ValueError(f"activation must be None or 'silu', got {activation!r}")


def conv1d_fwd(x, w, bias=None, state=None, *, activation="silu", y=None, state_out=None,
               return_state=True):
    """Short causal convolution ahead of the scan (ssm_conv1d_fwd).

    x: (B, L, D) float32 or bfloat16; w: (D, K) float32; bias: (D,) float32;
    state: (B, D, K-1) float32, the K-1 previous inputs of each channel,
    oldest first (zeros when None).  Returns (y, state_out); y has the input
    dtype, state_out (B, D, K-1) float32 (None if return_state is False).
    """
    if x.dim() != 3 or w.dim() != 2:
        raise ValueError("x must be (B, L, D) and w (D, K)")
    B, L, D = x.shape
    K = w.shape[1]
    dev, dt = x.device, x.dtype
    code = _dtype_code(x)
    _check("x", x, (B, L, D), dt, dev)
    _check("w", w, (D, K), torch.float32, dev)
    _check("bias", bias, (D,), torch.float32, dev)
    _check("state", state, (B, D, K - 1), torch.float32, dev)
    if y is None:
        y = torch.empty((B, L, D), dtype=dt, device=dev)
    _check("y", y, (B, L, D), dt, dev)
    if state_out is None and return_state:
        state_out = torch.empty((B, D, K - 1), dtype=torch.float32, device=dev)
    _check("state_out", state_out, (B, D, K - 1), torch.float32, dev)
    _call("ssm_conv1d_fwd", B, L, D, K, code, _ptr(x), _ptr(w), _ptr(bias), _ptr(state),
          _act_code(activation), _ptr(y), _ptr(state_out), _stream(dev))
    return y, state_out


def conv1d_update(state, x, w, bias=None, *, activation="silu", y=None):
    """One decode step of the causal convolution (ssm_conv1d_update); `state`
    (S, D, K-1) float32 is updated in place.  x: (S, D).  Returns y (S, D)."""
    S, D, Km1 = state.shape
    K = Km1 + 1
    dev, dt = x.device, x.dtype
    code = _dtype_code(x)
    _check("state", state, (S, D, Km1), torch.float32, dev)
    _check("x", x, (S, D), dt, dev)
    _check("w", w, (D, K), torch.float32, dev)
    _check("bias", bias, (D,), torch.float32, dev)
    if y is None:
        y = torch.empty((S, D), dtype=dt, device=dev)
    _check("y", y, (S, D), dt, dev)
    _call("ssm_conv1d_update", S, D, K, code, _ptr(state), _ptr(x), _ptr(w), _ptr(bias),
          _act_code(activation), _ptr(y), _stream(dev))
    return y


def decode_steps(state_pool, x, delta, A, Bm, Cm, D_skip=None, z=None, *, slots=None, y=None,
                 delta_bias=None, delta_softplus=False):
    """T decode tokens for S sequences whose states are rows of a pool
    (ssm_decode_steps).  state_pool (P, D, N) float32 is updated in place;
    x, delta, z: (S, T, D); Bm, Cm: (S, T, N); slots: (S,) int32 device tensor
    of pool rows (None: row s for sequence s; negative: skip).  Returns y."""
    if x.dim() != 3:
        raise ValueError("x must be (S, T, D)")
    S, T, D = x.shape
    Pr, Dp, N = state_pool.shape
    if Dp != D:
        raise ValueError("state_pool must be (pool_rows, D, N)")
    dev, dt = x.device, x.dtype
    code = _dtype_code(x)
    _check("state_pool", state_pool, (Pr, D, N), torch.float32, dev)
    for nm, t in (("x", x), ("delta", delta), ("z", z)):
        _check(nm, t, (S, T, D), dt, dev)
    _check("Bm", Bm, (S, T, N), dt, dev)
    _check("Cm", Cm, (S, T, N), dt, dev)
    _check("A", A, (D, N), torch.float32, dev)
    _check("D_skip", D_skip, (D,), torch.float32, dev)
    _check("delta_bias", delta_bias, (D,), torch.float32, dev)
    _check("slots", slots, (S,), torch.int32, dev)
    if y is None:
        y = torch.empty((S, T, D), dtype=dt, device=dev)
    _check("y", y, (S, T, D), dt, dev)
    _call("ssm_decode_steps", S, T, D, N, code, _ptr(state_pool), Pr, _ptr(slots), _ptr(x),
          _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D_skip), _ptr(z), _ptr(y),
          _dopts(delta_bias, delta_softplus), _stream(dev))
    return y


def scan_bwd_workspace_size(B, L, D, N, saved_states=False) -> int:
    """Workspace bytes of scan_bwd; saved_states: the call passes h_ckpt."""
    return int(lib().ssm_scan_bwd_workspace_size_ex(B, L, D, N, 1 if saved_states else 0))


def scan_fwd_train(x, delta, A, Bm, Cm, D_skip=None, z=None, h0=None, *, delta_bias=None,
                   delta_softplus=False):
    """scan_fwd for a training step (ssm_scan_fwd_train): returns y, h_final
    and h_ckpt (B, ceil(L/8), D, N), the state entering every 8-token
    segment, for scan_bwd(..., h_ckpt=h_ckpt)."""
    B, L, D = x.shape
    N = A.shape[1]
    dev, dt = x.device, x.dtype
    code = _dtype_code(x)
    for nm, t in (("x", x), ("delta", delta), ("z", z)):
        _check(nm, t, (B, L, D), dt, dev)
    _check("Bm", Bm, (B, L, N), dt, dev)
    _check("Cm", Cm, (B, L, N), dt, dev)
    _check("A", A, (D, N), torch.float32, dev)
    _check("D_skip", D_skip, (D,), torch.float32, dev)
    _check("h0", h0, (B, D, N), torch.float32, dev)
    _check("delta_bias", delta_bias, (D,), torch.float32, dev)
    y = torch.empty((B, L, D), dtype=dt, device=dev)
    hf = torch.empty((B, D, N), dtype=torch.float32, device=dev)
    ck = torch.empty((B, (L + 7) // 8, D, N), dtype=torch.float32, device=dev)
    _call("ssm_scan_fwd_train", B, L, D, N, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
          _ptr(D_skip), _ptr(z), _ptr(h0), _ptr(y), _ptr(hf), _ptr(ck), _dopts(delta_bias, delta_softplus),
          _stream(dev))
    return y, hf, ck


def scan_bwd(x, delta, A, Bm, Cm, D_skip=None, z=None, h0=None, dy=None, dh_final=None, *,
             delta_bias=None, delta_softplus=False, want_dh0=True, want_dbias=False, workspace=None,
             h_ckpt=None):
    """Gradients of scan_fwd (ssm_scan_bwd) for the output gradient dy and
    the final-state gradient dh_final (None = zero).  Returns a dict: dx,
    ddelta, dz (input dtype; dz None without z), dA, dB, dC (float32), dD
    (None without D_skip), dh0 (None unless want_dh0), dbias (None unless
    want_dbias)."""
    B, L, D = x.shape
    N = A.shape[1]
    dev, dt = x.device, x.dtype
    code = _dtype_code(x)
    for nm, t in (("x", x), ("delta", delta), ("z", z), ("dy", dy)):
        _check(nm, t, (B, L, D), dt, dev)
    if dy is None:
        raise ValueError("dy is required")
    _check("Bm", Bm, (B, L, N), dt, dev)
    _check("Cm", Cm, (B, L, N), dt, dev)
    _check("A", A, (D, N), torch.float32, dev)
    _check("D_skip", D_skip, (D,), torch.float32, dev)
    _check("h0", h0, (B, D, N), torch.float32, dev)
    _check("dh_final", dh_final, (B, D, N), torch.float32, dev)
    _check("delta_bias", delta_bias, (D,), torch.float32, dev)
    _check("h_ckpt", h_ckpt, (B, (L + 7) // 8, D, N), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dx": torch.empty((B, L, D), dtype=dt, device=dev),
           "ddelta": torch.empty((B, L, D), dtype=dt, device=dev),
           "dz": torch.empty((B, L, D), dtype=dt, device=dev) if z is not None else None,
           "dA": torch.empty((D, N), **f32), "dB": torch.empty((B, L, N), **f32),
           "dC": torch.empty((B, L, N), **f32),
           "dD": torch.empty((D,), **f32) if D_skip is not None else None,
           "dh0": torch.empty((B, D, N), **f32) if want_dh0 else None,
           "dbias": torch.empty((D,), **f32) if want_dbias else None}
    need = scan_bwd_workspace_size(B, L, D, N, saved_states=h_ckpt is not None)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("ssm_scan_bwd", B, L, D, N, code, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
          _ptr(D_skip), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dh_final), _ptr(h_ckpt), _ptr(out["dx"]),
          _ptr(out["ddelta"]), _ptr(out["dz"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
          _ptr(out["dD"]), _ptr(out["dh0"]), _ptr(out["dbias"]), _dopts(delta_bias, delta_softplus),
          _ptr(workspace), wsb, _stream(dev))
    return out
