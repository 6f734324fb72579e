"""ctypes binding of libfalcon.so.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind ``falcon_fwd``, every step of the Falcon-1 backward pass in
those behind ``falcon_bwd``.  PyTorch provides device memory and the
current stream.  The binding raises if the library is missing; there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
import pathlib
from dataclasses import dataclass
from typing import Optional

PKG = pathlib.Path(__file__).resolve().parent
LIB_PATH = PKG / "libfalcon.so"

ABI_VERSION = 1
MAX_WINDOW = 8
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
VARIANTS = {"F1": 1, "F2": 2, "F3": 3, "F1A": 11, "F2A": 12, "F3A": 13}
PER_COLUMN = (2, 12)
DTYPES = {"bf16": 0, "f32": 1}
PHIS = {"rmsnorm": 0, "identity": 1}


class FalconStateC(ctypes.Structure):
    _fields_ = [("S", ctypes.c_void_p), ("x_next", ctypes.c_void_p),
                ("tail_x", ctypes.c_void_p), ("tail_y", ctypes.c_void_p),
                ("n_tail", ctypes.c_int), ("fresh", ctypes.c_int)]


class FalconFwdArgsC(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int), ("variant", ctypes.c_int), ("dtype", ctypes.c_int),
                ("phi", ctypes.c_int),
                ("batch", ctypes.c_int), ("heads", ctypes.c_int), ("seqlen", ctypes.c_int),
                ("dk", ctypes.c_int), ("dv", ctypes.c_int),
                ("chunk", ctypes.c_int), ("window", ctypes.c_int),
                ("eps", ctypes.c_float), ("eps_gamma", ctypes.c_float), ("eps_rms", ctypes.c_float),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("lambda_", ctypes.c_void_p),
                ("state_in", ctypes.POINTER(FalconStateC)), ("state_out", ctypes.POINTER(FalconStateC)),
                ("o", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class FalconBwdArgsC(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int), ("variant", ctypes.c_int), ("dtype", ctypes.c_int),
                ("phi", ctypes.c_int),
                ("batch", ctypes.c_int), ("heads", ctypes.c_int), ("seqlen", ctypes.c_int),
                ("dk", ctypes.c_int), ("dv", ctypes.c_int),
                ("eps", ctypes.c_float), ("eps_gamma", ctypes.c_float), ("eps_rms", ctypes.c_float),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("lambda_", ctypes.c_void_p),
                ("state_in", ctypes.POINTER(FalconStateC)),
                ("d_o", ctypes.c_void_p), ("d_S_out", ctypes.c_void_p), ("d_x_next_out", ctypes.c_void_p),
                ("d_q", ctypes.c_void_p), ("d_k", ctypes.c_void_p), ("d_v", ctypes.c_void_p),
                ("d_beta", ctypes.c_void_p), ("d_lambda", ctypes.c_void_p),
                ("d_S_in", ctypes.c_void_p), ("d_x_next_in", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


EXPORTS = ("falcon_fwd", "falcon_fwd_validate", "falcon_fwd_workspace_size",
           "falcon_fwd_profile", "falcon_fwd_noalloc", "falcon_kernel_name", "falcon_status_str",
           "falcon_abi_version", "falcon_bwd", "falcon_bwd_validate", "falcon_bwd_workspace_size",
           "falcon_bwd_profile", "falcon_bwd_kernel_name")
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


def load_library(path: Optional[os.PathLike] = None) -> ctypes.CDLL:
    """Load libfalcon.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = pathlib.Path(path) if path else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"{p} not found: build it with `python -m linear_recurrent_weight_amd.build`")
    lib = ctypes.CDLL(str(p))
    lib.falcon_fwd.argtypes = [ctypes.POINTER(FalconFwdArgsC), ctypes.c_void_p]
    lib.falcon_fwd.restype = ctypes.c_int
    lib.falcon_fwd_validate.argtypes = [ctypes.POINTER(FalconFwdArgsC)]
    lib.falcon_fwd_validate.restype = ctypes.c_int
    lib.falcon_fwd_workspace_size.argtypes = [ctypes.POINTER(FalconFwdArgsC)]
    lib.falcon_fwd_workspace_size.restype = ctypes.c_size_t
    lib.falcon_status_str.argtypes = [ctypes.c_int]
    lib.falcon_status_str.restype = ctypes.c_char_p
    lib.falcon_fwd_profile.argtypes = [ctypes.POINTER(FalconFwdArgsC), ctypes.c_void_p,
                                       ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    lib.falcon_fwd_profile.restype = ctypes.c_int
    lib.falcon_fwd_noalloc.argtypes = [ctypes.POINTER(FalconFwdArgsC), ctypes.c_void_p]
    lib.falcon_fwd_noalloc.restype = ctypes.c_int
    lib.falcon_kernel_name.argtypes = [ctypes.POINTER(FalconFwdArgsC), ctypes.c_int]
    lib.falcon_kernel_name.restype = ctypes.c_char_p
    lib.falcon_bwd.argtypes = [ctypes.POINTER(FalconBwdArgsC), ctypes.c_void_p]
    lib.falcon_bwd.restype = ctypes.c_int
    lib.falcon_bwd_validate.argtypes = [ctypes.POINTER(FalconBwdArgsC)]
    lib.falcon_bwd_validate.restype = ctypes.c_int
    lib.falcon_bwd_workspace_size.argtypes = [ctypes.POINTER(FalconBwdArgsC)]
    lib.falcon_bwd_workspace_size.restype = ctypes.c_size_t
    lib.falcon_bwd_profile.argtypes = [ctypes.POINTER(FalconBwdArgsC), ctypes.c_void_p,
                                       ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    lib.falcon_bwd_profile.restype = ctypes.c_int
    lib.falcon_bwd_kernel_name.argtypes = [ctypes.POINTER(FalconBwdArgsC), ctypes.c_int]
    lib.falcon_bwd_kernel_name.restype = ctypes.c_char_p
    lib.falcon_abi_version.argtypes = []
    lib.falcon_abi_version.restype = ctypes.c_int
    if lib.falcon_abi_version() != ABI_VERSION:
        raise RuntimeError("libfalcon.so ABI version mismatch")
    if path is None:
        _lib = lib
    return lib


class FalconError(RuntimeError):
    def __init__(self, status: int, lib=None):
        lib = lib or load_library()
        super().__init__(f"falcon call failed: {lib.falcon_status_str(status).decode()} ({status})")
        self.status = status


@dataclass
class FalconState:
    """Boundary state (torch tensors on the device): S [B,H,dk,dv],
    x_next [B,H,dk], tail_x [B,H,W-1,dk], tail_y [B,H,W-1,dv], fp32."""
    S: "object"
    x_next: "object"
    tail_x: "object"
    tail_y: "object"
    n_tail: int = 0
    fresh: bool = False

    @staticmethod
    def empty(batch, heads, dk, dv, window, device):
        import torch
        f = dict(dtype=torch.float32, device=device)
        h = max(window - 1, 0)
        return FalconState(torch.zeros(batch, heads, dk, dv, **f), torch.zeros(batch, heads, dk, **f),
                           torch.zeros(batch, heads, h, dk, **f), torch.zeros(batch, heads, h, dv, **f))

    def to_c(self) -> FalconStateC:
        def ptr(t):
            return t.data_ptr() if (t is not None and t.numel() > 0) else None
        return FalconStateC(ptr(self.S), ptr(self.x_next), ptr(self.tail_x), ptr(self.tail_y),
                            int(self.n_tail), int(bool(self.fresh)))


def make_args(*, variant, dtype, batch, heads, seqlen, dk, dv, chunk=64, window=1, eps=1e-6,
              eps_gamma=1e-3, eps_rms=1e-6, phi="rmsnorm", q=None, k=None, v=None, beta=None,
              lam=None, o=None, state_in=None, state_out=None, workspace=None,
              workspace_bytes=0) -> FalconFwdArgsC:
    """Fill the C argument struct.  Tensor arguments may be torch tensors or
    raw integer addresses."""
    def addr(t):
        if t is None:
            return None
        return t if isinstance(t, int) else t.data_ptr()
    a = FalconFwdArgsC()
    a.abi_version = ABI_VERSION
    a.variant = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    a.dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    a.phi = PHIS[phi] if isinstance(phi, str) else int(phi)
    a.batch, a.heads, a.seqlen, a.dk, a.dv = batch, heads, seqlen, dk, dv
    a.chunk, a.window = chunk, window
    a.eps, a.eps_gamma, a.eps_rms = eps, eps_gamma, eps_rms
    a.q, a.k, a.v, a.beta, a.lambda_, a.o = map(addr, (q, k, v, beta, lam, o))
    a.state_in = ctypes.pointer(state_in) if state_in is not None else None
    a.state_out = ctypes.pointer(state_out) if state_out is not None else None
    a.workspace = addr(workspace)
    a.workspace_bytes = workspace_bytes
    return a


def _check_tensor(name, t, shape, dtype, device):
    """Raise ValueError unless `t` is a contiguous tensor of exactly this
    shape and dtype on `device`."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def check_fwd_tensors(q, k, v, beta, lam, *, variant, window, state=None, out=None, workspace=None):
    """Validate every tensor of a forward call against the shapes the C ABI
    assumes (the library sees only pointers and sizes, so a mismatch here
    would read or write past a buffer on the GPU).  Returns
    (B, H, T, dk, dv, torch dtype, device).  Raises ValueError."""
    import torch
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-d tensor [B,H,T,dk]")
    dt = q.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    dev = q.device
    B, H, T, dk = q.shape
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("v must be a 4-d tensor [B,H,T,dv]")
    dv = v.shape[-1]
    var = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    if window < 1 or window > MAX_WINDOW:
        raise ValueError(f"window must lie in [1, {MAX_WINDOW}]")
    _check_tensor("q", q, (B, H, T, dk), dt, dev)
    _check_tensor("k", k, (B, H, T, dk), dt, dev)
    _check_tensor("v", v, (B, H, T, dv), dt, dev)
    f32 = torch.float32
    _check_tensor("beta", beta, (B, H, T, dv) if var in PER_COLUMN else (B, H, T), f32, dev)
    _check_tensor("lambda", lam, (B, H, T), f32, dev)
    if out is not None:
        _check_tensor("out", out, (B, H, T, dv), dt, dev)
    if state is not None:
        _check_tensor("state.S", state.S, (B, H, dk, dv), f32, dev)
        if not state.fresh:
            _check_tensor("state.x_next", state.x_next, (B, H, dk), f32, dev)
        if not 0 <= int(state.n_tail) <= window - 1:
            raise ValueError(f"state.n_tail = {state.n_tail} must lie in [0, window - 1 = {window - 1}]")
        if state.fresh and state.n_tail:
            raise ValueError("a fresh state carries no tail pairs")
        if state.n_tail > 0:
            _check_tensor("state.tail_x", state.tail_x, (B, H, window - 1, dk), f32, dev)
            _check_tensor("state.tail_y", state.tail_y, (B, H, window - 1, dv), f32, dev)
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return B, H, T, dk, dv, dt, dev


def fwd(q, k, v, beta, lam, *, variant="F1", chunk=64, window=1, eps=1e-6, eps_gamma=1e-3,
        eps_rms=1e-6, phi="rmsnorm", state: Optional[FalconState] = None, want_state=True,
        out=None, workspace=None, stream=None):
    """Falcon forward pass on the GPU.

    q, k: [B,H,T,dk]; v: [B,H,T,dv] (all bf16 or all fp32, contiguous, on the
    device); beta: [B,H,T] fp32 ([B,H,T,dv] for F2 and F2A); lam: [B,H,T] fp32.
    `stream` is a torch.cuda.Stream (default: the current stream); the
    output, the state and any temporary workspace are allocated on it, so the
    caching allocator never hands them to other streams while the kernels run.
    Returns (o [B,H,T,dv], FalconState or None).  Raises ValueError on a
    tensor whose shape, dtype, device or layout does not match.
    """
    import torch
    lib = load_library()
    if not (isinstance(q, torch.Tensor) and q.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    B, H, T, dk, dv, dt, dev = check_fwd_tensors(q, k, v, beta, lam, variant=variant, window=window,
                                                  state=state, out=out, workspace=workspace)
    dtype = "bf16" if dt == torch.bfloat16 else "f32"
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif not isinstance(stream, torch.cuda.Stream):
        raise ValueError("stream must be a torch.cuda.Stream")
    with torch.cuda.stream(stream):
        o = out if out is not None else torch.empty(B, H, T, dv, dtype=dt, device=dev)
        st_in = state.to_c() if state is not None else None
        st_out_t = FalconState.empty(B, H, dk, dv, window, dev) if want_state else None
        st_out = st_out_t.to_c() if st_out_t is not None else None
        args = make_args(variant=variant, dtype=dtype, batch=B, heads=H, seqlen=T, dk=dk, dv=dv,
                         chunk=chunk, window=window, eps=eps, eps_gamma=eps_gamma, eps_rms=eps_rms,
                         phi=phi, q=q, k=k, v=v, beta=beta, lam=lam, o=o, state_in=st_in,
                         state_out=st_out)
        nbytes = lib.falcon_fwd_workspace_size(ctypes.byref(args))
        if nbytes:
            if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
                workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            args.workspace = workspace.data_ptr()
            args.workspace_bytes = workspace.numel() * workspace.element_size()
        rc = lib.falcon_fwd(ctypes.byref(args), ctypes.c_void_p(stream.cuda_stream))
    if rc != OK:
        raise FalconError(rc, lib)
    if st_out_t is not None:
        st_out_t.n_tail = args.state_out.contents.n_tail
        st_out_t.fresh = bool(args.state_out.contents.fresh)
    return o, st_out_t


def workspace_size(**kw) -> int:
    lib = load_library()
    return int(lib.falcon_fwd_workspace_size(ctypes.byref(make_args(**kw))))


def validate(**kw) -> int:
    lib = load_library()
    return int(lib.falcon_fwd_validate(ctypes.byref(make_args(**kw))))


def make_bwd_args(*, dtype, batch, heads, seqlen, dk, dv, variant="F1", eps=1e-6, eps_gamma=1e-3,
                  eps_rms=1e-6, phi="rmsnorm", q=None, k=None, v=None, beta=None, lam=None,
                  state_in=None, d_o=None, d_S_out=None, d_x_next_out=None, d_q=None, d_k=None,
                  d_v=None, d_beta=None, d_lam=None, d_S_in=None, d_x_next_in=None, workspace=None,
                  workspace_bytes=0) -> FalconBwdArgsC:
    """Fill the backward's C argument struct (tensors or raw addresses)."""
    def addr(t):
        if t is None:
            return None
        return t if isinstance(t, int) else t.data_ptr()
    a = FalconBwdArgsC()
    a.abi_version = ABI_VERSION
    a.variant = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    a.dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    a.phi = PHIS[phi] if isinstance(phi, str) else int(phi)
    a.batch, a.heads, a.seqlen, a.dk, a.dv = batch, heads, seqlen, dk, dv
    a.eps, a.eps_gamma, a.eps_rms = eps, eps_gamma, eps_rms
    a.q, a.k, a.v, a.beta, a.lambda_ = map(addr, (q, k, v, beta, lam))
    a.state_in = ctypes.pointer(state_in) if state_in is not None else None
    a.d_o, a.d_S_out, a.d_x_next_out = map(addr, (d_o, d_S_out, d_x_next_out))
    a.d_q, a.d_k, a.d_v, a.d_beta, a.d_lambda = map(addr, (d_q, d_k, d_v, d_beta, d_lam))
    a.d_S_in, a.d_x_next_in = addr(d_S_in), addr(d_x_next_in)
    a.workspace = addr(workspace)
    a.workspace_bytes = workspace_bytes
    return a


def bwd(q, k, v, beta, lam, d_o, *, d_S_out=None, d_x_next_out=None, eps=1e-6, eps_gamma=1e-3,
        eps_rms=1e-6, phi="rmsnorm", state: Optional[FalconState] = None, workspace=None, stream=None):
    """Falcon-1 backward pass on the GPU: the gradients of a loss through
    ``fwd(..., variant="F1")`` on the same inputs and state, given d_o
    [B,H,T,dv] (the inputs' dtype) and optionally d_S_out [B,H,dk,dv] and
    d_x_next_out [B,H,dk] (fp32).  Returns a dict with dq, dk, dv (inputs'
    dtype), dbeta, dlam [B,H,T], dS_in [B,H,dk,dv] and dx_next_in [B,H,dk]
    (fp32).  Raises ValueError on a tensor that does not match."""
    import torch
    lib = load_library()
    if not (isinstance(q, torch.Tensor) and q.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if state is not None and int(state.n_tail) != 0:
        raise ValueError("the Falcon-1 backward takes no tail pairs")
    B, H, T, dk, dv, dt, dev = check_fwd_tensors(q, k, v, beta, lam, variant="F1", window=1,
                                                  state=state, workspace=workspace)
    f32 = torch.float32
    _check_tensor("d_o", d_o, (B, H, T, dv), dt, dev)
    if d_S_out is not None:
        _check_tensor("d_S_out", d_S_out, (B, H, dk, dv), f32, dev)
    if d_x_next_out is not None:
        _check_tensor("d_x_next_out", d_x_next_out, (B, H, dk), f32, dev)
    dtype = "bf16" if dt == torch.bfloat16 else "f32"
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif not isinstance(stream, torch.cuda.Stream):
        raise ValueError("stream must be a torch.cuda.Stream")
    with torch.cuda.stream(stream):
        g = dict(dq=torch.empty(B, H, T, dk, dtype=dt, device=dev),
                 dk=torch.empty(B, H, T, dk, dtype=dt, device=dev),
                 dv=torch.empty(B, H, T, dv, dtype=dt, device=dev),
                 dbeta=torch.empty(B, H, T, dtype=f32, device=dev),
                 dlam=torch.empty(B, H, T, dtype=f32, device=dev),
                 dS_in=torch.empty(B, H, dk, dv, dtype=f32, device=dev),
                 dx_next_in=torch.empty(B, H, dk, dtype=f32, device=dev))
        st_in = state.to_c() if state is not None else None
        args = make_bwd_args(dtype=dtype, batch=B, heads=H, seqlen=T, dk=dk, dv=dv, eps=eps,
                             eps_gamma=eps_gamma, eps_rms=eps_rms, phi=phi, q=q, k=k, v=v, beta=beta,
                             lam=lam, state_in=st_in, d_o=d_o, d_S_out=d_S_out,
                             d_x_next_out=d_x_next_out, d_q=g["dq"], d_k=g["dk"], d_v=g["dv"],
                             d_beta=g["dbeta"], d_lam=g["dlam"], d_S_in=g["dS_in"],
                             d_x_next_in=g["dx_next_in"])
        nbytes = lib.falcon_bwd_workspace_size(ctypes.byref(args))
        if nbytes:
            if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
                workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            args.workspace = workspace.data_ptr()
            args.workspace_bytes = workspace.numel() * workspace.element_size()
        rc = lib.falcon_bwd(ctypes.byref(args), ctypes.c_void_p(stream.cuda_stream))
    if rc != OK:
        raise FalconError(rc, lib)
    return g
