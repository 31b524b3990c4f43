"""ctypes binding of libgdn.so: the C ABI of include/gdn.h under the same names.

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's kernels. There
is no fallback: if libgdn.so is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn.so")

VARIANTS = {"fg2": 0, "kda": 1, "gdn": 2, "deltaproduct": 3, "asym": 4}
DTYPE_F32, DTYPE_BF16 = 0, 1
STABILIZE_MODES = {"clip_decay": 1, "project_j": 2}
STATUS = {0: "GDN_OK", -1: "GDN_ERR_ARG", -2: "GDN_ERR_UNSUPPORTED", -3: "GDN_ERR_WORKSPACE",
          -4: "GDN_ERR_HIP"}


class GdnArgs(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("dk", ctypes.c_int64), ("dv", ctypes.c_int64),
                ("chunk", ctypes.c_int32), ("n_h", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("alpha", ctypes.c_void_p), ("beta", ctypes.c_void_p),
                ("beta_v", ctypes.c_void_p), ("j", ctypes.c_void_p), ("eta", ctypes.c_void_p),
                ("s0", ctypes.c_void_p), ("s_final", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("stabilize", ctypes.c_int32)]


class GdnGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dq", "dk", "dv", "dalpha", "dbeta", "dbeta_v", "dj", "deta", "ds0")]


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({gdn_status_str(status)})")


_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it first "
                               "(python -m gated_delta_rule_69_amd.build)")
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER(GdnArgs)
        lib.gdn_workspace_bytes.argtypes = [P]
        lib.gdn_workspace_bytes.restype = ctypes.c_size_t
        lib.gdn_chunk_fwd.argtypes = [P, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.gdn_chunk_fwd.restype = ctypes.c_int
        lib.gdn_final_state.argtypes = [P, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.gdn_final_state.restype = ctypes.c_int
        for name in ("gdn_chunk_prepare", "gdn_chunk_scan"):
            fn = getattr(lib, name)
            fn.argtypes = [P, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
            fn.restype = ctypes.c_int
        lib.gdn_chunk_fwd_static.argtypes = [P, ctypes.c_void_p]
        lib.gdn_chunk_fwd_static.restype = ctypes.c_int
        lib.gdn_recurrent_step.argtypes = [P, ctypes.c_void_p, ctypes.c_void_p]
        lib.gdn_recurrent_step.restype = ctypes.c_int
        lib.gdn_bwd_workspace_bytes.argtypes = [P]
        lib.gdn_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.gdn_recurrent_bwd.argtypes = [P, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(GdnGrads),
                                          ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.gdn_recurrent_bwd.restype = ctypes.c_int
        lib.gdn_asym_stabilize.argtypes = [P, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.gdn_asym_stabilize.restype = ctypes.c_int
        lib.gdn_status_str.argtypes = [ctypes.c_int]
        lib.gdn_status_str.restype = ctypes.c_char_p
        lib.gdn_abi_version.argtypes = []
        lib.gdn_abi_version.restype = ctypes.c_int
        _lib = lib
        return lib


def gdn_status_str(status: int) -> str:
    return load_library().gdn_status_str(int(status)).decode()


def gdn_abi_version() -> int:
    return int(load_library().gdn_abi_version())


# ---- tensor marshalling -----------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, device, dtype=None):
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a device tensor on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def make_args(variant, q, k, v, alpha, beta=None, *, chunk=64, n_h=None, beta_v=None, j=None,
              eta=None, s0=None, s_final=None, o=None, stabilize=None) -> GdnArgs:
    import torch
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    dev = k.device
    io = k.dtype
    if io not in (torch.float32, torch.bfloat16):
        raise ValueError("inputs must be float32 or bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta),
                    ("beta_v", beta_v), ("j", j), ("eta", eta), ("o", o)):
        _check(t, name, dev, io)
    for name, t in (("s0", s0), ("s_final", s_final)):
        _check(t, name, dev, torch.float32)
    dp = variant == "deltaproduct"
    B, T, H = k.shape[0], k.shape[1], k.shape[2]
    if dp:
        nh = k.shape[3]
        if n_h is not None and n_h != nh:
            raise ValueError("n_h does not match k.shape[3]")
    else:
        nh = 1
    a = GdnArgs()
    a.variant = VARIANTS[variant]
    a.dtype = DTYPE_BF16 if io == torch.bfloat16 else DTYPE_F32
    a.B, a.T, a.H = B, T, H
    a.dk, a.dv = k.shape[-1], v.shape[-1]
    a.chunk, a.n_h = int(chunk), int(nh)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.alpha, a.beta, a.beta_v = _ptr(alpha), _ptr(beta), _ptr(beta_v)
    a.j, a.eta = _ptr(j), _ptr(eta)
    a.s0, a.s_final, a.o = _ptr(s0), _ptr(s_final), _ptr(o)
    if stabilize is not None and stabilize not in STABILIZE_MODES:
        raise ValueError(f"unknown stabilizer mode {stabilize!r}")
    a.stabilize = 0 if stabilize is None else STABILIZE_MODES[stabilize]
    a._keep = (q, k, v, alpha, beta, beta_v, j, eta, s0, s_final, o)  # lifetimes
    return a


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def gdn_workspace_bytes(args: GdnArgs) -> int:
    return int(load_library().gdn_workspace_bytes(ctypes.byref(args)))


def _workspace(args, ws, device):
    import torch
    need = gdn_workspace_bytes(args)
    if need == 0:
        raise GdnError(-1, "gdn_workspace_bytes")
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    if ws.numel() < need:
        raise GdnError(-3, "workspace")
    return ws


def gdn_chunk_fwd(variant, q, k, v, alpha, beta=None, *, chunk=64, beta_v=None, j=None,
                  eta=None, s0=None, s_final=None, o=None, workspace=None, stream=None,
                  want_state=True, stabilize=None):
    """Chunkwise forward. Returns (o, s_final); allocates o / s_final / workspace
    when not given (torch device memory). s_final may be s0 (updated in place).
    stabilize ("clip_decay" / "project_j", ASYM only) applies that GDN2 stabiliser
    to every token inside the pass."""
    import torch
    dev = k.device
    B, T, H = k.shape[:3]
    dk, dv = k.shape[-1], v.shape[-1]
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=k.dtype, device=dev)
    if s_final is None and want_state:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    a = make_args(variant, q, k, v, alpha, beta, chunk=chunk, beta_v=beta_v, j=j, eta=eta,
                  s0=s0, s_final=s_final, o=o, stabilize=stabilize)
    ws = _workspace(a, workspace, dev)
    st = load_library().gdn_chunk_fwd(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()),
                                      ctypes.c_size_t(ws.numel()), _stream(stream))
    if st != 0:
        raise GdnError(st, "gdn_chunk_fwd")
    return o, s_final


def gdn_final_state(variant, k, v, alpha, beta=None, *, chunk=64, beta_v=None, j=None,
                    eta=None, s0=None, s_final=None, workspace=None, stream=None, stabilize=None):
    """State-only chunkwise forward. Returns s_final."""
    import torch
    dev = k.device
    B, T, H = k.shape[:3]
    dk, dv = k.shape[-1], v.shape[-1]
    if s_final is None:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    a = make_args(variant, None, k, v, alpha, beta, chunk=chunk, beta_v=beta_v, j=j, eta=eta,
                  s0=s0, s_final=s_final, o=None, stabilize=stabilize)
    ws = _workspace(a, workspace, dev)
    st = load_library().gdn_final_state(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()),
                                        ctypes.c_size_t(ws.numel()), _stream(stream))
    if st != 0:
        raise GdnError(st, "gdn_final_state")
    return s_final


def gdn_recurrent_step(variant, q, k, v, alpha, beta=None, *, state, beta_v=None, j=None,
                       eta=None, o=None, stream=None, stabilize=None):
    """Token-sequential update of ``state`` (in place) over k.shape[1] tokens; returns o."""
    import torch
    B, T, H = k.shape[:3]
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=k.dtype, device=k.device)
    _check(state, "state", k.device, torch.float32)
    a = make_args(variant, q, k, v, alpha, beta, chunk=16, beta_v=beta_v, j=j, eta=eta,
                  s0=None, s_final=None, o=o, stabilize=stabilize)
    st = load_library().gdn_recurrent_step(ctypes.byref(a), ctypes.c_void_p(state.data_ptr()),
                                           _stream(stream))
    if st != 0:
        raise GdnError(st, "gdn_recurrent_step")
    return o


def _staged(name, args: GdnArgs, workspace, stream):
    fn = getattr(load_library(), name)
    st = fn(ctypes.byref(args), ctypes.c_void_p(workspace.data_ptr()),
            ctypes.c_size_t(workspace.numel()), _stream(stream))
    if st != 0:
        raise GdnError(st, name)


def gdn_chunk_prepare(args: GdnArgs, workspace, stream=None):
    """First stage of gdn_chunk_fwd on prebuilt args (see make_args) and a workspace
    tensor of at least gdn_workspace_bytes(args) bytes."""
    _staged("gdn_chunk_prepare", args, workspace, stream)


def gdn_chunk_scan(args: GdnArgs, workspace, stream=None):
    """Second stage of gdn_chunk_fwd (same args and workspace as the prepare call)."""
    _staged("gdn_chunk_scan", args, workspace, stream)


def gdn_chunk_fwd_args(args: GdnArgs, workspace, stream=None):
    """gdn_chunk_fwd on prebuilt args (no per-call marshalling)."""
    _staged("gdn_chunk_fwd", args, workspace, stream)


def gdn_chunk_fwd_static(args: GdnArgs, stream=None):
    """gdn_chunk_fwd on prebuilt args (o and, optionally, s_final given) with the
    library's own record buffer instead of a workspace: nothing is allocated."""
    st = load_library().gdn_chunk_fwd_static(ctypes.byref(args), _stream(stream))
    if st != 0:
        raise GdnError(st, "gdn_chunk_fwd_static")


def gdn_asym_stabilize(mode, k, j, alpha, eta, *, out=None, stream=None):
    """GDN2 stabiliser on ASYM inputs (k, j, alpha = D of shape [B, T, H, dk], eta of
    shape [B, T, H]). mode "clip_decay" returns D' = min(D, 1/rho); mode "project_j"
    returns the projected j'. out may be alpha (clip_decay) or j (project_j) to update
    in place; it is allocated when not given."""
    import torch
    if mode not in STABILIZE_MODES:
        raise ValueError(f"unknown stabilizer mode {mode!r}")
    if k.dim() != 4 or j.shape != k.shape or alpha.shape != k.shape or eta.shape != k.shape[:3]:
        raise ValueError("k, j, alpha must be [B, T, H, dk] and eta [B, T, H]")
    dev, io = k.device, k.dtype
    if io not in (torch.float32, torch.bfloat16):
        raise ValueError("inputs must be float32 or bfloat16")
    if out is None:
        out = torch.empty_like(k)
    for name, t in (("k", k), ("j", j), ("alpha", alpha), ("eta", eta), ("out", out)):
        _check(t, name, dev, io)
    if out.shape != k.shape:
        raise ValueError("out must have the shape of k")
    a = GdnArgs()
    a.variant = VARIANTS["asym"]
    a.dtype = DTYPE_BF16 if io == torch.bfloat16 else DTYPE_F32
    a.B, a.T, a.H = k.shape[0], k.shape[1], k.shape[2]
    a.dk = a.dv = k.shape[-1]
    a.chunk, a.n_h = 64, 1
    a.k, a.j, a.alpha, a.eta = _ptr(k), _ptr(j), _ptr(alpha), _ptr(eta)
    st = load_library().gdn_asym_stabilize(ctypes.byref(a), STABILIZE_MODES[mode],
                                           ctypes.c_void_p(out.data_ptr()), _stream(stream))
    if st != 0:
        raise GdnError(st, "gdn_asym_stabilize")
    return out


def gdn_recurrent_bwd(variant, q, k, v, alpha, beta=None, *, d_o, s0=None, ds_final=None,
                      beta_v=None, j=None, eta=None, workspace=None, stream=None):
    """Gradients (float32 tensors, named after the inputs: dq, dk, dv, dalpha, dbeta,
    dbeta_v, dj, deta, ds0) of the token recurrence for upstream d_o (shape of o, input
    dtype) and ds_final (float32 state shape, optional); the library computes them in
    the chunkwise form on 16-step chunks. A workspace of gdn_bwd_workspace_bytes is
    allocated when none is given."""
    import torch
    dev = k.device
    _check(d_o, "d_o", dev, k.dtype)
    _check(ds_final, "ds_final", dev, torch.float32)
    a = make_args(variant, q, k, v, alpha, beta, chunk=16, beta_v=beta_v, j=j, eta=eta, s0=s0,
                  s_final=None, o=None)
    out = {}
    f32 = dict(dtype=torch.float32, device=dev)
    for name, ref in (("dq", q), ("dk", k), ("dv", v), ("dalpha", alpha), ("dbeta", beta),
                      ("dbeta_v", beta_v), ("dj", j), ("deta", eta)):
        if ref is not None:
            out[name] = torch.empty(ref.shape, **f32)
    B, H = k.shape[0], k.shape[2]
    out["ds0"] = torch.empty((B, H, k.shape[-1], v.shape[-1]), **f32)
    gr = GdnGrads(**{n: (t.data_ptr() if t is not None else None) for n, t in out.items()})
    need = int(load_library().gdn_bwd_workspace_bytes(ctypes.byref(a)))
    if need == 0:
        raise GdnError(-2, "gdn_bwd_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load_library().gdn_recurrent_bwd(ctypes.byref(a), _ptr(d_o), _ptr(ds_final), ctypes.byref(gr),
                                          ctypes.c_void_p(workspace.data_ptr()),
                                          ctypes.c_size_t(workspace.numel()), _stream(stream))
    if st != 0:
        raise GdnError(st, "gdn_recurrent_bwd")
    return out
