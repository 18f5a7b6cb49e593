"""MI355X (gfx950) delta-rule forward pass: chunkwise prefill and recurrent decode.

Thin Python binding over the C ABI of libdelta.so (include/delta.h).  It only
marshals arguments: every step of the computation runs in the library's HIP
kernels.  PyTorch provides device memory (tensors, allocated by torch's caching
allocator) and the current HIP stream.  There is no CPU fallback: if the HIP
library is missing or a tensor is not on the GPU, the call raises.

    import torch, chunkwise_delta_rule_chunked_amd as delta
    O, S_final = delta.fwd(q, k, v, beta, g_log, S0, n_h=1, chunk=64)
    O = delta.decode(q, k, v, beta, g_log, S)        # S updated in place

Layouts (contiguous): q [B,L,H,dk]; k [B,L*n_h,H,dk]; v [B,L*n_h,H,dv] in bf16 or
fp32; beta [B,L*n_h,H] and g_log [B,L,H] (log of the gate) in fp32; states
[B,H,dk,dv] fp32.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

__all__ = ["fwd", "fwd_noalloc", "NOALLOC_MAX_BYTES", "bwd", "bwd_workspace_bytes", "layer_prologue", "layer_prologue_step", "layer_epilogue", "fwd_intra", "fwd_inter", "decode", "decode_kda", "fwd_kda", "fwd_kda_chunked", "kda_chunked_workspace_bytes", "chunk_wy", "workspace_bytes", "strerror", "DeltaError", "lib_path",
           "load_library", "F32", "BF16"]

F32, BF16 = 0, 1
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "libdelta.so")
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "delta.h")
_lib = None


class DeltaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %d (%s)" % (where, code, strerror(code)))


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("L", ctypes.c_int32), ("H", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("n_h", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


def lib_path() -> str:
    return _LIB


def load_library():
    """Load libdelta.so (built by chunkwise_delta_rule_chunked_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        raise ImportError("libdelta.so not found at %s; build it with "
                          "`python -m chunkwise_delta_rule_chunked_amd.build`" % _LIB)
    lib = ctypes.CDLL(_LIB)
    P, SP = ctypes.c_void_p, ctypes.POINTER(Shape)
    lib.delta_fwd_workspace_bytes.argtypes = [SP, ctypes.POINTER(ctypes.c_size_t)]
    lib.delta_fwd.argtypes = [SP, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.delta_fwd_noalloc.argtypes = [SP, P, P, P, P, P, P, P, P, P]
    lib.delta_fwd_intra.argtypes = [SP, P, P, P, P, ctypes.c_size_t, P]
    lib.delta_fwd_inter.argtypes = [SP, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.delta_fwd_segments.argtypes = [SP, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.delta_fwd_scan_summary.argtypes = [SP, P, P, P, P, ctypes.c_size_t, P]
    lib.delta_fwd_scan_combine.argtypes = [SP, P, ctypes.c_size_t, P]
    lib.delta_fwd_scan_outputs.argtypes = [SP, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.delta_chunk_wy.argtypes = [SP, P, P, P, P, P, P, P, P, P]
    lib.delta_decode.argtypes = [SP, P, P, P, P, P, P, P, P]
    lib.delta_decode_kda.argtypes = [SP, P, P, P, P, P, P, P, P]
    lib.delta_fwd_kda.argtypes = [SP, P, P, P, P, P, P, P, P, P]
    lib.delta_fwd_kda_chunked_workspace_bytes.argtypes = [SP, ctypes.POINTER(ctypes.c_size_t)]
    lib.delta_fwd_kda_chunked.argtypes = [SP, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.delta_bwd_workspace_bytes.argtypes = [SP, ctypes.POINTER(ctypes.c_size_t)]
    lib.delta_bwd.argtypes = [SP] + [P] * 15 + [ctypes.c_size_t, P]
    lib.delta_layer_prologue.argtypes = [SP, ctypes.c_int32, ctypes.c_float] + [P] * 9 + [P]
    lib.delta_layer_epilogue.argtypes = [SP, ctypes.c_float, P, P, P, P, P]
    lib.delta_layer_prologue_step.argtypes = [SP, ctypes.c_int32, ctypes.c_float] + [P] * 12 + [P]
    lib.delta_layer_prologue_step.restype = ctypes.c_int
    lib.delta_measure_copy.argtypes = [P, P, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]
    lib.delta_measure_copy.restype = ctypes.c_int
    lib.delta_strerror.argtypes = [ctypes.c_int]
    lib.delta_strerror.restype = ctypes.c_char_p
    for f in (lib.delta_fwd_workspace_bytes, lib.delta_fwd, lib.delta_fwd_noalloc, lib.delta_fwd_intra, lib.delta_fwd_inter,
              lib.delta_chunk_wy, lib.delta_decode, lib.delta_decode_kda, lib.delta_fwd_kda, lib.delta_bwd_workspace_bytes,
              lib.delta_bwd, lib.delta_layer_prologue, lib.delta_layer_epilogue):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def header_functions(header: str = _HEADER) -> list:
    """Names of the functions a header of include/ declares (default include/delta.h)."""
    txt = open(header).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(delta_\w+)\s*\(", txt, flags=re.M)


def strerror(code: int) -> str:
    return load_library().delta_strerror(int(code)).decode()


def _check(rc: int, where: str):
    if rc != 0:
        raise DeltaError(rc, where)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _dev(t, name, dtype=None):
    """Pointer of a contiguous GPU tensor (or None)."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def make_shape(B, L, H, dk, dv, n_h=1, chunk=64, dtype=BF16, scale=1.0) -> Shape:
    return Shape(int(B), int(L), int(H), int(dk), int(dv), int(n_h), int(chunk), int(dtype), float(scale))


def workspace_bytes(B, L, H, dk, dv, n_h=1, chunk=64, dtype=BF16) -> int:
    n = ctypes.c_size_t(0)
    sh = make_shape(B, L, H, dk, dv, n_h, chunk, dtype)
    _check(load_library().delta_fwd_workspace_bytes(ctypes.byref(sh), ctypes.byref(n)),
           "delta_fwd_workspace_bytes")
    return int(n.value)


def fwd(q, k, v, beta, g_log=None, S0=None, *, n_h: int = 1, chunk: int = 64, scale: float = 1.0,
        O=None, S_final=None, workspace=None, stream=None, want_state: bool = True):
    """Chunkwise forward pass.  Returns (O, S_final); S_final is None if want_state is False
    and no S_final buffer is given.  Pass S_final=S0 to update the state in place."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, L, H, d]")
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    sh = make_shape(B, L, H, dk, dv, n_h, chunk, dt, scale)
    if O is None:
        O = torch.empty((B, L, H, dv), dtype=q.dtype, device=q.device)
    if S_final is None and want_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    need = workspace_bytes(B, L, H, dk, dv, n_h, chunk, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    rc = lib.delta_fwd(ctypes.byref(sh), _dev(q, "q", q.dtype), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
                       _dev(beta, "beta", torch.float32), _dev(g_log, "g_log", torch.float32),
                       _dev(S0, "S0", torch.float32), _dev(O, "O", q.dtype), _dev(S_final, "S_final", torch.float32),
                       _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                       _stream(stream))
    _check(rc, "delta_fwd")
    return O, S_final


# include/delta.h: DELTA_NOALLOC_MAX_BYTES, the fixed device workspace of delta_fwd_noalloc
NOALLOC_MAX_BYTES = 96 << 20


def fwd_noalloc(q, k, v, beta, g_log, S0, O, S_final, *, n_h: int = 1, chunk: int = 64, scale: float = 1.0,
                stream=None):
    """fwd through delta_fwd_noalloc: the workspace is the library's fixed device array, and the
    caller provides O (and S_final, or None), so nothing is allocated.  Calls that overlap on one
    device race (they share that array)."""
    torch = _torch()
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    sh = make_shape(B, L, H, dk, dv, n_h, chunk, _dtype_code(q), scale)
    rc = load_library().delta_fwd_noalloc(
        ctypes.byref(sh), _dev(q, "q", q.dtype), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
        _dev(beta, "beta", torch.float32), _dev(g_log, "g_log", torch.float32), _dev(S0, "S0", torch.float32),
        _dev(O, "O", q.dtype), _dev(S_final, "S_final", torch.float32), _stream(stream))
    _check(rc, "delta_fwd_noalloc")
    return O, S_final


def measure_copy(src, dst, *, unroll: int = 4, blocks: int = 4096, nontemporal: bool = False, stream=None):
    """delta_measure_copy (include/delta_measure.h): a plain streaming copy of src into dst (GPU
    tensors of equal byte size), the measured ceiling of a kernel that moves each byte once."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst sizes differ")
    _check(load_library().delta_measure_copy(_dev(src, "src"), _dev(dst, "dst"), nbytes, int(unroll), int(blocks),
                                             int(bool(nontemporal)), _stream(stream)), "delta_measure_copy")


def bwd_workspace_bytes(B, L, H, dk, dv, n_h=1, chunk=64, dtype=BF16) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().delta_bwd_workspace_bytes(ctypes.byref(make_shape(B, L, H, dk, dv, n_h, chunk, dtype)),
                                                    ctypes.byref(n)), "delta_bwd_workspace_bytes")
    return n.value


def bwd(q, k, v, beta, g_log=None, S0=None, dO=None, dS_final=None, *, n_h: int = 1, chunk: int = 64,
        scale: float = 1.0, want_dS0: bool = True, grads=None, workspace=None, stream=None):
    """Backward pass of fwd for the same arguments: returns a dict of float32 gradients dq, dk,
    dv, dbeta, dg_log (None when g_log is None) and dS0 (None unless want_dS0).  dO (same dtype
    as q) is required; dS_final (float32) may be None for zero.  `grads` may hold preallocated
    outputs under the same names."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, L, H, d]")
    if dO is None:
        raise ValueError("dO is required")
    B, L, H, dk = q.shape
    Lx, dv = k.shape[1], v.shape[-1]
    dt = _dtype_code(q)
    sh = make_shape(B, L, H, dk, dv, n_h, chunk, dt, scale)
    g = dict(grads or {})
    f32, dev = torch.float32, q.device
    shapes = {"dq": (B, L, H, dk), "dk": (B, Lx, H, dk), "dv": (B, Lx, H, dv), "dbeta": (B, Lx, H),
              "dg_log": (B, L, H) if g_log is not None else None, "dS0": (B, H, dk, dv) if want_dS0 else None}
    for name, shp in shapes.items():
        if g.get(name) is None and shp is not None:
            g[name] = torch.empty(shp, dtype=f32, device=dev)
        g.setdefault(name, None)
    if g_log is None:
        g["dg_log"] = None
    need = bwd_workspace_bytes(B, L, H, dk, dv, n_h, chunk, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib.delta_bwd(ctypes.byref(sh), _dev(q, "q", q.dtype), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
                       _dev(beta, "beta", f32), _dev(g_log, "g_log", f32), _dev(S0, "S0", f32),
                       _dev(dO, "dO", q.dtype), _dev(dS_final, "dS_final", f32), _dev(g["dq"], "dq", f32),
                       _dev(g["dk"], "dk", f32), _dev(g["dv"], "dv", f32), _dev(g["dbeta"], "dbeta", f32),
                       _dev(g["dg_log"], "dg_log", f32), _dev(g["dS0"], "dS0", f32), _dev(workspace, "workspace"),
                       workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "delta_bwd")
    return g


def layer_prologue(xq, xk, xv, wq, wk, wv, *, n_h: int = 1, eps: float = 1e-6, q=None, k=None, v=None,
                   stream=None):
    """q, k = L2norm(SiLU(ShortConv(xq | xk))), v = SiLU(ShortConv(xv)) (delta_layer_prologue).
    xq [B, L, H, dk], xk [B, L*n_h, H, dk], xv [B, L*n_h, H, dv]; w* float32 [H*d, width]."""
    torch = _torch()
    B, L, H, dk = xq.shape
    dv, width = xv.shape[-1], wq.shape[-1]
    sh = make_shape(B, L, H, dk, dv, n_h, 64 if 64 % n_h == 0 else n_h, _dtype_code(xq))
    q = torch.empty_like(xq) if q is None else q
    k = torch.empty_like(xk) if k is None else k
    v = torch.empty_like(xv) if v is None else v
    f32 = torch.float32
    rc = load_library().delta_layer_prologue(ctypes.byref(sh), int(width), float(eps), _dev(xq, "xq", xq.dtype),
                                             _dev(xk, "xk", xq.dtype), _dev(xv, "xv", xq.dtype), _dev(wq, "wq", f32),
                                             _dev(wk, "wk", f32), _dev(wv, "wv", f32), _dev(q, "q", xq.dtype),
                                             _dev(k, "k", xq.dtype), _dev(v, "v", xq.dtype), _stream(stream))
    _check(rc, "delta_layer_prologue")
    return q, k, v


def layer_prologue_step(xq, xk, xv, wq, wk, wv, conv_q, conv_k, conv_v, *, n_h: int = 1, eps: float = 1e-6,
                        q=None, k=None, v=None, stream=None):
    """One decode token through the layer prologue (delta_layer_prologue_step): xq [B,1,H,dk],
    xk [B,n_h,H,dk], xv [B,n_h,H,dv]; conv_* [B,width-1,H,d] (the filters' recent inputs, updated
    in place; None when width = 1).  Returns (q, k, v)."""
    torch = _torch()
    B, _, H, dk = xq.shape
    dv = xv.shape[-1]
    width = wq.shape[1]
    sh = make_shape(B, 1, H, dk, dv, n_h, 64, _dtype_code(xq))
    q = torch.empty_like(xq) if q is None else q
    k = torch.empty_like(xk) if k is None else k
    v = torch.empty_like(xv) if v is None else v
    f32 = torch.float32
    rc = load_library().delta_layer_prologue_step(
        ctypes.byref(sh), int(width), float(eps), _dev(xq, "xq", xq.dtype), _dev(xk, "xk", xq.dtype),
        _dev(xv, "xv", xq.dtype), _dev(wq, "wq", f32), _dev(wk, "wk", f32), _dev(wv, "wv", f32),
        _dev(conv_q, "conv_q", xq.dtype), _dev(conv_k, "conv_k", xq.dtype), _dev(conv_v, "conv_v", xq.dtype),
        _dev(q, "q", xq.dtype), _dev(k, "k", xq.dtype), _dev(v, "v", xq.dtype), _stream(stream))
    _check(rc, "delta_layer_prologue_step")
    return q, k, v


def layer_epilogue(o, g, weight, *, eps: float = 1e-6, y=None, stream=None):
    """y = RMSNorm(o) * weight * SiLU(g) per head (delta_layer_epilogue); o, g [B, L, H, dv]."""
    torch = _torch()
    B, L, H, dv = o.shape
    sh = make_shape(B, L, H, 16, dv, 1, 64, _dtype_code(o))
    y = torch.empty_like(o) if y is None else y
    rc = load_library().delta_layer_epilogue(ctypes.byref(sh), float(eps), _dev(o, "o", o.dtype), _dev(g, "g", o.dtype),
                                             _dev(weight, "weight", torch.float32), _dev(y, "y", o.dtype),
                                             _stream(stream))
    _check(rc, "delta_layer_epilogue")
    return y


def fwd_intra(k, beta, g_log, workspace, *, n_h: int = 1, chunk: int = 64, dv: int = None, stream=None):
    """Intra-chunk phase of fwd: T and the gate prefix into `workspace` (a uint8 GPU tensor of at
    least workspace_bytes(...)).  dv (default dk) sizes the workspace check."""
    torch = _torch()
    B, Lx, H, dk = k.shape
    sh = make_shape(B, Lx // n_h, H, dk, dv or dk, n_h, chunk, _dtype_code(k))
    rc = load_library().delta_fwd_intra(ctypes.byref(sh), _dev(k, "k", k.dtype),
                                        _dev(beta, "beta", torch.float32),
                                        _dev(g_log, "g_log", torch.float32), _dev(workspace, "workspace"),
                                        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "delta_fwd_intra")


def fwd_inter(q, k, v, S0, workspace, *, n_h: int = 1, chunk: int = 64, scale: float = 1.0, O=None,
              S_final=None, stream=None):
    """Inter-chunk phase of fwd, using a workspace filled by fwd_intra for the same k/beta/g_log."""
    torch = _torch()
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    sh = make_shape(B, L, H, dk, dv, n_h, chunk, _dtype_code(q), scale)
    rc = load_library().delta_fwd_inter(ctypes.byref(sh), _dev(q, "q", q.dtype), _dev(k, "k", q.dtype),
                                        _dev(v, "v", q.dtype), _dev(S0, "S0", torch.float32),
                                        _dev(O, "O", q.dtype), _dev(S_final, "S_final", torch.float32),
                                        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                        _stream(stream))
    _check(rc, "delta_fwd_inter")
    return O, S_final


def segments(B, L, H, dk, dv, n_h=1, chunk=64, dtype=BF16):
    """(segments, chunks per segment) of the inter-chunk phase's sequence split."""
    sh = make_shape(B, L, H, dk, dv, n_h, chunk, dtype)
    P, NS = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load_library().delta_fwd_segments(ctypes.byref(sh), ctypes.byref(P), ctypes.byref(NS)),
           "delta_fwd_segments")
    return P.value, NS.value


def scan_summary(k, v, S0, workspace, *, n_h: int = 1, chunk: int = 64, stream=None):
    """First launch of fwd_inter: per-segment summaries into the workspace."""
    torch = _torch()
    B, Lx, H, dk = k.shape
    sh = make_shape(B, Lx // n_h, H, dk, v.shape[-1], n_h, chunk, _dtype_code(k))
    rc = load_library().delta_fwd_scan_summary(ctypes.byref(sh), _dev(k, "k", k.dtype), _dev(v, "v", k.dtype),
                                               _dev(S0, "S0", torch.float32), _dev(workspace, "workspace"),
                                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "delta_fwd_scan_summary")


def scan_combine(workspace, *, B, L, H, dk, dv, n_h: int = 1, chunk: int = 64, dtype=BF16, stream=None):
    """Second launch of fwd_inter: segment start states from the summaries."""
    sh = make_shape(B, L, H, dk, dv, n_h, chunk, dtype)
    rc = load_library().delta_fwd_scan_combine(ctypes.byref(sh), _dev(workspace, "workspace"),
                                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "delta_fwd_scan_combine")


def scan_outputs(q, k, v, S0, workspace, *, n_h: int = 1, chunk: int = 64, scale: float = 1.0, O=None,
                 S_final=None, stream=None):
    """Third launch of fwd_inter: every segment from its start state, writing O and S_final."""
    torch = _torch()
    B, L, H, dk = q.shape
    sh = make_shape(B, L, H, dk, v.shape[-1], n_h, chunk, _dtype_code(q), scale)
    rc = load_library().delta_fwd_scan_outputs(ctypes.byref(sh), _dev(q, "q", q.dtype), _dev(k, "k", q.dtype),
                                               _dev(v, "v", q.dtype), _dev(S0, "S0", torch.float32),
                                               _dev(O, "O", q.dtype), _dev(S_final, "S_final", torch.float32),
                                               _dev(workspace, "workspace"),
                                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "delta_fwd_scan_outputs")
    return O, S_final


def chunk_wy(k, v, beta, g_log=None, *, L: int, n_h: int = 1, chunk: int = 64, want_wu: bool = True,
             stream=None):
    """Intra-chunk factors T, W, U, gc (fp32) per (b, h, chunk)."""
    torch = _torch()
    lib = load_library()
    B, Lx, H, dk = k.shape
    dv = v.shape[-1]
    if Lx != L * n_h:
        raise ValueError("k has %d positions, expected L*n_h = %d" % (Lx, L * n_h))
    dt = _dtype_code(k)
    sh = make_shape(B, L, H, dk, dv, n_h, chunk, dt)
    NT = -(-Lx // chunk)
    dev = k.device
    T = torch.empty((B, H, NT, chunk, chunk), dtype=torch.float32, device=dev)
    gc = torch.empty((B, H, NT, chunk), dtype=torch.float32, device=dev)
    W = torch.empty((B, H, NT, chunk, dk), dtype=torch.float32, device=dev) if want_wu else None
    U = torch.empty((B, H, NT, chunk, dv), dtype=torch.float32, device=dev) if want_wu else None
    rc = lib.delta_chunk_wy(ctypes.byref(sh), _dev(k, "k", k.dtype), _dev(v, "v", k.dtype),
                            _dev(beta, "beta", torch.float32), _dev(g_log, "g_log", torch.float32),
                            _dev(T, "T"), _dev(W, "W"), _dev(U, "U"), _dev(gc, "gc"), _stream(stream))
    _check(rc, "delta_chunk_wy")
    return {"T": T, "W": W, "U": U, "gc": gc}


def decode(q, k, v, beta, g_log, S, *, n_h: int = 1, scale: float = 1.0, O=None, stream=None):
    """One recurrent step per (b, h); S [B,H,dk,dv] fp32 is updated in place.  Returns O [B,1,H,dv]."""
    torch = _torch()
    lib = load_library()
    B, one, H, dk = q.shape
    if one != 1:
        raise ValueError("decode takes one token: q must be [B, 1, H, dk]")
    dv = v.shape[-1]
    dt = _dtype_code(q)
    sh = make_shape(B, 1, H, dk, dv, n_h, 64, dt, scale)
    if O is None:
        O = torch.empty((B, 1, H, dv), dtype=q.dtype, device=q.device)
    rc = lib.delta_decode(ctypes.byref(sh), _dev(q, "q", q.dtype), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
                          _dev(beta, "beta", torch.float32), _dev(g_log, "g_log", torch.float32),
                          _dev(S, "S", torch.float32), _dev(O, "O", q.dtype), _stream(stream))
    _check(rc, "delta_decode")
    return O


def fwd_kda(q, k, v, beta, a_log, S0=None, *, scale: float = 1.0, O=None, S_final=None, want_state: bool = True,
            stream=None):
    """KDA over a sequence (delta_fwd_kda): q, k [B,L,H,dk], v [B,L,H,dv] (bf16 or fp32), beta
    [B,L,H] and a_log [B,L,H,dk] (log of the per-channel decay) fp32, S0 [B,H,dk,dv] fp32 or None.
    Returns (O, S_final); pass S_final=S0 to update the state in place."""
    torch = _torch()
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    sh = make_shape(B, L, H, dk, dv, 1, 64, _dtype_code(q), scale)
    if O is None:
        O = torch.empty((B, L, H, dv), dtype=q.dtype, device=q.device)
    if S_final is None and want_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    rc = load_library().delta_fwd_kda(ctypes.byref(sh), _dev(q, "q", q.dtype), _dev(k, "k", q.dtype),
                                      _dev(v, "v", q.dtype), _dev(beta, "beta", torch.float32),
                                      _dev(a_log, "a_log", torch.float32), _dev(S0, "S0", torch.float32),
                                      _dev(O, "O", q.dtype), _dev(S_final, "S_final", torch.float32), _stream(stream))
    _check(rc, "delta_fwd_kda")
    return O, S_final


def kda_chunked_workspace_bytes(B, L, H, dk=128, dv=128, chunk=64, dtype=BF16) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().delta_fwd_kda_chunked_workspace_bytes(ctypes.byref(make_shape(B, L, H, dk, dv, 1, chunk, dtype)),
                                                                ctypes.byref(n)), "delta_fwd_kda_chunked_workspace_bytes")
    return n.value


def fwd_kda_chunked(q, k, v, beta, a_log, S0=None, *, scale: float = 1.0, chunk: int = 64, O=None, S_final=None,
                    want_state: bool = True, workspace=None, stream=None):
    """KDA over a sequence in chunks (delta_fwd_kda_chunked; bf16, dk = dv = 128, chunk 64): the
    arguments and result of fwd_kda.  Returns (O, S_final)."""
    torch = _torch()
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    sh = make_shape(B, L, H, dk, dv, 1, chunk, _dtype_code(q), scale)
    if O is None:
        O = torch.empty((B, L, H, dv), dtype=q.dtype, device=q.device)
    if S_final is None and want_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = kda_chunked_workspace_bytes(B, L, H, dk, dv, chunk, _dtype_code(q))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    rc = load_library().delta_fwd_kda_chunked(ctypes.byref(sh), _dev(q, "q", q.dtype), _dev(k, "k", q.dtype),
                                              _dev(v, "v", q.dtype), _dev(beta, "beta", torch.float32),
                                              _dev(a_log, "a_log", torch.float32), _dev(S0, "S0", torch.float32),
                                              _dev(O, "O", q.dtype), _dev(S_final, "S_final", torch.float32),
                                              _dev(workspace, "workspace"),
                                              workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "delta_fwd_kda_chunked")
    return O, S_final


def decode_kda(q, k, v, beta, a_log, S, *, scale: float = 1.0, O=None, stream=None):
    """One KDA step per (b, h) (per-key-channel decay exp(a_log) of the state's rows, then the
    delta-rule write and the readout); a_log [B,1,H,dk] fp32, S [B,H,dk,dv] fp32 updated in
    place.  Returns O [B,1,H,dv]."""
    torch = _torch()
    lib = load_library()
    B, one, H, dk = q.shape
    if one != 1:
        raise ValueError("decode_kda takes one token: q must be [B, 1, H, dk]")
    dv = v.shape[-1]
    sh = make_shape(B, 1, H, dk, dv, 1, 64, _dtype_code(q), scale)
    if O is None:
        O = torch.empty((B, 1, H, dv), dtype=q.dtype, device=q.device)
    rc = lib.delta_decode_kda(ctypes.byref(sh), _dev(q, "q", q.dtype), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
                              _dev(beta, "beta", torch.float32), _dev(a_log, "a_log", torch.float32),
                              _dev(S, "S", torch.float32), _dev(O, "O", q.dtype), _stream(stream))
    _check(rc, "delta_decode_kda")
    return O
