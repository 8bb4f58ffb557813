"""ctypes binding of librope_attn.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
turns torch tensors into device pointers, allocates outputs and the
workspace with torch on the inputs' device, and passes torch's current HIP
stream.  There is no fallback: if the library is missing, importing the
functions below raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librope_attn.so")

FP32, BF16 = 0, 1
# rope_attn_stage bits
STAGE_PREP, STAGE_EXACT, STAGE_MAIN, STAGE_DKDV, STAGE_DQ, STAGE_DALPHA = 1, 2, 4, 8, 16, 32
STAGE_ALL = 63
STAGE_PREP_GRAD = 64   # backward: dO plane and D only, reusing the forward's workspace
STATUS = {0: "OK", -1: "ERR_NULL", -2: "ERR_SHAPE", -3: "ERR_DTYPE", -4: "ERR_ALIGN",
          -5: "ERR_WORKSPACE", -6: "ERR_HIP", -7: "ERR_ARG"}

_lib = None


class Options(ctypes.Structure):
    """rope_attn_options: unrotated_pairs (the slowest bands left unrotated,
    partial RoPE), scale (softmax scale, 0 = 1/sqrt(D)), pos_offset (position
    of row 0), and block lists (device int32 CSR pointers over the B*H*nb
    query blocks of 128 rows, and the number of entries)."""
    _fields_ = [("unrotated_pairs", ctypes.c_int), ("scale", ctypes.c_float),
                ("pos_offset", ctypes.c_int), ("block_ptr", ctypes.c_void_p),
                ("block_idx", ctypes.c_void_p), ("block_nnz", ctypes.c_int)]


def _opts(opts):
    """None, an Options, or a dict with any of its fields; a dict may give
    ``blocks`` = (ptr, idx) int32 device tensors instead of the raw fields."""
    if opts is None or isinstance(opts, Options):
        return opts
    opts = dict(opts)
    blocks = opts.pop("blocks", None)
    if blocks is not None:
        import torch
        ptr, idx = blocks
        for name, t in (("ptr", ptr), ("idx", idx)):
            if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"block {name} must be a contiguous int32 device tensor")
        opts["block_ptr"] = ptr.data_ptr()
        opts["block_idx"] = idx.data_ptr() if idx.numel() else None
        opts["block_nnz"] = int(idx.numel())
    return Options(**opts)


def block_csr(lists, device=None):
    """CSR (ptr, idx) int32 tensors from nested lists ``lists[b][h][qb]`` of
    key-block indices (every query block of every head, in order)."""
    import torch
    ptr, idx = [0], []
    for per_b in lists:
        for per_h in per_b:
            for sel in per_h:
                idx.extend(int(x) for x in sel)
                ptr.append(len(idx))
    mk = lambda a: torch.tensor(a, dtype=torch.int32, device=device)
    return mk(ptr), mk(idx)


class RopeAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: status {status} ({STATUS.get(status, '?')}): {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not found: build it with `python -m bwd_rope_apply_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i, d = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_double
    lib.rope_attn_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.rope_attn_fwd_workspace_bytes.restype = sz
    lib.rope_attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.rope_attn_bwd_workspace_bytes.restype = sz
    lib.rope_attn_bwd_workspace_bytes_min.argtypes = [i, i, i, i, i, i]
    lib.rope_attn_bwd_workspace_bytes_min.restype = sz
    lib.rope_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, d, vp, i, vp, sz, vp]
    lib.rope_attn_fwd.restype = i
    lib.rope_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, d, vp, i,
                                  vp, sz, vp]
    lib.rope_attn_bwd.restype = i
    lib.rope_attn_fwd_stages.argtypes = [ctypes.c_uint] + lib.rope_attn_fwd.argtypes
    lib.rope_attn_fwd_stages.restype = i
    lib.rope_attn_bwd_stages.argtypes = [ctypes.c_uint] + lib.rope_attn_bwd.argtypes
    lib.rope_attn_bwd_stages.restype = i
    lib.rope_attn_fwd_ex.argtypes = [ctypes.c_uint, vp] + lib.rope_attn_fwd.argtypes
    lib.rope_attn_fwd_ex.restype = i
    lib.rope_attn_bwd_ex.argtypes = [ctypes.c_uint, vp] + lib.rope_attn_bwd.argtypes
    lib.rope_attn_bwd_ex.restype = i
    lib.rope_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, d, vp, i, vp]
    lib.rope_attn_fwd_noalloc.restype = i
    lib.rope_attn_workspace_flags.argtypes = [vp, sz, ctypes.POINTER(ctypes.c_uint), vp]
    lib.rope_attn_workspace_flags.restype = i
    lib.rope_attn_status_string.argtypes = [i]
    lib.rope_attn_status_string.restype = ctypes.c_char_p
    f = ctypes.c_float
    lib.gram_select_workspace_bytes.argtypes = [i, i, i]
    lib.gram_select_workspace_bytes.restype = sz
    lib.gram_cascade_workspace_bytes.argtypes = [i, i]
    lib.gram_cascade_workspace_bytes.restype = sz
    lib.gram_select.argtypes = [vp, i, i, i, i, f, vp, vp, vp, vp, sz, vp]
    lib.gram_select.restype = i
    lib.gram_select_stages.argtypes = [ctypes.c_uint] + lib.gram_select.argtypes
    lib.gram_select_stages.restype = i
    lib.gram_cascade.argtypes = [vp, i, i, i, f, vp, vp, vp, vp, vp, sz, vp]
    lib.gram_cascade.restype = i
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise RopeAttnError(fn, status, load().rope_attn_status_string(status).decode())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"q/k/v/dO must be bfloat16 or float32, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _shape(q, k, v):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, D]")
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in shape, dtype and device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    return tuple(int(x) for x in q.shape)


def _same_device(name, t, device):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a device tensor on {device}")


def _check_tensor(name, t, shape, dtype, device):
    """A caller-supplied tensor the library reads or writes: the given shape
    and dtype, contiguous, on ``device`` (the kernels write exactly
    prod(shape) elements of dtype through its pointer)."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")
    _same_device(name, t, device)


def _workspace(workspace, nbytes, device):
    """The workspace tensor (any dtype, contiguous, on ``device``) and its
    size in bytes; a new one of ``nbytes`` when None."""
    import torch
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _same_device("workspace", workspace, device)
    return workspace, workspace.numel() * workspace.element_size()


def _alpha(alpha, q, D):
    import torch
    if alpha is None:
        return None
    if tuple(alpha.shape) != (D // 2,) or alpha.dtype != torch.float32 or alpha.device != q.device:
        raise ValueError("alpha must be a float32 [D/2] tensor on q's device")
    return alpha.contiguous()


def workspace_bytes(kind: str, B: int, H: int, N: int, D: int, dtype: int, causal: bool) -> int:
    """kind "fwd", "bwd" (with the dS panels where they apply) or "bwd_min"
    (the smallest backward workspace: dQ recomputes the scores)."""
    lib = load()
    f = {"fwd": lib.rope_attn_fwd_workspace_bytes, "bwd": lib.rope_attn_bwd_workspace_bytes,
         "bwd_min": lib.rope_attn_bwd_workspace_bytes_min}[kind]
    return int(f(B, H, N, D, dtype, int(causal)))


def fwd(q, k, v, base: float, alpha=None, causal: bool = True, workspace=None,
        out: Optional[Tuple] = None, stages: int = STAGE_ALL, opts=None):
    """O [B,H,N,D] float32 and LSE [B,H,N] float32 for rotated attention.
    ``stages`` selects stage bits (default: the whole pass); ``opts`` is None,
    an Options or a dict of its fields (frequency-schedule options)."""
    import torch
    lib = load()
    B, H, N, D = _shape(q, k, v)
    dt = _dtype_code(q)
    alpha = _alpha(alpha, q, D)
    if out is None:
        o = torch.empty((B, H, N, D), dtype=torch.float32, device=q.device)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _check_tensor("o", o, (B, H, N, D), torch.float32, q.device)
        _check_tensor("lse", lse, (B, H, N), torch.float32, q.device)
    nbytes = workspace_bytes("fwd", B, H, N, D, dt, causal)
    workspace, wbytes = _workspace(workspace, nbytes, q.device)
    op = _opts(opts)
    st = lib.rope_attn_fwd_ex(stages, None if op is None else ctypes.addressof(op), _ptr(q), _ptr(k),
                              _ptr(v), _ptr(o), _ptr(lse), B, H, N, D, dt, float(base), _ptr(alpha),
                              int(causal), _ptr(workspace), wbytes, _stream(q.device))
    _check("rope_attn_fwd", st)
    return o, lse


def bwd(q, k, v, o, do, lse, base: float, alpha=None, causal: bool = True, workspace=None,
        want_dalpha: bool = True, out: Optional[Tuple] = None, stages: int = STAGE_ALL, opts=None):
    """(dQ, dK, dV [B,H,N,D] float32, dalpha [D/2] float32 or None).
    ``stages`` selects stage bits (default: the whole pass); ``opts`` as for
    fwd (the same options as the forward that produced o, lse)."""
    import torch
    lib = load()
    B, H, N, D = _shape(q, k, v)
    dt = _dtype_code(q)
    _check_tensor("dO", do, (B, H, N, D), q.dtype, q.device)
    _check_tensor("O", o, (B, H, N, D), torch.float32, q.device)
    _check_tensor("LSE", lse, (B, H, N), torch.float32, q.device)
    alpha = _alpha(alpha, q, D)
    if out is None:
        dq = torch.empty((B, H, N, D), dtype=torch.float32, device=q.device)
        dk = torch.empty_like(dq)
        dv = torch.empty_like(dq)
        da = torch.empty((D // 2,), dtype=torch.float32, device=q.device) if want_dalpha else None
    else:
        dq, dk, dv, da = out
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            _check_tensor(name, t, (B, H, N, D), torch.float32, q.device)
        if da is not None:
            _check_tensor("dalpha", da, (D // 2,), torch.float32, q.device)
    nbytes = workspace_bytes("bwd", B, H, N, D, dt, causal)
    workspace, wbytes = _workspace(workspace, nbytes, q.device)
    op = _opts(opts)
    st = lib.rope_attn_bwd_ex(stages, None if op is None else ctypes.addressof(op), _ptr(q), _ptr(k),
                              _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                              _ptr(da), B, H, N, D, dt, float(base), _ptr(alpha), int(causal),
                              _ptr(workspace), wbytes, _stream(q.device))
    _check("rope_attn_bwd", st)
    return dq, dk, dv, da


def fwd_noalloc(q, k, v, base: float, alpha=None, causal: bool = True, out: Optional[Tuple] = None):
    """The forward through rope_attn_fwd_noalloc: the library's own fixed
    device array is the workspace (no workspace argument).  ``out`` (o, lse)
    as for fwd; the binding allocates them with torch only when not given."""
    import torch
    lib = load()
    B, H, N, D = _shape(q, k, v)
    dt = _dtype_code(q)
    alpha = _alpha(alpha, q, D)
    if out is None:
        o = torch.empty((B, H, N, D), dtype=torch.float32, device=q.device)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _check_tensor("o", o, (B, H, N, D), torch.float32, q.device)
        _check_tensor("lse", lse, (B, H, N), torch.float32, q.device)
    st = lib.rope_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, D, dt,
                                   float(base), _ptr(alpha), int(causal), _stream(q.device))
    _check("rope_attn_fwd_noalloc", st)
    return o, lse


FLAG_FP16_RANGE = 1   # an entry of the scaled Q~, of K~ or of V exceeded fp16's range


def workspace_flags(workspace) -> int:
    """The range flags that the last PREP stage left in ``workspace`` (a
    device tensor passed to fwd or bwd).  Synchronises the current stream."""
    lib = load()
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    v = ctypes.c_uint(0)
    st = lib.rope_attn_workspace_flags(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                       ctypes.byref(v), _stream(workspace.device))
    _check("rope_attn_workspace_flags", st)
    return int(v.value)


# ------------------------------------------------------------ token selection
GRAM_BF16, GRAM_FP16 = 1, 2
GRAM_STAGE_PREP, GRAM_STAGE_GRAM, GRAM_STAGE_DECIDE, GRAM_STAGE_ALL = 1, 2, 4, 7


def _gram_dtype(x) -> int:
    import torch
    if x.dtype == torch.bfloat16:
        return GRAM_BF16
    if x.dtype == torch.float16:
        return GRAM_FP16
    raise TypeError(f"tokens must be bfloat16 or float16, got {x.dtype}")


def gram_select(x, tau: float, workspace=None, out=None, stages: int = GRAM_STAGE_ALL):
    """Gram-threshold selection of each sequence of ``x`` ([B, T, d] or
    [T, d], bf16 or fp16, on the device).  Returns (max_cos float32, rep
    uint8, count int32 [B]) with the leading shape of ``x``.  ``stages``
    selects stage bits (default: all)."""
    import torch
    lib = load()
    if not x.is_cuda or not x.is_contiguous() or x.dim() not in (2, 3):
        raise ValueError("x must be a contiguous [B, T, d] or [T, d] device tensor")
    xb = x if x.dim() == 3 else x.unsqueeze(0)
    B, T, d = (int(v) for v in xb.shape)
    dt = _gram_dtype(x)
    if out is None:
        m = torch.empty((B, T), dtype=torch.float32, device=x.device)
        rep = torch.empty((B, T), dtype=torch.uint8, device=x.device)
        cnt = torch.empty((B,), dtype=torch.int32, device=x.device)
    else:
        m, rep, cnt = out
        _check_tensor("max_cos", m, (B, T), torch.float32, x.device)
        _check_tensor("rep", rep, (B, T), torch.uint8, x.device)
        _check_tensor("count", cnt, (B,), torch.int32, x.device)
    nbytes = int(lib.gram_select_workspace_bytes(B, T, d))
    workspace, wbytes = _workspace(workspace, nbytes, x.device)
    st = lib.gram_select_stages(stages, _ptr(xb), B, T, d, dt, float(tau), _ptr(m), _ptr(rep),
                                _ptr(cnt), _ptr(workspace), wbytes, _stream(x.device))
    _check("gram_select", st)
    if x.dim() == 2:
        return m[0], rep[0], cnt
    return m, rep, cnt


def gram_cascade(x, tau: float, prev, workspace=None, out=None):
    """One cascade step on one sequence ``x`` [T, d] (bf16 or fp16, on the
    device) with the inherited set ``prev`` ([T] uint8 flags on the device).
    Returns (max_cos float32 [T], rep uint8 [T], count int32 [1])."""
    import torch
    lib = load()
    if not x.is_cuda or not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous [T, d] device tensor")
    T, d = (int(v) for v in x.shape)
    if prev.shape != (T,) or prev.dtype != torch.uint8 or not prev.is_contiguous() or not prev.is_cuda:
        raise ValueError("prev must be a contiguous uint8 [T] device tensor")
    dt = _gram_dtype(x)
    if out is None:
        m = torch.empty((T,), dtype=torch.float32, device=x.device)
        rep = torch.empty((T,), dtype=torch.uint8, device=x.device)
        cnt = torch.empty((1,), dtype=torch.int32, device=x.device)
    else:
        m, rep, cnt = out
        _check_tensor("max_cos", m, (T,), torch.float32, x.device)
        _check_tensor("rep", rep, (T,), torch.uint8, x.device)
        _check_tensor("count", cnt, (1,), torch.int32, x.device)
    if prev.device != x.device:
        raise ValueError("prev must be on x's device")
    nbytes = int(lib.gram_cascade_workspace_bytes(T, d))
    workspace, wbytes = _workspace(workspace, nbytes, x.device)
    st = lib.gram_cascade(_ptr(x), T, d, dt, float(tau), _ptr(prev), _ptr(m), _ptr(rep), _ptr(cnt),
                          _ptr(workspace), wbytes, _stream(x.device))
    _check("gram_cascade", st)
    return m, rep, cnt
