"""MonarchAttention for MI355X (gfx950): thin Python binding.

Every step of the computation runs in ``libmonarch_attn.so`` (HIP kernels for
gfx950); this module only marshals arguments: device pointers of torch
tensors, sizes, and the current HIP stream.  The C entry points are exposed
under the same names.  If the library is missing or fails to load, every
call raises: there is no fallback path.

The library is loaded lazily, so ``structured_attention_video_monarch_amd.inputs``
imports without it.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmonarch_attn.so")

MONARCH_OK = 0
MONARCH_EINVAL = -1
MONARCH_EUNSUPPORTED = -2
MONARCH_EHIP = -3
MONARCH_ENOMEM = -4
MONARCH_BF16 = 0
MONARCH_F32 = 1
MONARCH_NUM_KERNELS = 13

_lib = None


class MonarchError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _declare(lib):
    c_int, c_void_p, c_size_t = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    dims = [c_int] * 10  # B, H, f, h, w, d, b1, b2, tiles, iters
    lib.monarch_attn_fwd.argtypes = [c_void_p] * 4 + dims + [c_void_p]
    lib.monarch_attn_fwd.restype = c_int
    lib.monarch_attn_fwd_f32.argtypes = [c_void_p] * 4 + dims + [c_void_p]
    lib.monarch_attn_fwd_f32.restype = c_int
    lib.monarch_attn_debug_factors_f32.argtypes = [c_void_p] * 5 + dims + [c_void_p]
    lib.monarch_attn_debug_factors_f32.restype = c_int
    lib.monarch_attn_workspace_bytes.argtypes = dims + [c_int]
    lib.monarch_attn_workspace_bytes.restype = c_size_t
    lib.monarch_attn_fwd_ws.argtypes = [c_void_p] * 4 + dims + [c_int, c_void_p, c_size_t, c_void_p]
    lib.monarch_attn_fwd_ws.restype = c_int
    lib.monarch_attn_fwd_scratch.argtypes = [c_void_p] * 4 + dims + [c_int, c_void_p]
    lib.monarch_attn_fwd_scratch.restype = c_int
    lib.monarch_attn_adaptive_workspace_bytes.argtypes = dims + [c_int]
    lib.monarch_attn_adaptive_workspace_bytes.restype = c_size_t
    lib.monarch_attn_fwd_adaptive_ws.argtypes = ([c_void_p] * 4 + dims + [ctypes.c_float, c_int, c_void_p,
                                                 c_void_p, c_size_t, c_void_p])
    lib.monarch_attn_fwd_adaptive_ws.restype = c_int
    kdims = [c_int] * 11  # B, H, fq, f, h, w, d, b1, b2, tiles, iters
    lib.monarch_attn_kv_workspace_bytes.argtypes = kdims + [c_int]
    lib.monarch_attn_kv_workspace_bytes.restype = c_size_t
    lib.monarch_attn_fwd_kv.argtypes = [c_void_p] * 4 + kdims + [c_int, c_void_p]
    lib.monarch_attn_fwd_kv.restype = c_int
    lib.monarch_attn_fwd_kv_ws.argtypes = [c_void_p] * 4 + kdims + [c_int, c_void_p, c_size_t, c_void_p]
    lib.monarch_attn_fwd_kv_ws.restype = c_int
    tdims = [c_int] * 10  # B, H, f, h, w, d, b1, b2, tiles, iters
    lib.monarch_attn_train_state_bytes.argtypes = tdims + [c_int]
    lib.monarch_attn_train_state_bytes.restype = c_size_t
    lib.monarch_attn_fwd_train.argtypes = [c_void_p] * 4 + tdims + [c_int, c_void_p, c_size_t, c_void_p]
    lib.monarch_attn_fwd_train.restype = c_int
    lib.monarch_attn_bwd.argtypes = [c_void_p] * 8 + tdims + [c_int, c_void_p, c_size_t, c_void_p]
    lib.monarch_attn_bwd.restype = c_int
    lib.monarch_attn_adaptive_kv_workspace_bytes.argtypes = kdims + [c_int]
    lib.monarch_attn_adaptive_kv_workspace_bytes.restype = c_size_t
    lib.monarch_attn_fwd_adaptive_kv_ws.argtypes = ([c_void_p] * 4 + kdims
                                                    + [ctypes.c_float, c_int, c_void_p, c_void_p, c_size_t, c_void_p])
    lib.monarch_attn_fwd_adaptive_kv_ws.restype = c_int
    lib.monarch_attn_train_state_bytes_kv.argtypes = kdims + [c_int]
    lib.monarch_attn_train_state_bytes_kv.restype = c_size_t
    lib.monarch_attn_fwd_train_kv.argtypes = [c_void_p] * 4 + kdims + [c_int, c_void_p, c_size_t, c_void_p]
    lib.monarch_attn_fwd_train_kv.restype = c_int
    lib.monarch_attn_bwd_kv.argtypes = [c_void_p] * 8 + kdims + [c_int, c_void_p, c_size_t, c_void_p]
    lib.monarch_attn_bwd_kv.restype = c_int
    lib.monarch_attn_status_string.argtypes = [c_int]
    lib.monarch_attn_status_string.restype = ctypes.c_char_p
    lib.monarch_attn_last_hip_error.argtypes = []
    lib.monarch_attn_last_hip_error.restype = c_int
    lib.monarch_attn_profile_enable.argtypes = [c_int]
    lib.monarch_attn_profile_enable.restype = c_int
    lib.monarch_attn_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_double),
                                                 ctypes.POINTER(ctypes.c_long), c_int]
    lib.monarch_attn_profile_collect.restype = c_int
    lib.monarch_attn_kernel_name.argtypes = [c_int]
    lib.monarch_attn_kernel_name.restype = ctypes.c_char_p
    return lib


def lib():
    """The loaded C library (builds it first only if no built copy exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from .build import build_library
            build_library()
        # torch ships its own HIP runtime under the same soname: load torch
        # first so that the library binds to that one runtime instead of
        # bringing in a second copy that torch would then pick up
        import torch  # noqa: F401
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def monarch_attn_status_string(status: int) -> str:
    return lib().monarch_attn_status_string(int(status)).decode()


def _check(rc: int, what: str):
    if rc != MONARCH_OK:
        extra = ""
        if rc == MONARCH_EHIP:
            extra = f" (hipError {lib().monarch_attn_last_hip_error()})"
        raise MonarchError(rc, f"{what}: {monarch_attn_status_string(rc)}{extra}")


def _dims(q, f, h, w, b1, b2, tiles, iters):
    if q.dim() != 4:
        raise ValueError("q, k, v, out must be [B, H, N, d]")
    B, H, N, d = q.shape
    if f * h * w != N:
        raise ValueError(f"f*h*w = {f * h * w} != N = {N}")
    return [B, H, f, h, w, d, b1, b2, tiles, iters]


def _ptr(t):
    """Device address of a tensor on the current GPU: the kernels run on the
    current device, so a tensor elsewhere is refused before any launch."""
    import torch
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"tensor on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    return ctypes.c_void_p(t.data_ptr())


def _tensors(q, k, v, out, dtype):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.shape != q.shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != q shape {tuple(q.shape)}")
    return [_ptr(t) for t in (q, k, v, out)]


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def monarch_attn_fwd(q, k, v, out, f, h, w, b1, b2, tiles=1, iters=1, stream=None):
    """bf16: out <- M V (in place), enqueued on ``stream`` (default: current)."""
    import torch
    ptrs = _tensors(q, k, v, out, torch.bfloat16)
    _check(lib().monarch_attn_fwd(*ptrs, *_dims(q, f, h, w, b1, b2, tiles, iters), _stream(stream)),
           "monarch_attn_fwd")
    return out


def monarch_attn_fwd_f32(q, k, v, out, f, h, w, b1, b2, tiles=1, iters=1, stream=None):
    """float32 variant of :func:`monarch_attn_fwd`."""
    import torch
    ptrs = _tensors(q, k, v, out, torch.float32)
    _check(lib().monarch_attn_fwd_f32(*ptrs, *_dims(q, f, h, w, b1, b2, tiles, iters), _stream(stream)),
           "monarch_attn_fwd_f32")
    return out


def monarch_attn_debug_factors_f32(q, k, v, f, h, w, b1, b2, tiles=1, iters=1, stream=None):
    """Test-only: the factors of the last iteration of the float32 forward,
    L [B,H,b2,b1,b1] (L[a2][a1][c1]) and R [B,H,t,b1,b2,b2] (R[g][c1][a2][c2]),
    as new GPU tensors."""
    import torch
    dims = _dims(q, f, h, w, b1, b2, tiles, iters)
    B, H = dims[0], dims[1]
    L = torch.empty((B, H, b2, b1, b1), dtype=torch.float32, device=q.device)
    R = torch.empty((B, H, tiles, b1, b2, b2), dtype=torch.float32, device=q.device)
    ptrs = _tensors(q, k, v, q, torch.float32)[:3] + [_ptr(L), _ptr(R)]
    _check(lib().monarch_attn_debug_factors_f32(*ptrs, *dims, _stream(stream)), "monarch_attn_debug_factors_f32")
    return L, R


def monarch_attn_workspace_bytes(B, H, f, h, w, d, b1, b2, tiles, iters, dtype=MONARCH_BF16) -> int:
    return int(lib().monarch_attn_workspace_bytes(B, H, f, h, w, d, b1, b2, tiles, iters, dtype))


def monarch_attn_fwd_ws(q, k, v, out, f, h, w, b1, b2, tiles, iters, workspace, stream=None):
    """Either dtype, with a caller-provided workspace (a uint8 GPU tensor)."""
    import torch
    dtype = _dtype_code(q)
    ptrs = _tensors(q, k, v, out, q.dtype)
    if not workspace.is_cuda or workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 GPU tensor")
    nbytes = workspace.numel()
    _check(lib().monarch_attn_fwd_ws(*ptrs, *_dims(q, f, h, w, b1, b2, tiles, iters), dtype,
                                     _ptr(workspace), nbytes, _stream(stream)),
           "monarch_attn_fwd_ws")
    return out


MONARCH_SCRATCH_BYTES = 128 << 20


def monarch_attn_fwd_scratch(q, k, v, out, f, h, w, b1, b2, tiles=1, iters=1, stream=None):
    """Either dtype, with the library's static device scratch array instead of
    a workspace: allocates nothing (MonarchError ENOMEM when the workspace
    would exceed MONARCH_SCRATCH_BYTES).  Calls that overlap on one GPU race."""
    dtype = _dtype_code(q)
    ptrs = _tensors(q, k, v, out, q.dtype)
    _check(lib().monarch_attn_fwd_scratch(*ptrs, *_dims(q, f, h, w, b1, b2, tiles, iters), dtype,
                                          _stream(stream)), "monarch_attn_fwd_scratch")
    return out


def monarch_attn(q, k, v, f, h, w, b1=None, b2=None, tiles=1, iters=1):
    """Allocate the output and run the forward; aligned blocks by default."""
    import torch
    b1 = f * h if b1 is None else b1
    b2 = w if b2 is None else b2
    out = torch.empty_like(q)
    if q.dtype == torch.bfloat16:
        return monarch_attn_fwd(q, k, v, out, f, h, w, b1, b2, tiles, iters)
    return monarch_attn_fwd_f32(q, k, v, out, f, h, w, b1, b2, tiles, iters)


def monarch_attn_adaptive_workspace_bytes(B, H, f, h, w, d, b1, b2, tiles, max_iters, dtype=MONARCH_BF16) -> int:
    return int(lib().monarch_attn_adaptive_workspace_bytes(B, H, f, h, w, d, b1, b2, tiles, max_iters, dtype))


def monarch_attn_fwd_adaptive(q, k, v, out, f, h, w, b1, b2, tiles, max_iters, tol, iters_used=None,
                              workspace=None, stream=None):
    """Up to max_iters iterations, each head stopping when its objective gain
    per token is <= tol.  Returns (out, iters_used) with iters_used an int32
    GPU tensor [B, H] (allocated if not given)."""
    import torch
    ptrs = _tensors(q, k, v, out, q.dtype)
    B, H, _, d = q.shape
    dt = _dtype_code(q)
    if iters_used is None:
        iters_used = torch.empty((B, H), dtype=torch.int32, device=q.device)
    if not iters_used.is_cuda or iters_used.dtype != torch.int32 or iters_used.numel() != B * H:
        raise ValueError("iters_used must be an int32 GPU tensor of B*H elements")
    if workspace is None:
        nb = monarch_attn_adaptive_workspace_bytes(B, H, f, h, w, d, b1, b2, tiles, max_iters, dt)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=q.device)
    _check(lib().monarch_attn_fwd_adaptive_ws(*ptrs, *_dims(q, f, h, w, b1, b2, tiles, max_iters), float(tol), dt,
                                              _ptr(iters_used),
                                              _ptr(workspace), workspace.numel(),
                                              _stream(stream)), "monarch_attn_fwd_adaptive_ws")
    return out, iters_used


def monarch_attn_kv_workspace_bytes(B, H, fq, f, h, w, d, b1, b2, tiles, iters, dtype=MONARCH_BF16) -> int:
    return int(lib().monarch_attn_kv_workspace_bytes(B, H, fq, f, h, w, d, b1, b2, tiles, iters, dtype))


def _kv_tensors(q, fq, f, h, w, query_side, key_side):
    """Check [B,H,rows,d] GPU tensors of q's dtype: query_side ones have the
    chunk's fq*h*w rows, key_side ones all f*h*w."""
    named = [(n, t, fq * h * w) for n, t in query_side] + [(n, t, f * h * w) for n, t in key_side]
    for name, t, rows in named:
        if not t.is_cuda or t.dtype != q.dtype or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-d GPU tensor of q's dtype")
        if t.shape[0] != q.shape[0] or t.shape[1] != q.shape[1] or t.shape[3] != q.shape[3] \
                or t.shape[2] != rows:
            raise ValueError(f"{name} shape {tuple(t.shape)} does not match the chunk/frame sizes")


def monarch_attn_fwd_kv(q, k, v, out, fq, f, h, w, b1, b2, tiles=1, iters=1, workspace=None,
                        stream=None):
    """Chunk of fq frames (q, out [B,H,fq*h*w,d]) against all f frames (k, v
    [B,H,f*h*w,d]); (b1, b2) block the keys.  Either dtype; with ``workspace``
    (a uint8 GPU tensor) nothing is allocated."""
    import torch
    _kv_tensors(q, fq, f, h, w, [("q", q), ("out", out)], [("k", k), ("v", v)])
    B, H, _, d = q.shape
    ptrs = [_ptr(t) for t in (q, k, v, out)]
    dims = [B, H, fq, f, h, w, d, b1, b2, tiles, iters]
    if workspace is None:
        _check(lib().monarch_attn_fwd_kv(*ptrs, *dims, _dtype_code(q), _stream(stream)), "monarch_attn_fwd_kv")
    else:
        if not workspace.is_cuda or workspace.dtype != torch.uint8:
            raise ValueError("workspace must be a uint8 GPU tensor")
        _check(lib().monarch_attn_fwd_kv_ws(*ptrs, *dims, _dtype_code(q), _ptr(workspace),
                                            workspace.numel(), _stream(stream)), "monarch_attn_fwd_kv_ws")
    return out


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return MONARCH_BF16
    if t.dtype == torch.float32:
        return MONARCH_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def monarch_attn_train_state_bytes(B, H, f, h, w, d, b1, b2, tiles, iters, dtype=MONARCH_BF16) -> int:
    return int(lib().monarch_attn_train_state_bytes(B, H, f, h, w, d, b1, b2, tiles, iters, dtype))


def _state(state):
    import torch
    if not state.is_cuda or state.dtype != torch.uint8:
        raise ValueError("state must be a uint8 GPU tensor")
    return _ptr(state), state.numel()


def monarch_attn_fwd_train(q, k, v, out, f, h, w, b1, b2, tiles, iters, state, stream=None):
    """Forward (``iters`` iterations) that also fills ``state`` for the backward."""
    ptrs = _tensors(q, k, v, out, q.dtype)
    sp, sn = _state(state)
    dims = _dims(q, f, h, w, b1, b2, tiles, iters)
    _check(lib().monarch_attn_fwd_train(*ptrs, *dims, _dtype_code(q), sp, sn, _stream(stream)),
           "monarch_attn_fwd_train")
    return out


def monarch_attn_bwd(q, k, v, out, dout, dq, dk, dv, f, h, w, b1, b2, tiles, iters, state, stream=None):
    """dq, dk, dv <- gradients of sum(dout * out) (state from monarch_attn_fwd_train)."""
    if dout.shape != q.shape:
        raise ValueError(f"dout shape {tuple(dout.shape)} != q shape {tuple(q.shape)}")
    ptrs = _tensors(q, k, v, out, q.dtype) + _tensors(dout, dq, dk, dv, q.dtype)
    sp, sn = _state(state)
    dims = _dims(q, f, h, w, b1, b2, tiles, iters)
    _check(lib().monarch_attn_bwd(*ptrs, *dims, _dtype_code(q), sp, sn, _stream(stream)),
           "monarch_attn_bwd")
    return dq, dk, dv


def monarch_attn_adaptive_kv_workspace_bytes(B, H, fq, f, h, w, d, b1, b2, tiles, max_iters,
                                              dtype=MONARCH_BF16) -> int:
    return int(lib().monarch_attn_adaptive_kv_workspace_bytes(B, H, fq, f, h, w, d, b1, b2, tiles, max_iters,
                                                              dtype))


def monarch_attn_fwd_adaptive_kv(q, k, v, out, fq, f, h, w, b1, b2, tiles, max_iters, tol, iters_used=None,
                                 workspace=None, stream=None):
    """monarch_attn_fwd_adaptive for a chunk of fq frames against all f frames.
    Returns (out, iters_used)."""
    import torch
    _kv_tensors(q, fq, f, h, w, [("q", q), ("out", out)], [("k", k), ("v", v)])
    B, H, _, d = q.shape
    dt = _dtype_code(q)
    if iters_used is None:
        iters_used = torch.empty((B, H), dtype=torch.int32, device=q.device)
    if not iters_used.is_cuda or iters_used.dtype != torch.int32 or iters_used.numel() != B * H:
        raise ValueError("iters_used must be an int32 GPU tensor of B*H elements")
    if workspace is None:
        nb = monarch_attn_adaptive_kv_workspace_bytes(B, H, fq, f, h, w, d, b1, b2, tiles, max_iters, dt)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=q.device)
    ptrs = [_ptr(t) for t in (q, k, v, out)]
    _check(lib().monarch_attn_fwd_adaptive_kv_ws(*ptrs, B, H, fq, f, h, w, d, b1, b2, tiles, max_iters, float(tol),
                                                 dt, _ptr(iters_used),
                                                 _ptr(workspace), workspace.numel(),
                                                 _stream(stream)), "monarch_attn_fwd_adaptive_kv_ws")
    return out, iters_used


def monarch_attn_train_state_bytes_kv(B, H, fq, f, h, w, d, b1, b2, tiles, iters, dtype=MONARCH_BF16) -> int:
    return int(lib().monarch_attn_train_state_bytes_kv(B, H, fq, f, h, w, d, b1, b2, tiles, iters, dtype))


def monarch_attn_fwd_train_kv(q, k, v, out, fq, f, h, w, b1, b2, tiles, iters, state, stream=None):
    """Training forward of a chunk of fq frames against all f frames (fills ``state``)."""
    _kv_tensors(q, fq, f, h, w, [("q", q), ("out", out)], [("k", k), ("v", v)])
    sp, sn = _state(state)
    B, H, _, d = q.shape
    ptrs = [_ptr(t) for t in (q, k, v, out)]
    _check(lib().monarch_attn_fwd_train_kv(*ptrs, B, H, fq, f, h, w, d, b1, b2, tiles, iters, _dtype_code(q),
                                           sp, sn, _stream(stream)), "monarch_attn_fwd_train_kv")
    return out


def monarch_attn_bwd_kv(q, k, v, out, dout, dq, dk, dv, fq, f, h, w, b1, b2, tiles, iters, state, stream=None):
    """dq [B,H,fq*h*w,d], dk, dv [B,H,f*h*w,d] <- gradients of sum(dout * out) of a chunk."""
    _kv_tensors(q, fq, f, h, w, [("q", q), ("out", out), ("dout", dout), ("dq", dq)],
                [("k", k), ("v", v), ("dk", dk), ("dv", dv)])
    sp, sn = _state(state)
    B, H, _, d = q.shape
    ptrs = [_ptr(t) for t in (q, k, v, out, dout, dq, dk, dv)]
    _check(lib().monarch_attn_bwd_kv(*ptrs, B, H, fq, f, h, w, d, b1, b2, tiles, iters, _dtype_code(q),
                                     sp, sn, _stream(stream)), "monarch_attn_bwd_kv")
    return dq, dk, dv


def monarch_attn_profile_enable(on: bool = True):
    _check(lib().monarch_attn_profile_enable(1 if on else 0), "monarch_attn_profile_enable")


def monarch_attn_profile_collect():
    """{kernel name: (total ms, launches)} since the last collect."""
    n = MONARCH_NUM_KERNELS
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_long * n)()
    _check(lib().monarch_attn_profile_collect(ms, cnt, n), "monarch_attn_profile_collect")
    return {monarch_attn_kernel_name(i): (ms[i], cnt[i]) for i in range(n)}


def monarch_attn_kernel_name(i: int) -> str:
    return lib().monarch_attn_kernel_name(int(i)).decode()
