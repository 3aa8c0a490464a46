"""The C ABI on the CPU: every declared symbol is exported, arguments are
checked before any GPU call, and the workspace formula (no GPU needed)."""
import ctypes
import os
import re

import pytest

import structured_attention_video_monarch_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "monarch_attn.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(monarch_\w+)\s*\(", txt, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("monarch_attn_fwd", "monarch_attn_fwd_f32", "monarch_attn_fwd_ws",
              "monarch_attn_workspace_bytes", "monarch_attn_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = M.lib()
    raw = ctypes.CDLL(M.LIB_PATH)
    for n in declared_functions():
        assert hasattr(raw, n), n
    assert lib is not None


def _fwd(q=1, k=2, v=3, out=4, B=1, H=2, f=3, h=30, w=52, d=128, b1=90, b2=52, t=1, T=1):
    P = ctypes.c_void_p
    return M.lib().monarch_attn_fwd(P(q), P(k), P(v), P(out), B, H, f, h, w, d, b1, b2, t, T, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), M.MONARCH_EINVAL),
    (dict(out=0), M.MONARCH_EINVAL),
    (dict(B=0), M.MONARCH_EINVAL),
    (dict(d=-1), M.MONARCH_EINVAL),
    (dict(b1=91), M.MONARCH_EINVAL),
    (dict(t=0), M.MONARCH_EINVAL),
    (dict(t=91), M.MONARCH_EINVAL),
    (dict(T=0), M.MONARCH_EINVAL),
    (dict(d=48), M.MONARCH_EUNSUPPORTED),
    (dict(d=256), M.MONARCH_EUNSUPPORTED),
    (dict(f=1, h=1, w=16400, b1=1, b2=16400), M.MONARCH_EUNSUPPORTED),  # key blocks beyond 16384
    (dict(out=1 + 1000), M.MONARCH_EINVAL),  # overlaps q (bytes 1 .. 1 + 2*N*d*2)
])
def test_bad_arguments_rejected_before_any_gpu_call(kw, status):
    # pointers are fake: the check must fail before anything touches them
    assert _fwd(**kw) == status


def test_status_strings():
    for s in (0, -1, -2, -3, -4, 12345):
        assert isinstance(M.monarch_attn_status_string(s), str)
    assert M.monarch_attn_status_string(M.MONARCH_EINVAL) == "invalid argument"


def test_kernel_names():
    names = [M.monarch_attn_kernel_name(i) for i in range(M.MONARCH_NUM_KERNELS)]
    assert len(set(names)) == M.MONARCH_NUM_KERNELS
    assert M.monarch_attn_kernel_name(99) == "unknown"


def _align(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("shape", [
    (1, 12, 3, 30, 52, 128, 90, 52, 1, 1, 0),
    (1, 40, 21, 45, 80, 128, 945, 80, 4, 1, 0),
    (2, 3, 3, 7, 13, 32, 21, 13, 2, 2, 1),
])
def test_workspace_bytes(shape):
    B, H, f, h, w, d, b1, b2, t, T, dt = shape
    e = 2 if dt == 0 else 4
    N, BH = f * h * w, B * H
    expect = _align(BH * b1 * d * e) + _align(BH * b1 * 4) + _align(BH * N * 4) + _align(BH * t * N * d * e)
    if T > 1:
        expect += _align(BH * t * N * d * e) + _align(BH * t * N * 4)
    assert M.monarch_attn_workspace_bytes(*shape) == expect


def test_workspace_bytes_zero_when_invalid():
    assert M.monarch_attn_workspace_bytes(1, 1, 2, 4, 4, 16, 8, 5, 1, 1, 1) == 0
    assert M.monarch_attn_workspace_bytes(1, 1, 2, 4, 4, 16, 8, 4, 1, 1, 7) == 0


# ---- training entry points (fake, widely spaced pointers: checks only)
_GAP = 1 << 40


def _train_ptrs(n):
    return [ctypes.c_void_p((i + 1) * _GAP) for i in range(n)]


def _bwd(state_bytes=None, B=1, H=2, f=3, h=30, w=52, d=128, b1=90, b2=52, t=1, T=1, dtype=0, null=None,
         alias=None):
    p = _train_ptrs(9)  # q k v out dout dq dk dv state
    if null is not None:
        p[null] = ctypes.c_void_p(0)
    if alias is not None:
        p[alias[0]] = p[alias[1]]
    if state_bytes is None:
        state_bytes = M.monarch_attn_train_state_bytes(B, H, f, h, w, d, b1, b2, t, T, dtype)
    return M.lib().monarch_attn_bwd(*p[:8], B, H, f, h, w, d, b1, b2, t, T, dtype, p[8], state_bytes, None)


@pytest.mark.parametrize("T", [1, 2, 5])
def test_train_state_bytes_formula(T):
    B, H, f, h, w, d, b1, b2, t = 1, 40, 21, 45, 80, 128, 945, 80, 4
    N, BH, e = f * h * w, B * H, 2
    per_iter = _align(BH * N * 4) + _align(BH * t * N * 4) + _align(BH * t * N * d * e)
    expect = (_align(BH * b1 * d * e) + _align(BH * b1 * 4) + T * per_iter + _align(BH * t * N * d * e)
              + (T - 1) * (_align(BH * t * N * d * e) + _align(BH * t * N * 4)))
    assert M.monarch_attn_train_state_bytes(B, H, f, h, w, d, b1, b2, t, T, 0) == expect
    assert M.monarch_attn_train_state_bytes(B, H, f, h, w, d, b1 + 1, b2, t, T, 0) == 0
    assert M.monarch_attn_train_state_bytes(B, H, f, h, w, d, b1, b2, t, 0, 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(null=4), M.MONARCH_EINVAL),                     # dout NULL
    (dict(null=5), M.MONARCH_EINVAL),                     # dq NULL
    (dict(null=8), M.MONARCH_ENOMEM),                     # state NULL
    (dict(state_bytes=1024), M.MONARCH_ENOMEM),           # state too small
    (dict(alias=(5, 0)), M.MONARCH_EINVAL),               # dq aliases q
    (dict(alias=(7, 6)), M.MONARCH_EINVAL),               # dv aliases dk
    (dict(alias=(6, 8)), M.MONARCH_EINVAL),               # dk aliases the state
    (dict(b1=91), M.MONARCH_EINVAL),
    (dict(d=48), M.MONARCH_EUNSUPPORTED),
    (dict(f=1, h=1, w=16400, b1=1, b2=16400), M.MONARCH_EUNSUPPORTED),  # key blocks beyond 16384
    (dict(T=0, state_bytes=1 << 30), M.MONARCH_EINVAL),
    (dict(T=2, state_bytes="T1"), M.MONARCH_ENOMEM),  # state of a one-iteration forward
])
def test_bwd_bad_arguments_rejected_before_any_gpu_call(kw, status):
    if kw.get("state_bytes") == "T1":
        kw = dict(kw, state_bytes=M.monarch_attn_train_state_bytes(1, 2, 3, 30, 52, 128, 90, 52, 1, 1, 0))
    assert _bwd(**kw) == status


def test_long_key_blocks_sizes():
    # blocks of whole frames (b2 = h*w > 128): the state of short blocks plus
    # every R-step's row log-sum-exps
    B, H, f, h, w, d, b1, b2, t, T = 1, 2, 3, 20, 26, 64, 3, 520, 1, 2
    assert M.monarch_attn_workspace_bytes(B, H, f, h, w, d, b1, b2, t, T, 0) > 0
    assert M.monarch_attn_kv_workspace_bytes(B, H, 1, f, h, w, d, b1, b2, t, T, 0) > 0
    N, e = f * h * w, 2
    expect = (_align(B * H * b1 * d * e) + _align(B * H * b1 * 4)
              + T * (_align(B * H * N * 4) + _align(B * H * t * N * 4) + _align(B * H * t * N * d * e))
              + _align(B * H * t * N * d * e) + (T - 1) * (_align(B * H * t * N * d * e) + _align(B * H * t * N * 4)))
    assert M.monarch_attn_train_state_bytes(B, H, f, h, w, d, b1, b2, t, T, 0) == expect + T * _align(B * H * t * N * 4)
    assert M.monarch_attn_train_state_bytes_kv(B, H, 1, f, h, w, d, b1, b2, t, T, 0) > 0


def test_fwd_train_rejects_small_state():
    p = _train_ptrs(5)
    rc = M.lib().monarch_attn_fwd_train(*p[:4], 1, 2, 3, 30, 52, 128, 90, 52, 1, 1, 0, p[4], 256, None)
    assert rc == M.MONARCH_ENOMEM


# ---- chunked queries against cached keys
def _kv(B=1, H=2, fq=3, f=21, h=30, w=52, d=128, b1=630, b2=52, t=1, T=1, dtype=0, out=None):
    p = _train_ptrs(4)
    if out is not None:
        p[3] = p[out]
    return M.lib().monarch_attn_fwd_kv(*p, B, H, fq, f, h, w, d, b1, b2, t, T, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(b1=629), M.MONARCH_EINVAL),                  # b1*b2 != f*h*w
    (dict(fq=0), M.MONARCH_EINVAL),
    (dict(t=91), M.MONARCH_EINVAL),                    # tiles > query blocks (90)
    (dict(fq=1, h=3, w=5, f=4, b1=12, b2=5, t=1, d=64), None),  # valid shape: checked below
    (dict(fq=1, h=3, w=5, f=4, b1=6, b2=10, t=1, d=64), M.MONARCH_EINVAL),  # Nq = 15 not a multiple of b2
    (dict(out=0), M.MONARCH_EINVAL),                   # out aliases q
    (dict(d=48), M.MONARCH_EUNSUPPORTED),
])
def test_kv_bad_arguments_rejected_before_any_gpu_call(kw, status):
    if status is None:
        assert M.monarch_attn_kv_workspace_bytes(1, 2, 1, 4, 3, 5, 64, 12, 5, 1, 1, 0) > 0
        return
    assert _kv(**kw) == status


def test_kv_workspace_bytes():
    B, H, fq, f, h, w, d, b1, b2, t, T = 1, 40, 3, 21, 45, 80, 128, 945, 80, 1, 2
    N, Nq, BH, e = f * h * w, fq * h * w, B * H, 2
    expect = (_align(BH * b1 * d * e) + _align(BH * b1 * 4) + _align(BH * Nq * 4) + _align(BH * t * N * d * e)
              + _align(BH * t * N * d * e) + _align(BH * t * N * 4))
    assert M.monarch_attn_kv_workspace_bytes(B, H, fq, f, h, w, d, b1, b2, t, T, 0) == expect
    # fq == f is the square layer
    assert (M.monarch_attn_kv_workspace_bytes(B, H, f, f, h, w, d, b1, b2, 4, 1, 0)
            == M.monarch_attn_workspace_bytes(B, H, f, h, w, d, b1, b2, 4, 1, 0))


def test_adaptive_workspace_and_bad_arguments():
    shape = (1, 40, 21, 45, 80, 128, 945, 80, 4, 10, 0)
    nb = M.monarch_attn_adaptive_workspace_bytes(*shape)
    # the forward's workspace, then the previous objective per head (double)
    # and the counts of heads stopped after each iteration (max_iters + 1 ints)
    assert nb == M.monarch_attn_workspace_bytes(*shape) + _align(40 * 8) + _align(11 * 4)
    p = _train_ptrs(6)  # q k v out iters_used workspace
    base = (1, 2, 3, 30, 52, 128, 90, 52, 1, 10)
    lib = M.lib()
    need = M.monarch_attn_adaptive_workspace_bytes(*base, 0)
    rc = lib.monarch_attn_fwd_adaptive_ws(*p[:4], *base, float("nan"), 0, p[4], p[5], need, None)
    assert rc == M.MONARCH_EINVAL
    rc = lib.monarch_attn_fwd_adaptive_ws(*p[:4], *base, 1e-3, 0, None, p[5], need, None)
    assert rc == M.MONARCH_EINVAL
    rc = lib.monarch_attn_fwd_adaptive_ws(*p[:4], *base, 1e-3, 0, p[4], p[5], need - 256, None)
    assert rc == M.MONARCH_ENOMEM


# ---- training for a chunk against cached keys
def test_kv_train_state_bytes():
    B, H, fq, f, h, w, d, b1, b2, t = 1, 40, 3, 21, 45, 80, 128, 945, 80, 1
    N, Nq, BH, e = f * h * w, fq * h * w, B * H, 2
    for T in (1, 2):
        per_iter = _align(BH * Nq * 4) + _align(BH * t * N * 4) + _align(BH * t * N * d * e)
        expect = (_align(BH * b1 * d * e) + _align(BH * b1 * 4) + T * per_iter + _align(BH * t * N * d * e)
                  + (T - 1) * (_align(BH * t * N * d * e) + _align(BH * t * N * 4)))
        assert M.monarch_attn_train_state_bytes_kv(B, H, fq, f, h, w, d, b1, b2, t, T, 0) == expect
        # fq == f is the square layer
        assert (M.monarch_attn_train_state_bytes_kv(B, H, f, f, h, w, d, b1, b2, 4, T, 0)
                == M.monarch_attn_train_state_bytes(B, H, f, h, w, d, b1, b2, 4, T, 0))
    assert M.monarch_attn_train_state_bytes_kv(B, H, fq, f, h, w, d, b1 + 1, b2, t, 1, 0) == 0


def _bwd_kv(state_bytes=None, fq=1, f=4, h=3, w=5, d=64, b1=12, b2=5, t=1, T=1, alias=None):
    p = _train_ptrs(9)  # q k v out dout dq dk dv state
    if alias is not None:
        p[alias[0]] = p[alias[1]]
    if state_bytes is None:
        state_bytes = M.monarch_attn_train_state_bytes_kv(1, 2, fq, f, h, w, d, b1, b2, t, T, 0)
    return M.lib().monarch_attn_bwd_kv(*p[:8], 1, 2, fq, f, h, w, d, b1, b2, t, T, 0, p[8], state_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(alias=(5, 0)), M.MONARCH_EINVAL),          # dq aliases q
    (dict(alias=(6, 3)), M.MONARCH_EINVAL),          # dk aliases out
    (dict(t=4), M.MONARCH_EINVAL),                   # tiles > query blocks (3)
    (dict(b1=6, b2=10), M.MONARCH_EINVAL),           # Nq = 15 not a multiple of b2
    (dict(state_bytes=4096), M.MONARCH_ENOMEM),
    (dict(d=48, state_bytes=1 << 30), M.MONARCH_EUNSUPPORTED),
])
def test_kv_bwd_bad_arguments_rejected_before_any_gpu_call(kw, status):
    assert _bwd_kv(**kw) == status


def test_adaptive_kv_workspace_and_bad_arguments():
    shape = (1, 40, 3, 21, 45, 80, 128, 945, 80, 1, 10, 0)
    nb = M.monarch_attn_adaptive_kv_workspace_bytes(*shape)
    assert nb == M.monarch_attn_kv_workspace_bytes(*shape) + _align(40 * 8) + _align(11 * 4)
    p = _train_ptrs(6)  # q k v out iters_used workspace
    base = (1, 2, 1, 4, 3, 5, 64, 12, 5, 1, 10)
    lib = M.lib()
    need = M.monarch_attn_adaptive_kv_workspace_bytes(*base, 0)
    assert lib.monarch_attn_fwd_adaptive_kv_ws(*p[:4], *base, float("nan"), 0, p[4], p[5], need,
                                               None) == M.MONARCH_EINVAL
    assert lib.monarch_attn_fwd_adaptive_kv_ws(*p[:4], *base, 1e-3, 0, None, p[5], need, None) == M.MONARCH_EINVAL
    assert lib.monarch_attn_fwd_adaptive_kv_ws(*p[:4], *base, 1e-3, 0, p[4], p[5], need - 256,
                                               None) == M.MONARCH_ENOMEM
    bad = (1, 2, 1, 4, 3, 5, 64, 12, 5, 4, 10)      # tiles 4 > query blocks 3
    assert lib.monarch_attn_fwd_adaptive_kv_ws(*p[:4], *bad, 1e-3, 0, p[4], p[5], 1 << 30,
                                               None) == M.MONARCH_EINVAL


# ---- the factors (test-only export)
def _factors(q=1, k=2, v=3, L=4, R=5, B=1, H=2, f=2, h=4, w=4, d=16, b1=8, b2=4, t=1, T=1):
    P = ctypes.c_void_p
    return M.lib().monarch_attn_debug_factors_f32(P(q), P(k), P(v), P(L), P(R), B, H, f, h, w, d, b1, b2, t, T, None)


@pytest.mark.parametrize("kw,status", [
    (dict(L=0), M.MONARCH_EINVAL),
    (dict(R=0), M.MONARCH_EINVAL),
    (dict(b1=7), M.MONARCH_EINVAL),
    (dict(T=0), M.MONARCH_EINVAL),
    (dict(d=48), M.MONARCH_EUNSUPPORTED),
    (dict(H=1 << 20, f=4, h=16, w=16, b1=64, b2=16), M.MONARCH_EUNSUPPORTED),  # more than 2^28 factor entries
    (dict(L=_GAP, R=_GAP + 64), M.MONARCH_EINVAL),  # L and R overlap
])
def test_factors_bad_arguments_rejected_before_any_gpu_call(kw, status):
    if "L" in kw and kw["L"] == _GAP:
        kw = dict(kw, q=2 * _GAP, k=3 * _GAP, v=4 * _GAP)
    assert _factors(**kw) == status


def test_binding_refuses_host_tensors_before_any_call():
    """The Python binding passes device addresses only: host tensors are
    refused with ValueError before the library is called."""
    import torch
    q = torch.zeros(1, 1, 12, 16, dtype=torch.bfloat16)
    ws = torch.zeros(64, dtype=torch.uint8)
    calls = [
        lambda: M.monarch_attn_fwd(q, q, q, q.clone(), 1, 3, 4, 3, 4),
        lambda: M.monarch_attn_fwd_f32(q.float(), q.float(), q.float(), q.float().clone(), 1, 3, 4, 3, 4),
        lambda: M.monarch_attn_fwd_ws(q, q, q, q.clone(), 1, 3, 4, 3, 4, 1, 1, ws),
        lambda: M.monarch_attn_fwd_kv(q, q, q, q.clone(), 1, 1, 3, 4, 3, 4),
        lambda: M.monarch_attn_fwd_adaptive(q, q, q, q.clone(), 1, 3, 4, 3, 4, 1, 3, 1e-3),
        lambda: M.monarch_attn_fwd_train(q, q, q, q.clone(), 1, 3, 4, 3, 4, 1, 1, ws),
        lambda: M.monarch_attn_bwd(q, q, q, q, q, q.clone(), q.clone(), q.clone(), 1, 3, 4, 3, 4, 1, 1, ws),
    ]
    for call in calls:
        with pytest.raises(ValueError):
            call()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: when the library is absent and the build produces none,
    the first call into the binding raises instead of computing anything."""
    import structured_attention_video_monarch_amd.build as B
    monkeypatch.setattr(M, "LIB_PATH", str(tmp_path / "libmonarch_attn.so"))
    monkeypatch.setattr(M, "_lib", None)
    monkeypatch.setattr(B, "build_library", lambda *a, **k: None)
    with pytest.raises(OSError):
        M.lib()
    with pytest.raises(OSError):
        M.monarch_attn_workspace_bytes(1, 1, 2, 4, 4, 16, 8, 4, 1, 1)


def test_binding_refuses_a_tensor_on_another_device(monkeypatch):
    """The kernels run on the current device: a GPU tensor elsewhere is
    refused before any call (a stand-in tensor and a patched current device,
    so no GPU is needed)."""
    import torch

    class OnDevice1:
        is_cuda = True
        device = torch.device("cuda", 1)

        def data_ptr(self):
            return 4096

    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    with pytest.raises(ValueError, match="current device"):
        M._ptr(OnDevice1())
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 1)
    assert M._ptr(OnDevice1()).value == 4096


class _StandIn:
    """A stand-in for a contiguous GPU tensor (no GPU needed): the attributes
    the binding reads before it calls the library."""

    def __init__(self, shape, dtype):
        import torch
        self.shape = torch.Size(shape)
        self.dtype = dtype
        self.is_cuda = True
        self.device = torch.device("cuda", 0)

    def is_contiguous(self):
        return True

    def dim(self):
        return len(self.shape)

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def data_ptr(self):
        return 1 << 20


class _NoCalls:
    """A library stub: any entry point that is reached fails the test."""

    def __getattr__(self, name):
        def called(*args):
            raise AssertionError(f"library entry point {name} was called")
        return called


def test_binding_refuses_other_dtypes_and_bad_gradient_shapes(monkeypatch):
    """fp16 and fp64 tensors are refused with ValueError before the library
    is called (the library has bf16 and fp32 kernels only), and so is a
    gradient whose shape differs from q's: the dimensions passed down are
    q's, so a smaller dout/dq/dk/dv would be read and written out of bounds."""
    import torch
    monkeypatch.setattr(M, "_lib", _NoCalls())
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    shp = (1, 1, 12, 16)
    ws = _StandIn((4096,), torch.uint8)
    for dt in (torch.float16, torch.float64):
        q = _StandIn(shp, dt)
        with pytest.raises(ValueError):
            M.monarch_attn_fwd_ws(q, q, q, _StandIn(shp, dt), 1, 3, 4, 3, 4, 1, 1, ws)
        with pytest.raises(ValueError):
            M.monarch_attn_fwd_train(q, q, q, _StandIn(shp, dt), 1, 3, 4, 3, 4, 1, 1, ws)
        with pytest.raises(ValueError):
            M.monarch_attn_fwd_adaptive(q, q, q, _StandIn(shp, dt), 1, 3, 4, 3, 4, 1, 3, 1e-3,
                                        iters_used=_StandIn((1, 1), torch.int32), workspace=ws)
        with pytest.raises(ValueError):
            M.monarch_attn_fwd_kv(q, q, q, _StandIn(shp, dt), 1, 1, 3, 4, 3, 4, workspace=ws)
    q = _StandIn((1, 12, 4680, 128), torch.bfloat16)
    small = _StandIn((1, 1, 32, 16), torch.bfloat16)
    with pytest.raises(ValueError):
        M.monarch_attn_bwd(q, q, q, _StandIn(q.shape, torch.bfloat16), small, small, small, small,
                           3, 30, 52, 90, 52, 1, 1, ws)
