"""head_wise_lstm_amd -- Python binding of libfrnn, the gfx950 head-wise LSTM / Elman / GRU
forward recurrence library (C ABI in include/frnn.h).

The binding only marshals arguments: it checks tensor shapes and dtypes, allocates the outputs and
the workspace with torch (device memory is torch's), and passes raw device pointers and torch's
current stream to the C entry points of the same names. Every step of the computation runs in the
library's HIP kernels. There is no fallback: if libfrnn.so is missing or no gfx950 device is
present, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "FRNN_PATH_ALTERNATING", "FRNN_PATH_FUSED", "FrnnError", "Desc", "lib_path", "load",
    "frnn_abi_version", "frnn_status_str", "frnn_workspace_bytes", "frnn_plan_str", "frnn_fwd",
    "frnn_check", "frnn_lstm_stack_workspace_bytes", "frnn_lstm_stack_fwd", "frnn_bwd_workspace_bytes",
    "frnn_bwd_plan_str", "frnn_bwd", "flashrnn", "frnn_lstm_stack_bwd_workspace_bytes", "frnn_lstm_stack_bwd",
    "frnn_init", "frnn_fwd_noalloc",
]

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfrnn.so"

FRNN_OK = 0
FRNN_CELL_LSTM, FRNN_CELL_ELMAN, FRNN_CELL_GRU = 0, 1, 2
FRNN_F32, FRNN_BF16 = 0, 1
FRNN_PATH_ALTERNATING, FRNN_PATH_FUSED = 0, 1

_CELLS = {"lstm": FRNN_CELL_LSTM, "elman": FRNN_CELL_ELMAN, "gru": FRNN_CELL_GRU}
_GATES_STATES = {"lstm": (4, 2), "elman": (1, 1), "gru": (3, 1)}
_PATHS = {"alternating": FRNN_PATH_ALTERNATING, "fused": FRNN_PATH_FUSED}
_DTYPES = {torch.float32: FRNN_F32, torch.bfloat16: FRNN_BF16}


class FrnnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {frnn_status_str(status)} ({status})")


class Desc(ctypes.Structure):
    """frnn_desc: sizes, cell, dtypes, then element strides (0 = the dense default)."""
    _fields_ = ([(n, ctypes.c_int32) for n in ("B", "T", "N", "D", "cell", "in_dtype", "out_dtype", "reserved")]
                + [(n, ctypes.c_int64) for n in ("wx_sb", "wx_st", "st_ss", "st_sb", "st_st", "r_sg", "r_sn", "r_sd")])


_lib = None


def lib_path() -> str:
    return os.path.join(HERE, _LIB_NAME)


def load():
    """Load libfrnn.so from this package folder (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m head_wise_lstm_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    dptr = ctypes.POINTER(Desc)
    lib.frnn_abi_version.restype = i32
    lib.frnn_abi_version.argtypes = []
    lib.frnn_init.restype = i32
    lib.frnn_init.argtypes = []
    lib.frnn_status_str.restype = ctypes.c_char_p
    lib.frnn_status_str.argtypes = [i32]
    lib.frnn_workspace_bytes.restype = i32
    lib.frnn_workspace_bytes.argtypes = [dptr, i32, ctypes.POINTER(sz)]
    lib.frnn_plan_str.restype = i32
    lib.frnn_plan_str.argtypes = [dptr, i32, ctypes.c_char_p, sz]
    lib.frnn_fwd.restype = i32
    lib.frnn_fwd.argtypes = [dptr, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.frnn_check.restype = i32
    lib.frnn_check.argtypes = [vp, vp]
    lib.frnn_fwd_noalloc.restype = i32
    lib.frnn_fwd_noalloc.argtypes = [dptr, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.frnn_bwd_workspace_bytes.restype = i32
    lib.frnn_bwd_workspace_bytes.argtypes = [dptr, i32, ctypes.POINTER(sz)]
    lib.frnn_bwd_plan_str.restype = i32
    lib.frnn_bwd_plan_str.argtypes = [dptr, i32, ctypes.c_char_p, sz]
    lib.frnn_bwd.restype = i32
    lib.frnn_bwd.argtypes = [dptr, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.frnn_lstm_stack_workspace_bytes.restype = i32
    lib.frnn_lstm_stack_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.frnn_lstm_stack_bwd_workspace_bytes.restype = i32
    lib.frnn_lstm_stack_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.frnn_lstm_stack_bwd.restype = i32
    lib.frnn_lstm_stack_bwd.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                        ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp, vp, vp, vp,
                                        ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                        ctypes.POINTER(vp), vp, vp, vp, sz, vp]
    lib.frnn_lstm_stack_fwd.restype = i32
    lib.frnn_lstm_stack_fwd.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                        ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp, vp, vp, vp, sz, vp]
    _lib = lib
    return lib


def frnn_abi_version() -> int:
    return load().frnn_abi_version()


_initialised = set()


def frnn_init(device=None) -> None:
    """frnn_init() on ``device`` (default: torch's current device), once per device: the one call
    that allocates device memory and waits for the device. Every compute wrapper below calls it
    for its tensors' device before its first call there."""
    idx = torch.cuda.current_device() if device is None else torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    if idx in _initialised:
        return
    with torch.cuda.device(idx):
        rc = load().frnn_init()
    if rc != FRNN_OK:
        raise FrnnError(rc, "frnn_init")
    _initialised.add(idx)


def frnn_status_str(status: int) -> str:
    return load().frnn_status_str(int(status)).decode()


def _desc(B, T, N, D, cell, in_dtype, out_dtype=FRNN_F32) -> Desc:
    return Desc(B, T, N, D, _CELLS[cell] if isinstance(cell, str) else cell,
                _DTYPES[in_dtype] if isinstance(in_dtype, torch.dtype) else in_dtype, out_dtype, 0)


def _path(path) -> int:
    return _PATHS[path] if isinstance(path, str) else int(path)


def frnn_workspace_bytes(desc: Desc, path="fused") -> int:
    n = ctypes.c_size_t(0)
    rc = load().frnn_workspace_bytes(ctypes.byref(desc), _path(path), ctypes.byref(n))
    if rc != FRNN_OK:
        raise FrnnError(rc, "frnn_workspace_bytes")
    return n.value


def frnn_plan_str(desc: Desc, path="fused") -> str:
    buf = ctypes.create_string_buffer(1024)
    rc = load().frnn_plan_str(ctypes.byref(desc), _path(path), buf, 1024)
    if rc != FRNN_OK:
        raise FrnnError(rc, "frnn_plan_str")
    return buf.value.decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def frnn_check(workspace: torch.Tensor, stream=None) -> None:
    """Wait for the stream, then raise if the device reported an error into the workspace."""
    st = _stream_handle(workspace.device) if stream is None else ctypes.c_void_p(stream)
    rc = load().frnn_check(_ptr(workspace), st)
    if rc != FRNN_OK:
        raise FrnnError(rc, "frnn_check")


def _check_tensor(t, name, shape, dtype, device, dense_inner=None):
    """Check device, dtype and shape. Without ``dense_inner`` the tensor must be contiguous; with
    it, only its last ``dense_inner`` dimensions must be dense, and its strides are returned."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device != device or t.dtype != dtype:
        raise ValueError(f"{name}: expected a {dtype} tensor on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dense_inner is None:
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
        return None
    st, expect = t.stride(), 1
    for k in range(t.dim() - 1, t.dim() - 1 - dense_inner, -1):
        if t.shape[k] > 1 and st[k] != expect:
            raise ValueError(f"{name}: its last {dense_inner} dimensions must be dense")
        expect *= t.shape[k]
    return st


def _set_strides(desc: Desc, wx=None, st=None, r=None) -> None:
    """Element strides of strided views into the description (None keeps the dense default)."""
    if wx is not None:
        desc.wx_sb, desc.wx_st = wx[0], wx[1]
    if st is not None:
        desc.st_ss, desc.st_sb, desc.st_st = st[0], st[1], st[2]
    if r is not None:
        desc.r_sg, desc.r_sn, desc.r_sd = r[0], r[1], r[2]


def frnn_fwd(Wx: torch.Tensor, R: torch.Tensor, b: Optional[torch.Tensor] = None,
             states: Optional[torch.Tensor] = None, cell: str = "lstm", path="fused",
             out: Optional[Sequence[torch.Tensor]] = None, workspace: Optional[torch.Tensor] = None,
             check: bool = True):
    """Head-wise forward: (states [S,B,T,N,D] fp32, last_states [S,B,1,N,D] fp32).

    Wx [B,T,G,N,D], R [G,N,D,D], b [G,N,D] or None, states (initial) [S,B,1,N,D] or None; all of
    one dtype (float32 or bfloat16) on one device. ``out`` may pass preallocated (states,
    last_states); ``workspace`` a preallocated uint8 tensor of at least frnn_workspace_bytes().
    With ``check`` the call waits for the stream and raises on a device-side error.
    """
    if cell not in _GATES_STATES:
        raise ValueError(f"unknown cell {cell!r}")
    G, S = _GATES_STATES[cell]
    if Wx.dim() != 5:
        raise ValueError("Wx must be [B,T,G,N,D]")
    B, T, G_, N, D = Wx.shape
    dev, dt = Wx.device, Wx.dtype
    if G_ != G or dt not in _DTYPES:
        raise ValueError("Wx: wrong gate count or dtype")
    wx_st = _check_tensor(Wx, "Wx", (B, T, G, N, D), dt, dev, dense_inner=3)
    r_st = _check_tensor(R, "R", (G, N, D, D), dt, dev, dense_inner=1)
    _check_tensor(b, "b", (G, N, D), dt, dev)
    _check_tensor(states, "states", (S, B, 1, N, D), dt, dev)
    desc = _desc(B, T, N, D, cell, dt)
    p = _path(path)
    if out is None:
        st_out = torch.empty((S, B, T, N, D), dtype=torch.float32, device=dev)
        last = torch.empty((S, B, 1, N, D), dtype=torch.float32, device=dev)
    else:
        st_out, last = out
        _check_tensor(last, "out[1]", (S, B, 1, N, D), torch.float32, dev)
    st_st = _check_tensor(st_out, "out[0]", (S, B, T, N, D), torch.float32, dev, dense_inner=2)
    _set_strides(desc, wx_st, st_st, r_st)
    need = frnn_workspace_bytes(desc, p)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() < need or workspace.device != dev:
        raise ValueError("workspace too small")
    frnn_init(dev)
    rc = load().frnn_fwd(ctypes.byref(desc), p, _ptr(Wx), _ptr(R), _ptr(b), _ptr(states), _ptr(st_out),
                         _ptr(last), _ptr(workspace), workspace.numel(), _stream_handle(dev))
    if rc != FRNN_OK:
        raise FrnnError(rc, "frnn_fwd")
    if check:
        frnn_check(workspace)
    return st_out, last


def frnn_fwd_noalloc(Wx: torch.Tensor, R: torch.Tensor, b: Optional[torch.Tensor], states: Optional[torch.Tensor],
                     out: Sequence[torch.Tensor], cell: str = "lstm", path="fused", check: bool = True):
    """frnn_fwd into the caller's ``out`` = (states [S,B,T,N,D], last_states [S,B,1,N,D]) fp32, with
    the library's own per-device array as the workspace: the call allocates nothing (for callers
    that cannot). Calls on one device share the array and must not overlap. Returns ``out``."""
    if cell not in _GATES_STATES:
        raise ValueError(f"unknown cell {cell!r}")
    G, S = _GATES_STATES[cell]
    B, T, G_, N, D = Wx.shape
    dev, dt = Wx.device, Wx.dtype
    if G_ != G or dt not in _DTYPES:
        raise ValueError("Wx: wrong gate count or dtype")
    wx_st = _check_tensor(Wx, "Wx", (B, T, G, N, D), dt, dev, dense_inner=3)
    r_st = _check_tensor(R, "R", (G, N, D, D), dt, dev, dense_inner=1)
    _check_tensor(b, "b", (G, N, D), dt, dev)
    _check_tensor(states, "states", (S, B, 1, N, D), dt, dev)
    st_out, last = out
    st_st = _check_tensor(st_out, "out[0]", (S, B, T, N, D), torch.float32, dev, dense_inner=2)
    _check_tensor(last, "out[1]", (S, B, 1, N, D), torch.float32, dev)
    desc = _desc(B, T, N, D, cell, dt)
    _set_strides(desc, wx_st, st_st, r_st)
    frnn_init(dev)
    stream = _stream_handle(dev)
    rc = load().frnn_fwd_noalloc(ctypes.byref(desc), _path(path), _ptr(Wx), _ptr(R), _ptr(b), _ptr(states),
                                 _ptr(st_out), _ptr(last), stream)
    if rc != FRNN_OK:
        raise FrnnError(rc, "frnn_fwd_noalloc")
    if check:
        rc = load().frnn_check(None, stream)
        if rc != FRNN_OK:
            raise FrnnError(rc, "frnn_check")
    return st_out, last


def frnn_bwd_workspace_bytes(desc: Desc, path="alternating") -> int:
    n = ctypes.c_size_t(0)
    rc = load().frnn_bwd_workspace_bytes(ctypes.byref(desc), _path(path), ctypes.byref(n))
    if rc != FRNN_OK:
        raise FrnnError(rc, "frnn_bwd_workspace_bytes")
    return n.value


def frnn_bwd_plan_str(desc: Desc, path="alternating") -> str:
    buf = ctypes.create_string_buffer(1024)
    rc = load().frnn_bwd_plan_str(ctypes.byref(desc), _path(path), buf, 1024)
    if rc != FRNN_OK:
        raise FrnnError(rc, "frnn_bwd_plan_str")
    return buf.value.decode()


def frnn_bwd(Wx: torch.Tensor, R: torch.Tensor, b: Optional[torch.Tensor], states0: Optional[torch.Tensor],
             states: torch.Tensor, dstates: Optional[torch.Tensor], dlast: Optional[torch.Tensor],
             cell: str = "lstm", path="alternating", workspace: Optional[torch.Tensor] = None, check: bool = True):
    """Backward of frnn_fwd: (dWx [B,T,G,N,D], dR [G,N,D,D], db [G,N,D], dstates0 [S,B,1,N,D]), fp32.

    Wx, R, b, states0 as for frnn_fwd; states [S,B,T,N,D] fp32 is what frnn_fwd returned for them;
    dstates [S,B,T,N,D] and dlast [S,B,1,N,D] (fp32 or None) are the gradients of its two outputs.
    """
    if cell not in _GATES_STATES:
        raise ValueError(f"unknown cell {cell!r}")
    G, S = _GATES_STATES[cell]
    B, T, G_, N, D = Wx.shape
    dev, dt = Wx.device, Wx.dtype
    if G_ != G or dt not in _DTYPES:
        raise ValueError("Wx: wrong gate count or dtype")
    wx_st = _check_tensor(Wx, "Wx", (B, T, G, N, D), dt, dev, dense_inner=3)
    r_st = _check_tensor(R, "R", (G, N, D, D), dt, dev, dense_inner=1)
    _check_tensor(b, "b", (G, N, D), dt, dev)
    _check_tensor(states0, "states0", (S, B, 1, N, D), dt, dev)
    st_st = _check_tensor(states, "states", (S, B, T, N, D), torch.float32, dev, dense_inner=2)
    if dstates is not None and dstates.stride() != states.stride():
        # dstates is read with the states' strides
        ds = torch.empty_strided(states.shape, states.stride(), dtype=torch.float32, device=dev)
        ds.copy_(dstates)
        dstates = ds
    _check_tensor(dstates, "dstates", (S, B, T, N, D), torch.float32, dev, dense_inner=2)
    _check_tensor(dlast, "dlast", (S, B, 1, N, D), torch.float32, dev)
    desc = _desc(B, T, N, D, cell, dt)
    _set_strides(desc, wx_st, st_st, r_st)
    p = _path(path)
    f = torch.float32
    # dWx and dR take the layouts (strides) of Wx and R
    dWx = torch.empty_strided((B, T, G, N, D), Wx.stride(), dtype=f, device=dev)
    dR = torch.empty_strided((G, N, D, D), R.stride(), dtype=f, device=dev)
    db = torch.empty((G, N, D), dtype=f, device=dev)
    ds0 = torch.empty((S, B, 1, N, D), dtype=f, device=dev)
    need = frnn_bwd_workspace_bytes(desc, p)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() < need or workspace.device != dev:
        raise ValueError("workspace too small")
    frnn_init(dev)
    rc = load().frnn_bwd(ctypes.byref(desc), p, _ptr(Wx), _ptr(R), _ptr(b), _ptr(states0), _ptr(states),
                         _ptr(dstates), _ptr(dlast), _ptr(dWx), _ptr(dR), _ptr(db), _ptr(ds0), _ptr(workspace),
                         workspace.numel(), _stream_handle(dev))
    if rc != FRNN_OK:
        raise FrnnError(rc, "frnn_bwd")
    if check:
        frnn_check(workspace)
    return dWx, dR, db, ds0


class _FlashRNNFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, Wx, R, b, states0, cell, path, bwd_path, check):
        states, last = frnn_fwd(Wx, R, b, states0, cell=cell, path=path, check=check)
        ctx.save_for_backward(Wx, R, b, states0, states)
        ctx.cell, ctx.bwd_path, ctx.check = cell, bwd_path, check
        return states, last

    @staticmethod
    def backward(ctx, dstates, dlast):
        Wx, R, b, states0, states = ctx.saved_tensors
        c = lambda t: None if t is None else t.float().contiguous()
        dWx, dR, db, ds0 = frnn_bwd(Wx, R, b, states0, states, c(dstates), c(dlast), cell=ctx.cell,
                                    path=ctx.bwd_path, check=ctx.check)
        cast = lambda g, like: None if like is None else g.to(like.dtype)
        return cast(dWx, Wx), cast(dR, R), cast(db, b), cast(ds0, states0), None, None, None, None


def flashrnn(Wx: torch.Tensor, R: torch.Tensor, b: Optional[torch.Tensor] = None,
             states: Optional[torch.Tensor] = None, cell: str = "lstm", path="fused", bwd_path=None,
             check: bool = False):
    """Differentiable head-wise forward (the FlashRNN page's functional call): returns (states,
    last_states) like frnn_fwd; torch autograd runs frnn_bwd for the gradients of Wx, R, b and the
    initial states (cast to their dtypes). bwd_path None: the fused backward where this build has
    a design for the shape and dtype, else the alternating one (both are HIP paths). Neither pass
    waits for the stream unless ``check`` is set (then each waits and raises on a device-side
    error, as frnn_check does)."""
    if bwd_path is None:
        B, T, _, N, D = Wx.shape
        try:
            frnn_bwd_plan_str(_desc(B, T, N, D, cell, Wx.dtype), "fused")
            bwd_path = "fused"
        except FrnnError as e:
            if e.status != -2:
                raise
            bwd_path = "alternating"
    return _FlashRNNFunction.apply(Wx, R, b, states, cell, path, bwd_path, check)


def frnn_lstm_stack_workspace_bytes(L, T, B, I, H, path="fused", dirs: int = 1) -> int:
    n = ctypes.c_size_t(0)
    rc = load().frnn_lstm_stack_workspace_bytes(L, dirs, T, B, I, H, _path(path), ctypes.byref(n))
    if rc != FRNN_OK:
        raise FrnnError(rc, "frnn_lstm_stack_workspace_bytes")
    return n.value


def frnn_lstm_stack_fwd(x: torch.Tensor, Wi: Sequence[torch.Tensor], Wh: Sequence[torch.Tensor],
                        b_ih: Sequence[Optional[torch.Tensor]], b_hh: Sequence[Optional[torch.Tensor]],
                        h0: Optional[torch.Tensor] = None, c0: Optional[torch.Tensor] = None, path="fused",
                        out: Optional[Sequence[torch.Tensor]] = None, workspace: Optional[torch.Tensor] = None,
                        check: bool = True, bidirectional: bool = False):
    """Multi-layer LSTM with input projection: (out [T,B,dirs*H], hn [L*dirs,B,H], cn [L*dirs,B,H]), fp32.

    x [T,B,I]; per layer l and direction k (index l*dirs + k, dirs = 2 when ``bidirectional``):
    Wi [in,4H] (in = I for l = 0, else dirs*H); Wh [H,4H]; b_ih, b_hh [4H] or None; h0, c0
    [L*dirs,B,H] or None; every tensor bfloat16 on one device. Direction 1 runs the sequence
    backwards; a layer's output is [h of direction 0, h of direction 1] at each step.
    """
    T, B, I = x.shape
    dirs = 2 if bidirectional else 1
    if len(Wi) % dirs or len(Wh) != len(Wi) or len(b_ih) != len(Wi) or len(b_hh) != len(Wi):
        raise ValueError("one Wi, Wh, b_ih and b_hh per layer and direction")
    L = len(Wi) // dirs
    H = Wh[0].shape[0]
    dev, bf = x.device, torch.bfloat16
    _check_tensor(x, "x", (T, B, I), bf, dev)
    for j in range(L * dirs):
        _check_tensor(Wi[j], f"Wi[{j}]", ((I if j < dirs else dirs * H), 4 * H), bf, dev)
        _check_tensor(Wh[j], f"Wh[{j}]", (H, 4 * H), bf, dev)
        _check_tensor(b_ih[j], f"b_ih[{j}]", (4 * H,), bf, dev)
        _check_tensor(b_hh[j], f"b_hh[{j}]", (4 * H,), bf, dev)
    _check_tensor(h0, "h0", (L * dirs, B, H), bf, dev)
    _check_tensor(c0, "c0", (L * dirs, B, H), bf, dev)
    p = _path(path)
    if out is None:
        o = torch.empty((T, B, dirs * H), dtype=torch.float32, device=dev)
        hn = torch.empty((L * dirs, B, H), dtype=torch.float32, device=dev)
        cn = torch.empty((L * dirs, B, H), dtype=torch.float32, device=dev)
    else:
        o, hn, cn = out
        _check_tensor(o, "out[0]", (T, B, dirs * H), torch.float32, dev)
        _check_tensor(hn, "out[1]", (L * dirs, B, H), torch.float32, dev)
        _check_tensor(cn, "out[2]", (L * dirs, B, H), torch.float32, dev)
    need = frnn_lstm_stack_workspace_bytes(L, T, B, I, H, p, dirs)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() < need:
        raise ValueError("workspace too small")
    frnn_init(dev)
    arr = ctypes.c_void_p * (L * dirs)
    ptrs = lambda ts: arr(*[0 if t is None else t.data_ptr() for t in ts])
    rc = load().frnn_lstm_stack_fwd(
        L, dirs, T, B, I, H, p, _ptr(x), ptrs(Wi), ptrs(Wh), ptrs(b_ih), ptrs(b_hh),
        _ptr(h0), _ptr(c0), _ptr(o), _ptr(hn), _ptr(cn), _ptr(workspace), workspace.numel(), _stream_handle(dev))
    if rc != FRNN_OK:
        raise FrnnError(rc, "frnn_lstm_stack_fwd")
    if check:
        frnn_check(workspace)
    return o, hn, cn


def frnn_lstm_stack_bwd_workspace_bytes(L, T, B, I, H, path="fused", dirs: int = 1) -> int:
    n = ctypes.c_size_t(0)
    rc = load().frnn_lstm_stack_bwd_workspace_bytes(L, dirs, T, B, I, H, _path(path), ctypes.byref(n))
    if rc != FRNN_OK:
        raise FrnnError(rc, "frnn_lstm_stack_bwd_workspace_bytes")
    return n.value


def frnn_lstm_stack_bwd(x: torch.Tensor, Wi: Sequence[torch.Tensor], Wh: Sequence[torch.Tensor],
                        b_ih: Sequence[Optional[torch.Tensor]], b_hh: Sequence[Optional[torch.Tensor]],
                        h0: Optional[torch.Tensor] = None, c0: Optional[torch.Tensor] = None,
                        dout: Optional[torch.Tensor] = None, dhn: Optional[torch.Tensor] = None,
                        dcn: Optional[torch.Tensor] = None, path="fused", workspace: Optional[torch.Tensor] = None,
                        check: bool = True, bidirectional: bool = False):
    """Backward of frnn_lstm_stack_fwd: (dx [T,B,I], dWi[], dWh[], db_ih[], db_hh[], dh0, dc0 [L*dirs,B,H]),
    fp32, for the loss sum(dout * out) + sum(dhn * hn) + sum(dcn * cn); dout [T,B,dirs*H], dhn, dcn
    [L*dirs,B,H] fp32 or None. The weight lists hold L*dirs entries, layer l direction k at
    l*dirs + k (dirs = 2 with ``bidirectional``), as for frnn_lstm_stack_fwd."""
    T, B, I = x.shape
    dirs = 2 if bidirectional else 1
    if len(Wi) % dirs:
        raise ValueError("two directions need two weights per layer")
    J = len(Wi)
    L = J // dirs
    H = Wh[0].shape[0]
    dev, bf, f = x.device, torch.bfloat16, torch.float32
    _check_tensor(x, "x", (T, B, I), bf, dev)
    ins = [(I if j < dirs else dirs * H) for j in range(J)]
    for j in range(J):
        _check_tensor(Wi[j], f"Wi[{j}]", (ins[j], 4 * H), bf, dev)
        _check_tensor(Wh[j], f"Wh[{j}]", (H, 4 * H), bf, dev)
        _check_tensor(b_ih[j], f"b_ih[{j}]", (4 * H,), bf, dev)
        _check_tensor(b_hh[j], f"b_hh[{j}]", (4 * H,), bf, dev)
    _check_tensor(h0, "h0", (J, B, H), bf, dev)
    _check_tensor(c0, "c0", (J, B, H), bf, dev)
    _check_tensor(dout, "dout", (T, B, dirs * H), f, dev)
    _check_tensor(dhn, "dhn", (J, B, H), f, dev)
    _check_tensor(dcn, "dcn", (J, B, H), f, dev)
    p = _path(path)
    dx = torch.empty((T, B, I), dtype=f, device=dev)
    dWi = [torch.empty((ins[j], 4 * H), dtype=f, device=dev) for j in range(J)]
    dWh = [torch.empty((H, 4 * H), dtype=f, device=dev) for _ in range(J)]
    dbi = [torch.empty((4 * H,), dtype=f, device=dev) for _ in range(J)]
    dbh = [torch.empty((4 * H,), dtype=f, device=dev) for _ in range(J)]
    dh0 = torch.empty((J, B, H), dtype=f, device=dev)
    dc0 = torch.empty((J, B, H), dtype=f, device=dev)
    need = frnn_lstm_stack_bwd_workspace_bytes(L, T, B, I, H, p, dirs)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() < need:
        raise ValueError("workspace too small")
    frnn_init(dev)
    arr = ctypes.c_void_p * J
    ptrs = lambda ts: arr(*[0 if t is None else t.data_ptr() for t in ts])
    rc = load().frnn_lstm_stack_bwd(
        L, dirs, T, B, I, H, p, _ptr(x), ptrs(Wi), ptrs(Wh), ptrs(b_ih), ptrs(b_hh), _ptr(h0), _ptr(c0), _ptr(dout),
        _ptr(dhn), _ptr(dcn), _ptr(dx), ptrs(dWi), ptrs(dWh), ptrs(dbi), ptrs(dbh), _ptr(dh0), _ptr(dc0),
        _ptr(workspace), workspace.numel(), _stream_handle(dev))
    if rc != FRNN_OK:
        raise FrnnError(rc, "frnn_lstm_stack_bwd")
    if check:
        frnn_check(workspace)
    return dx, dWi, dWh, dbi, dbh, dh0, dc0
