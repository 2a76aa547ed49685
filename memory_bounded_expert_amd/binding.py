"""Thin Python binding of libmoebound.so (ctypes).

Argument marshalling only: the functions carry the C ABI's names, check that
torch tensors have the shapes, dtypes and devices the C ABI expects, allocate
missing outputs and the workspace with torch, and pass raw device pointers
and the current HIP stream.  Every step of the layer runs in the library's
HIP kernels; there is no fallback.  Loading fails loudly when the library is
not built.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoebound.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
HEADERS = (os.path.join(INCLUDE, "moebound.h"), os.path.join(INCLUDE, "cce.h"))

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, 1, 2, 3, 4
STAGES = {"router": 0, "topk": 1, "plan": 2, "gather": 3, "gemm_up": 4, "gemm_down": 5,
          "combine": 6}
BSTAGES = {"zero": 0, "transpose": 1, "plan": 2, "recompute": 3, "dh": 4, "wgrad_down": 5,
           "wgrad_gate_up": 6, "dx": 7, "combine_bwd": 8, "dwr": 9}
MOE_F32, MOE_BF16 = 0, 1
CCE_STAGES = {"logits": 0, "fold": 1, "grad": 2, "dx": 3, "dw": 4}

_c = ctypes
_vp = _c.c_void_p


class MoePlan(_c.Structure):
    _fields_ = [
        ("magic", _c.c_uint32), ("dtype", _c.c_int32), ("N", _c.c_int64),
        ("H", _c.c_int32), ("F", _c.c_int32), ("E", _c.c_int32), ("k", _c.c_int32),
        ("c", _c.c_int32), ("K_max", _c.c_int32), ("K", _c.c_int32), ("flags", _c.c_int32),
        ("c_eff", _c.c_int64), ("max_pairs_per_chunk", _c.c_int64),
        ("dispatch_bound_bytes", _c.c_int64), ("fwd_workspace_bytes", _c.c_int64),
        ("bwd_workspace_bytes", _c.c_int64), ("debug_workspace_bytes", _c.c_int64),
    ]


class MoeStats(_c.Structure):
    _fields_ = [
        ("K", _c.c_int32), ("launches", _c.c_int32), ("c_eff", _c.c_int64),
        ("max_pairs_per_chunk", _c.c_int64), ("dispatch_bytes", _c.c_int64),
        ("dispatch_bound_bytes", _c.c_int64), ("intermediate_bytes", _c.c_int64),
        ("workspace_bytes", _c.c_int64),
    ]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class CcePlan(_c.Structure):
    _fields_ = [
        ("magic", _c.c_uint32), ("dtype", _c.c_int32), ("N", _c.c_int64), ("V", _c.c_int64),
        ("H", _c.c_int32), ("v_chunk", _c.c_int32), ("S", _c.c_int32), ("reserved0", _c.c_int32),
        ("strip_bound_bytes", _c.c_int64), ("unchunked_logit_bytes", _c.c_int64),
        ("fwd_workspace_bytes", _c.c_int64), ("bwd_workspace_bytes", _c.c_int64),
    ]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded after torch, so that it binds to the HIP
    runtime torch already uses)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    L.moe_status_string.restype = _c.c_char_p
    L.moe_status_string.argtypes = [_c.c_int]
    L.moe_plan_chunks.restype = _c.c_int
    L.moe_plan_chunks.argtypes = [_c.c_int64, _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int32,
                                  _c.c_int32, _c.c_int32, _c.c_int32, _c.POINTER(MoePlan)]
    L.moe_plan_set_flags.restype = _c.c_int
    L.moe_plan_set_flags.argtypes = [_c.POINTER(MoePlan), _c.c_int32]
    L.moe_bounded_forward.restype = _c.c_int
    L.moe_bounded_forward.argtypes = [_c.POINTER(MoePlan)] + [_vp] * 10 + [_vp, _c.c_size_t, _vp,
                                                                         _c.POINTER(MoeStats)]
    L.moe_bounded_forward_static.restype = _c.c_int
    L.moe_bounded_forward_static.argtypes = [_c.POINTER(MoePlan)] + [_vp] * 10 + [
        _vp, _c.POINTER(MoeStats)]
    L.moe_bounded_backward.restype = _c.c_int
    L.moe_bounded_backward.argtypes = [_c.POINTER(MoePlan)] + [_vp] * 15 + [_vp, _c.c_size_t, _vp,
                                                                          _c.POINTER(MoeStats)]
    L.moe_debug_topk.restype = _c.c_int
    L.moe_debug_topk.argtypes = [_vp, _c.c_int64, _c.c_int32, _c.c_int32, _vp, _vp, _vp]
    L.moe_debug_plan.restype = _c.c_int
    L.moe_debug_plan.argtypes = [_c.POINTER(MoePlan), _vp, _vp, _vp, _vp, _vp, _c.c_size_t, _vp]
    L.moe_debug_stage.restype = _c.c_int
    L.moe_debug_stage.argtypes = [_c.POINTER(MoePlan), _c.c_int32, _c.c_int32] + [_vp] * 9 + [
        _vp, _c.c_size_t, _vp]
    L.moe_debug_stage_bwd.restype = _c.c_int
    L.moe_debug_stage_bwd.argtypes = [_c.POINTER(MoePlan), _c.c_int32, _c.c_int32] + [_vp] * 15 + [
        _vp, _c.c_size_t, _vp]
    L.cce_plan.restype = _c.c_int
    L.cce_plan.argtypes = [_c.c_int64, _c.c_int32, _c.c_int64, _c.c_int32, _c.c_int32,
                           _c.POINTER(CcePlan)]
    L.cce_forward.restype = _c.c_int
    L.cce_forward.argtypes = [_c.POINTER(CcePlan)] + [_vp] * 5 + [_vp, _c.c_size_t, _vp]
    L.cce_backward.restype = _c.c_int
    L.cce_backward.argtypes = [_c.POINTER(CcePlan)] + [_vp] * 7 + [_vp, _c.c_size_t, _vp]
    L.cce_debug_stage.restype = _c.c_int
    L.cce_debug_stage.argtypes = [_c.POINTER(CcePlan), _c.c_int32, _c.c_int32] + [_vp] * 8 + [
        _vp, _c.c_size_t, _vp]
    _LIB = L
    return L


def declared_functions() -> list:
    """Function names declared in include/moebound.h and include/cce.h."""
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:moe|cce)_[a-z_]+)\s*\(", text))
    return sorted(names)


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else _vp(t.data_ptr())


def torch_dtype(dtype: int) -> torch.dtype:
    return torch.bfloat16 if dtype == MOE_BF16 else torch.float32


def moe_dtype(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return MOE_BF16
    if t == torch.float32:
        return MOE_F32
    raise ValueError(f"unsupported dtype {t}")


def _expect(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: device {t.device} != {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return _vp(stream.cuda_stream)


def moe_plan_chunks(N: int, H: int, F: int, E: int, k: int, c: int, K_max: int,
                    dtype: int) -> MoePlan:
    plan = MoePlan()
    _check(lib().moe_plan_chunks(N, H, F, E, k, c, K_max, dtype, ctypes.byref(plan)),
           "moe_plan_chunks")
    return plan


MOE_PLAN_EXACT_DW = 1


def moe_plan_set_flags(plan: MoePlan, flags: int) -> MoePlan:
    """Set the plan's options in place (MOE_PLAN_EXACT_DW: order-invariant
    expert weight gradients); returns the plan."""
    _check(lib().moe_plan_set_flags(ctypes.byref(plan), flags), "moe_plan_set_flags")
    return plan


def workspace(plan, kind: str, device) -> torch.Tensor:
    """Workspace of a MoePlan ("fwd", "bwd", "debug") or CcePlan ("fwd", "bwd")."""
    n = getattr(plan, {"fwd": "fwd_workspace_bytes", "bwd": "bwd_workspace_bytes",
                       "debug": "debug_workspace_bytes"}[kind])
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


def moe_bounded_forward(plan: MoePlan, X, W_r, router_bias, W_gate, W_up, W_down,
                        Y=None, topk_idx=None, gates=None, logits=None, want_logits=True,
                        ws=None, stream=None):
    """Returns (Y, topk_idx, gates, logits or None, stats dict)."""
    dev = X.device
    dt = torch_dtype(plan.dtype)
    N, H, F, E, k = plan.N, plan.H, plan.F, plan.E, plan.k
    _expect(X, "X", (N, H), dt, dev)
    _expect(W_r, "W_r", (H, E), dt, dev)
    if router_bias is not None:
        _expect(router_bias, "router_bias", (E,), torch.float32, dev)
    _expect(W_gate, "W_gate", (E, H, F), dt, dev)
    _expect(W_up, "W_up", (E, H, F), dt, dev)
    _expect(W_down, "W_down", (E, F, H), dt, dev)
    Y = torch.empty((N, H), dtype=dt, device=dev) if Y is None else Y
    topk_idx = torch.empty((N, k), dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
    gates = torch.empty((N, k), dtype=torch.float32, device=dev) if gates is None else gates
    if logits is None and want_logits:
        logits = torch.empty((N, E), dtype=torch.float32, device=dev)
    _expect(Y, "Y", (N, H), dt, dev)
    _expect(topk_idx, "topk_idx", (N, k), torch.int32, dev)
    _expect(gates, "gates", (N, k), torch.float32, dev)
    if logits is not None:
        _expect(logits, "logits", (N, E), torch.float32, dev)
    ws = workspace(plan, "fwd", dev) if ws is None else ws
    st = MoeStats()
    _check(lib().moe_bounded_forward(
        ctypes.byref(plan), _ptr(X), _ptr(W_r), _ptr(router_bias), _ptr(W_gate), _ptr(W_up),
        _ptr(W_down), _ptr(Y), _ptr(topk_idx), _ptr(gates), _ptr(logits), _ptr(ws),
        ws.numel(), _stream(dev, stream), ctypes.byref(st)), "moe_bounded_forward")
    return Y, topk_idx, gates, logits, st.as_dict()


def moe_bounded_forward_static(plan: MoePlan, X, W_r, router_bias, W_gate, W_up, W_down,
                               Y=None, topk_idx=None, gates=None, logits=None,
                               want_logits=True, stream=None):
    """moe_bounded_forward on the library's static scratch array (no
    workspace).  Returns (Y, topk_idx, gates, logits or None, stats dict)."""
    dev = X.device
    dt = torch_dtype(plan.dtype)
    N, H, F, E, k = plan.N, plan.H, plan.F, plan.E, plan.k
    _expect(X, "X", (N, H), dt, dev)
    _expect(W_r, "W_r", (H, E), dt, dev)
    if router_bias is not None:
        _expect(router_bias, "router_bias", (E,), torch.float32, dev)
    _expect(W_gate, "W_gate", (E, H, F), dt, dev)
    _expect(W_up, "W_up", (E, H, F), dt, dev)
    _expect(W_down, "W_down", (E, F, H), dt, dev)
    Y = torch.empty((N, H), dtype=dt, device=dev) if Y is None else Y
    topk_idx = torch.empty((N, k), dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
    gates = torch.empty((N, k), dtype=torch.float32, device=dev) if gates is None else gates
    if logits is None and want_logits:
        logits = torch.empty((N, E), dtype=torch.float32, device=dev)
    _expect(Y, "Y", (N, H), dt, dev)
    _expect(topk_idx, "topk_idx", (N, k), torch.int32, dev)
    _expect(gates, "gates", (N, k), torch.float32, dev)
    if logits is not None:
        _expect(logits, "logits", (N, E), torch.float32, dev)
    st = MoeStats()
    _check(lib().moe_bounded_forward_static(
        ctypes.byref(plan), _ptr(X), _ptr(W_r), _ptr(router_bias), _ptr(W_gate), _ptr(W_up),
        _ptr(W_down), _ptr(Y), _ptr(topk_idx), _ptr(gates), _ptr(logits),
        _stream(dev, stream), ctypes.byref(st)), "moe_bounded_forward_static")
    return Y, topk_idx, gates, logits, st.as_dict()


def moe_bounded_backward(plan: MoePlan, X, W_r, W_gate, W_up, W_down, dY, topk_idx, gates,
                         dX=None, dW_gate=None, dW_up=None, dW_down=None, dlogits=None,
                         dgates=None, want_dgates=True, dW_r=None, want_dW_r=True, ws=None,
                         stream=None):
    """Returns dict with dX, dW_gate, dW_up, dW_down, dlogits, dgates, dW_r, stats."""
    dev = X.device
    dt = torch_dtype(plan.dtype)
    N, H, F, E, k = plan.N, plan.H, plan.F, plan.E, plan.k
    f32 = torch.float32
    for t, n, s, d in ((X, "X", (N, H), dt), (W_r, "W_r", (H, E), dt),
                       (W_gate, "W_gate", (E, H, F), dt), (W_up, "W_up", (E, H, F), dt),
                       (W_down, "W_down", (E, F, H), dt), (dY, "dY", (N, H), dt),
                       (topk_idx, "topk_idx", (N, k), torch.int32), (gates, "gates", (N, k), f32)):
        _expect(t, n, s, d, dev)
    new = lambda shape, d=f32: torch.empty(shape, dtype=d, device=dev)
    dX = new((N, H), dt) if dX is None else dX
    dW_gate = new((E, H, F)) if dW_gate is None else dW_gate
    dW_up = new((E, H, F)) if dW_up is None else dW_up
    dW_down = new((E, F, H)) if dW_down is None else dW_down
    dlogits = new((N, E)) if dlogits is None else dlogits
    if dgates is None and want_dgates:
        dgates = new((N, k))
    if dW_r is None and want_dW_r:
        dW_r = new((H, E))
    _expect(dX, "dX", (N, H), dt, dev)
    _expect(dW_gate, "dW_gate", (E, H, F), f32, dev)
    _expect(dW_up, "dW_up", (E, H, F), f32, dev)
    _expect(dW_down, "dW_down", (E, F, H), f32, dev)
    _expect(dlogits, "dlogits", (N, E), f32, dev)
    if dgates is not None:
        _expect(dgates, "dgates", (N, k), f32, dev)
    if dW_r is not None:
        _expect(dW_r, "dW_r", (H, E), f32, dev)
    ws = workspace(plan, "bwd", dev) if ws is None else ws
    st = MoeStats()
    _check(lib().moe_bounded_backward(
        ctypes.byref(plan), _ptr(X), _ptr(W_r), _ptr(W_gate), _ptr(W_up), _ptr(W_down),
        _ptr(dY), _ptr(topk_idx), _ptr(gates), _ptr(dX), _ptr(dW_gate), _ptr(dW_up),
        _ptr(dW_down), _ptr(dlogits), _ptr(dgates), _ptr(dW_r), _ptr(ws), ws.numel(),
        _stream(dev, stream), ctypes.byref(st)), "moe_bounded_backward")
    return dict(dX=dX, dW_gate=dW_gate, dW_up=dW_up, dW_down=dW_down, dlogits=dlogits,
                dgates=dgates, dW_r=dW_r, stats=st.as_dict())


def moe_debug_topk(logits: torch.Tensor, k: int, stream=None):
    dev = logits.device
    N, E = logits.shape
    _expect(logits, "logits", (N, E), torch.float32, dev)
    idx = torch.empty((N, k), dtype=torch.int32, device=dev)
    gates = torch.empty((N, k), dtype=torch.float32, device=dev)
    _check(lib().moe_debug_topk(_ptr(logits), N, E, k, _ptr(idx), _ptr(gates),
                                _stream(dev, stream)), "moe_debug_topk")
    return idx, gates


def moe_debug_plan(plan: MoePlan, topk_idx: torch.Tensor, stream=None):
    """Returns (offsets [K, E+1], perm [N*k], pos [N*k]) as int32 device tensors."""
    dev = topk_idx.device
    _expect(topk_idx, "topk_idx", (plan.N, plan.k), torch.int32, dev)
    offsets = torch.empty((plan.K, plan.E + 1), dtype=torch.int32, device=dev)
    perm = torch.empty(plan.N * plan.k, dtype=torch.int32, device=dev)
    pos = torch.empty(plan.N * plan.k, dtype=torch.int32, device=dev)
    ws = workspace(plan, "debug", dev)
    _check(lib().moe_debug_plan(ctypes.byref(plan), _ptr(topk_idx), _ptr(offsets), _ptr(perm),
                                _ptr(pos), _ptr(ws), ws.numel(), _stream(dev, stream)),
           "moe_debug_plan")
    return offsets, perm, pos


def moe_debug_stage(plan: MoePlan, stage: str, chunk: int, X, W_r, router_bias, W_gate, W_up,
                    W_down, Y, topk_idx, gates, ws, stream=None):
    """Re-launch one forward stage for one chunk (state from the last forward
    call on ``ws``, which must have been made with logits=None)."""
    _check(lib().moe_debug_stage(ctypes.byref(plan), STAGES[stage], chunk, _ptr(X), _ptr(W_r),
                                 _ptr(router_bias), _ptr(W_gate), _ptr(W_up), _ptr(W_down),
                                 _ptr(Y), _ptr(topk_idx), _ptr(gates), _ptr(ws), ws.numel(),
                                 _stream(X.device, stream)), "moe_debug_stage")


def moe_debug_stage_bwd(plan: MoePlan, stage: str, chunk: int, X, W_r, W_gate, W_up, W_down, dY,
                        topk_idx, gates, grads: dict, ws, stream=None):
    """Re-launch one backward stage (for one chunk) on the state of the last
    backward call on ``ws``; ``grads`` holds that call's output tensors (the
    dict moe_bounded_backward returns, or the tensors passed to it)."""
    _check(lib().moe_debug_stage_bwd(
        ctypes.byref(plan), BSTAGES[stage], chunk, _ptr(X), _ptr(W_r), _ptr(W_gate), _ptr(W_up),
        _ptr(W_down), _ptr(dY), _ptr(topk_idx), _ptr(gates), _ptr(grads["dX"]),
        _ptr(grads["dW_gate"]), _ptr(grads["dW_up"]), _ptr(grads["dW_down"]),
        _ptr(grads["dlogits"]), _ptr(grads.get("dgates")), _ptr(grads.get("dW_r")), _ptr(ws),
        ws.numel(), _stream(X.device, stream)), "moe_debug_stage_bwd")


# ---- vocabulary projection with cross-entropy over vocabulary strips


def cce_plan(N: int, H: int, V: int, v_chunk: int, dtype: int = MOE_BF16) -> CcePlan:
    plan = CcePlan()
    _check(lib().cce_plan(N, H, V, v_chunk, dtype, ctypes.byref(plan)), "cce_plan")
    return plan


def cce_forward(plan: CcePlan, X, W, targets, loss=None, lse=None, ws=None, stream=None):
    """Returns (loss [N], lse [N]) fp32."""
    dev = X.device
    N, H, V = plan.N, plan.H, plan.V
    _expect(X, "X", (N, H), torch.bfloat16, dev)
    _expect(W, "W", (V, H), torch.bfloat16, dev)
    _expect(targets, "targets", (N,), torch.int32, dev)
    loss = torch.empty(N, dtype=torch.float32, device=dev) if loss is None else loss
    lse = torch.empty(N, dtype=torch.float32, device=dev) if lse is None else lse
    _expect(loss, "loss", (N,), torch.float32, dev)
    _expect(lse, "lse", (N,), torch.float32, dev)
    ws = workspace(plan, "fwd", dev) if ws is None else ws
    _check(lib().cce_forward(ctypes.byref(plan), _ptr(X), _ptr(W), _ptr(targets), _ptr(loss),
                             _ptr(lse), _ptr(ws), ws.numel(), _stream(dev, stream)),
           "cce_forward")
    return loss, lse


def cce_backward(plan: CcePlan, X, W, targets, lse, dloss, dX=None, dW=None, ws=None,
                 stream=None):
    """Returns (dX [N, H] bf16, dW [V, H] fp32)."""
    dev = X.device
    N, H, V = plan.N, plan.H, plan.V
    f32 = torch.float32
    for t, n, shp, d in ((X, "X", (N, H), torch.bfloat16), (W, "W", (V, H), torch.bfloat16),
                         (targets, "targets", (N,), torch.int32), (lse, "lse", (N,), f32),
                         (dloss, "dloss", (N,), f32)):
        _expect(t, n, shp, d, dev)
    dX = torch.empty((N, H), dtype=torch.bfloat16, device=dev) if dX is None else dX
    dW = torch.empty((V, H), dtype=f32, device=dev) if dW is None else dW
    _expect(dX, "dX", (N, H), torch.bfloat16, dev)
    _expect(dW, "dW", (V, H), f32, dev)
    ws = workspace(plan, "bwd", dev) if ws is None else ws
    _check(lib().cce_backward(ctypes.byref(plan), _ptr(X), _ptr(W), _ptr(targets), _ptr(lse),
                              _ptr(dloss), _ptr(dX), _ptr(dW), _ptr(ws), ws.numel(),
                              _stream(dev, stream)), "cce_backward")
    return dX, dW


def cce_debug_stage(plan: CcePlan, stage: str, strip: int, X, W, targets, loss, lse, dloss, dX,
                    dW, ws, stream=None):
    """Re-launch one kernel of one strip (state from the last cce_forward or
    cce_backward call on ``ws``)."""
    _check(lib().cce_debug_stage(ctypes.byref(plan), CCE_STAGES[stage], strip, _ptr(X), _ptr(W),
                                 _ptr(targets), _ptr(loss), _ptr(lse), _ptr(dloss), _ptr(dX),
                                 _ptr(dW), _ptr(ws), ws.numel(), _stream(X.device, stream)),
           "cce_debug_stage")
