"""PyTorch-facing binding of the CARVE C ABI.

Argument marshalling only: tensors are checked, outputs and workspace are
allocated with torch on the GPU, and the C entry point is called on torch's
current HIP stream. Every step of the forward pass runs in the HIP library;
there is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.CARVE_F32, torch.bfloat16: _lib.CARVE_BF16}


def make_config(B, H, T, dk, dv, L, rank, dtype, decay_logits=False, qk_l2norm=False,
                detach_mean=False) -> _lib.CarveConfig:
    flags = ((_lib.CARVE_DECAY_LOGITS if decay_logits else 0) | (_lib.CARVE_QK_L2NORM if qk_l2norm else 0)
             | (_lib.CARVE_DETACH_MEAN if detach_mean else 0))
    return _lib.CarveConfig(B, H, T, dk, dv, L, rank, _DTYPES[dtype] if isinstance(dtype, torch.dtype) else dtype,
                            flags)


def recurrent_ref_shapes(B, H, T, dk, dv, L, rank=0, dtype=torch.bfloat16, decay_logits=False, qk_l2norm=False,
                         detach_mean=False) -> _lib.CarveShapes:
    return _lib.ref_shapes(make_config(B, H, T, dk, dv, L, rank, dtype, decay_logits, qk_l2norm, detach_mean))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def chunk_fwd(q, k, v, g, bx, w, L=64, ub_down=None, ub_up=None, state_in=None, mean_in=None,
              return_state=False, out=None, workspace=None, stream=None, decay_logits=False, qk_l2norm=False):
    """CARVE forward pass. Shapes: q, k, g, bx [B,T,H,dk]; v [B,T,H,dv]; w [B,T,H];
    ub_down [H,r,dv]; ub_up [H,dk,r]; state_in [B,H,dv,dk] fp32; mean_in [B,H,dv] fp32.
    With decay_logits, g holds raw decay logits a and the kernels use the
    log-decay -softplus(a). With qk_l2norm, q and k are divided per token by
    their L2 norms inside the kernels. Returns o [B,T,H,dv] (and (state_out,
    mean_out) when return_state)."""
    if q.device.type != "cuda":
        raise ValueError("chunk_fwd runs on the GPU only; move the inputs to a cuda device")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    rank = 0 if ub_down is None else int(ub_down.shape[1])
    if (ub_down is None) != (ub_up is None):
        raise ValueError("ub_down and ub_up come together")
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("v", v, (B, T, H, dv)),
                         ("g", g, (B, T, H, dk)), ("bx", bx, (B, T, H, dk)), ("w", w, (B, T, H))):
        _need(t, name, shp, dt, dev)
    if rank:
        _need(ub_down, "ub_down", (H, rank, dv), dt, dev)
        _need(ub_up, "ub_up", (H, dk, rank), dt, dev)
    _need(state_in, "state_in", (B, H, dv, dk), torch.float32, dev)
    _need(mean_in, "mean_in", (B, H, dv), torch.float32, dev)

    cfg = make_config(B, H, T, dk, dv, L, rank, dt, decay_logits, qk_l2norm)
    sh = _lib.ref_shapes(cfg)
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _need(o, "out", (B, T, H, dv), dt, dev)
    state_out = mean_out = None
    if return_state:
        state_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
        mean_out = torch.empty((B, H, dv), dtype=torch.float32, device=dev)
    ws_bytes = int(sh.workspace_bytes)
    if ws_bytes and (workspace is None or workspace.numel() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    code = _lib.lib().carve_chunk_fwd(
        ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(bx), _ptr(w),
        _ptr(ub_down), _ptr(ub_up), _ptr(state_in), _ptr(mean_in),
        _ptr(o), _ptr(state_out), _ptr(mean_out),
        _ptr(workspace) if ws_bytes else None, ctypes.c_size_t(ws_bytes if ws_bytes else 0),
        ctypes.c_void_p(stream))
    _lib.check(code)
    if return_state:
        return o, state_out, mean_out
    return o


def chunk_bwd(q, k, v, g, bx, w, d_o, L=64, ub_down=None, ub_up=None, state_in=None, mean_in=None,
              d_state_out=None, d_mean_out=None, decay_logits=False, workspace=None, stream=None,
              d_state_in=None, d_mean_in=None, out=None, qk_l2norm=False, detach_mean=False):
    """Gradients of chunk_fwd's inputs from the gradients of its outputs.
    q .. mean_in and L as given to chunk_fwd; d_o [B,T,H,dv] in the input
    dtype; d_state_out [B,H,dv,dk] and d_mean_out [B,H,dv] fp32 or None.
    d_state_in / d_mean_in: optional fp32 output buffers (may be d_state_out /
    d_mean_out themselves); allocated when None. Returns a dict with dq, dk,
    dv, dg, dbx, dw (input dtype), dub_down, dub_up (fp32, None without a
    projection), d_state_in and d_mean_in (fp32). `out`: an earlier call's
    returned dict, whose tensors are written again instead of new ones.
    detach_mean: the content gate's chunk means are constants (no gradient
    through them to earlier outputs or mean_in; U_down, U_up still get theirs)."""
    if q.device.type != "cuda":
        raise ValueError("chunk_bwd runs on the GPU only; move the inputs to a cuda device")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    if (ub_down is None) != (ub_up is None):
        raise ValueError("ub_down and ub_up come together")
    rank = 0 if ub_down is None else int(ub_down.shape[1])
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("v", v, (B, T, H, dv)),
                         ("g", g, (B, T, H, dk)), ("bx", bx, (B, T, H, dk)), ("w", w, (B, T, H)),
                         ("d_o", d_o, (B, T, H, dv))):
        _need(t, name, shp, dt, dev)
    if rank:
        _need(ub_down, "ub_down", (H, rank, dv), dt, dev)
        _need(ub_up, "ub_up", (H, dk, rank), dt, dev)
    for name, t, shp in (("state_in", state_in, (B, H, dv, dk)), ("mean_in", mean_in, (B, H, dv)),
                         ("d_state_out", d_state_out, (B, H, dv, dk)), ("d_mean_out", d_mean_out, (B, H, dv))):
        _need(t, name, shp, torch.float32, dev)
    cfg = make_config(B, H, T, dk, dv, L, rank, dt, decay_logits, qk_l2norm, detach_mean)
    sh = _lib.ref_shapes(cfg)
    empty = lambda shp, dtype=dt: torch.empty(shp, dtype=dtype, device=dev)
    if out is not None:
        out = dict(out)
        for n, shp, dtype in (("dq", (B, T, H, dk), dt), ("dk", (B, T, H, dk), dt), ("dv", (B, T, H, dv), dt),
                              ("dg", (B, T, H, dk), dt), ("dbx", (B, T, H, dk), dt), ("dw", (B, T, H), dt)):
            _need(out[n], n, shp, dtype, dev)
        if rank:
            _need(out["dub_down"], "dub_down", (H, rank, dv), torch.float32, dev)
            _need(out["dub_up"], "dub_up", (H, dk, rank), torch.float32, dev)
        if d_state_in is not None:
            out["d_state_in"] = d_state_in
        if d_mean_in is not None:
            out["d_mean_in"] = d_mean_in
    else:
        out = {"dq": empty((B, T, H, dk)), "dk": empty((B, T, H, dk)), "dv": empty((B, T, H, dv)),
               "dg": empty((B, T, H, dk)), "dbx": empty((B, T, H, dk)), "dw": empty((B, T, H)),
               "dub_down": empty((H, rank, dv), torch.float32) if rank else None,
               "dub_up": empty((H, dk, rank), torch.float32) if rank else None,
               "d_state_in": d_state_in if d_state_in is not None else empty((B, H, dv, dk), torch.float32),
               "d_mean_in": d_mean_in if d_mean_in is not None else empty((B, H, dv), torch.float32)}
    _need(out["d_state_in"], "d_state_in", (B, H, dv, dk), torch.float32, dev)
    _need(out["d_mean_in"], "d_mean_in", (B, H, dv), torch.float32, dev)
    ws_bytes = int(sh.bwd_workspace_bytes)
    if ws_bytes and (workspace is None or workspace.numel() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    code = _lib.lib().carve_chunk_bwd(
        ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(bx), _ptr(w), _ptr(ub_down), _ptr(ub_up),
        _ptr(state_in), _ptr(mean_in), _ptr(d_o), _ptr(d_state_out), _ptr(d_mean_out),
        *(_ptr(out[n]) for n in ("dq", "dk", "dv", "dg", "dbx", "dw", "dub_down", "dub_up", "d_state_in",
                                 "d_mean_in")),
        _ptr(workspace) if ws_bytes else None, ctypes.c_size_t(ws_bytes if ws_bytes else 0), ctypes.c_void_p(stream))
    _lib.check(code)
    return out


def recurrent_step(q, k, v, g, bx, w, state, mean_prev, chunk_acc, pos, L, ub_down=None, ub_up=None,
                   out=None, stream=None, decay_logits=False, qk_l2norm=False):
    """One decode step for every (batch, head). Shapes: q, k, g, bx [B,H,dk];
    v [B,H,dv]; w [B,H]; state [B,H,dv,dk] fp32, mean_prev and chunk_acc
    [B,H,dv] fp32 (all three updated in place); pos is the token's position
    within its chunk of L tokens; decay_logits as for chunk_fwd. Returns
    o [B,H,dv]."""
    if q.device.type != "cuda":
        raise ValueError("recurrent_step runs on the GPU only; move the inputs to a cuda device")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    if (ub_down is None) != (ub_up is None):
        raise ValueError("ub_down and ub_up come together")
    rank = 0 if ub_down is None else int(ub_down.shape[1])
    for name, t, shp in (("q", q, (B, H, dk)), ("k", k, (B, H, dk)), ("v", v, (B, H, dv)),
                         ("g", g, (B, H, dk)), ("bx", bx, (B, H, dk)), ("w", w, (B, H))):
        _need(t, name, shp, dt, dev)
    if rank:
        _need(ub_down, "ub_down", (H, rank, dv), dt, dev)
        _need(ub_up, "ub_up", (H, dk, rank), dt, dev)
    for name, t, shp in (("state", state, (B, H, dv, dk)), ("mean_prev", mean_prev, (B, H, dv)),
                         ("chunk_acc", chunk_acc, (B, H, dv))):
        if t is None:
            raise ValueError(f"{name} is required")
        _need(t, name, shp, torch.float32, dev)
    o = out if out is not None else torch.empty((B, H, dv), dtype=dt, device=dev)
    _need(o, "out", (B, H, dv), dt, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    code = _lib.lib().carve_recurrent_step(
        ctypes.byref(make_config(B, H, 1, dk, dv, L, rank, dt, decay_logits, qk_l2norm)), ctypes.c_int32(pos),
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(bx), _ptr(w), _ptr(ub_down), _ptr(ub_up),
        _ptr(state), _ptr(mean_prev), _ptr(chunk_acc), _ptr(o), ctypes.c_void_p(stream))
    _lib.check(code)
    return o
