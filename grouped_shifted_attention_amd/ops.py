"""Thin torch-facing binding of the C ABI (include/s2attn.h).

Argument marshalling only: tensors are checked for device, dtype, layout and
shape, outputs and workspaces are allocated with torch, and the raw device
pointers plus torch's current HIP stream go to libs2attn.so.  Every step of
the computation runs in the library's HIP kernels.

Function names match the C entry points.  Tensors: q/out/dout/dq
[B, N, H, D] bf16, k/v/dk/dv [B, N, Hkv, D] bf16, lse [B, H, N] float32, all
contiguous on one GPU.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import check, lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dims(q, k, v):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, N, H, D] and k, v [B, N, Hkv, D]")
    B, N, H, D = q.shape
    Hkv = k.shape[2]
    _need(q, "q", torch.bfloat16, (B, N, H, D), None)
    _need(k, "k", torch.bfloat16, (B, N, Hkv, D), q.device)
    _need(v, "v", torch.bfloat16, (B, N, Hkv, D), q.device)
    return B, N, H, Hkv, D


def _workspace(nbytes, device):
    # torch's caching allocator hands out 512-byte aligned blocks.
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def s2attn_fwd(q, k, v, G, shift, out=None, lse=None, with_lse=True):
    """Forward pass; returns (out, lse) (lse is None when with_lse is False)."""
    B, N, H, Hkv, D = _dims(q, k, v)
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", torch.bfloat16, (B, N, H, D), q.device)
    if with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
        _need(lse, "lse", torch.float32, (B, H, N), q.device)
    else:
        lse = None
    check(lib().s2attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                           B, N, H, Hkv, D, int(G), int(shift), _stream(q)))
    return out, lse


def s2attn_fwd_rope(q, k, v, G, shift, rope_base, pos_scale, out=None, lse=None, with_lse=True,
                    workspace=None):
    """Forward pass with the fused RoPE + linear position interpolation."""
    B, N, H, Hkv, D = _dims(q, k, v)
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", torch.bfloat16, (B, N, H, D), q.device)
    if with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
        _need(lse, "lse", torch.float32, (B, H, N), q.device)
    else:
        lse = None
    L = lib()
    nbytes = L.s2attn_fwd_rope_workspace_size(B, N, H, Hkv, D)
    ws = _workspace(nbytes, q.device) if workspace is None else workspace
    check(L.s2attn_fwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                            B, N, H, Hkv, D, int(G), int(shift), float(rope_base), float(pos_scale),
                            _ptr(ws), ws.numel() * ws.element_size(), _stream(q)))
    return out, lse


def _bwd_common(q, k, v, out, lse, dout, dq, dk, dv):
    B, N, H, Hkv, D = _dims(q, k, v)
    _need(out, "out", torch.bfloat16, (B, N, H, D), q.device)
    _need(dout, "dout", torch.bfloat16, (B, N, H, D), q.device)
    _need(lse, "lse", torch.float32, (B, H, N), q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", torch.bfloat16, (B, N, H, D), q.device)
    _need(dk, "dk", torch.bfloat16, (B, N, Hkv, D), q.device)
    _need(dv, "dv", torch.bfloat16, (B, N, Hkv, D), q.device)
    return (B, N, H, Hkv, D), dq, dk, dv


def s2attn_bwd(q, k, v, out, lse, dout, G, shift, dq=None, dk=None, dv=None, workspace=None):
    """Backward pass; returns (dq, dk, dv)."""
    (B, N, H, Hkv, D), dq, dk, dv = _bwd_common(q, k, v, out, lse, dout, dq, dk, dv)
    L = lib()
    ws = _workspace(L.s2attn_bwd_workspace_size(B, N, H, Hkv, D), q.device) if workspace is None else workspace
    check(L.s2attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                       _ptr(dq), _ptr(dk), _ptr(dv), B, N, H, Hkv, D, int(G), int(shift),
                       _ptr(ws), ws.numel() * ws.element_size(), _stream(q)))
    return dq, dk, dv


def s2attn_bwd_noalloc(q, k, v, out, lse, dout, G, shift, dq=None, dk=None, dv=None):
    """s2attn_bwd without a workspace: the library's own device scratch holds
    the row statistics (B*H*N <= 4,194,304; calls on one GPU must not
    overlap).  Returns (dq, dk, dv)."""
    (B, N, H, Hkv, D), dq, dk, dv = _bwd_common(q, k, v, out, lse, dout, dq, dk, dv)
    # The library takes the scratch of the current device: make it q's.
    with torch.cuda.device(q.device):
        check(lib().s2attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                                       _ptr(dq), _ptr(dk), _ptr(dv), B, N, H, Hkv, D, int(G), int(shift),
                                       _stream(q)))
    return dq, dk, dv


def s2attn_bwd_preprocess(out, dout, lse, workspace):
    """Stage 1 of the backward: the row statistics (-Delta, -lse*log2 e) into
    the workspace."""
    B, N, H, D = out.shape
    _need(out, "out", torch.bfloat16, (B, N, H, D), None)
    _need(dout, "dout", torch.bfloat16, (B, N, H, D), out.device)
    _need(lse, "lse", torch.float32, (B, H, N), out.device)
    check(lib().s2attn_bwd_preprocess(_ptr(out), _ptr(dout), _ptr(lse), B, N, H, D, _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(out)))


def _stage_dims(q, k, v, dout):
    B, N, H, D = dout.shape
    _need(dout, "dout", torch.bfloat16, (B, N, H, D), None)
    _need(q, "q", torch.bfloat16, (B, N, H, D), dout.device)
    Hkv = k.shape[2] if k.dim() == 4 else -1
    _need(k, "k", torch.bfloat16, (B, N, Hkv, D), dout.device)
    _need(v, "v", torch.bfloat16, (B, N, Hkv, D), dout.device)
    return B, N, H, Hkv, D


def s2attn_bwd_dkdv(q, k, v, dout, G, shift, workspace, dk=None, dv=None):
    """Stage 2 of the backward: dk, dv (needs the preprocess stage's workspace)."""
    B, N, H, Hkv, D = _stage_dims(q, k, v, dout)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dk, "dk", torch.bfloat16, (B, N, Hkv, D), k.device)
    _need(dv, "dv", torch.bfloat16, (B, N, Hkv, D), k.device)
    check(lib().s2attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dk), _ptr(dv),
                                B, N, H, Hkv, D, int(G), int(shift), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(k)))
    return dk, dv


def s2attn_bwd_dq(q, k, v, dout, G, shift, workspace, dq=None):
    """Stage 3 of the backward: dq (needs the preprocess stage's workspace)."""
    B, N, H, Hkv, D = _stage_dims(q, k, v, dout)
    dq = torch.empty_like(dout) if dq is None else dq
    _need(dq, "dq", torch.bfloat16, (B, N, H, D), k.device)
    check(lib().s2attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq),
                              B, N, H, Hkv, D, int(G), int(shift), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(k)))
    return dq


def s2attn_bwd_rope(q, k, v, out, lse, dout, G, shift, rope_base, pos_scale, dq=None, dk=None, dv=None,
                    workspace=None):
    """Backward of s2attn_fwd_rope; dq and dk refer to the unrotated q and k."""
    (B, N, H, Hkv, D), dq, dk, dv = _bwd_common(q, k, v, out, lse, dout, dq, dk, dv)
    L = lib()
    nbytes = L.s2attn_bwd_rope_workspace_size(B, N, H, Hkv, D)
    ws = _workspace(nbytes, q.device) if workspace is None else workspace
    check(L.s2attn_bwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                            _ptr(dq), _ptr(dk), _ptr(dv), B, N, H, Hkv, D, int(G), int(shift),
                            float(rope_base), float(pos_scale),
                            _ptr(ws), ws.numel() * ws.element_size(), _stream(q)))
    return dq, dk, dv


HEAD_PATTERNS = {"second_half": 0, "alternate": 1}


def _pattern(head_pattern):
    if head_pattern not in HEAD_PATTERNS:
        raise ValueError(f"head_pattern must be one of {sorted(HEAD_PATTERNS)}, got {head_pattern!r}")
    return HEAD_PATTERNS[head_pattern]


def s2attn_fwd_ex(q, k, v, G, shift, head_pattern="second_half", rope=None, out=None, lse=None, with_lse=True,
                  workspace=None):
    """Forward with every option: which heads are shifted ("second_half" or
    "alternate") and, when ``rope`` is a (base, pos_scale) pair, RoPE with
    position interpolation."""
    B, N, H, Hkv, D = _dims(q, k, v)
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", torch.bfloat16, (B, N, H, D), q.device)
    if with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
        _need(lse, "lse", torch.float32, (B, H, N), q.device)
    else:
        lse = None
    L = lib()
    base, scale = (0.0, 1.0) if rope is None else (float(rope[0]), float(rope[1]))
    ws = workspace
    if ws is None and rope is not None:
        ws = _workspace(L.s2attn_fwd_rope_workspace_size(B, N, H, Hkv, D), q.device)
    check(L.s2attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, N, H, Hkv, D, int(G), int(shift),
                          _pattern(head_pattern), base, scale, _ptr(ws),
                          0 if ws is None else ws.numel() * ws.element_size(), _stream(q)))
    return out, lse


def s2attn_bwd_ex(q, k, v, out, lse, dout, G, shift, head_pattern="second_half", rope=None, dq=None, dk=None,
                  dv=None, workspace=None):
    """Backward of s2attn_fwd_ex (same head_pattern and rope)."""
    (B, N, H, Hkv, D), dq, dk, dv = _bwd_common(q, k, v, out, lse, dout, dq, dk, dv)
    L = lib()
    base, scale = (0.0, 1.0) if rope is None else (float(rope[0]), float(rope[1]))
    size = L.s2attn_bwd_workspace_size if rope is None else L.s2attn_bwd_rope_workspace_size
    ws = _workspace(size(B, N, H, Hkv, D), q.device) if workspace is None else workspace
    check(L.s2attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                          _ptr(dq), _ptr(dk), _ptr(dv), B, N, H, Hkv, D, int(G), int(shift),
                          _pattern(head_pattern), base, scale,
                          _ptr(ws), ws.numel() * ws.element_size(), _stream(q)))
    return dq, dk, dv


def bwd_workspace(q, k, rope=False):
    """A workspace tensor large enough for s2attn_bwd and its stages (or for
    s2attn_bwd_rope when rope is true)."""
    B, N, H, D = q.shape
    L = lib()
    size = L.s2attn_bwd_rope_workspace_size if rope else L.s2attn_bwd_workspace_size
    return _workspace(size(B, N, H, k.shape[2], D), q.device)


def fwd_rope_workspace(q, k):
    """A workspace tensor large enough for s2attn_fwd_rope."""
    B, N, H, D = q.shape
    return _workspace(lib().s2attn_fwd_rope_workspace_size(B, N, H, k.shape[2], D), q.device)


def s2attn_workspace_sizes(B, N, H, Hkv, D):
    """Workspace bytes of the four entry points that take one."""
    L = lib()
    return {
        "bwd": L.s2attn_bwd_workspace_size(B, N, H, Hkv, D),
        "fwd_rope": L.s2attn_fwd_rope_workspace_size(B, N, H, Hkv, D),
        "bwd_rope": L.s2attn_bwd_rope_workspace_size(B, N, H, Hkv, D),
    }


def lora_qkv_workspace(M, r, device):
    """A workspace tensor large enough for s2attn_lora_qkv_fwd (None when r = 0)."""
    n = lib().s2attn_lora_qkv_workspace_size(int(M), int(r))
    return None if n == 0 else _workspace(n, device)


def s2attn_lora_qkv_fwd(x, wt, at=None, bt=None, scale=1.0, out=None, workspace=None):
    """LoRA-adapted q/k/v projections: y_p = x W_p + scale (x A_p) B_p.

    x [M, d_in]; wt = (wq_t, wk_t, wv_t) with wq_t [width_q, d_in] and wk_t,
    wv_t [width_kv, d_in]; at = three [r, d_in] (A transposed) and bt =
    (bq_t [width_q, r], bk_t, bv_t [width_kv, r]) (B transposed), or both None
    for plain projections.  All bf16, contiguous, on one GPU.  Returns
    (q, k, v, workspace): q [M, width_q], k, v [M, width_kv] and the workspace,
    which then holds scale * x A_p for the three targets ([M, 3r] bf16).
    """
    if x.dim() != 2 or len(wt) != 3:
        raise ValueError("x must be [M, d_in] and wt three weights")
    M, d_in = x.shape
    dev = x.device
    _need(x, "x", torch.bfloat16, (M, d_in), None)
    wq = wt[0].shape[0]
    wkv = wt[1].shape[0]
    for name, t, w in (("wq_t", wt[0], wq), ("wk_t", wt[1], wkv), ("wv_t", wt[2], wkv)):
        _need(t, name, torch.bfloat16, (w, d_in), dev)
    if (at is None) != (bt is None):
        raise ValueError("at and bt must both be given or both be None")
    r = 0 if at is None else at[0].shape[0]
    if at is not None:
        for p, (a, b) in enumerate(zip(at, bt)):
            _need(a, f"at[{p}]", torch.bfloat16, (r, d_in), dev)
            _need(b, f"bt[{p}]", torch.bfloat16, (wq if p == 0 else wkv, r), dev)
    if out is None:
        out = (torch.empty(M, wq, dtype=torch.bfloat16, device=dev),
               torch.empty(M, wkv, dtype=torch.bfloat16, device=dev),
               torch.empty(M, wkv, dtype=torch.bfloat16, device=dev))
    for name, t, w in (("q", out[0], wq), ("k", out[1], wkv), ("v", out[2], wkv)):
        _need(t, name, torch.bfloat16, (M, w), dev)
    ws = lora_qkv_workspace(M, r, dev) if workspace is None else workspace
    none3 = (None, None, None)
    a3 = none3 if at is None else at
    b3 = none3 if bt is None else bt
    check(lib().s2attn_lora_qkv_fwd(
        _ptr(x), M, d_in, _ptr(wt[0]), _ptr(wt[1]), _ptr(wt[2]), wq, wkv,
        _ptr(a3[0]), _ptr(a3[1]), _ptr(a3[2]), _ptr(b3[0]), _ptr(b3[1]), _ptr(b3[2]), r, float(scale),
        _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(x)))
    return out[0], out[1], out[2], ws


def lora_qkv_bwd_workspace(M, d_in, width_q, width_kv, r, device):
    """A workspace tensor large enough for s2attn_lora_qkv_bwd (None when r = 0)."""
    n = lib().s2attn_lora_qkv_bwd_workspace_size(int(M), int(d_in), int(width_q), int(width_kv), int(r))
    return None if n == 0 else _workspace(n, device)


def s2attn_lora_qkv_bwd(x, wt, at, bt, scale, t, dys, out=None, workspace=None):
    """Backward of s2attn_lora_qkv_fwd for upstream gradients dys = (dq, dk, dv).

    x, wt, at, bt, scale as for the forward; t is the forward's low-rank
    activations ([M, 3r] bf16, e.g. a view of the forward's workspace), or
    None with r = 0.  Returns (dx [M, d_in], [dA_q^T, dA_k^T, dA_v^T] each
    [r, d_in], [dB_q^T [width_q, r], dB_k^T, dB_v^T [width_kv, r]]); the
    adapter lists are None when r = 0.
    """
    M, d_in = x.shape
    dev = x.device
    _need(x, "x", torch.bfloat16, (M, d_in), None)
    wq, wkv = wt[0].shape[0], wt[1].shape[0]
    widths = (wq, wkv, wkv)
    for name, w, n in zip(("wq_t", "wk_t", "wv_t"), wt, widths):
        _need(w, name, torch.bfloat16, (n, d_in), dev)
    for name, d, n in zip(("dq", "dk", "dv"), dys, widths):
        _need(d, name, torch.bfloat16, (M, n), dev)
    if (at is None) != (bt is None):
        raise ValueError("at and bt must both be given or both be None")
    r = 0 if at is None else at[0].shape[0]
    if r > 0:
        for p in range(3):
            _need(at[p], f"at[{p}]", torch.bfloat16, (r, d_in), dev)
            _need(bt[p], f"bt[{p}]", torch.bfloat16, (widths[p], r), dev)
        _need(t, "t", torch.bfloat16, (M, 3 * r), dev)
    if out is None:
        dx = torch.empty(M, d_in, dtype=torch.bfloat16, device=dev)
        dat = [torch.empty(r, d_in, dtype=torch.bfloat16, device=dev) for _ in range(3)] if r > 0 else None
        dbt = [torch.empty(n, r, dtype=torch.bfloat16, device=dev) for n in widths] if r > 0 else None
    else:
        dx, dat, dbt = out
    _need(dx, "dx", torch.bfloat16, (M, d_in), dev)
    ws = lora_qkv_bwd_workspace(M, d_in, wq, wkv, r, dev) if workspace is None else workspace
    n3 = (None, None, None)
    a3, b3 = (n3, n3) if r == 0 else (at, bt)
    da3, db3 = (n3, n3) if r == 0 else (dat, dbt)
    check(lib().s2attn_lora_qkv_bwd(
        _ptr(x), M, d_in, _ptr(wt[0]), _ptr(wt[1]), _ptr(wt[2]), wq, wkv,
        _ptr(a3[0]), _ptr(a3[1]), _ptr(a3[2]), _ptr(b3[0]), _ptr(b3[1]), _ptr(b3[2]), r, float(scale),
        _ptr(t) if r > 0 else None, _ptr(dys[0]), _ptr(dys[1]), _ptr(dys[2]), _ptr(dx),
        _ptr(da3[0]), _ptr(da3[1]), _ptr(da3[2]), _ptr(db3[0]), _ptr(db3[1]), _ptr(db3[2]),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(x)))
    return dx, dat, dbt


class S2AttnFunction(torch.autograd.Function):
    """Autograd wrapper: forward saves q, k, v, out and lse; backward calls the
    library's backward entry point."""

    @staticmethod
    def forward(ctx, q, k, v, G, shift, rope):
        if rope is None:
            out, lse = s2attn_fwd(q, k, v, G, shift)
        else:
            out, lse = s2attn_fwd_rope(q, k, v, G, shift, rope[0], rope[1])
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.cfg = (G, shift, rope)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse = ctx.saved_tensors
        G, shift, rope = ctx.cfg
        dout = dout.contiguous()
        if rope is None:
            dq, dk, dv = s2attn_bwd(q, k, v, out, lse, dout, G, shift)
        else:
            dq, dk, dv = s2attn_bwd_rope(q, k, v, out, lse, dout, G, shift, rope[0], rope[1])
        return dq, dk, dv, None, None, None


class LoraQKVFunction(torch.autograd.Function):
    """Autograd wrapper of the LoRA q/k/v projections: forward keeps the
    low-rank activations the library leaves in its workspace; backward calls
    s2attn_lora_qkv_bwd (the frozen weights get no gradient)."""

    @staticmethod
    def forward(ctx, x, wq_t, wk_t, wv_t, aq_t, ak_t, av_t, bq_t, bk_t, bv_t, scale):
        wt, at, bt = (wq_t, wk_t, wv_t), (aq_t, ak_t, av_t), (bq_t, bk_t, bv_t)
        q, k, v, ws = s2attn_lora_qkv_fwd(x, wt, at, bt, scale)
        M, r = x.shape[0], aq_t.shape[0]
        t = ws[: M * 3 * r * 2].view(torch.bfloat16).view(M, 3 * r)
        ctx.save_for_backward(x, wq_t, wk_t, wv_t, aq_t, ak_t, av_t, bq_t, bk_t, bv_t, t)
        ctx.scale = scale
        return q, k, v

    @staticmethod
    def backward(ctx, dq, dk, dv):
        x, wq_t, wk_t, wv_t, aq_t, ak_t, av_t, bq_t, bk_t, bv_t, t = ctx.saved_tensors
        dx, dat, dbt = s2attn_lora_qkv_bwd(x, (wq_t, wk_t, wv_t), (aq_t, ak_t, av_t), (bq_t, bk_t, bv_t),
                                           ctx.scale, t, (dq.contiguous(), dk.contiguous(), dv.contiguous()))
        return (dx, None, None, None, dat[0], dat[1], dat[2], dbt[0], dbt[1], dbt[2], None)


def lora_qkv(x, wt, at, bt, scale=1.0):
    """LoRA-adapted q/k/v projections with autograd: returns (q, k, v) as
    [M, width] tensors; gradients flow to x and to the adapters (A^T, B^T),
    not to the frozen W^T."""
    return LoraQKVFunction.apply(x, *wt, *at, *bt, float(scale))


def s2attn(q, k, v, group_size, shift=None, rope=None):
    """S2-Attn with autograd.  shift defaults to group_size // 2 (the pages'
    half-group shift); rope is None or (rope_base, pos_scale)."""
    shift = group_size // 2 if shift is None else shift
    return S2AttnFunction.apply(q, k, v, int(group_size), int(shift), rope)
