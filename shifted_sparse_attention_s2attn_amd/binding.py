"""PyTorch-facing wrappers over the C ABI of libs2attn (argument marshalling only).

Tensors are token-major: q, o, dO [B, N, H, d]; k, v [B, N, Hkv, d]; lse [B, H, N]
float32.  Every step of the computation runs in the HIP kernels of libs2attn;
torch only provides device memory and the current stream.
"""

import ctypes

import torch

from . import _lib

__all__ = ["S2AttnError", "s2attn_fwd", "s2attn_bwd", "s2attn_bwd_workspace_bytes", "s2attn_bwd_noalloc",
           "s2attn_bwd_prep", "s2attn_bwd_dkdv", "s2attn_bwd_dq", "s2attn_bwd_prep_dq",
           "s2attn_status_str", "S2Attn", "s2attn", "s2attn_rope", "RoPE", "rope", "s2attn_fwd_rope",
           "s2attn_bwd_rope", "S2AttnRoPE", "s2attn_with_rope"]


class S2AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {s2attn_status_str(status)} (status {status})")


def s2attn_status_str(status):
    return _lib.load().s2attn_status_str(int(status)).decode()


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return _lib.S2ATTN_BF16
    if t.dtype == torch.float32:
        return _lib.S2ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _fptr(t):
    return ctypes.cast(ctypes.c_void_p(t.data_ptr()), ctypes.POINTER(ctypes.c_float))


def _check_tensors(q, k, v, extra=()):
    """q [B,N,H,d], k and v [B,N,Hkv,d] of one dtype, plus the named tensors of
    ``extra`` as (name, tensor, shape, dtype); shape None = q's, dtype None =
    q's.  Every tensor must be contiguous and on q's GPU: the library takes raw
    pointers, so a mismatch here would become an out-of-bounds access there."""
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError(f"bad shapes q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    for name, t, shape, dtype in (("q", q, None, None), ("k", k, k.shape, None), ("v", v, v.shape, None)) + tuple(extra):
        if not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be a GPU tensor on {q.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        want = tuple(q.shape if shape is None else shape)
        if tuple(t.shape) != want:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want}")
        if t.dtype != (q.dtype if dtype is None else dtype):
            raise TypeError(f"{name} has dtype {t.dtype}, expected {q.dtype if dtype is None else dtype}")


def _lse_shape(q):
    B, N, H, _ = q.shape
    return (B, H, N)


def _check_workspace(q, ws):
    if not ws.is_cuda or ws.device != q.device or not ws.is_contiguous() or ws.dtype != torch.uint8:
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {q.device}")


def _wrap_code(wrap):
    """Wrap handling of the shifted heads: "roll" (the method), "split" or "swap"
    (Table 8, Variants 2 and 3)."""
    if wrap not in _lib.WRAPS:
        raise ValueError(f"wrap must be one of {sorted(_lib.WRAPS)}, got {wrap!r}")
    return _lib.WRAPS[wrap]


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def s2attn_fwd(q, k, v, G, shift_heads=None, out=None, lse=None, stream=None, wrap="roll"):
    """S2-Attn forward.  Returns (o [B,N,H,d], lse [B,H,N] float32)."""
    _check_tensors(q, k, v)
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    if shift_heads is None:
        shift_heads = H // 2
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensors(q, k, v, (("out", o, None, None), ("lse", lse_t, (B, H, N), torch.float32)))
    with torch.cuda.device(q.device):
        st = _lib.load().s2attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _fptr(lse_t),
                                       B, H, Hkv, N, d, G, shift_heads, _wrap_code(wrap), _dtype_code(q),
                                       _stream(stream))
    if st != _lib.S2ATTN_OK:
        raise S2AttnError(st, "s2attn_fwd")
    return o, lse_t


def s2attn_bwd_workspace_bytes(B, H, Hkv, N, d, G, shift_heads, dtype):
    code = _lib.S2ATTN_BF16 if dtype == torch.bfloat16 else _lib.S2ATTN_F32
    return int(_lib.load().s2attn_bwd_workspace_bytes(B, H, Hkv, N, d, G, shift_heads, code))


def s2attn_bwd(q, k, v, o, lse, do, G, shift_heads=None, workspace=None, stream=None, grads=None, wrap="roll"):
    """S2-Attn backward of sum(o * do).  Returns (dq, dk, dv)."""
    _check_tensors(q, k, v, (("o", o, None, None), ("lse", lse, _lse_shape(q), torch.float32),
                             ("do", do, None, None)))
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    if shift_heads is None:
        shift_heads = H // 2
    need = s2attn_bwd_workspace_bytes(B, H, Hkv, N, d, G, shift_heads, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = grads
        _check_tensors(q, k, v, (("dq", dq, None, None), ("dk", dk, k.shape, None), ("dv", dv, k.shape, None)))
    _check_workspace(q, workspace)
    with torch.cuda.device(q.device):
        st = _lib.load().s2attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _fptr(lse), _ptr(do),
                                       _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                                       B, H, Hkv, N, d, G, shift_heads, _wrap_code(wrap), _dtype_code(q),
                                       _stream(stream))
    if st != _lib.S2ATTN_OK:
        raise S2AttnError(st, "s2attn_bwd")
    return dq, dk, dv


def s2attn_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, G, shift_heads=None, stream=None, wrap="roll"):
    """The backward of s2attn_bwd into caller-given dq, dk, dv, with no
    workspace: the library's own per-device scratch array holds the row sums
    (B * H * N <= S2ATTN_NOALLOC_MAX_ROWS), so the call allocates nothing.
    Calls that can overlap on one GPU race on that scratch."""
    _check_tensors(q, k, v, (("o", o, None, None), ("lse", lse, _lse_shape(q), torch.float32),
                             ("do", do, None, None), ("dq", dq, None, None), ("dk", dk, k.shape, None),
                             ("dv", dv, k.shape, None)))
    B, H, Hkv, N, d, S = _dims(q, k, shift_heads)
    with torch.cuda.device(q.device):
        _check(_lib.load().s2attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _fptr(lse), _ptr(do),
                                              _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, N, d, G, S,
                                              _wrap_code(wrap), _dtype_code(q), _stream(stream)),
               "s2attn_bwd_noalloc")


def _dims(q, k, shift_heads):
    B, N, H, d = q.shape
    return B, H, k.shape[2], N, d, (H // 2 if shift_heads is None else shift_heads)


def _check(st, where):
    if st != _lib.S2ATTN_OK:
        raise S2AttnError(st, where)


def s2attn_bwd_prep(q, k, o, lse, do, workspace, G, shift_heads=None, stream=None):
    """Stage 1 of the backward: Dvec = rowsum(dO * o) and lse * log2(e) into the workspace."""
    _check_tensors(q, k, k, (("o", o, None, None), ("lse", lse, _lse_shape(q), torch.float32),
                             ("do", do, None, None)))
    _check_workspace(q, workspace)
    B, H, Hkv, N, d, S = _dims(q, k, shift_heads)
    with torch.cuda.device(q.device):
        _check(_lib.load().s2attn_bwd_prep(_ptr(o), _fptr(lse), _ptr(do), _ptr(workspace), workspace.numel(),
                                           B, H, Hkv, N, d, G, S, _dtype_code(q), _stream(stream)),
               "s2attn_bwd_prep")


def s2attn_bwd_dkdv(q, k, v, do, dk, dv, workspace, G, shift_heads=None, stream=None, wrap="roll"):
    """Stage 2 of the backward: dk, dv (needs prep's workspace)."""
    _check_tensors(q, k, v, (("do", do, None, None), ("dk", dk, k.shape, None), ("dv", dv, k.shape, None)))
    _check_workspace(q, workspace)
    B, H, Hkv, N, d, S = _dims(q, k, shift_heads)
    with torch.cuda.device(q.device):
        _check(_lib.load().s2attn_bwd_dkdv_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dk), _ptr(dv),
                                              _ptr(workspace), workspace.numel(),
                                              B, H, Hkv, N, d, G, S, _wrap_code(wrap), _dtype_code(q),
                                              _stream(stream)),
               "s2attn_bwd_dkdv")


def s2attn_bwd_dq(q, k, v, do, dq, workspace, G, shift_heads=None, stream=None, wrap="roll"):
    """Stage 3 of the backward: dq (needs prep's workspace)."""
    _check_tensors(q, k, v, (("do", do, None, None), ("dq", dq, None, None)))
    _check_workspace(q, workspace)
    B, H, Hkv, N, d, S = _dims(q, k, shift_heads)
    with torch.cuda.device(q.device):
        _check(_lib.load().s2attn_bwd_dq_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq),
                                            _ptr(workspace), workspace.numel(),
                                            B, H, Hkv, N, d, G, S, _wrap_code(wrap), _dtype_code(q),
                                            _stream(stream)),
               "s2attn_bwd_dq")


def s2attn_bwd_prep_dq(q, k, v, o, lse, do, dq, workspace, G, shift_heads=None, stream=None, wrap="roll"):
    """Stages 1 and 3 together: dq, and Dvec and lse * log2(e) into the workspace (dk, dv follow)."""
    _check_tensors(q, k, v, (("o", o, None, None), ("lse", lse, _lse_shape(q), torch.float32),
                             ("do", do, None, None), ("dq", dq, None, None)))
    _check_workspace(q, workspace)
    B, H, Hkv, N, d, S = _dims(q, k, shift_heads)
    with torch.cuda.device(q.device):
        _check(_lib.load().s2attn_bwd_prep_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _fptr(lse), _ptr(do), _ptr(dq),
                                              _ptr(workspace), workspace.numel(),
                                              B, H, Hkv, N, d, G, S, _wrap_code(wrap), _dtype_code(q),
                                              _stream(stream)),
               "s2attn_bwd_prep_dq")


class S2Attn(torch.autograd.Function):
    """autograd wrapper: forward and backward both run in libs2attn."""

    @staticmethod
    def forward(ctx, q, k, v, G, shift_heads, wrap="roll"):
        o, lse = s2attn_fwd(q, k, v, G, shift_heads, wrap=wrap)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.G, ctx.shift_heads, ctx.wrap = G, shift_heads, wrap
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = s2attn_bwd(q, k, v, o, lse, do.contiguous(), ctx.G, ctx.shift_heads, wrap=ctx.wrap)
        return dq, dk, dv, None, None, None


def s2attn(q, k, v, G, shift_heads=None, wrap="roll"):
    """Differentiable S2-Attn on [B, N, H, d] tensors (shift_heads defaults to H // 2).

    ``wrap="split"`` selects Variant 2 of Table 8: the tokens the roll carries
    from the front of the sequence form their own group; ``wrap="swap"``
    Variant 3: they stay in the last group but come before its end tokens.
    """
    return S2Attn.apply(q, k, v, G, q.shape[2] // 2 if shift_heads is None else shift_heads, wrap)


def s2attn_rope(x, pos_scale=1.0, base=10000.0, inverse=False, out=None, stream=None):
    """Rotary position embedding with Position Interpolation on x [B, N, heads, d]
    (q or k): pair (i, i + d/2) of token n turned by n * pos_scale * base^(-2i/d)
    (by minus that with ``inverse``).  ``out`` may be ``x`` (in place)."""
    if x.dim() != 4:
        raise ValueError(f"x must be [B, N, heads, d], got {tuple(x.shape)}")
    y = torch.empty_like(x) if out is None else out
    for name, t in (("x", x), ("out", y)):
        if not t.is_cuda or t.device != x.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor on {x.device}")
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError(f"out {tuple(y.shape)} {y.dtype} does not match x {tuple(x.shape)} {x.dtype}")
    B, N, Hx, d = x.shape
    with torch.cuda.device(x.device):
        st = _lib.load().s2attn_rope(_ptr(x), _ptr(y), B, N, Hx, d, float(pos_scale), float(base), int(bool(inverse)),
                                     _dtype_code(x), _stream(stream))
    if st != _lib.S2ATTN_OK:
        raise S2AttnError(st, "s2attn_rope")
    return y


class RoPE(torch.autograd.Function):
    """autograd wrapper: the backward is the inverse rotation (its transpose)."""

    @staticmethod
    def forward(ctx, x, pos_scale, base):
        ctx.pos_scale, ctx.base = pos_scale, base
        return s2attn_rope(x.contiguous(), pos_scale, base)

    @staticmethod
    def backward(ctx, g):
        return s2attn_rope(g.contiguous(), ctx.pos_scale, ctx.base, inverse=True), None, None


def rope(x, pos_scale=1.0, base=10000.0):
    """Differentiable rotary embedding with Position Interpolation (see s2attn_rope)."""
    return RoPE.apply(x, pos_scale, base)


def s2attn_fwd_rope(q, k_rot, v, G, shift_heads=None, pos_scale=1.0, base=10000.0, wrap="roll", out=None, lse=None,
                    q_rot=None, stream=None):
    """S2-Attn forward with the rotary embedding of q fused in (bf16): q is
    unrotated, k_rot = s2attn_rope(k).  Returns (o, lse, q_rot), q_rot being q
    rotated (bit-equal to s2attn_rope(q)) for s2attn_bwd_rope."""
    _check_tensors(q, k_rot, v)
    B, N, H, d = q.shape
    Hkv = k_rot.shape[2]
    if shift_heads is None:
        shift_heads = H // 2
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    qr = torch.empty_like(q) if q_rot is None else q_rot
    _check_tensors(q, k_rot, v, (("out", o, None, None), ("lse", lse_t, (B, H, N), torch.float32),
                                 ("q_rot", qr, None, None)))
    with torch.cuda.device(q.device):
        _check(_lib.load().s2attn_fwd_rope(_ptr(q), _ptr(k_rot), _ptr(v), _ptr(o), _fptr(lse_t), _ptr(qr),
                                           B, H, Hkv, N, d, G, shift_heads, _wrap_code(wrap), float(pos_scale),
                                           float(base), _dtype_code(q), _stream(stream)),
               "s2attn_fwd_rope")
    return o, lse_t, qr


def s2attn_bwd_rope(q_rot, k_rot, v, o, lse, do, G, shift_heads=None, pos_scale=1.0, base=10000.0, wrap="roll",
                    workspace=None, grads=None, stream=None):
    """Backward of s2attn_fwd_rope: (dq, dk, dv) with dq, dk the gradients with
    respect to the unrotated q and k (turned back inside the kernels)."""
    _check_tensors(q_rot, k_rot, v, (("o", o, None, None), ("lse", lse, _lse_shape(q_rot), torch.float32),
                                     ("do", do, None, None)))
    B, H, Hkv, N, d, S = _dims(q_rot, k_rot, shift_heads)
    need = s2attn_bwd_workspace_bytes(B, H, Hkv, N, d, G, S, q_rot.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_rot.device)
    _check_workspace(q_rot, workspace)
    if grads is None:
        dq, dk, dv = torch.empty_like(q_rot), torch.empty_like(k_rot), torch.empty_like(v)
    else:
        dq, dk, dv = grads
        _check_tensors(q_rot, k_rot, v, (("dq", dq, None, None), ("dk", dk, k_rot.shape, None),
                                         ("dv", dv, k_rot.shape, None)))
    with torch.cuda.device(q_rot.device):
        _check(_lib.load().s2attn_bwd_rope(_ptr(q_rot), _ptr(k_rot), _ptr(v), _ptr(o), _fptr(lse), _ptr(do),
                                           _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                                           B, H, Hkv, N, d, G, S, _wrap_code(wrap), float(pos_scale), float(base),
                                           _dtype_code(q_rot), _stream(stream)),
               "s2attn_bwd_rope")
    return dq, dk, dv


class S2AttnRoPE(torch.autograd.Function):
    """autograd wrapper of rotary embedding + S2-Attn with the q rotation and the
    inverse rotations of dq and dk fused into the attention kernels; k takes the
    stand-alone rotary pass."""

    @staticmethod
    def forward(ctx, q, k, v, G, shift_heads, pos_scale, base, wrap="roll"):
        k_rot = s2attn_rope(k, pos_scale, base)
        o, lse, q_rot = s2attn_fwd_rope(q, k_rot, v, G, shift_heads, pos_scale, base, wrap=wrap)
        ctx.save_for_backward(q_rot, k_rot, v, o, lse)
        ctx.args = (G, shift_heads, pos_scale, base, wrap)
        return o

    @staticmethod
    def backward(ctx, do):
        q_rot, k_rot, v, o, lse = ctx.saved_tensors
        G, shift_heads, pos_scale, base, wrap = ctx.args
        dq, dk, dv = s2attn_bwd_rope(q_rot, k_rot, v, o, lse, do.contiguous(), G, shift_heads, pos_scale, base,
                                     wrap=wrap)
        return dq, dk, dv, None, None, None, None, None


def s2attn_with_rope(q, k, v, G, shift_heads=None, pos_scale=1.0, base=10000.0, wrap="roll"):
    """Differentiable rotary embedding (Position Interpolation) of q and k followed
    by S2-Attn, bf16; q, k unrotated [B, N, heads, d]."""
    return S2AttnRoPE.apply(q, k, v, G, q.shape[2] // 2 if shift_heads is None else shift_heads, pos_scale, base,
                            wrap)
