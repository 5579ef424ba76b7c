"""PyTorch-facing wrappers over the C ABI of libs2attn (argument marshalling only).

Tensors are token-major: q, o, dO [B, N, H, d]; k, v [B, N, Hkv, d]; lse [B, H, N]
float32.  Every step of the computation runs in the HIP kernels of libs2attn;
torch only provides device memory and the current stream.
"""

import ctypes

import torch

from . import _lib

__all__ = ["S2AttnError", "s2attn_fwd", "s2attn_bwd", "s2attn_bwd_workspace_bytes",
           "s2attn_bwd_prep", "s2attn_bwd_dkdv", "s2attn_bwd_dq", "s2attn_bwd_prep_dq",
           "s2attn_status_str", "S2Attn", "s2attn"]


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
    for name, t in (("q", q), ("k", k), ("v", v)) + tuple(extra):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError(f"bad shapes q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")


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
    _check_tensors(q, k, v, (("o", o), ("lse", lse), ("do", do)))
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
    with torch.cuda.device(q.device):
        st = _lib.load().s2attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _fptr(lse), _ptr(do),
                                       _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                                       B, H, Hkv, N, d, G, shift_heads, _wrap_code(wrap), _dtype_code(q),
                                       _stream(stream))
    if st != _lib.S2ATTN_OK:
        raise S2AttnError(st, "s2attn_bwd")
    return dq, dk, dv


def _dims(q, k, shift_heads):
    B, N, H, d = q.shape
    return B, H, k.shape[2], N, d, (H // 2 if shift_heads is None else shift_heads)


def _check(st, where):
    if st != _lib.S2ATTN_OK:
        raise S2AttnError(st, where)


def s2attn_bwd_prep(q, k, o, lse, do, workspace, G, shift_heads=None, stream=None):
    """Stage 1 of the backward: Dvec = rowsum(dO * o) and lse * log2(e) into the workspace."""
    B, H, Hkv, N, d, S = _dims(q, k, shift_heads)
    with torch.cuda.device(q.device):
        _check(_lib.load().s2attn_bwd_prep(_ptr(o), _fptr(lse), _ptr(do), _ptr(workspace), workspace.numel(),
                                           B, H, Hkv, N, d, G, S, _dtype_code(q), _stream(stream)),
               "s2attn_bwd_prep")


def s2attn_bwd_dkdv(q, k, v, do, dk, dv, workspace, G, shift_heads=None, stream=None, wrap="roll"):
    """Stage 2 of the backward: dk, dv (needs prep's workspace)."""
    B, H, Hkv, N, d, S = _dims(q, k, shift_heads)
    with torch.cuda.device(q.device):
        _check(_lib.load().s2attn_bwd_dkdv_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dk), _ptr(dv),
                                              _ptr(workspace), workspace.numel(),
                                              B, H, Hkv, N, d, G, S, _wrap_code(wrap), _dtype_code(q),
                                              _stream(stream)),
               "s2attn_bwd_dkdv")


def s2attn_bwd_dq(q, k, v, do, dq, workspace, G, shift_heads=None, stream=None, wrap="roll"):
    """Stage 3 of the backward: dq (needs prep's workspace)."""
    B, H, Hkv, N, d, S = _dims(q, k, shift_heads)
    with torch.cuda.device(q.device):
        _check(_lib.load().s2attn_bwd_dq_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq),
                                            _ptr(workspace), workspace.numel(),
                                            B, H, Hkv, N, d, G, S, _wrap_code(wrap), _dtype_code(q),
                                            _stream(stream)),
               "s2attn_bwd_dq")


def s2attn_bwd_prep_dq(q, k, v, o, lse, do, dq, workspace, G, shift_heads=None, stream=None, wrap="roll"):
    """Stages 1 and 3 together: dq, and Dvec and lse * log2(e) into the workspace (dk, dv follow)."""
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
