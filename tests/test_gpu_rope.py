"""Rotary position embedding with Position Interpolation (s2attn_rope) against
the float64 oracle, element by element, and composed with the attention.

Bar: |y - y*| <= 2^-8 (|x_i| + |x_{i+d/2}|) per element for bf16 (the output
rounding alone is at most the bf16 unit roundoff 2^-8 of |y| <= |x_i| +
|x_{i+d/2}|; the float32 rotation and the hardware sine and cosine add far
less), 1e-6 of the same for fp32 (float32 rotation of an angle reduced in
float64)."""

import numpy as np
import pytest
import torch

from oracle import s2attn_oracle as orc
from shifted_sparse_attention_s2attn_amd import rope, s2attn_fwd, s2attn_rope
from shifted_sparse_attention_s2attn_amd.inputs import make_inputs, small_workload

pytestmark = pytest.mark.gpu


def f64(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def check(x, y, scale, base, inverse=False):
    xr = f64(x)
    ref = orc.rope(xr, scale, base, inverse)
    half = xr.shape[-1] // 2
    mag = np.abs(xr[..., :half]) + np.abs(xr[..., half:])
    bound = (2.0 ** -8 if x.dtype == torch.bfloat16 else 1e-6) * np.concatenate([mag, mag], axis=-1) + 1e-30
    err = np.abs(f64(y) - ref)
    worst = float(np.max(err / bound))
    print(f"  max err / bound = {worst:.3f}", flush=True)
    assert worst <= 1.0


CASES = [  # B, N, Hx, d, dtype, pos_scale, base
    (2, 300, 3, 128, torch.bfloat16, 1.0, 10000.0),
    (1, 4096, 4, 128, torch.bfloat16, 4096 / 32768, 10000.0),
    (1, 1000, 2, 64, torch.bfloat16, 0.5, 500000.0),
    (1, 777, 2, 128, torch.float32, 0.25, 10000.0),
    (2, 64, 3, 64, torch.float32, 1.0, 10000.0),
]


@pytest.mark.parametrize("B,N,Hx,d,dtype,scale,base", CASES)
def test_rope_matches_oracle(B, N, Hx, d, dtype, scale, base):
    print(f"case rope B={B} N={N} Hx={Hx} d={d} {dtype} scale={scale} base={base}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(N + d)
    x = torch.randn(B, N, Hx, d, device="cuda", generator=g).to(dtype)
    check(x, s2attn_rope(x, scale, base), scale, base)
    check(x, s2attn_rope(x, scale, base, inverse=True), scale, base, inverse=True)


def test_rope_long_positions():
    """Positions up to 102400 (7B at 100k, plain and interpolated): the float64
    angle reduction keeps every element within the bar."""
    print("case rope N=102400", flush=True)
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn(1, 102400, 1, 128, device="cuda", generator=g).bfloat16()
    for scale in (1.0, 4096 / 102400):
        check(x, s2attn_rope(x, scale), scale, 10000.0)


def test_rope_in_place_and_inverse():
    print("case rope in place", flush=True)
    g = torch.Generator(device="cuda").manual_seed(6)
    x = torch.randn(2, 513, 4, 128, device="cuda", generator=g)
    y = s2attn_rope(x, 0.125)
    z = x.clone()
    s2attn_rope(z, 0.125, out=z)
    assert torch.equal(y, z)
    back = s2attn_rope(y, 0.125, inverse=True)
    assert float((back - x).abs().max()) <= 1e-5


def test_rope_autograd_is_the_inverse_rotation():
    print("case rope autograd", flush=True)
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn(1, 256, 2, 64, device="cuda", generator=g).bfloat16().requires_grad_(True)
    gy = torch.randn(1, 256, 2, 64, device="cuda", generator=g).bfloat16()
    y = rope(x, 0.5)
    y.backward(gy)
    assert torch.equal(x.grad, s2attn_rope(gy, 0.5, inverse=True))


def test_rope_then_attention_matches_oracle():
    """Rotate q and k, then S2-Attn: against the oracle's rotation followed by the
    oracle's attention (both on the same bf16 inputs)."""
    w = small_workload("rope-attn", B=1, H=4, Hkv=2, d=128, N=1024, G=256, shift_heads=2)
    print(f"case {w} with rope", flush=True)
    inp = make_inputs(w, seed=12)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    scale = 4096 / 32768
    o, lse = s2attn_fwd(s2attn_rope(q, scale), s2attn_rope(k, scale), v, w.G, w.shift_heads)
    torch.cuda.synchronize()
    qr = torch.tensor(orc.rope(f64(inp["q"]), scale)).bfloat16()   # rounded like the kernel's output
    kr = torch.tensor(orc.rope(f64(inp["k"]), scale)).bfloat16()
    o_ref, lse_ref = orc.forward(f64(qr), f64(kr), f64(inp["v"]), w.G, w.shift_heads)
    err = float(np.max(np.abs(f64(o) - o_ref)))
    print(f"  max|dO| = {err:.3e}", flush=True)
    assert err <= 2e-2
