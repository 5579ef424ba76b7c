"""The rotary embedding (Position Interpolation) fused into the attention
(s2attn_fwd_rope / s2attn_bwd_rope, bf16), through the C ABI.

* Against the stand-alone route on the same inputs: the fused forward's q_rot
  equals s2attn_rope(q) bit for bit, and o and lse equal s2attn_fwd on
  (s2attn_rope(q), s2attn_rope(k)) bit for bit (the same rotation helpers, the
  same attention kernel); dv equals the unfused backward's bit for bit; dq and
  dk equal the unfused gradients turned back by s2attn_rope(.., inverse) up to
  the roundings: the fused kernels turn the fp32 sums g and round once, the
  stand-alone route rounds g to bf16, turns it and rounds again.  With the bf16
  unit roundoff u = 2^-8 (8 significant bits), the first rounding moves the
  turned pair by at most u (|g_i| + |g_{i+d/2}|) and each final rounding by
  at most u times the same, so |diff| <= 3u (|g_i| + |g_{i+d/2}|) per element.
* Against the float64 oracle: q and k rotated by the oracle's rope (rounded to
  bf16 as the kernel rounds q_rot and k_rot), the oracle's attention and
  gradients, dq and dk turned back by the oracle's inverse rope; the bars of
  the attention parity tests (max |O - O*| <= 2e-2, rel-L2 <= 3e-2 on dq, dk,
  dv).
"""

import numpy as np
import pytest
import torch

from oracle import s2attn_oracle as orc
from shifted_sparse_attention_s2attn_amd import (S2AttnError, s2attn_bwd, s2attn_bwd_rope, s2attn_fwd,
                                                 s2attn_fwd_rope, s2attn_rope, s2attn_with_rope)
from shifted_sparse_attention_s2attn_amd.inputs import make_inputs, small_workload

pytestmark = pytest.mark.gpu


def f64(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


CASES = [  # workload, wrap, pos_scale, base
    (small_workload("rope-mha", B=2, H=4, Hkv=4, d=128, N=1024, G=256, shift_heads=2), "roll", 4096 / 32768, 1e4),
    (small_workload("rope-gqa-d64", B=1, H=8, Hkv=2, d=64, N=2048, G=512, shift_heads=4), "roll", 0.5, 5e5),
    (small_workload("rope-split", B=1, H=4, Hkv=2, d=128, N=1024, G=256, shift_heads=2), "split", 0.25, 1e4),
    (small_workload("rope-swap", B=1, H=4, Hkv=4, d=128, N=1024, G=512, shift_heads=2), "swap", 1.0, 1e4),
    (small_workload("rope-unaligned", B=1, H=2, Hkv=2, d=128, N=1000, G=300, shift_heads=1), "roll", 0.125, 1e4),
    # a key/value head shared by shifted and unshifted query heads, G/2 = 192
    # not a multiple of 128: the two-pass dK/dV with the rotary epilogue
    (small_workload("rope-mixed-two-pass", B=1, H=6, Hkv=2, d=128, N=768, G=384, shift_heads=2), "split", 0.25, 1e4),
]


@pytest.mark.parametrize("w,wrap,scale,base", CASES, ids=[c[0].name for c in CASES])
def test_fused_rope_matches_standalone_and_oracle(w, wrap, scale, base):
    print(f"case {w} wrap={wrap} pos_scale={scale} base={base}", flush=True)
    inp = make_inputs(w, seed=21)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    # stand-alone route
    qr_s, kr_s = s2attn_rope(q, scale, base), s2attn_rope(k, scale, base)
    o_s, lse_s = s2attn_fwd(qr_s, kr_s, v, w.G, w.shift_heads, wrap=wrap)
    dqr_s, dkr_s, dv_s = s2attn_bwd(qr_s, kr_s, v, o_s, lse_s, do, w.G, w.shift_heads, wrap=wrap)
    dq_s, dk_s = s2attn_rope(dqr_s, scale, base, inverse=True), s2attn_rope(dkr_s, scale, base, inverse=True)
    # fused route (k still takes the stand-alone pass)
    o, lse, q_rot = s2attn_fwd_rope(q, kr_s, v, w.G, w.shift_heads, scale, base, wrap=wrap)
    dq, dk, dv = s2attn_bwd_rope(q_rot, kr_s, v, o, lse, do, w.G, w.shift_heads, scale, base, wrap=wrap)
    torch.cuda.synchronize()
    print(f"  q_rot vs s2attn_rope(q): {int((q_rot != qr_s).sum())} elements differ, "
          f"max {float((q_rot.float() - qr_s.float()).abs().max()):.3e}", flush=True)
    assert torch.equal(q_rot, qr_s)
    assert torch.equal(o, o_s) and torch.equal(lse, lse_s)
    assert torch.equal(dv, dv_s)
    for name, a, ref, raw in (("dq", dq, dq_s, dqr_s), ("dk", dk, dk_s, dkr_s)):
        g = f64(raw)
        half = g.shape[-1] // 2
        mag = np.abs(g[..., :half]) + np.abs(g[..., half:])
        bound = 3 * 2.0 ** -8 * np.concatenate([mag, mag], axis=-1) + 1e-30
        worst = float(np.max(np.abs(f64(a) - f64(ref)) / bound))
        print(f"  {name}: fused vs stand-alone max diff / bound = {worst:.3f}", flush=True)
        assert worst <= 1.0, name
    # the oracle: rope, attention, gradients, inverse rope
    qr = f64(torch.tensor(orc.rope(f64(inp["q"]), scale, base)).bfloat16())
    kr = f64(torch.tensor(orc.rope(f64(inp["k"]), scale, base)).bfloat16())
    vv, dd = f64(inp["v"]), f64(inp["do"])
    o_ref, _ = orc.forward(qr, kr, vv, w.G, w.shift_heads, wrap)
    dqr, dkr, dv_ref = orc.backward(qr, kr, vv, dd, w.G, w.shift_heads, wrap)
    dq_ref, dk_ref = orc.rope(dqr, scale, base, inverse=True), orc.rope(dkr, scale, base, inverse=True)
    err_o = float(np.max(np.abs(f64(o) - o_ref)))
    errs = {"dq": rel_l2(f64(dq), dq_ref), "dk": rel_l2(f64(dk), dk_ref), "dv": rel_l2(f64(dv), dv_ref)}
    print(f"  vs oracle: max|dO|={err_o:.3e} relL2 {errs}", flush=True)
    assert err_o <= 2e-2
    for n, e in errs.items():
        assert e <= 3e-2, (n, e)


def test_fused_rope_autograd_wrapper():
    w = small_workload("rope-autograd", B=1, H=4, Hkv=2, d=128, N=512, G=256, shift_heads=2)
    print(f"case {w}", flush=True)
    t = {n: x.cuda() for n, x in make_inputs(w, seed=22).items()}
    q, k, v = (t[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = s2attn_with_rope(q, k, v, w.G, w.shift_heads, 0.125)
    (o.float() * t["do"].float()).sum().backward()
    kr = s2attn_rope(t["k"], 0.125)
    o2, lse2, qr2 = s2attn_fwd_rope(t["q"], kr, t["v"], w.G, w.shift_heads, 0.125)
    g2 = s2attn_bwd_rope(qr2, kr, t["v"], o2, lse2, t["do"], w.G, w.shift_heads, 0.125)
    assert torch.equal(o, o2)
    assert torch.equal(q.grad, g2[0]) and torch.equal(k.grad, g2[1]) and torch.equal(v.grad, g2[2])


def test_fused_rope_full_size_32k():
    """The 7B 32k workload with Position Interpolation from 4096: the forward's
    q_rot and o bit-equal to the stand-alone route; a shifted head's wrap group
    and an unshifted group of dq, dk against the oracle route on those slices."""
    from shifted_sparse_attention_s2attn_amd.inputs import WORKLOADS
    w = WORKLOADS["llama2-7b-32k"]
    scale = 4096 / w.N
    print(f"case {w} pos_scale={scale} (generating inputs on the GPU)", flush=True)
    t = make_inputs(w, seed=0, device="cuda")
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    kr = s2attn_rope(k, scale)
    o, lse, q_rot = s2attn_fwd_rope(q, kr, v, w.G, w.shift_heads, scale)
    dq, dk, dv = s2attn_bwd_rope(q_rot, kr, v, o, lse, do, w.G, w.shift_heads, scale)
    torch.cuda.synchronize()
    assert torch.equal(q_rot, s2attn_rope(q, scale))
    o_s, _ = s2attn_fwd(q_rot, kr, v, w.G, w.shift_heads)
    assert torch.equal(o, o_s)
    for x in (dq, dk, dv):
        assert bool(torch.isfinite(x).all())
    N, G = w.N, w.G
    for h, g in ((w.H - 1, 3), (0, 1)):
        sig = orc.head_shift(h, w.H, w.shift_heads, G)
        rows = orc.rolled_order(N, sig)[g * G:(g + 1) * G]
        qh = f64(q_rot[:, :, h:h + 1])
        kh = f64(kr[:, :, h:h + 1])
        vh, doh = f64(v[:, :, h:h + 1]), f64(do[:, :, h:h + 1])
        S1 = 1 if sig else 0
        rr, dQg, dKg, dVg = orc.head_group_backward(qh, kh, vh, doh, G, S1, 0, 0, g)
        # turn the oracle's rotated-frame gradients back at their tokens
        pos_rows = torch.as_tensor(rr, device="cuda")

        def back(x):
            full = np.zeros((1, N, 1, w.d))
            full[0, rr, 0] = x
            return orc.rope(full, scale, inverse=True)[0, rr, 0]

        e_dq = rel_l2(f64(dq[0, pos_rows, h]), back(dQg))
        e_dk = rel_l2(f64(dk[0, pos_rows, h]), back(dKg))
        e_dv = rel_l2(f64(dv[0, pos_rows, h]), dVg)
        print(f"  head {h} group {g}: relL2 dq={e_dq:.3e} dk={e_dk:.3e} dv={e_dv:.3e}", flush=True)
        assert max(e_dq, e_dk, e_dv) <= 3e-2


def test_fused_rope_rejects_fp32_and_bad_parameters():
    w = small_workload("rope-reject", B=1, H=2, Hkv=2, d=64, N=256, G=128, shift_heads=1, dtype="f32")
    t = {n: x.cuda() for n, x in make_inputs(w, seed=23).items()}
    with pytest.raises(S2AttnError):
        s2attn_fwd_rope(t["q"], t["k"], t["v"], w.G, w.shift_heads, 1.0)
    qb, kb, vb = (t[n].bfloat16() for n in ("q", "k", "v"))
    with pytest.raises(S2AttnError):
        s2attn_fwd_rope(qb, kb, vb, w.G, w.shift_heads, -1.0)
    with pytest.raises(S2AttnError):
        s2attn_fwd_rope(qb, kb, vb, w.G, w.shift_heads, 1.0, base=1.0)
    torch.cuda.synchronize()
