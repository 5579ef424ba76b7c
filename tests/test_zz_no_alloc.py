"""s2attn_bwd_noalloc (the backward with the library's own scratch array, for
callers that cannot allocate) against s2attn_bwd_ex, through the C ABI.

Four calls in a row share the GPU's scratch array, each smaller than the one
before, so the later ones run on scratch still holding the earlier rows: the
7B 32k workload, a bf16 shape whose groups are not whole tiles, a bf16 shape
whose dK/dV takes two passes (a key/value head shared by shifted and
unshifted query heads, G = 100: the first pass's sums also sit in the
scratch), and an fp32 shape with the split option.  Each must equal s2attn_bwd_ex on the same inputs
bit for bit (the same kernels, no atomics), which is within the bf16 / fp32
bars of the oracle parity tests; the smallest one is also checked against the
oracle.
"""

import numpy as np
import pytest
import torch

from oracle import s2attn_oracle as orc
from shifted_sparse_attention_s2attn_amd import s2attn_bwd, s2attn_bwd_noalloc, s2attn_fwd
from shifted_sparse_attention_s2attn_amd.inputs import WORKLOADS, make_inputs, small_workload

pytestmark = pytest.mark.gpu

CASES = [
    (WORKLOADS["llama2-7b-32k"], "roll", "cuda"),
    (small_workload("edge", B=2, H=4, Hkv=2, d=128, N=1000, G=256, shift_heads=2), "roll", "cpu"),
    (small_workload("mixed-two-pass", B=1, H=6, Hkv=2, d=64, N=500, G=100, shift_heads=2), "swap", "cpu"),
    (small_workload("f32-split", B=1, H=2, Hkv=2, d=64, N=512, G=128, shift_heads=1, dtype="f32"), "split", "cpu"),
]


def f64(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def test_noalloc_matches_bwd_ex_on_successive_calls():
    for w, wrap, gen in CASES:
        print(f"case {w} wrap={wrap}", flush=True)
        inp = make_inputs(w, seed=11, device=gen)
        t = {n: x.cuda() for n, x in inp.items()}
        q, k, v, do = t["q"], t["k"], t["v"], t["do"]
        o, lse = s2attn_fwd(q, k, v, w.G, w.shift_heads, wrap=wrap)
        ref = s2attn_bwd(q, k, v, o, lse, do, w.G, w.shift_heads, wrap=wrap)
        got = (torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan")))
        s2attn_bwd_noalloc(q, k, v, o, lse, do, *got, w.G, w.shift_heads, wrap=wrap)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"{w.name}: {name} differs from s2attn_bwd_ex"
        if w.N <= 512:
            qa, ka, va, doa = (f64(inp[n]) for n in ("q", "k", "v", "do"))
            g_ref = orc.backward(qa, ka, va, doa, w.G, w.shift_heads, wrap)
            for name, a, b in zip(("dq", "dk", "dv"), got, g_ref):
                rel = float(np.linalg.norm(f64(a) - b) / np.linalg.norm(b))
                assert rel <= (1e-4 if w.dtype == "f32" else 3e-2), (name, rel)
        del t, q, k, v, do, o, lse, ref, got
