"""The library from plain C: tests/_bin/c_abi_client (tests/c_abi_client.c)
allocates device memory with the HIP runtime, calls s2attn_fwd_ex,
s2attn_bwd_ex and s2attn_rope (q, Position Interpolation by 1/4) through
include/s2attn.h, and writes the outputs to a file.  They
must meet the float64 oracle's bars and equal, bit for bit, what the Python
binding gets from the same library on the same inputs (every kernel is
deterministic)."""

import os
import subprocess

import numpy as np
import pytest
import torch

from oracle import s2attn_oracle as orc
from shifted_sparse_attention_s2attn_amd import s2attn_bwd, s2attn_fwd, s2attn_rope
from shifted_sparse_attention_s2attn_amd.inputs import make_inputs, small_workload

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_bin", "c_abi_client")
WRAP_CODE = {"roll": 0, "split": 1, "swap": 2}

CASES = [
    (small_workload("c-gqa2-roll", B=2, H=4, Hkv=2, d=128, N=1024, G=256, shift_heads=2), "roll"),
    (small_workload("c-gqa2-split", B=1, H=4, Hkv=2, d=64, N=1024, G=512, shift_heads=2), "split"),
    (small_workload("c-gqa2-swap", B=1, H=4, Hkv=2, d=128, N=1024, G=256, shift_heads=2), "swap"),
    (small_workload("c-short-last-group", B=1, H=4, Hkv=2, d=128, N=1000, G=300, shift_heads=2), "roll"),
]


def bf16_bytes(x):
    return x.contiguous().view(torch.int16).numpy().tobytes()


@pytest.mark.parametrize("w,wrap", CASES, ids=[w.name for w, _ in CASES])
def test_c_client_matches_oracle_and_binding(w, wrap, tmp_path):
    print(f"case {w} wrap={wrap}", flush=True)
    assert os.path.exists(CLIENT), "tests/_bin/c_abi_client is missing: run __graft_entry__.build()"
    inp = make_inputs(w, seed=11)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    src.write_bytes(b"".join(bf16_bytes(inp[n]) for n in ("q", "k", "v", "do")))
    args = [CLIENT, str(src), str(dst), *map(str, (w.B, w.H, w.Hkv, w.N, w.d, w.G, w.shift_heads, WRAP_CODE[wrap]))]
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"client exit {r.returncode}: {r.stdout} {r.stderr}"

    raw = dst.read_bytes()
    nq, nkv, nl = w.B * w.N * w.H * w.d, w.B * w.N * w.Hkv * w.d, w.B * w.H * w.N
    assert len(raw) == 2 * (3 * nq + 2 * nkv) + 4 * nl
    pos = 0

    def take(n, dtype, shape):
        nonlocal pos
        size = n * np.dtype(dtype).itemsize
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=pos).reshape(shape)
        pos += size
        return torch.from_numpy(a.copy())

    qs, ks = (w.B, w.N, w.H, w.d), (w.B, w.N, w.Hkv, w.d)
    o = take(nq, np.int16, qs).view(torch.bfloat16)
    lse = take(nl, np.float32, (w.B, w.H, w.N))
    dq = take(nq, np.int16, qs).view(torch.bfloat16)
    dk = take(nkv, np.int16, ks).view(torch.bfloat16)
    dv = take(nkv, np.int16, ks).view(torch.bfloat16)
    qr = take(nq, np.int16, qs).view(torch.bfloat16)

    # the same library through the Python binding
    t = {k: v.cuda() for k, v in inp.items()}
    o_b, lse_b = s2attn_fwd(t["q"], t["k"], t["v"], w.G, w.shift_heads, wrap=wrap)
    g_b = s2attn_bwd(t["q"], t["k"], t["v"], o_b, lse_b, t["do"], w.G, w.shift_heads, wrap=wrap)
    torch.cuda.synchronize()
    qr_b = s2attn_rope(t["q"], 0.25)
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv", "rope(q)"), (o, lse, dq, dk, dv, qr),
                          (o_b, lse_b) + tuple(g_b) + (qr_b,)):
        assert torch.equal(a, b.cpu()), f"{name}: C client and Python binding differ"

    # against the oracle (bars of the bf16 parity tests)
    f = lambda x: x.float().numpy().astype(np.float64)   # noqa: E731
    q, k, v, do = (f(inp[n]) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = orc.forward(q, k, v, w.G, w.shift_heads, wrap)
    refs = orc.backward(q, k, v, do, w.G, w.shift_heads, wrap)
    assert float(np.max(np.abs(f(o) - o_ref))) <= 2e-2
    assert float(np.max(np.abs(f(lse) - lse_ref))) <= 4e-3   # -ln(1 - 2^-8): bf16 row sums
    for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        e = float(np.linalg.norm(f(a) - b) / np.linalg.norm(b))
        assert e <= 3e-2, (name, e)
    # rotary embedding: the per-element bar of the rotary parity tests
    half = w.d // 2
    mag = np.abs(q[..., :half]) + np.abs(q[..., half:])
    bound = 2.0 ** -8 * np.concatenate([mag, mag], axis=-1) + 1e-30
    assert float(np.max(np.abs(f(qr) - orc.rope(q, 0.25, 10000.0, False)) / bound)) <= 1.0
