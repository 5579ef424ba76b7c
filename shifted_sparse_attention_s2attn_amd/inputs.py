"""Seeded synthetic inputs for S2-Attn, shared by the tests, the benchmark and the smoke check.

This module draws random tensors and nothing else: it holds none of the
attention arithmetic, so both the GPU library and the float64 oracle can be fed
from it without sharing any computation.

Workloads (the attention shapes of the pages' Llama2 fine-tuning runs: 32 heads
of width 128 for 7B, 64 query heads over 8 key/value heads for 70B, group size
G = N/4 as in "LongLoRA: Efficient Fine-tuning of Long-Context Large Language
Models", section 3.2 item 3 and the Table 7 discussion).  The pages train on
RedPajama text and evaluate on PG19 / proof-pile; no activations of those runs
exist here, so i.i.d. Gaussians of the same shapes stand in for them.

Recipe: one CPU ``torch.Generator`` seeded with ``seed``; q, k, v, dO drawn in
that order with ``torch.randn`` in float32 at shapes [B,N,H,d], [B,N,Hkv,d],
[B,N,Hkv,d], [B,N,H,d]; q and k multiplied by d**-0.25 when ``qk_quarter_scale``
is set (the 8k workload); then rounded to the workload dtype (round to nearest
even for bf16).
"""

from dataclasses import dataclass

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "small_workload"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    d: int
    N: int
    G: int
    shift_heads: int
    dtype: str               # "bf16" or "f32"
    qk_quarter_scale: bool = False

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


WORKLOADS = {
    "tiny-f32": Workload("tiny-f32", 1, 4, 4, 64, 512, 128, 2, "f32"),
    "llama2-7b-8k": Workload("llama2-7b-8k", 1, 32, 32, 128, 8192, 2048, 16, "bf16", True),
    "llama2-7b-32k": Workload("llama2-7b-32k", 1, 32, 32, 128, 32768, 8192, 16, "bf16"),
    "llama2-7b-100k": Workload("llama2-7b-100k", 1, 32, 32, 128, 102400, 25600, 16, "bf16"),
    "llama2-70b-gqa-32k": Workload("llama2-70b-gqa-32k", 1, 64, 8, 128, 32768, 8192, 32, "bf16"),
    # Table 7's 1/6 group at context 8192: G = 1365 does not divide N (the last
    # group holds 2 tokens) and is odd (shift 682); runs the kernels' EDGE instantiations
    "llama2-7b-8k-g1365": Workload("llama2-7b-8k-g1365", 1, 32, 32, 128, 8192, 1365, 16, "bf16", True),
    # full causal attention over the whole context (G = N, no shifted heads): what the
    # fine-tuned model runs at inference (section 3.2, "Inference")
    "llama2-7b-100k-fullattn": Workload("llama2-7b-100k-fullattn", 1, 32, 32, 128, 102400, 102400, 0, "bf16"),
}


def small_workload(name="custom", B=1, H=4, Hkv=4, d=64, N=512, G=128, shift_heads=None,
                   dtype="bf16", qk_quarter_scale=False):
    """A workload of arbitrary (small) shape; shift_heads defaults to H // 2."""
    if shift_heads is None:
        shift_heads = H // 2
    return Workload(name, B, H, Hkv, d, N, G, shift_heads, dtype, qk_quarter_scale)


def make_inputs(w, seed=0, device="cpu"):
    """Return dict(q, k, v, do) of the workload dtype on ``device``.

    The generator lives on ``device`` (torch's CPU generator, or the GPU's
    Philox generator for the large workloads), so values depend on the device;
    a run that checks against the oracle copies the very tensors it used.
    """
    g = torch.Generator(device=device).manual_seed(seed)
    qs = (w.B, w.N, w.H, w.d)
    kvs = (w.B, w.N, w.Hkv, w.d)
    kw = dict(dtype=torch.float32, generator=g, device=device)
    q = torch.randn(qs, **kw)
    k = torch.randn(kvs, **kw)
    v = torch.randn(kvs, **kw)
    do = torch.randn(qs, **kw)
    if w.qk_quarter_scale:
        f = float(w.d) ** -0.25
        q.mul_(f)
        k.mul_(f)
    dt = w.torch_dtype
    return {"q": q.to(dt), "k": k.to(dt), "v": v.to(dt), "do": do.to(dt)}
