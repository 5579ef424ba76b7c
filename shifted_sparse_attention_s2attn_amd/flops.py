"""Algorithmic work and traffic of S2-Attn, used to turn measured times into rates.

Work is counted on the group-local causal pairs only: one (query, key) pair of
one (batch, head) is counted when both tokens sit in the same group of that
head's rolled frame and the key is not after the query.
"""

__all__ = ["allowed_pairs", "fwd_flops", "bwd_flops", "fwd_bytes", "bwd_bytes",
           "dense_fwd_attention_flops", "MI355X_BF16_PEAK_TFLOPS", "MI355X_F32_PEAK_TFLOPS",
           "MI355X_HBM_PEAK_GBS"]

MI355X_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk/CU (dense bf16 MFMA)
MI355X_F32_PEAK_TFLOPS = 157.3     # dense fp32 MFMA
MI355X_HBM_PEAK_GBS = 8000.0


def allowed_pairs(B, H, N, G, shift_heads=0, wrap="roll"):
    """B * H * (N/G) groups, each a causal G x G triangle with G(G+1)/2 pairs
    (when G does not divide N, a last group of N mod G tokens).

    With the split wrap option each shifted head's wrap group loses the pairs of
    the wrapped tokens (the last floor(G/2) of the group) with the tokens before
    them, (G - floor(G/2)) floor(G/2) of them.  The swap option only reorders
    the wrap group, which stays one causal triangle: the count is the main
    method's.
    """
    rem = N % G
    pairs = B * H * ((N // G) * G * (G + 1) // 2 + rem * (rem + 1) // 2)
    if wrap == "split":
        pairs -= B * shift_heads * (G - G // 2) * (G // 2)
    return pairs


def fwd_flops(B, H, N, G, d, shift_heads=0, wrap="roll"):
    """QK^T (2d) and PV (2d) per allowed pair."""
    return 4 * d * allowed_pairs(B, H, N, G, shift_heads, wrap)


def bwd_flops(B, H, N, G, d, shift_heads=0, wrap="roll"):
    """Five contractions per allowed pair (QK^T, dO V^T, P^T dO, dS^T Q, dS K); recompute not counted."""
    return 10 * d * allowed_pairs(B, H, N, G, shift_heads, wrap)


def fwd_bytes(B, H, Hkv, N, d, elt):
    """Compulsory HBM traffic of the forward: read q, k, v; write o and lse (fp32)."""
    return elt * B * N * d * (2 * H + 2 * Hkv) + 4 * B * H * N


def bwd_bytes(B, H, Hkv, N, d, elt):
    """Compulsory traffic of the backward.

    Reads q, k, v, o, dO, lse; writes dq, dk, dv; writes and reads the fp32
    row-sum Dvec once each.
    """
    return elt * B * N * d * (3 * H + 2 * Hkv + H + 2 * Hkv) + 4 * B * H * N * 3


def dense_fwd_attention_flops(N, G, d, H, L):
    """The pages' convention for attention FLOPs of one sequence forward.

    4 N G d per head per layer: dense (not causally halved) QK^T and PV over
    groups of G ("LongLoRA..." page, Table 11; G = N is full attention).
    """
    return 4 * N * G * d * H * L
