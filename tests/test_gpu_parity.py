"""HIP path (through the C ABI) against the float64 oracle, element by element.

Small problems are checked on every output element.  The five named workloads
run at full size in the library's only launch configuration; their outputs are
checked on sampled (key/value head, group) slices that the oracle computes one
by one, plus properties that hold everywhere (finite values, the closed form of
the first row of every group).

Bars: bf16 inputs with fp32 accumulation: max |O - O*| <= 2e-2 and
||x - x*||_2 / ||x*||_2 <= 3e-2 for each of dQ, dK, dV; fp32 inputs: both
metrics <= 1e-4.  lse is compared as a diagnostic: fp32 1e-4; bf16 4e-3,
because the bf16 kernels normalise by the sum of the bf16-rounded P they feed to
the matrix cores: with the bf16 unit roundoff u = 2^-8 (8 significant bits),
|sum bf16(p) - sum p| <= u sum p bounds the lse deviation by
-ln(1 - 2^-8) ~ 3.92e-3 (reached only if every rounding of a row goes one way;
largest on rows with few keys).
"""

import numpy as np
import pytest
import torch

from oracle import s2attn_oracle as orc
from shifted_sparse_attention_s2attn_amd import (S2AttnError, s2attn, s2attn_bwd, s2attn_bwd_dq, s2attn_bwd_prep,
                                                 s2attn_bwd_prep_dq, s2attn_bwd_workspace_bytes, s2attn_fwd)
from shifted_sparse_attention_s2attn_amd.inputs import WORKLOADS, make_inputs, small_workload

pytestmark = pytest.mark.gpu

TOL = {"bf16": dict(o=2e-2, grad=3e-2, lse=4e-3), "f32": dict(o=1e-4, grad=1e-4, lse=1e-4)}


def say(*a):
    print(*a, flush=True)


def to_gpu(inp):
    return {k: v.cuda() for k, v in inp.items()}


def run_gpu(w, t, wrap="roll"):
    o, lse = s2attn_fwd(t["q"], t["k"], t["v"], w.G, w.shift_heads, wrap=wrap)
    dq, dk, dv = s2attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], w.G, w.shift_heads, wrap=wrap)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def f64(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def check_full(w, inp, out, wrap="roll"):
    tol = TOL[w.dtype]
    o, lse, dq, dk, dv = (f64(x) for x in out)
    q, k, v, do = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = orc.forward(q, k, v, w.G, w.shift_heads, wrap)
    dq_ref, dk_ref, dv_ref = orc.backward(q, k, v, do, w.G, w.shift_heads, wrap)
    err_o = float(np.max(np.abs(o - o_ref)))
    err_lse = float(np.max(np.abs(lse - lse_ref)))
    errs = {n: rel_l2(a, b) for n, a, b in (("dq", dq, dq_ref), ("dk", dk, dk_ref), ("dv", dv, dv_ref))}
    say(f"  max|dO|={err_o:.3e} max|dlse|={err_lse:.3e} relL2 {errs}")
    assert err_o <= tol["o"]
    assert err_lse <= tol["lse"]
    for n, e in errs.items():
        assert e <= tol["grad"], (n, e)


SMALL = [
    small_workload("bf16-d128-mha", B=2, H=4, Hkv=4, d=128, N=1024, G=256, shift_heads=2),
    small_workload("bf16-d64-gqa2", B=1, H=4, Hkv=2, d=64, N=1024, G=512, shift_heads=2),
    small_workload("bf16-gqa3-mixed-shift", B=1, H=6, Hkv=2, d=128, N=1024, G=256, shift_heads=2),
    small_workload("bf16-gqa8", B=1, H=16, Hkv=2, d=128, N=1024, G=256, shift_heads=8),
    small_workload("bf16-only-unshifted", B=1, H=2, Hkv=2, d=128, N=768, G=256, shift_heads=0),
    small_workload("bf16-only-shifted", B=1, H=2, Hkv=2, d=64, N=768, G=256, shift_heads=2),
    small_workload("bf16-full-causal", B=1, H=2, Hkv=1, d=128, N=1024, G=1024, shift_heads=0),
    small_workload("bf16-single-group-shifted", B=2, H=2, Hkv=2, d=128, N=128, G=128, shift_heads=1),
    small_workload("bf16-qk-scaled", B=1, H=4, Hkv=4, d=128, N=512, G=128, shift_heads=2, qk_quarter_scale=True),
    small_workload("f32-d128", B=1, H=2, Hkv=2, d=128, N=512, G=256, shift_heads=1, dtype="f32"),
    small_workload("f32-gqa2", B=2, H=4, Hkv=2, d=64, N=256, G=128, shift_heads=2, dtype="f32"),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_parity(w):
    say(f"case {w}")
    inp = make_inputs(w, seed=1)
    out = run_gpu(w, to_gpu(inp))
    check_full(w, inp, out)


# the split wrap option (Table 8, Variant 2) on every kernel path: bf16 fast
# kernels (G a multiple of 256: the last group's G/2 boundary inside a 256-row
# query tile; G = 128: inside a 128-key tile), the generic kernels (fp32, and
# bf16 with G = 128), GQA with mixed shifts
SPLIT = [w for w in SMALL if w.shift_heads > 0] + [
    small_workload("bf16-g128-split", B=1, H=4, Hkv=2, d=128, N=512, G=128, shift_heads=2),
    small_workload("bf16-d64-g384", B=1, H=2, Hkv=2, d=64, N=768, G=384, shift_heads=2),
]


@pytest.mark.parametrize("w", SPLIT, ids=[w.name for w in SPLIT])
def test_small_parity_split(w):
    say(f"case {w} wrap=split")
    inp = make_inputs(w, seed=2)
    out = run_gpu(w, to_gpu(inp), wrap="split")
    check_full(w, inp, out, wrap="split")


# the swap option (Table 8, Variant 3) on the same shapes: its row map breaks at
# N - G and N - G/2, tile boundaries of every kernel for these G
@pytest.mark.parametrize("w", SPLIT, ids=[w.name for w in SPLIT])
def test_small_parity_swap(w):
    say(f"case {w} wrap=swap")
    inp = make_inputs(w, seed=8)
    out = run_gpu(w, to_gpu(inp), wrap="swap")
    check_full(w, inp, out, wrap="swap")


# group sizes that do not divide the sequence, or are not whole 128-row tiles
# (EDGE instantiations of the bf16 kernels, generic kernels for fp32): the last
# group is short, the shift floor(G/2).  The forward and dq run 4-wave
# workgroups (128 query rows) for groups shorter than 4096 that are not whole
# 256-row tiles, 8-wave ones otherwise: both counts appear below.
UNALIGNED = [
    small_workload("bf16-short-last-group", B=1, H=4, Hkv=4, d=128, N=1000, G=256, shift_heads=2),
    # G not a multiple of 256 but long enough that the forward and dq keep 8
    # waves (256-row tiles): partial tiles in every group, a short last group
    small_workload("bf16-g4100", B=1, H=2, Hkv=2, d=128, N=9000, G=4100, shift_heads=1),
    small_workload("bf16-g100-gqa", B=2, H=2, Hkv=1, d=64, N=777, G=100, shift_heads=2),
    small_workload("bf16-table7-sixth", B=1, H=2, Hkv=2, d=128, N=8192, G=1365, shift_heads=1),
    small_workload("bf16-g3", B=1, H=2, Hkv=2, d=64, N=100, G=3, shift_heads=1),
    small_workload("f32-odd-g103", B=1, H=4, Hkv=2, d=64, N=515, G=103, shift_heads=2, dtype="f32"),
    small_workload("f32-g-equals-n-300", B=1, H=2, Hkv=2, d=128, N=300, G=300, shift_heads=1, dtype="f32"),
]


@pytest.mark.parametrize("w", UNALIGNED, ids=[w.name for w in UNALIGNED])
def test_small_parity_unaligned(w):
    say(f"case {w}")
    inp = make_inputs(w, seed=3)
    out = run_gpu(w, to_gpu(inp))
    check_full(w, inp, out)


# the split and swap options on the same shapes: the wrap group is the rolled
# group containing the wrap from token N-1 to token 0 (not necessarily the last
# one), and its cut (split) or the boundary between its front and end tokens
# (swap) falls inside tiles of every kernel
@pytest.mark.parametrize("wrap", ["split", "swap"])
@pytest.mark.parametrize("w", UNALIGNED, ids=[w.name for w in UNALIGNED])
def test_small_parity_unaligned_wrap_options(w, wrap):
    say(f"case {w} wrap={wrap}")
    inp = make_inputs(w, seed=13)
    out = run_gpu(w, to_gpu(inp), wrap=wrap)
    check_full(w, inp, out, wrap=wrap)


# a key/value head read by shifted and unshifted query heads on shapes whose two
# frames (G/2 apart) cut the keys into different 128-row tiles: dK/dV in two
# passes, the first leaving fp32 sums in the workspace (groups that are whole
# tiles with G/2 not a multiple of 128, groups that are not whole tiles, bf16
# fast kernels and fp32 generic ones, d 64 and 128), under every wrap option
MIXED = [
    small_workload("bf16-mixed-g128", B=1, H=6, Hkv=2, d=128, N=1024, G=128, shift_heads=2),
    small_workload("bf16-mixed-g384", B=2, H=4, Hkv=2, d=128, N=768, G=384, shift_heads=1),
    small_workload("bf16-mixed-g300", B=1, H=6, Hkv=2, d=64, N=1000, G=300, shift_heads=4),
    small_workload("bf16-mixed-g100-gqa4", B=1, H=4, Hkv=1, d=128, N=777, G=100, shift_heads=1),
    small_workload("f32-mixed-g103", B=1, H=6, Hkv=2, d=64, N=515, G=103, shift_heads=2, dtype="f32"),
    small_workload("f32-mixed-g128", B=1, H=4, Hkv=2, d=128, N=512, G=128, shift_heads=1, dtype="f32"),
    # Table 7's 1/6 group at N = 8192: 6 groups (the last of 2 rows) per head, many key tiles each
    small_workload("bf16-mixed-table7-8k", B=1, H=6, Hkv=2, d=128, N=8192, G=1365, shift_heads=2),
]


@pytest.mark.parametrize("wrap", ["roll", "split", "swap"])
@pytest.mark.parametrize("w", MIXED, ids=[w.name for w in MIXED])
def test_small_parity_mixed_shift_two_pass(w, wrap):
    say(f"case {w} wrap={wrap}")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    assert s2attn_bwd_workspace_bytes(w.B, w.H, w.Hkv, w.N, w.d, w.G, w.shift_heads, dt) >= \
        2 * w.B * w.H * w.N * 4 + 2 * w.B * w.N * w.Hkv * w.d * 4      # the two-pass workspace
    inp = make_inputs(w, seed=17)
    out = run_gpu(w, to_gpu(inp), wrap=wrap)
    check_full(w, inp, out, wrap=wrap)


def random_cases(n=24, seed=2024, wide=False):
    """Seeded random small problems over every option the ABI accepts: d, dtype,
    B, GQA ratio, shifted-head count, aligned and unaligned G, every wrap mode
    (key/value heads shared by shifted and unshifted query heads included).
    ``wide``: larger batches, GQA ratios and groups (bf16 only, N up to 4096)."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        d = int(rng.choice([64, 128]))
        dtype = "bf16" if wide else str(rng.choice(["bf16", "bf16", "f32"]))
        Hkv = int(rng.choice([1, 2, 3] if wide else [1, 2]))
        r = int(rng.choice([1, 2, 4] if wide else [1, 2, 3]))
        H = Hkv * r
        S = int(rng.integers(0, H + 1))
        G = int(rng.choice([768, 1024, 1536, 640, 1200, 333] if wide else [128, 256, 384, 512, 100, 7, 250, 1000]))
        N = int(rng.choice([G, 2 * G, 3 * G, G + int(rng.integers(1, G)) if G > 1 else G]))
        N = min(N, 4096 if wide else 2048)
        if G > N:
            continue
        B = int(rng.choice([1, 2, 3] if wide else [1, 2]))
        wrap = str(rng.choice(["roll", "split", "swap"]))
        cases.append((small_workload(f"rand{len(cases)}", B=B, H=H, Hkv=Hkv, d=d, N=N, G=G, shift_heads=S,
                                     dtype=dtype), wrap))
    return cases


RANDOM = random_cases()


@pytest.mark.parametrize("w,wrap", RANDOM, ids=[f"{w.name}-{w.dtype}-d{w.d}-N{w.N}-G{w.G}-H{w.H}x{w.Hkv}-S{w.shift_heads}-{wrap}"
                                                for w, wrap in RANDOM])
def test_random_shapes(w, wrap):
    say(f"case {w} wrap={wrap}")
    inp = make_inputs(w, seed=7)
    out = run_gpu(w, to_gpu(inp), wrap=wrap)
    check_full(w, inp, out, wrap=wrap)


RANDOM_WIDE = random_cases(n=12, seed=77, wide=True)


@pytest.mark.parametrize("w,wrap", RANDOM_WIDE, ids=[f"{w.name}-d{w.d}-B{w.B}-N{w.N}-G{w.G}-H{w.H}x{w.Hkv}-S{w.shift_heads}-{wrap}"
                                                     for w, wrap in RANDOM_WIDE])
def test_random_wide_shapes(w, wrap):
    say(f"case {w} wrap={wrap}")
    inp = make_inputs(w, seed=8)
    out = run_gpu(w, to_gpu(inp), wrap=wrap)
    check_full(w, inp, out, wrap=wrap)


@pytest.mark.parametrize("seed", range(10))
def test_tiny_f32_workload(seed):
    """B=1, H=4 (2 shifted), d=64, N=512, G=128, fp32; seeds 0-9."""
    w = WORKLOADS["tiny-f32"]
    say(f"case {w.name} seed {seed}")
    inp = make_inputs(w, seed=seed)
    out = run_gpu(w, to_gpu(inp))
    check_full(w, inp, out)


# ---------------------------------------------------------------------------
# full-size workloads: sampled slices + global properties
# ---------------------------------------------------------------------------

# (key/value head, group index in the frame of that KV head's first query head).
# The kernels number their blocks in chunks of 32 (batch, head, group) pairs
# (4 groups per head here, so a chunk is 8 consecutive query heads): the MHA
# workloads sample one slice in each of their 4 chunks, the GQA workload 5 of its
# 8 KV heads (one chunk each), wrap groups of shifted heads included.
SAMPLES = {
    "llama2-7b-8k": [(0, 1), (10, 2), (20, 0), (31, 3)],
    "llama2-7b-32k": [(0, 0), (12, 1), (17, 3), (31, 3)],
    "llama2-7b-100k": [(5, 2), (9, 0), (22, 1), (31, 3)],
    "llama2-70b-gqa-32k": [(0, 2), (2, 1), (4, 3), (5, 0), (7, 3)],
}


def check_sampled(w, t, out, c, g0, b=0, wrap="roll"):
    tol = TOL[w.dtype]
    o, lse, dq, dk, dv = out
    r = w.H // w.Hkv
    S_sub = max(0, min(r, (c + 1) * r - (w.H - w.shift_heads)))
    hs = slice(c * r, (c + 1) * r)
    q = f64(t["q"][:, :, hs])
    k = f64(t["k"][:, :, c:c + 1])
    v = f64(t["v"][:, :, c:c + 1])
    do = f64(t["do"][:, :, hs])
    N, G = w.N, w.G
    R = orc.rolled_order(N, orc.head_shift(0, r, S_sub, G))[g0 * G:(g0 + 1) * G]
    dk_acc = np.zeros((N, w.d))
    dv_acc = np.zeros((N, w.d))
    o_err, lse_err = 0.0, 0.0
    dq_num, dq_den = 0.0, 0.0
    for hh in range(r):
        h = c * r + hh
        sig = orc.head_shift(hh, r, S_sub, G)
        for g in sorted(set(((R - sig) % N) // G)):
            rows, Og, lseg = orc.head_group_forward(q, k, v, G, S_sub, b, hh, g, wrap)
            ridx = torch.as_tensor(rows, device=o.device)
            o_err = max(o_err, float(np.max(np.abs(f64(o[b, ridx, h]) - Og))))
            lse_err = max(lse_err, float(np.max(np.abs(f64(lse[b, h, ridx]) - lseg))))
            rows, dQg, dKg, dVg = orc.head_group_backward(q, k, v, do, G, S_sub, b, hh, g, wrap)
            dq_num += float(np.sum((f64(dq[b, ridx, h]) - dQg) ** 2))
            dq_den += float(np.sum(dQg ** 2))
            dk_acc[rows] += dKg
            dv_acc[rows] += dVg
    Ridx = torch.as_tensor(R, device=o.device)
    e_dk = rel_l2(f64(dk[b, Ridx, c]), dk_acc[R])
    e_dv = rel_l2(f64(dv[b, Ridx, c]), dv_acc[R])
    e_dq = (dq_num / dq_den) ** 0.5
    say(f"  kv head {c} group {g0} ({wrap}): max|dO|={o_err:.3e} max|dlse|={lse_err:.3e} "
        f"relL2 dq={e_dq:.3e} dk={e_dk:.3e} dv={e_dv:.3e}")
    assert o_err <= tol["o"]
    assert lse_err <= tol["lse"]
    assert e_dq <= tol["grad"] and e_dk <= tol["grad"] and e_dv <= tol["grad"]


def check_global(w, t, out):
    o, lse, dq, dk, dv = out
    for name, x in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(x).all()), f"non-finite values in {name}"
    # first row of every group attends to itself only: O = V exactly, lse = scale q.k
    r = w.H // w.Hkv
    for h in range(w.H):
        sig = w.G // 2 if h >= w.H - w.shift_heads else 0
        first = (torch.arange(0, w.N, w.G, device=o.device) + sig) % w.N
        c = h // r
        assert torch.equal(o[:, first, h], t["v"][:, first, c]), f"first-row O head {h}"
        ref = (t["q"][:, first, h].float() * t["k"][:, first, c].float()).sum(-1) / w.d ** 0.5
        assert float((lse[:, h, first] - ref).abs().max()) <= 1e-3, f"first-row lse head {h}"


@pytest.mark.parametrize("name", list(SAMPLES))
def test_full_size_workload(name):
    w = WORKLOADS[name]
    say(f"case {w} (generating inputs on the GPU)")
    t = make_inputs(w, seed=0, device="cuda")
    out = run_gpu(w, t)
    say("  kernels done; global checks")
    check_global(w, t, out)
    for c, g0 in SAMPLES[name]:
        check_sampled(w, t, out, c, g0)


@pytest.mark.parametrize("wrap", ["split", "swap"])
def test_full_size_table7_sixth_group_wrap_options(wrap):
    """Table 7's 1/6 group (G = 1365 at N = 8192, shift 682) with the split and
    swap options: the wrap group is rolled group 5 (rows 6825..8189, the wrap
    after row 7509, 680 front tokens), followed by the 2-row group 6; sampled
    for a shifted head, with an unshifted head's group."""
    w = WORKLOADS["llama2-7b-8k-g1365"]
    say(f"case {w} wrap={wrap} (generating inputs on the GPU)")
    t = make_inputs(w, seed=0, device="cuda")
    out = run_gpu(w, t, wrap=wrap)
    say("  kernels done")
    for name, x in zip(("o", "lse", "dq", "dk", "dv"), out):
        assert bool(torch.isfinite(x).all()), f"non-finite values in {name}"
    for c, g0 in [(31, 5), (31, 6), (0, 5)]:
        check_sampled(w, t, out, c, g0, wrap=wrap)


def test_full_size_table7_sixth_group():
    """Table 7's 1/6 group at the 7B 8k shape: G = 1365 (odd, does not divide
    8192), shift 682.  Sampled: a shifted head's wrap group (rolled group 5)
    and its 2-token last group, and an unshifted head's last group."""
    w = WORKLOADS["llama2-7b-8k-g1365"]
    say(f"case {w} (generating inputs on the GPU)")
    t = make_inputs(w, seed=0, device="cuda")
    out = run_gpu(w, t)
    say("  kernels done")
    for name, x in zip(("o", "lse", "dq", "dk", "dv"), out):
        assert bool(torch.isfinite(x).all()), f"non-finite values in {name}"
    for c, g0 in [(31, 5), (31, 6), (0, 6), (0, 0)]:
        check_sampled(w, t, out, c, g0)


def test_slice_over_2gib():
    """One batch's q / dO slice of 2 GiB (B=1, H=64, d=128, N=131072): the
    dK/dV kernel reads query tiles 2 GiB into the slice, through buffers based
    at each tile.  Sampled as the other full-size workloads: a shifted and an
    unshifted KV head."""
    w = small_workload("gqa-131k", B=1, H=64, Hkv=8, d=128, N=131072, G=8192, shift_heads=32)
    assert w.N * w.H * w.d * 2 >= 2 ** 31
    say(f"case {w} (generating inputs on the GPU)")
    t = make_inputs(w, seed=0, device="cuda")
    out = run_gpu(w, t)
    say("  kernels done; global checks")
    check_global(w, t, out)
    for c, g0 in [(7, 15), (0, 3)]:
        check_sampled(w, t, out, c, g0)


def test_kv_slice_over_2gib():
    """K / V slices of 2.5 GiB per batch (B=1, H=Hkv=32, d=128, N=327680,
    G=8192): the forward and dQ kernels read key tiles past byte offset 2^31 of
    the slice (every tensor is 2.5 GiB, 20 GiB in all), with the same kernels as
    every other bf16 size.  Sampled: the wrap group of a shifted head, which
    reads the last and the first tokens, and an unshifted group wholly past
    2 GiB (tokens 286720..294911)."""
    w = small_workload("mha-320k", B=1, H=32, Hkv=32, d=128, N=327680, G=8192, shift_heads=16)
    assert 286720 * w.Hkv * w.d * 2 >= 2 ** 31
    say(f"case {w} (generating inputs on the GPU)")
    t = make_inputs(w, seed=0, device="cuda")
    out = run_gpu(w, t)
    say("  kernels done; global checks")
    check_global(w, t, out)
    for c, g0 in [(31, 39), (0, 35)]:
        check_sampled(w, t, out, c, g0)


def test_full_size_split():
    """The split option at the 7B-32k size: the wrap group of a shifted head
    (its group 3, whose second half is tokens 0..G/2-1) and a plain group."""
    w = WORKLOADS["llama2-7b-32k"]
    say(f"case {w} wrap=split (generating inputs on the GPU)")
    t = make_inputs(w, seed=0, device="cuda")
    out = run_gpu(w, t, wrap="split")
    say("  kernels done")
    for name, x in zip(("o", "lse", "dq", "dk", "dv"), out):
        assert bool(torch.isfinite(x).all()), f"non-finite values in {name}"
    # the first wrapped token of a shifted head attends to itself only
    h = w.H - 1
    assert torch.equal(out[0][:, 0, h], t["v"][:, 0, h // (w.H // w.Hkv)])
    for c, g0 in [(31, 3), (0, 3)]:
        check_sampled(w, t, out, c, g0, wrap="split")


def test_full_size_swap():
    """The swap option at the 7B-32k size: the wrap group of a shifted head
    (tokens 0..G/2-1 first, then N-G/2..N-1) and a plain group."""
    w = WORKLOADS["llama2-7b-32k"]
    say(f"case {w} wrap=swap (generating inputs on the GPU)")
    t = make_inputs(w, seed=0, device="cuda")
    out = run_gpu(w, t, wrap="swap")
    say("  kernels done")
    for name, x in zip(("o", "lse", "dq", "dk", "dv"), out):
        assert bool(torch.isfinite(x).all()), f"non-finite values in {name}"
    # token 0 now opens the wrap group of a shifted head: it attends to itself only
    h = w.H - 1
    assert torch.equal(out[0][:, 0, h], t["v"][:, 0, h // (w.H // w.Hkv)])
    for c, g0 in [(31, 3), (0, 3)]:
        check_sampled(w, t, out, c, g0, wrap="swap")


@pytest.mark.parametrize("wrap", ["split", "swap"])
def test_full_size_gqa_wrap_options(wrap):
    """The split and swap options at the 70B GQA shape (64 query heads over 8
    KV heads, 32 shifted): the wrap group of a shifted KV head (8 query heads,
    dk / dv summed over them) and a group of an unshifted one."""
    w = WORKLOADS["llama2-70b-gqa-32k"]
    say(f"case {w} wrap={wrap} (generating inputs on the GPU)")
    t = make_inputs(w, seed=0, device="cuda")
    out = run_gpu(w, t, wrap=wrap)
    say("  kernels done")
    for name, x in zip(("o", "lse", "dq", "dk", "dv"), out):
        assert bool(torch.isfinite(x).all()), f"non-finite values in {name}"
    # token 0 of a shifted head opens a causal group of its own (split) or the wrap group (swap)
    h = w.H - 1
    assert torch.equal(out[0][:, 0, h], t["v"][:, 0, h // (w.H // w.Hkv)])
    for c, g0 in [(6, 3), (1, 2)]:
        check_sampled(w, t, out, c, g0, wrap=wrap)


def test_full_size_full_attention():
    """G = N = 102400, no shift: full causal attention at the 7B 100k shape.

    One group holds the whole sequence, so the oracle checks rows: o, lse and dq
    of sampled tokens of two heads, and dk, dv of the last 64 keys (which only
    the last 64 tokens see), each from the tokens' own rows.
    """
    w = WORKLOADS["llama2-7b-100k-fullattn"]
    tol = TOL[w.dtype]
    say(f"case {w} (generating inputs on the GPU)")
    t = make_inputs(w, seed=0, device="cuda")
    o, lse, dq, dk, dv = run_gpu(w, t)
    say("  kernels done")
    N, d = w.N, w.d
    for h in (0, w.H - 1):
        # this head alone, as a one-head problem (its own KV head: H = Hkv here)
        qh, kh, vh, doh = (f64(t[n][:, :, h:h + 1]) for n in ("q", "k", "v", "do"))
        o_err = lse_err = 0.0
        num = den = 0.0
        for tok in (0, 1, 4095, 51200, N - 1):
            row = orc.row_attention(qh, kh, vh, doh, N, 0, 0, 0, tok)
            o_err = max(o_err, float(np.max(np.abs(f64(o[0, tok, h]) - row["o"]))))
            lse_err = max(lse_err, abs(float(lse[0, h, tok]) - row["lse"]))
            num += float(np.sum((f64(dq[0, tok, h]) - row["dq"]) ** 2))
            den += float(np.sum(row["dq"] ** 2))
        last = 64
        dk_ref = np.zeros((last, d))
        dv_ref = np.zeros((last, d))
        for tok in range(N - last, N):
            row = orc.row_attention(qh, kh, vh, doh, N, 0, 0, 0, tok)
            sel = row["keys"] >= N - last
            idx = row["keys"][sel] - (N - last)
            dv_ref[idx] += row["p"][sel][:, None] * doh[0, tok, 0][None, :]
            dk_ref[idx] += row["ds"][sel][:, None] * qh[0, tok, 0][None, :] / np.sqrt(d)
        e_dk = rel_l2(f64(dk[0, N - last:, h]), dk_ref)
        e_dv = rel_l2(f64(dv[0, N - last:, h]), dv_ref)
        e_dq = (num / den) ** 0.5
        say(f"  head {h}: max|dO|={o_err:.3e} max|dlse|={lse_err:.3e} relL2 dq={e_dq:.3e} "
            f"dk={e_dk:.3e} dv={e_dv:.3e}")
        assert o_err <= tol["o"] and lse_err <= tol["lse"]
        assert e_dq <= tol["grad"] and e_dk <= tol["grad"] and e_dv <= tol["grad"]


# ---------------------------------------------------------------------------
# determinism, autograd wrapper, error path
# ---------------------------------------------------------------------------

def test_repeatability():
    """Every output is bitwise repeatable: no kernel uses atomics, so the order of
    every sum is fixed by the code."""
    w = small_workload("rep", B=1, H=8, Hkv=2, d=128, N=2048, G=512, shift_heads=4)
    say(f"case {w}")
    t = to_gpu(make_inputs(w, seed=3))
    a = run_gpu(w, t)
    b = run_gpu(w, t)
    for i in range(5):
        assert torch.equal(a[i], b[i])


@pytest.mark.parametrize("wrap", ["roll", "split", "swap"])
def test_autograd_wrapper(wrap):
    w = small_workload("autograd", B=1, H=4, Hkv=4, d=64, N=512, G=256, shift_heads=2)
    say(f"case {w} wrap={wrap}")
    t = to_gpu(make_inputs(w, seed=4))
    q, k, v = (t[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = s2attn(q, k, v, w.G, w.shift_heads, wrap=wrap)
    (o.float() * t["do"].float()).sum().backward()
    ref = run_gpu(w, t, wrap=wrap)
    assert torch.equal(o, ref[0])
    assert torch.equal(q.grad, ref[2]) and torch.equal(k.grad, ref[3]) and torch.equal(v.grad, ref[4])


@pytest.mark.parametrize("G,dtype", [(256, "bf16"), (100, "bf16"), (256, "f32")])
def test_graph_capture_replays(G, dtype):
    """The forward and backward calls launch kernels only (no allocation, copy,
    memset or synchronisation), so they can be captured in a HIP graph: three
    replays, with eager work and synchronisations between them, each equal to
    the eager result bit for bit (fast and generic kernels)."""
    w = small_workload("graph", B=1, H=4, Hkv=2, d=128, N=1024, G=G, shift_heads=2, dtype=dtype)
    say(f"case {w}")
    t = to_gpu(make_inputs(w, seed=5))
    ref = run_gpu(w, t)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o, lse = torch.empty_like(q), torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = torch.empty(s2attn_bwd_workspace_bytes(w.B, w.H, w.Hkv, w.N, w.d, w.G, w.shift_heads, q.dtype),
                     dtype=torch.uint8, device="cuda")

    def step():
        s2attn_fwd(q, k, v, w.G, w.shift_heads, out=o, lse=lse)
        s2attn_bwd(q, k, v, o, lse, do, w.G, w.shift_heads, workspace=ws, grads=grads)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    outs = (o, lse) + grads
    for rep in range(3):
        for x in outs:
            x.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(("o", "lse", "dq", "dk", "dv"), outs, ref):
            assert torch.equal(x, r), f"replay {rep}: {name} differs from the eager result"


@pytest.mark.parametrize("G,dtype", [(256, "bf16"), (256, "f32"), (100, "bf16")])
def test_prep_fused_into_dq(G, dtype):
    """s2attn_bwd_prep_dq (one launch on the fast bf16 path) against prep then dq:
    lse * log2(e) bit-equal, Dvec and dq equal up to the rounding of Dvec."""
    w = small_workload("prep-dq", B=2, H=4, Hkv=2, d=128, N=1024, G=G, shift_heads=2, dtype=dtype)
    say(f"case {w}")
    t = to_gpu(make_inputs(w, seed=6))
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o, lse = s2attn_fwd(q, k, v, w.G, w.shift_heads)
    nbytes = s2attn_bwd_workspace_bytes(w.B, w.H, w.Hkv, w.N, w.d, w.G, w.shift_heads, q.dtype)
    ws_a = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros_like(ws_a)
    dq_a, dq_b = torch.empty_like(q), torch.empty_like(q)
    s2attn_bwd_prep(q, k, o, lse, do, ws_a, w.G, w.shift_heads)
    s2attn_bwd_dq(q, k, v, do, dq_a, ws_a, w.G, w.shift_heads)
    s2attn_bwd_prep_dq(q, k, v, o, lse, do, dq_b, ws_b, w.G, w.shift_heads)
    torch.cuda.synchronize()
    n = w.B * w.H * w.N
    half = nbytes // 2
    dvec_a, dvec_b = ws_a[:4 * n].view(torch.float32), ws_b[:4 * n].view(torch.float32)
    lse2_a, lse2_b = ws_a[half:half + 4 * n].view(torch.float32), ws_b[half:half + 4 * n].view(torch.float32)
    assert torch.equal(lse2_a, lse2_b)
    assert float((dvec_a - dvec_b).abs().max()) <= 1e-5 * max(1.0, float(dvec_a.abs().max()))
    err = float((dq_a.float() - dq_b.float()).norm() / dq_a.float().norm())
    assert err <= (1e-2 if dtype == "bf16" else 1e-5), err


@pytest.mark.parametrize("B,N", [(0, 512), (2, 0)])
def test_empty_inputs(B, N):
    """An empty batch or sequence: outputs of the right (empty) shapes, no error."""
    say(f"case empty B={B} N={N}")
    q = torch.zeros((B, N, 4, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, N, 2, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = s2attn_fwd(q, k, k, 128, 2)
    assert o.shape == q.shape and lse.shape == (B, 4, N)
    dq, dk, dv = s2attn_bwd(q, k, k, o, lse, q, 128, 2)
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == k.shape
    qg, kg, vg = (x.clone().requires_grad_(True) for x in (q, k, k))
    s2attn(qg, kg, vg, 128, 2).float().sum().backward()
    assert qg.grad.shape == q.shape and kg.grad.shape == k.shape
    torch.cuda.synchronize()


def test_binding_rejects_mismatched_tensors():
    """Wrong shapes, dtypes or workspaces raise in the binding, before any launch."""
    w = small_workload("mismatch", B=1, H=4, Hkv=2, d=64, N=512, G=128, shift_heads=2)
    t = to_gpu(make_inputs(w, seed=9))
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o, lse = s2attn_fwd(q, k, v, w.G, w.shift_heads)
    with pytest.raises(ValueError, match="lse"):
        s2attn_fwd(q, k, v, w.G, w.shift_heads, lse=torch.empty(1, 4, 256, device="cuda"))
    with pytest.raises(TypeError, match="lse"):
        s2attn_bwd(q, k, v, o, lse.double(), do, w.G, w.shift_heads)
    with pytest.raises(ValueError, match="do"):
        s2attn_bwd(q, k, v, o, lse, do[:, :256].contiguous(), w.G, w.shift_heads)
    with pytest.raises(ValueError, match="dk"):
        s2attn_bwd(q, k, v, o, lse, do, w.G, w.shift_heads, grads=(torch.empty_like(q), torch.empty_like(q),
                                                                      torch.empty_like(k)))
    with pytest.raises(ValueError, match="workspace"):
        s2attn_bwd(q, k, v, o, lse, do, w.G, w.shift_heads, workspace=torch.empty(1 << 20, device="cuda"))
    with pytest.raises(ValueError, match="contiguous"):
        s2attn_fwd(q.transpose(1, 2).contiguous().transpose(1, 2), k, v, w.G, w.shift_heads)
    torch.cuda.synchronize()


def test_rejected_shape_raises():
    q = torch.zeros((1, 500, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(S2AttnError):
        s2attn_fwd(q, q, q, 1024, 1)            # group longer than the sequence
    with pytest.raises(S2AttnError):
        s2attn_fwd(q, q, q, 100, 3)             # more shifted heads than heads
