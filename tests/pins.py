"""Independent checks that pin the float64 oracle to the method's definition.

Each ``pin_*`` function takes the oracle module and raises AssertionError when the
oracle disagrees with something other than itself: a brute-force dense masked
attention written in original token coordinates, a roll / regroup / causal-SDPA
formulation evaluated by torch, full causal attention, exact symmetries of the
method, closed forms, finite differences and the page's worked index example.
``test_oracle.py`` runs them on the real oracle; ``test_oracle_mutations.py``
runs them on copies of the oracle with planted mistakes and expects a failure.
"""

import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# (B, N, H, Hkv, d, G, S): small problems covering MHA, GQA, every shift count
SMALL_CASES = [
    (1, 16, 2, 2, 4, 8, 1),
    (2, 24, 4, 2, 3, 8, 2),
    (1, 32, 4, 4, 5, 8, 4),
    (1, 32, 4, 1, 4, 16, 0),
    (1, 12, 3, 3, 2, 4, 2),
    (1, 32, 6, 3, 4, 8, 3),   # GQA with the shifted/unshifted boundary inside a KV group
]


def rand_problem(B, N, H, Hkv, d, seed, scale_qk=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, H, d)) * scale_qk
    k = rng.standard_normal((B, N, Hkv, d)) * scale_qk
    v = rng.standard_normal((B, N, Hkv, d))
    do = rng.standard_normal((B, N, H, d))
    return q, k, v, do


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) / max(1.0, np.max(np.abs(b)))
    assert err <= tol, f"{what}: relative max error {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
# P1: brute force in original coordinates
# ---------------------------------------------------------------------------

def allowed_mask_original(N, G, shifted, split=False, swap=False):
    """M[t, u] = token t may attend token u, written without any roll.

    Unshifted heads: groups are [kG, (k+1)G) and a token sees the earlier tokens
    of its group and itself.  Shifted heads: the group boundaries move by G/2,
    so groups are [kG + G/2, (k+1)G + G/2) taken cyclically; the last one holds
    the final G/2 tokens followed by the first G/2, in that order, and "earlier"
    means earlier in that order.  Shifted heads with ``split`` (Table 8's
    Variant 2): additionally both tokens must lie on the same side of the wrap
    (both among the first G/2 tokens, or both not), so for N a multiple of G the
    groups are [0, G/2), [G/2 + jG, G/2 + (j+1)G) and [N - G/2, N).
    Shifted heads with ``swap`` (Variant 3): the groups of the main method, with
    "earlier" meaning a smaller token index in every group (the first G/2
    tokens come before the last G/2 in the group they share).
    When G does not divide N the groups are counted from the start of the
    (shifted) grid and the last one is short; the shift is floor(G/2).
    """
    M = np.zeros((N, N), dtype=bool)
    half = G // 2
    for t in range(N):
        for u in range(N):
            if not shifted:
                same = (t // G) == (u // G)
                before = u <= t
            elif split:
                ot = (t - half) % N
                ou = (u - half) % N
                same = (ot // G) == (ou // G) and ((t < half) == (u < half))
                before = ou <= ot
            elif swap:
                same = ((t - half) % N) // G == ((u - half) % N) // G
                before = u <= t
            else:
                # offset of each token from the start of the shifted grid
                ot = (t - half) % N
                ou = (u - half) % N
                same = (ot // G) == (ou // G)
                before = ou <= ot
            M[t, u] = same and before
    return M


def dense_masked_attention(q, k, v, G, S, grad_do=None, split=False, swap=False):
    """Dense N x N masked softmax attention in torch float64 (autograd for grads)."""
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    r = H // Hkv
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    masks = {False: torch.tensor(allowed_mask_original(N, G, False)),
             True: torch.tensor(allowed_mask_original(N, G, True, split, swap))}
    outs, lses = [], []
    for h in range(H):
        shifted = h >= H - S
        c = h // r
        s = torch.einsum("bnd,bmd->bnm", tq[:, :, h], tk[:, :, c]) / np.sqrt(d)
        s = s.masked_fill(~masks[shifted][None], float("-inf"))
        lses.append(torch.logsumexp(s, dim=-1))
        p = torch.softmax(s, dim=-1)
        outs.append(torch.einsum("bnm,bmd->bnd", p, tv[:, :, c]))
    o = torch.stack(outs, dim=2)
    lse = torch.stack(lses, dim=1)
    grads = None
    if grad_do is not None:
        (o * torch.tensor(grad_do, dtype=torch.float64)).sum().backward()
        grads = (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())
    return o.detach().numpy(), lse.detach().numpy(), grads


def pin_bruteforce_forward(orc):
    for i, (B, N, H, Hkv, d, G, S) in enumerate(SMALL_CASES):
        q, k, v, _ = rand_problem(B, N, H, Hkv, d, seed=10 + i)
        o, lse = orc.forward(q, k, v, G, S)
        o_ref, lse_ref, _ = dense_masked_attention(q, k, v, G, S)
        _close(o, o_ref, 1e-12, f"brute-force O case {i}")
        _close(lse, lse_ref, 1e-12, f"brute-force lse case {i}")


def pin_bruteforce_backward(orc):
    for i, (B, N, H, Hkv, d, G, S) in enumerate(SMALL_CASES):
        q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=20 + i)
        dq, dk, dv = orc.backward(q, k, v, do, G, S)
        _, _, (dq_ref, dk_ref, dv_ref) = dense_masked_attention(q, k, v, G, S, grad_do=do)
        _close(dq, dq_ref, 1e-11, f"brute-force dQ case {i}")
        _close(dk, dk_ref, 1e-11, f"brute-force dK case {i}")
        _close(dv, dv_ref, 1e-11, f"brute-force dV case {i}")


# ---------------------------------------------------------------------------
# P2: roll the shifted heads, regroup, causal SDPA per group, roll back
# ---------------------------------------------------------------------------

def roll_regroup_attention(q, k, v, G, S, grad_do=None):
    """S2-Attn as tensor operations: roll, view as groups, causal attention, unroll.

    The shifted heads' tokens are rolled by -G/2 along the sequence, the sequence
    is viewed as B*N/G independent groups, torch's causal scaled_dot_product_attention
    runs on every group, the result is viewed back as [B, N, H, d] and the shifted
    heads are rolled by +G/2.  Key/value heads are repeated for grouped queries.
    """
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    r = H // Hkv
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    kk = torch.repeat_interleave(tk, r, dim=2)
    vv = torch.repeat_interleave(tv, r, dim=2)
    split = H - S

    def shift(x):
        return torch.cat([x[:, :, :split], torch.roll(x[:, :, split:], -(G // 2), dims=1)], dim=2)

    def unshift(x):
        return torch.cat([x[:, :, :split], torch.roll(x[:, :, split:], G // 2, dims=1)], dim=2)

    def grouped(x):  # [B, N, H, d] -> [B*N/G, H, G, d]
        return x.reshape(B * N // G, G, H, d).transpose(1, 2)

    og = F.scaled_dot_product_attention(grouped(shift(tq)), grouped(shift(kk)), grouped(shift(vv)),
                                        is_causal=True)
    o = unshift(og.transpose(1, 2).reshape(B, N, H, d))
    grads = None
    if grad_do is not None:
        (o * torch.tensor(grad_do, dtype=torch.float64)).sum().backward()
        grads = (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())
    return o.detach().numpy(), grads


def pin_roll_regroup(orc):
    cases = SMALL_CASES + [(1, 64, 4, 2, 8, 16, 2), (2, 48, 2, 2, 4, 12, 1)]
    for i, (B, N, H, Hkv, d, G, S) in enumerate(cases):
        q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=30 + i)
        o, _ = orc.forward(q, k, v, G, S)
        dq, dk, dv = orc.backward(q, k, v, do, G, S)
        o_ref, (dq_ref, dk_ref, dv_ref) = roll_regroup_attention(q, k, v, G, S, grad_do=do)
        _close(o, o_ref, 1e-12, f"roll/regroup O case {i}")
        _close(dq, dq_ref, 1e-11, f"roll/regroup dQ case {i}")
        _close(dk, dk_ref, 1e-11, f"roll/regroup dK case {i}")
        _close(dv, dv_ref, 1e-11, f"roll/regroup dV case {i}")


# ---------------------------------------------------------------------------
# P3: G = N without shift is full causal attention
# ---------------------------------------------------------------------------

def pin_full_causal(orc):
    for i, (B, N, H, d) in enumerate([(1, 40, 2, 8), (2, 33, 3, 5)]):
        if N % 2:
            N += 1
        q, k, v, do = rand_problem(B, N, H, H, d, seed=40 + i)
        o, lse = orc.forward(q, k, v, N, 0)
        dq, dk, dv = orc.backward(q, k, v, do, N, 0)
        tq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        ref = F.scaled_dot_product_attention(tq.transpose(1, 2), tk.transpose(1, 2), tv.transpose(1, 2),
                                             is_causal=True).transpose(1, 2)
        (ref * torch.tensor(do)).sum().backward()
        _close(o, ref.detach().numpy(), 1e-12, "full causal O")
        _close(dq, tq.grad.numpy(), 1e-11, "full causal dQ")
        _close(dk, tk.grad.numpy(), 1e-11, "full causal dK")
        _close(dv, tv.grad.numpy(), 1e-11, "full causal dV")
        # lse of full causal attention: row t normalises over tokens 0..t
        s = np.einsum("bnhd,bmhd->bhnm", q, k) / np.sqrt(d)
        s = np.where(np.tril(np.ones((N, N), dtype=bool))[None, None], s, -np.inf)
        lse_ref = np.log(np.sum(np.exp(s), axis=-1))
        _close(lse, lse_ref, 1e-12, "full causal lse")


# ---------------------------------------------------------------------------
# P4: reversing the roll direction changes nothing (bitwise)
# ---------------------------------------------------------------------------

def pin_direction_reversal(orc):
    """Rolling by +G/2 instead of -G/2 shifts the grid by a whole group.

    With N a multiple of G both rolls give the same partition of the tokens into
    the same ordered groups, so every output must be bitwise identical.
    """
    B, N, H, Hkv, d, G, S = 1, 48, 4, 2, 4, 12, 2
    q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=50)
    o1, lse1 = orc.forward(q, k, v, G, S)
    g1 = orc.backward(q, k, v, do, G, S)
    original = orc.head_shift
    try:
        # -G/2 mod N: rolled position j then holds token (j - G/2) mod N
        orc.head_shift = lambda h, H_, S_, G_: (N - G_ // 2) % N if h >= H_ - S_ else 0
        o2, lse2 = orc.forward(q, k, v, G, S)
        g2 = orc.backward(q, k, v, do, G, S)
    finally:
        orc.head_shift = original
    assert np.array_equal(o1, o2), "O changed when the roll direction was reversed"
    assert np.array_equal(lse1, lse2), "lse changed when the roll direction was reversed"
    for a, b, n in zip(g1, g2, ("dQ", "dK", "dV")):
        assert np.array_equal(a, b), f"{n} changed when the roll direction was reversed"


# ---------------------------------------------------------------------------
# P5: rolling the input by G/2 swaps the roles of the two head halves
# ---------------------------------------------------------------------------

def pin_head_swap(orc):
    """With S = H/2: roll inputs by +G/2 and exchange the head halves.

    The unshifted grid of the rolled input is the shifted grid of the input and
    vice versa, so the output is the original output rolled by +G/2 with its
    head halves exchanged.  Key/value heads are exchanged the same way.
    """
    for (B, N, H, Hkv, d, G) in [(1, 32, 4, 4, 4, 8), (1, 48, 4, 2, 3, 12)]:
        S = H // 2
        q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=60 + N)
        o, lse = orc.forward(q, k, v, G, S)
        dq, dk, dv = orc.backward(q, k, v, do, G, S)

        def sw(x, nh):
            return np.roll(np.concatenate([x[:, :, nh // 2:], x[:, :, :nh // 2]], axis=2), G // 2, axis=1)

        o2, lse2 = orc.forward(sw(q, H), sw(k, Hkv), sw(v, Hkv), G, S)
        dq2, dk2, dv2 = orc.backward(sw(q, H), sw(k, Hkv), sw(v, Hkv), sw(do, H), G, S)
        _close(o2, sw(o, H), 1e-13, "head-swap O")
        lse_sw = np.roll(np.concatenate([lse[:, H // 2:], lse[:, :H // 2]], axis=1), G // 2, axis=2)
        _close(lse2, lse_sw, 1e-13, "head-swap lse")
        _close(dq2, sw(dq, H), 1e-12, "head-swap dQ")
        _close(dk2, sw(dk, Hkv), 1e-12, "head-swap dK")
        _close(dv2, sw(dv, Hkv), 1e-12, "head-swap dV")


# ---------------------------------------------------------------------------
# P6: closed forms
# ---------------------------------------------------------------------------

def pin_closed_forms(orc):
    B, N, H, Hkv, d, G, S = 1, 32, 4, 2, 6, 8, 2
    q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=70)
    o, lse = orc.forward(q, k, v, G, S)
    r = H // Hkv
    for h in range(H):
        c = h // r
        first = (np.arange(0, N, G) + (G // 2 if h >= H - S else 0)) % N
        # the first token of every group attends to itself only
        _close(o[0, first, h], v[0, first, c], 1e-14, f"first-row O head {h}")
        lse_first = np.sum(q[0, first, h] * k[0, first, c], axis=1) / np.sqrt(d)
        _close(lse[0, h, first], lse_first, 1e-14, f"first-row lse head {h}")
    # constant values: every output row equals that value
    vc = np.broadcast_to(np.arange(1.0, d + 1.0), v.shape).copy()
    oc, _ = orc.forward(q, k, vc, G, S)
    _close(oc, np.broadcast_to(np.arange(1.0, d + 1.0), oc.shape), 1e-13, "constant V")
    # zero queries: uniform weights over the allowed keys (position p of a group sees p + 1 keys)
    z = np.zeros_like(q)
    _, lse0 = orc.forward(z, k, v, G, S)
    for h in range(H):
        sig = G // 2 if h >= H - S else 0
        pos = (np.arange(N) - sig) % N % G
        _close(lse0[0, h], np.log(pos + 1.0), 1e-14, f"zero-query lse head {h}")
    # locality: without shift, changing keys/values outside group 1 leaves group 1 unchanged
    o_a, _ = orc.forward(q, k, v, G, 0)
    k2, v2 = k.copy(), v.copy()
    k2[:, :G] += 3.0
    v2[:, 2 * G:] -= 5.0
    o_b, _ = orc.forward(q, k2, v2, G, 0)
    assert np.array_equal(o_a[:, G:2 * G], o_b[:, G:2 * G]), "group 1 depends on other groups"


# ---------------------------------------------------------------------------
# P7: finite differences of L = sum(O * dO)
# ---------------------------------------------------------------------------

def pin_finite_differences(orc):
    for Hkv in (2, 1):
        B, N, H, d, G, S = 1, 16, 2, 4, 8, 1
        q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=80 + Hkv)
        dq, dk, dv = orc.backward(q, k, v, do, G, S)
        eps = 1e-6

        def loss(qq, kk, vv):
            o, _ = orc.forward(qq, kk, vv, G, S)
            return float(np.sum(o * do))

        for name, x, g in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp = x.copy()
                xp[idx] += eps
                xm = x.copy()
                xm[idx] -= eps
                args_p = [q, k, v]
                args_m = [q, k, v]
                pos = {"dQ": 0, "dK": 1, "dV": 2}[name]
                args_p[pos] = xp
                args_m[pos] = xm
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            err = np.linalg.norm(num - g) / np.linalg.norm(num)
            assert err <= 1e-6, f"finite differences {name} (Hkv={Hkv}): rel {err:.2e}"


# ---------------------------------------------------------------------------
# P8: grouped-query attention equals multi-head attention on repeated K/V
# ---------------------------------------------------------------------------

def pin_gqa_repeat(orc):
    B, N, H, Hkv, d, G, S = 1, 32, 6, 2, 4, 8, 3
    q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=90)
    r = H // Hkv
    o, lse = orc.forward(q, k, v, G, S)
    dq, dk, dv = orc.backward(q, k, v, do, G, S)
    kr = np.repeat(k, r, axis=2)
    vr = np.repeat(v, r, axis=2)
    o2, lse2 = orc.forward(q, kr, vr, G, S)
    dq2, dk2, dv2 = orc.backward(q, kr, vr, do, G, S)
    _close(o, o2, 1e-14, "GQA O")
    _close(lse, lse2, 1e-14, "GQA lse")
    _close(dq, dq2, 1e-13, "GQA dQ")
    _close(dk, dk2.reshape(B, N, Hkv, r, d).sum(axis=3), 1e-13, "GQA dK")
    _close(dv, dv2.reshape(B, N, Hkv, r, d).sum(axis=3), 1e-13, "GQA dV")


# ---------------------------------------------------------------------------
# P9: the page's worked index example
# ---------------------------------------------------------------------------

def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split()
            vals[key] = int(val)
    return vals


def pin_worked_example_index_map(orc):
    """Which token sits where after the roll (fixes the roll direction)."""
    ex = read_golden("shift_worked_example.txt")
    N, G = ex["N"], ex["G"]
    H, S = 2, 1
    assert orc.head_shift(1, H, S, G) == ex["shift"]
    assert orc.head_shift(0, H, S, G) == 0
    order = orc.rolled_order(N, orc.head_shift(1, H, S, G))
    assert order[0] == ex["rolled0_token"]
    assert int(np.where(order == 0)[0][0]) == ex["token0_rolled_position"]
    assert order[0] == ex["shifted_group0_first"] and order[G - 1] == ex["shifted_group0_last"]
    plain = orc.rolled_order(N, orc.head_shift(0, H, S, G))
    assert plain[0] == ex["unshifted_group0_first"] and plain[G - 1] == ex["unshifted_group0_last"]


def pin_worked_example_reach(orc):
    """Which tokens the probe token reaches (independent of the roll direction)."""
    ex = read_golden("shift_worked_example.txt")
    N, G = ex["N"], ex["G"]
    H, S = 2, 1
    # attention reach of the probe token, read off the oracle forward itself:
    # zero queries give uniform weights, one-hot value columns report which keys are reached
    t = ex["probe_token"]
    d = 4
    q = np.zeros((1, N, H, d))
    k = np.zeros((1, N, H, d))
    v = np.zeros((1, N, H, d))
    v[0, ex["shifted_group0_first"], :, 0] = 1.0        # first token of the shifted group
    v[0, ex["shifted_group0_first"] - 1, :, 1] = 1.0    # token just before it
    v[0, t + 1, :, 2] = 1.0                             # next token (future)
    v[0, t, :, 3] = 1.0                                 # itself
    o, _ = orc.forward(q, k, v, G, S)
    n_sh = ex["probe_shifted_group_position"] + 1
    _close(o[0, t, 1], [1.0 / n_sh, 0.0, 0.0, 1.0 / n_sh], 1e-15, "shifted head reach")
    n_un = t + 1
    _close(o[0, t, 0], [1.0 / n_un, 1.0 / n_un, 0.0, 1.0 / n_un], 1e-15, "unshifted head reach")


# ---------------------------------------------------------------------------
# Split wrap option (Table 8, Variant 2): the wrapped tokens form their own group
# ---------------------------------------------------------------------------

def pin_split_bruteforce(orc):
    """Oracle with wrap="split" against the dense mask of the split partition."""
    for i, (B, N, H, Hkv, d, G, S) in enumerate(SMALL_CASES):
        q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=110 + i)
        o, lse = orc.forward(q, k, v, G, S, "split")
        dq, dk, dv = orc.backward(q, k, v, do, G, S, "split")
        o_ref, lse_ref, (dq_ref, dk_ref, dv_ref) = dense_masked_attention(q, k, v, G, S, grad_do=do, split=True)
        _close(o, o_ref, 1e-12, f"split brute-force O case {i}")
        _close(lse, lse_ref, 1e-12, f"split brute-force lse case {i}")
        _close(dq, dq_ref, 1e-11, f"split brute-force dQ case {i}")
        _close(dk, dk_ref, 1e-11, f"split brute-force dK case {i}")
        _close(dv, dv_ref, 1e-11, f"split brute-force dV case {i}")


def pin_split_segments_sdpa(orc):
    """Every split group is a contiguous token range: causal SDPA on each range.

    Shifted heads: [0, G/2), [G/2 + jG, G/2 + (j+1)G), [N - G/2, N); unshifted
    heads: [jG, (j+1)G).  torch's scaled_dot_product_attention (float64, causal)
    on each range, autograd for the gradients; K/V repeated for grouped queries.
    """
    for i, (B, N, H, Hkv, d, G, S) in enumerate([(1, 32, 4, 2, 4, 8, 2), (2, 24, 2, 1, 3, 12, 1),
                                                  (1, 16, 2, 2, 4, 16, 2)]):
        q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=120 + i)
        o, lse = orc.forward(q, k, v, G, S, "split")
        dq, dk, dv = orc.backward(q, k, v, do, G, S, "split")
        r = H // Hkv
        tq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        kk = torch.repeat_interleave(tk, r, dim=2)
        vv = torch.repeat_interleave(tv, r, dim=2)
        heads = []
        for h in range(H):
            cuts = [0] + (list(range(G // 2, N, G)) if h >= H - S else list(range(G, N, G))) + [N]
            segs = []
            for a, e in zip(cuts[:-1], cuts[1:]):
                segs.append(F.scaled_dot_product_attention(tq[:, a:e, h][:, None], kk[:, a:e, h][:, None],
                                                           vv[:, a:e, h][:, None], is_causal=True)[:, 0])
            heads.append(torch.cat(segs, dim=1))
        ref = torch.stack(heads, dim=2)
        (ref * torch.tensor(do)).sum().backward()
        _close(o, ref.detach().numpy(), 1e-12, f"split SDPA O case {i}")
        _close(dq, tq.grad.numpy(), 1e-11, f"split SDPA dQ case {i}")
        _close(dk, tk.grad.numpy(), 1e-11, f"split SDPA dK case {i}")
        _close(dv, tv.grad.numpy(), 1e-11, f"split SDPA dV case {i}")


def pin_split_agrees_with_roll(orc):
    """The two wrap options differ only where their partitions differ.

    S = 0: no head is shifted, so every output is identical.  S > 0: unshifted
    heads are identical; in shifted heads O and lse differ only on tokens
    [0, G/2) (the wrapped tokens, which no longer see the last G/2 tokens), and
    the first wrapped token then attends to itself only (O = V, lse = scale q.k).
    """
    B, N, H, Hkv, d, G = 1, 32, 4, 2, 4, 8
    q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=130)
    for S in (0, 2):
        o_r, lse_r = orc.forward(q, k, v, G, S)
        o_s, lse_s = orc.forward(q, k, v, G, S, "split")
        if S == 0:
            assert np.array_equal(o_r, o_s) and np.array_equal(lse_r, lse_s), "split changed an unshifted problem"
            for a, b, n in zip(orc.backward(q, k, v, do, G, S), orc.backward(q, k, v, do, G, S, "split"),
                               ("dQ", "dK", "dV")):
                assert np.array_equal(a, b), f"split changed {n} of an unshifted problem"
            continue
        _close(o_s[:, :, :H - S], o_r[:, :, :H - S], 1e-14, "split: unshifted heads O")
        _close(o_s[:, G // 2:], o_r[:, G // 2:], 1e-13, "split: rows past the wrapped tokens")
        _close(lse_s[:, :, G // 2:], lse_r[:, :, G // 2:], 1e-13, "split: lse past the wrapped tokens")
        assert np.max(np.abs(o_s[:, :G // 2, H - S:] - o_r[:, :G // 2, H - S:])) > 1e-3, \
            "split did not change the wrapped tokens"
        r = H // Hkv
        for h in range(H - S, H):
            _close(o_s[0, 0, h], v[0, 0, h // r], 1e-14, f"split: first wrapped token O head {h}")
            _close(lse_s[0, h, 0], np.dot(q[0, 0, h], k[0, 0, h // r]) / np.sqrt(d), 1e-14,
                   f"split: first wrapped token lse head {h}")


def pin_split_finite_differences(orc):
    B, N, H, Hkv, d, G, S = 1, 16, 2, 1, 3, 8, 1
    q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=140)
    grads = orc.backward(q, k, v, do, G, S, "split")
    eps = 1e-6
    for pos, name in enumerate(("dQ", "dK", "dV")):
        x = (q, k, v)[pos]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args_p, args_m = [q, k, v], [q, k, v]
            args_p[pos] = x.copy()
            args_p[pos][idx] += eps
            args_m[pos] = x.copy()
            args_m[pos][idx] -= eps
            lp = float(np.sum(orc.forward(*args_p, G, S, "split")[0] * do))
            lm = float(np.sum(orc.forward(*args_m, G, S, "split")[0] * do))
            num[idx] = (lp - lm) / (2 * eps)
        err = np.linalg.norm(num - grads[pos]) / np.linalg.norm(num)
        assert err <= 1e-6, f"split finite differences {name}: rel {err:.2e}"


# ---------------------------------------------------------------------------
# Swap wrap option (Table 8, Variant 3): inside the wrap group the tokens from
# the front of the sequence come before those from its end
# ---------------------------------------------------------------------------

def pin_swap_bruteforce(orc):
    """Oracle with wrap="swap" against the dense mask: the main method's groups,
    causal in original token order."""
    for i, (B, N, H, Hkv, d, G, S) in enumerate(SMALL_CASES):
        q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=180 + i)
        o, lse = orc.forward(q, k, v, G, S, "swap")
        dq, dk, dv = orc.backward(q, k, v, do, G, S, "swap")
        o_ref, lse_ref, (dq_ref, dk_ref, dv_ref) = dense_masked_attention(q, k, v, G, S, grad_do=do, swap=True)
        _close(o, o_ref, 1e-12, f"swap brute-force O case {i}")
        _close(lse, lse_ref, 1e-12, f"swap brute-force lse case {i}")
        _close(dq, dq_ref, 1e-11, f"swap brute-force dQ case {i}")
        _close(dk, dk_ref, 1e-11, f"swap brute-force dK case {i}")
        _close(dv, dv_ref, 1e-11, f"swap brute-force dV case {i}")


def pin_swap_gathered_sdpa(orc, cases=((1, 32, 4, 2, 4, 8, 2), (2, 24, 2, 1, 3, 12, 1), (1, 16, 2, 2, 4, 16, 2))):
    """Every swap group gathered in token order, then torch's causal SDPA.

    Token t of a head shifted by s = floor(G/2) belongs to group ((t - s) mod N)
    // G (the main method's partition, last group short when G does not divide
    N); the tokens of each group are taken in increasing index, attended with
    is_causal=True and scattered back; autograd for the gradients; K/V repeated
    for grouped queries.
    """
    for i, (B, N, H, Hkv, d, G, S) in enumerate(cases):
        q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=190 + i)
        o, lse = orc.forward(q, k, v, G, S, "swap")
        dq, dk, dv = orc.backward(q, k, v, do, G, S, "swap")
        r = H // Hkv
        tq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        kk = torch.repeat_interleave(tk, r, dim=2)
        vv = torch.repeat_interleave(tv, r, dim=2)
        heads = []
        for h in range(H):
            sh = G // 2 if h >= H - S else 0
            gid = ((np.arange(N) - sh) % N) // G
            out = [None] * N
            for g in np.unique(gid):
                toks = torch.tensor(np.nonzero(gid == g)[0])      # increasing token index
                og = F.scaled_dot_product_attention(tq[:, toks, h][:, None], kk[:, toks, h][:, None],
                                                    vv[:, toks, h][:, None], is_causal=True)[:, 0]
                for n, t in enumerate(toks.tolist()):
                    out[t] = og[:, n]
            heads.append(torch.stack(out, dim=1))
        ref = torch.stack(heads, dim=2)
        (ref * torch.tensor(do)).sum().backward()
        _close(o, ref.detach().numpy(), 1e-12, f"swap SDPA O case {i}")
        _close(dq, tq.grad.numpy(), 1e-11, f"swap SDPA dQ case {i}")
        _close(dk, tk.grad.numpy(), 1e-11, f"swap SDPA dK case {i}")
        _close(dv, tv.grad.numpy(), 1e-11, f"swap SDPA dV case {i}")


def pin_swap_agrees_with_roll_and_split(orc):
    """Where the options coincide.

    S = 0: identical to the main method.  S > 0: unshifted heads, and in shifted
    heads every token outside the wrap group ([G/2, N - G/2)), equal the main
    method; the first G/2 tokens see exactly what they see under the split
    option (the tokens before them), so they equal split; the first token
    attends to itself only (O = V, lse = scale q.k); the last G/2 tokens differ
    from both (they now also see the first G/2).
    """
    B, N, H, Hkv, d, G = 1, 32, 4, 2, 4, 8
    q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=200)
    for S in (0, 2):
        o_r, lse_r = orc.forward(q, k, v, G, S)
        o_w, lse_w = orc.forward(q, k, v, G, S, "swap")
        if S == 0:
            assert np.array_equal(o_r, o_w) and np.array_equal(lse_r, lse_w), "swap changed an unshifted problem"
            for a, b, n in zip(orc.backward(q, k, v, do, G, S), orc.backward(q, k, v, do, G, S, "swap"),
                               ("dQ", "dK", "dV")):
                assert np.array_equal(a, b), f"swap changed {n} of an unshifted problem"
            continue
        o_s, lse_s = orc.forward(q, k, v, G, S, "split")
        h2, half = H - S, G // 2
        _close(o_w[:, :, :h2], o_r[:, :, :h2], 1e-14, "swap: unshifted heads O")
        _close(o_w[:, half:N - half], o_r[:, half:N - half], 1e-13, "swap: tokens outside the wrap group")
        _close(o_w[:, :half, h2:], o_s[:, :half, h2:], 1e-13, "swap: front tokens equal split")
        _close(lse_w[:, h2:, :half], lse_s[:, h2:, :half], 1e-13, "swap: front tokens lse equal split")
        assert np.max(np.abs(o_w[:, N - half:, h2:] - o_r[:, N - half:, h2:])) > 1e-3, \
            "swap did not change the end tokens"
        assert np.max(np.abs(o_w[:, N - half:, h2:] - o_s[:, N - half:, h2:])) > 1e-3, \
            "swap equals split on the end tokens"
        r = H // Hkv
        for h in range(h2, H):
            _close(o_w[0, 0, h], v[0, 0, h // r], 1e-14, f"swap: first token O head {h}")
            _close(lse_w[0, h, 0], np.dot(q[0, 0, h], k[0, 0, h // r]) / np.sqrt(d), 1e-14,
                   f"swap: first token lse head {h}")


def pin_swap_finite_differences(orc):
    B, N, H, Hkv, d, G, S = 1, 16, 2, 1, 3, 8, 1
    q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=210)
    grads = orc.backward(q, k, v, do, G, S, "swap")
    eps = 1e-6
    for pos, name in enumerate(("dQ", "dK", "dV")):
        x = (q, k, v)[pos]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args_p, args_m = [q, k, v], [q, k, v]
            args_p[pos] = x.copy()
            args_p[pos][idx] += eps
            args_m[pos] = x.copy()
            args_m[pos][idx] -= eps
            lp = float(np.sum(orc.forward(*args_p, G, S, "swap")[0] * do))
            lm = float(np.sum(orc.forward(*args_m, G, S, "swap")[0] * do))
            num[idx] = (lp - lm) / (2 * eps)
        err = np.linalg.norm(num - grads[pos]) / np.linalg.norm(num)
        assert err <= 1e-6, f"swap finite differences {name}: rel {err:.2e}"


# ---------------------------------------------------------------------------
# One token's row (used for sampled checks of long groups)
# ---------------------------------------------------------------------------

def pin_row_attention(orc, cases=SMALL_CASES[:4] + [(1, 16, 2, 1, 3, 16, 0)]):
    """row_attention of every token against the brute-force dense attention:
    o, lse and dq per row; dk and dv assembled from the rows' p and ds."""
    for i, (B, N, H, Hkv, d, G, S) in enumerate(cases):
        for wrap in ("roll", "split", "swap"):
            q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=150 + i)
            o_ref, lse_ref, (dq_ref, dk_ref, dv_ref) = dense_masked_attention(
                q, k, v, G, S, grad_do=do, split=wrap == "split", swap=wrap == "swap")
            dk = np.zeros_like(k)
            dv = np.zeros_like(v)
            r = H // Hkv
            for b in range(B):
                for h in range(H):
                    for t in range(N):
                        row = orc.row_attention(q, k, v, do, G, S, b, h, t, wrap)
                        _close(row["o"], o_ref[b, t, h], 1e-12, f"row O case {i} {wrap}")
                        _close(row["lse"], lse_ref[b, h, t], 1e-12, f"row lse case {i} {wrap}")
                        _close(row["dq"], dq_ref[b, t, h], 1e-11, f"row dQ case {i} {wrap}")
                        dv[b, row["keys"], h // r] += row["p"][:, None] * do[b, t, h][None, :]
                        dk[b, row["keys"], h // r] += row["ds"][:, None] * q[b, t, h][None, :] / np.sqrt(d)
            _close(dk, dk_ref, 1e-11, f"rows -> dK case {i} {wrap}")
            _close(dv, dv_ref, 1e-11, f"rows -> dV case {i} {wrap}")


# ---------------------------------------------------------------------------
# Group sizes that do not divide the sequence (Table 7's 1/6 group): the last
# group is short, the shift is floor(G/2)
# ---------------------------------------------------------------------------

UNALIGNED_CASES = [   # (B, N, H, Hkv, d, G, S)
    (1, 30, 2, 2, 4, 8, 1),      # remainder 6
    (1, 21, 2, 1, 3, 7, 2),      # odd G dividing N
    (1, 23, 3, 3, 4, 7, 2),      # odd G, remainder 2
    (1, 13, 2, 2, 3, 13, 1),     # G = N, odd
    (2, 18, 2, 2, 2, 5, 1),      # remainder 3, B = 2
    (1, 9, 2, 2, 3, 1, 2),       # G = 1: every token alone
    (1, 26, 4, 2, 3, 6, 2),      # GQA, remainder 2
]


def pin_unaligned_bruteforce(orc):
    for i, (B, N, H, Hkv, d, G, S) in enumerate(UNALIGNED_CASES):
        for wrap in ("roll", "split", "swap"):
            q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=160 + i)
            o, lse = orc.forward(q, k, v, G, S, wrap)
            dq, dk, dv = orc.backward(q, k, v, do, G, S, wrap)
            o_ref, lse_ref, (dq_ref, dk_ref, dv_ref) = dense_masked_attention(
                q, k, v, G, S, grad_do=do, split=wrap == "split", swap=wrap == "swap")
            _close(o, o_ref, 1e-12, f"unaligned brute-force O case {i} {wrap}")
            _close(lse, lse_ref, 1e-12, f"unaligned brute-force lse case {i} {wrap}")
            _close(dq, dq_ref, 1e-11, f"unaligned brute-force dQ case {i} {wrap}")
            _close(dk, dk_ref, 1e-11, f"unaligned brute-force dK case {i} {wrap}")
            _close(dv, dv_ref, 1e-11, f"unaligned brute-force dV case {i} {wrap}")


def pin_unaligned_row_attention(orc):
    pin_row_attention(orc, cases=[(1, 23, 3, 3, 4, 7, 2), (1, 26, 4, 2, 3, 6, 2)])


def pin_unaligned_swap_gathered_sdpa(orc):
    pin_swap_gathered_sdpa(orc, cases=UNALIGNED_CASES)


def pin_unaligned_cut_sdpa(orc):
    """Roll the shifted heads by floor(G/2), cut the sequence at every multiple
    of G (and, for split, at the wrap), run torch's causal SDPA on every piece,
    roll back; autograd for the gradients."""
    for i, (B, N, H, Hkv, d, G, S) in enumerate(UNALIGNED_CASES):
        for split in (False, True):
            q, k, v, do = rand_problem(B, N, H, Hkv, d, seed=170 + i)
            wrap = "split" if split else "roll"
            o, _ = orc.forward(q, k, v, G, S, wrap)
            dq, dk, dv = orc.backward(q, k, v, do, G, S, wrap)
            r = H // Hkv
            tq = torch.tensor(q, requires_grad=True)
            tk = torch.tensor(k, requires_grad=True)
            tv = torch.tensor(v, requires_grad=True)
            kk = torch.repeat_interleave(tk, r, dim=2)
            vv = torch.repeat_interleave(tv, r, dim=2)
            heads = []
            for h in range(H):
                sh = G // 2 if h >= H - S else 0
                xs = [torch.roll(x[:, :, h], -sh, dims=1) for x in (tq, kk, vv)]
                cuts = set(range(0, N, G)) | {N}
                if split and sh:
                    cuts.add(N - sh)
                cuts = sorted(cuts)
                pieces = [F.scaled_dot_product_attention(xs[0][:, a:e][:, None], xs[1][:, a:e][:, None],
                                                         xs[2][:, a:e][:, None], is_causal=True)[:, 0]
                          for a, e in zip(cuts[:-1], cuts[1:])]
                heads.append(torch.roll(torch.cat(pieces, dim=1), sh, dims=1))
            ref = torch.stack(heads, dim=2)
            (ref * torch.tensor(do)).sum().backward()
            _close(o, ref.detach().numpy(), 1e-12, f"cut/SDPA O case {i} {wrap}")
            _close(dq, tq.grad.numpy(), 1e-11, f"cut/SDPA dQ case {i} {wrap}")
            _close(dk, tk.grad.numpy(), 1e-11, f"cut/SDPA dK case {i} {wrap}")
            _close(dv, tv.grad.numpy(), 1e-11, f"cut/SDPA dV case {i} {wrap}")


# ---------------------------------------------------------------------------
# Rotary position embedding with Position Interpolation (the step before the
# attention on the fine-tuning path)
# ---------------------------------------------------------------------------

def pin_rope_complex(orc):
    """Each pair (i, i + d/2) is the complex number x_i + j x_{i+d/2} multiplied
    by exp(j t), t = n * scale * base^(-2i/d): numpy complex arithmetic."""
    rng = np.random.default_rng(300)
    for (B, N, Hx, d, scale, base) in [(1, 9, 2, 8, 1.0, 10000.0), (2, 17, 3, 16, 0.125, 10000.0),
                                       (1, 5, 1, 4, 0.5, 500.0)]:
        x = rng.standard_normal((B, N, Hx, d))
        half = d // 2
        z = x[..., :half] + 1j * x[..., half:]
        freq = np.array([base ** (-2.0 * i / d) for i in range(half)])
        pos = np.arange(N) * scale
        rot = np.exp(1j * pos[:, None] * freq[None, :])[None, :, None, :]
        w = z * rot
        ref = np.concatenate([w.real, w.imag], axis=-1)
        _close(orc.rope(x, scale, base), ref, 1e-13, f"rope complex d={d}")
        winv = z * np.conj(rot)
        _close(orc.rope(x, scale, base, inverse=True), np.concatenate([winv.real, winv.imag], axis=-1), 1e-13,
               f"rope inverse complex d={d}")


def pin_rope_relative_position(orc):
    """A rotated query and key meet with a score that depends on their positions
    only through the difference (the defining property of rotary embeddings)."""
    rng = np.random.default_rng(301)
    d, N = 16, 64
    qv, kv = rng.standard_normal(d), rng.standard_normal(d)
    X = np.broadcast_to(qv, (1, N, 1, d)).copy()
    Y = np.broadcast_to(kv, (1, N, 1, d)).copy()
    for scale in (1.0, 0.125):
        rq, rk = orc.rope(X, scale)[0, :, 0], orc.rope(Y, scale)[0, :, 0]
        for m, n, t in [(5, 2, 11), (40, 40, 7), (3, 30, 20), (0, 9, 50)]:
            a, b = float(rq[m] @ rk[n]), float(rq[m + t] @ rk[n + t])
            assert abs(a - b) <= 1e-12 * max(1.0, abs(a)), f"rope score moved with the positions ({m},{n})+{t}"
        assert abs(float(rq[7] @ rk[7]) - float(qv @ kv)) <= 1e-12 * max(1.0, abs(float(qv @ kv))), \
            "equal positions must give the unrotated score"


def pin_rope_orthogonal(orc):
    """Position 0 (and scale 0) is the identity; norms are preserved; the inverse
    undoes the rotation and is its transpose: <rope(x), y> = <x, rope_inv(y)>."""
    rng = np.random.default_rng(302)
    x = rng.standard_normal((2, 33, 3, 8))
    y = rng.standard_normal((2, 33, 3, 8))
    r = orc.rope(x, 0.25)
    _close(r[:, 0], x[:, 0], 0.0, "rope at position 0")
    _close(orc.rope(x, 0.0), x, 0.0, "rope with scale 0")
    _close(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), 1e-14, "rope norm")
    _close(orc.rope(r, 0.25, inverse=True), x, 1e-14, "rope inverse")
    assert abs(float(np.sum(r * y)) - float(np.sum(x * orc.rope(y, 0.25, inverse=True)))) <= 1e-11, \
        "the inverse is not the transpose"


ALL_PINS = [
    pin_bruteforce_forward, pin_bruteforce_backward, pin_roll_regroup, pin_full_causal,
    pin_direction_reversal, pin_head_swap, pin_closed_forms, pin_finite_differences,
    pin_gqa_repeat, pin_worked_example_index_map, pin_worked_example_reach,
    pin_split_bruteforce, pin_split_segments_sdpa, pin_split_agrees_with_roll, pin_split_finite_differences,
    pin_swap_bruteforce, pin_swap_gathered_sdpa, pin_swap_agrees_with_roll_and_split, pin_swap_finite_differences,
    pin_row_attention, pin_unaligned_bruteforce, pin_unaligned_cut_sdpa, pin_unaligned_row_attention,
    pin_unaligned_swap_gathered_sdpa, pin_rope_complex, pin_rope_relative_position, pin_rope_orthogonal,
]
