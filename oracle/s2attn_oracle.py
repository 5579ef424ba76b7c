"""Plain float64 CPU oracle for Shifted Sparse Attention (S2-Attn), forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module.  The GPU library never imports, links or calls it, and it shares no
code with the GPU library: it imports NumPy and nothing else.

What it computes (page "LongLoRA: Efficient Fine-tuning of Long-Context Large
Language Models", paper-graph-ui summary, section 3.4):

* "The core computational problem": attention is o = softmax(q k^T) v on each
  head, under the causal mask of a causal language model.  The page drops the
  softmax scale; this oracle uses 1/sqrt(d) (the scale the 7B workload states).
* "The solution: group tokens and compute attention locally": the N tokens are
  cut into N/G groups of G consecutive tokens and attention runs inside each
  group only.
* "The shifting mechanism", Steps 1-3 and Figure 3, and "Algorithmic
  implementation" (Algorithm 1): the second chunk of heads has its tokens rolled
  cyclically by G/2 along the sequence before grouping (a torch.roll by -G/2:
  rolled position j holds original token (j + G/2) mod N), attention runs per
  group in that rolled order, and the output is rolled back by +G/2.  Here the
  "second chunk" is the last ``shift_heads`` heads (half of them by default).
  Causality is applied in the rolled frame, exactly as a causal attention call
  on the rolled groups would (section "Information leakage considerations"
  keeps that wrap-around in the main method).
* Wrap-group option ``wrap="split"`` (section 5, "Ablation Studies and
  Robustness Checks", Table 8 and Figure 6, Variant 2; section 3.4,
  "Information leakage considerations"): the tokens that the roll carries from
  the front of the sequence to its end form a group of their own instead of
  sharing the last rolled group with the last G/2 tokens.  Reading taken here:
  in a shifted head the rolled group that wraps from the end of the sequence
  to its start (the last one: the last G/2 tokens, then the first G/2) is cut
  at the wrap into two causal groups; every other group, and every unshifted
  head, is as in the main method (``wrap="roll"``).
* Wrap-group option ``wrap="swap"`` (the same Table 8, Variant 3: the shifted
  tokens swap places with the original front tokens).  Reading taken here: in
  a shifted head the rolled group that wraps keeps its tokens, but the part the
  roll carried from the front of the sequence (tokens 0, 1, ...) is placed
  before the part from the end, so that inside every group causal order is the
  original token order; every other group, and every unshifted head, is as in
  the main method.
* Group sizes that do not divide the sequence (section 5, "Ablation Studies
  and Robustness Checks", Table 7: a 1/6 group, 1365 tokens, at context 8192;
  Algorithm 1's reshape needs N to be a multiple of G there, and the pages do
  not say what was done).  Reading taken here: the (rolled) sequence is cut
  into consecutive groups of G tokens and the last group holds the N mod G
  tokens that remain; the shift is floor(G/2) tokens when G is odd.  Aligned
  shapes (N a multiple of an even G) are unchanged by this reading.
* Grouped-query attention (several query heads sharing one key/value head) is
  not on the pages; query head h reads key/value head h // (H // Hkv) and the
  key/value gradients are summed over the query heads that share them.

The backward pass is the textbook gradient of that function (the pages only say
gradients flow through the attention during fine-tuning, section 3.2 Phase 1
step 5):  P = exp(S - lse), dV = P^T dO, dP = dO V^T, Dvec = rowsum(dO * O),
dS = P * (dP - Dvec), dQ = scale dS K, dK = scale dS^T Q.

Evaluation order: one (batch, head, group) slice at a time; inside a group the
query rows are taken in chunks (rows are independent in softmax), each chunk
against the keys up to its last row (later keys are masked for every row of the
chunk and would add exact zeros).  Nothing else is blocked or reordered.

Pins (all in ``tests/test_oracle.py``): brute-force masked attention written in
original token coordinates, a roll/regroup/causal-SDPA formulation, full causal
attention at G = N without shift, exact invariance under reversing the roll
direction, head-swap equivariance, closed forms (first row of each group),
finite differences, GQA against repeated-KV MHA, and the worked index example
of "The shifting mechanism"; ``row_attention`` against the brute-force
attention row by row.  The split wrap option is pinned by the same
brute-force mask with the split partition, by causal SDPA over each split group
as a contiguous token range, by finite differences, and by its agreement with
the main method wherever the two partitions coincide.  The swap option is
pinned by the brute-force mask of the same partition with original-order
causality, by causal SDPA over each group gathered in token order, by finite
differences, and by its agreement with the main method and the split option
where they coincide.
"""

import numpy as np

WRAPS = ("roll", "split", "swap")

__all__ = [
    "WRAPS", "check_problem", "num_groups", "head_shift", "kv_head", "rolled_order", "group_order", "group_parts",
    "group_forward", "group_backward",
    "forward", "backward",
    "head_group_forward", "head_group_backward", "row_attention", "rope",
]


def check_problem(B, N, H, Hkv, d, G, shift_heads, wrap="roll"):
    """Reject problems the method does not define.

    Grouping cuts the sequence into groups of G tokens (Algorithm 1's reshape to
    [B*N/G, G, ...]; a last, shorter group when G does not divide N), so G must
    lie in [1, N].  ``wrap`` is "roll" (the main method), "split" or "swap".
    """
    if wrap not in WRAPS:
        raise ValueError(f"wrap must be one of {WRAPS}, got {wrap!r}")
    for name, val in (("B", B), ("N", N), ("H", H), ("Hkv", Hkv), ("d", d), ("G", G)):
        if val <= 0:
            raise ValueError(f"{name} must be positive, got {val}")
    if G > N:
        raise ValueError(f"the group size G={G} exceeds the sequence length N={N}")
    if not 0 <= shift_heads <= H:
        raise ValueError(f"shift_heads={shift_heads} must lie in [0, H={H}]")
    if H % Hkv:
        raise ValueError(f"H={H} is not a multiple of Hkv={Hkv}")


def num_groups(N, G):
    """Groups of one head: N/G rounded up (the last one may be shorter)."""
    return (N + G - 1) // G


def head_shift(h, H, shift_heads, G):
    """Roll amount of head h: G/2 for the last ``shift_heads`` heads, else 0.

    Step 1-2 of "The shifting mechanism": the heads are split in two chunks and
    only the second chunk is shifted by half a group.
    """
    return G // 2 if h >= H - shift_heads else 0


def kv_head(h, H, Hkv):
    """Key/value head read by query head h (consecutive query heads share one)."""
    return h // (H // Hkv)


def rolled_order(N, sigma):
    """Original token index held at each rolled position.

    Rolling a sequence by -sigma puts original token (j + sigma) mod N at
    position j (the first key line of Algorithm 1 with sigma = G/2).
    """
    return (np.arange(N) + sigma) % N


def _wrap_cut(rows):
    """Index in ``rows`` (a rolled group, original token indices) of the first
    token after the wrap from the end of the sequence to its start, or None."""
    wraps = np.nonzero(np.diff(rows) < 0)[0]
    return int(wraps[0]) + 1 if len(wraps) else None


def group_order(rows, sigma, wrap):
    """The order in which the tokens of one rolled group attend causally.

    Rolled order, except under ``wrap="swap"`` for the group of a shifted head
    in which the rolled order wraps: there the tokens after the wrap (carried
    from the front of the sequence) are moved before the tokens of the end.
    """
    if wrap == "swap" and sigma:
        cut = _wrap_cut(rows)
        if cut is not None:
            return np.concatenate([rows[cut:], rows[:cut]])
    return rows


def group_parts(rows, sigma, wrap):
    """The causal groups that one rolled group (original rows ``rows``, in
    rolled order) is made of.

    One group, except under ``wrap="split"`` for the group of a shifted head in
    which the rolled order wraps from the last token of the sequence to the
    first: it is cut at the wrap, so the tokens the roll carried from the front
    form a group apart from the tokens of the end.  Returns consecutive slices
    of ``rows`` that cover it.
    """
    if wrap == "split" and sigma:
        cut = _wrap_cut(rows)
        if cut is not None:
            return [slice(0, cut), slice(cut, len(rows))]
    return [slice(0, len(rows))]


def group_forward(Qg, Kg, Vg, scale, chunk=1024):
    """Causal softmax attention of one group, rows already in rolled order.

    Returns (O [G, d], lse [G]) with lse the natural-log normaliser of each row.
    """
    G = Qg.shape[0]
    O = np.empty((G, Vg.shape[1]), dtype=np.float64)
    lse = np.empty(G, dtype=np.float64)
    for r0 in range(0, G, chunk):
        r1 = min(G, r0 + chunk)
        S = scale * (Qg[r0:r1] @ Kg[:r1].T)
        allowed = np.arange(r1)[None, :] <= np.arange(r0, r1)[:, None]
        S = np.where(allowed, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        P = np.exp(S - m)
        l = P.sum(axis=1, keepdims=True)
        O[r0:r1] = (P / l) @ Vg[:r1]
        lse[r0:r1] = (m + np.log(l))[:, 0]
    return O, lse


def group_backward(Qg, Kg, Vg, Og, lseg, dOg, scale, chunk=1024):
    """Gradients of one group's causal attention given its output and lse.

    Returns (dQ [G, d], dK [G, d], dV [G, d]) for the group's rows in rolled order.
    """
    G = Qg.shape[0]
    Dvec = np.sum(dOg * Og, axis=1)
    dQ = np.empty_like(Qg, dtype=np.float64)
    dK = np.zeros_like(Kg, dtype=np.float64)
    dV = np.zeros_like(Vg, dtype=np.float64)
    for r0 in range(0, G, chunk):
        r1 = min(G, r0 + chunk)
        S = scale * (Qg[r0:r1] @ Kg[:r1].T)
        allowed = np.arange(r1)[None, :] <= np.arange(r0, r1)[:, None]
        P = np.where(allowed, np.exp(S - lseg[r0:r1, None]), 0.0)
        dV[:r1] += P.T @ dOg[r0:r1]
        dP = dOg[r0:r1] @ Vg[:r1].T
        dS = P * (dP - Dvec[r0:r1, None])
        dQ[r0:r1] = scale * (dS @ Kg[:r1])
        dK[:r1] += scale * (dS.T @ Qg[r0:r1])
    return dQ, dK, dV


def _dims(q, k, v, G, shift_heads, wrap="roll"):
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, N, Hkv, d) or v.shape != (B, N, Hkv, d):
        raise ValueError(f"k {k.shape} / v {v.shape} do not match q {q.shape}")
    check_problem(B, N, H, Hkv, d, G, shift_heads, wrap)
    return B, N, H, Hkv, d


def head_group_forward(q, k, v, G, shift_heads, b, h, g, wrap="roll"):
    """Forward of one (batch b, query head h, group g of h's rolled frame).

    Returns (rows, O, lse): ``rows`` are the original token indices of the group
    in the order its causal attention runs (rolled order; see ``group_order``);
    O[i] and lse[i] belong to original token rows[i].
    """
    B, N, H, Hkv, d = _dims(q, k, v, G, shift_heads, wrap)
    sigma = head_shift(h, H, shift_heads, G)
    rows = group_order(rolled_order(N, sigma)[g * G:(g + 1) * G], sigma, wrap)
    c = kv_head(h, H, Hkv)
    O = np.empty((len(rows), d), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    for part in group_parts(rows, sigma, wrap):
        pr = rows[part]
        Qg = np.asarray(q[b, pr, h], dtype=np.float64)
        Kg = np.asarray(k[b, pr, c], dtype=np.float64)
        Vg = np.asarray(v[b, pr, c], dtype=np.float64)
        O[part], lse[part] = group_forward(Qg, Kg, Vg, 1.0 / np.sqrt(d))
    return rows, O, lse


def head_group_backward(q, k, v, do, G, shift_heads, b, h, g, wrap="roll"):
    """Backward of one (b, h, g) slice.

    Returns (rows, dQ, dK_part, dV_part): dQ is complete for those rows (a query
    only sees its own group); dK_part / dV_part are head h's contribution to the
    gradients of key/value head kv_head(h) at the same original rows.
    """
    B, N, H, Hkv, d = _dims(q, k, v, G, shift_heads, wrap)
    sigma = head_shift(h, H, shift_heads, G)
    rows = group_order(rolled_order(N, sigma)[g * G:(g + 1) * G], sigma, wrap)
    c = kv_head(h, H, Hkv)
    scale = 1.0 / np.sqrt(d)
    dQ = np.empty((len(rows), d), dtype=np.float64)
    dK = np.empty((len(rows), d), dtype=np.float64)
    dV = np.empty((len(rows), d), dtype=np.float64)
    for part in group_parts(rows, sigma, wrap):
        pr = rows[part]
        Qg = np.asarray(q[b, pr, h], dtype=np.float64)
        Kg = np.asarray(k[b, pr, c], dtype=np.float64)
        Vg = np.asarray(v[b, pr, c], dtype=np.float64)
        dOg = np.asarray(do[b, pr, h], dtype=np.float64)
        O, lse = group_forward(Qg, Kg, Vg, scale)
        dQ[part], dK[part], dV[part] = group_backward(Qg, Kg, Vg, O, lse, dOg, scale)
    return rows, dQ, dK, dV


def row_attention(q, k, v, do, G, shift_heads, b, h, t, wrap="roll"):
    """Everything about one query token t of head h, from its own row only.

    The keys token t attends to are the tokens of its causal group that come at
    or before it in the group's causal order (``group_order``).  Returns a dict: ``keys`` (their
    original indices, in that order), ``o`` and ``lse`` of token t, the row of
    attention weights ``p`` and of score gradients ``ds`` over ``keys`` (for L =
    sum(o * do)), and ``dq`` of token t.  Key/value gradients of key u are then
    sums over the tokens whose ``keys`` contain u (p * do for dv, scale * ds * q
    for dk), which is how long groups are checked a few rows at a time.
    """
    B, N, H, Hkv, d = _dims(q, k, v, G, shift_heads, wrap)
    sigma = head_shift(h, H, shift_heads, G)
    order = rolled_order(N, sigma)
    g = int(np.nonzero(order == t)[0][0]) // G   # group of token t
    rows = group_order(order[g * G:(g + 1) * G], sigma, wrap)
    pos = int(np.nonzero(rows == t)[0][0])       # its place in the group's causal order
    part = next(pt for pt in group_parts(rows, sigma, wrap) if pt.start <= pos < pt.stop)
    keys = rows[part.start:pos + 1]
    c = kv_head(h, H, Hkv)
    scale = 1.0 / np.sqrt(d)
    qt = np.asarray(q[b, t, h], dtype=np.float64)
    dot = np.asarray(do[b, t, h], dtype=np.float64)
    Kr = np.asarray(k[b, keys, c], dtype=np.float64)
    Vr = np.asarray(v[b, keys, c], dtype=np.float64)
    s = scale * (Kr @ qt)
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    p = e / l
    o = p @ Vr
    dp = Vr @ dot
    ds = p * (dp - np.dot(dot, o))
    return {"keys": keys, "o": o, "lse": m + np.log(l), "p": p, "ds": ds, "dq": scale * (ds @ Kr)}


def forward(q, k, v, G, shift_heads, wrap="roll"):
    """S2-Attn forward.

    q [B, N, H, d], k and v [B, N, Hkv, d] (any float dtype; computed in float64).
    Returns o [B, N, H, d] and lse [B, H, N] (natural log), both in original
    token order: writing each group's rows back through ``rows`` is the roll-back
    (Step 2, last sentence; Algorithm 1's second key line).
    """
    B, N, H, Hkv, d = _dims(q, k, v, G, shift_heads, wrap)
    o = np.empty((B, N, H, d), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for g in range(num_groups(N, G)):
                rows, Og, lseg = head_group_forward(q, k, v, G, shift_heads, b, h, g, wrap)
                o[b, rows, h] = Og
                lse[b, h, rows] = lseg
    return o, lse


def backward(q, k, v, do, G, shift_heads, wrap="roll"):
    """S2-Attn backward: (dq, dk, dv) of L = sum(o * do), float64.

    dk and dv sum the contributions of every query head that reads them.
    """
    B, N, H, Hkv, d = _dims(q, k, v, G, shift_heads, wrap)
    dq = np.empty((B, N, H, d), dtype=np.float64)
    dk = np.zeros((B, N, Hkv, d), dtype=np.float64)
    dv = np.zeros((B, N, Hkv, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            c = kv_head(h, H, Hkv)
            for g in range(num_groups(N, G)):
                rows, dQg, dKg, dVg = head_group_backward(q, k, v, do, G, shift_heads, b, h, g, wrap)
                dq[b, rows, h] = dQg
                dk[b, rows, c] += dKg
                dv[b, rows, c] += dVg
    return dq, dk, dv


def rope(x, pos_scale=1.0, base=10000.0, inverse=False):
    """Rotary position embedding with Position Interpolation, on q or k.

    The step before the attention on the pages' fine-tuning path (page
    "LongLoRA: Efficient Fine-tuning of Long-Context Large Language Models",
    section 3.2 Phase 1 item 2, and "Training Procedure, Hyperparameters, and
    Dataset Configuration", "Model setup"): the rotary position embeddings of
    the pre-trained model are rescaled by Position Interpolation so that the
    extended context maps into the original position range.  The pages give
    neither formula; the readings taken here are the published definitions:
    rotary embedding (RoFormer) in the rotate-half pairing of Llama models,
    dimension i paired with i + d/2, frequencies base^(-2i/d) with base 10000;
    Position Interpolation multiplies every position by pos_scale = original
    context / target context (4096 / 32768 for the 7B model at 32k).

    x [B, N, heads, d] (any float dtype; computed in float64), token n at
    position n.  With angle t = n * pos_scale * base^(-2i/d):
        y_i       = x_i cos t - x_{i+d/2} sin t
        y_{i+d/2} = x_{i+d/2} cos t + x_i sin t
    ``inverse`` rotates by -t: the transpose, which maps gradients of the
    rotated tensor back to gradients of x.
    """
    x = np.asarray(x, dtype=np.float64)
    B, N, Hx, d = x.shape
    if d % 2:
        raise ValueError(f"the head dimension must be even, got {d}")
    half = d // 2
    inv_freq = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    t = (np.arange(N, dtype=np.float64) * pos_scale)[:, None] * inv_freq[None, :]   # [N, d/2]
    c = np.cos(t)[None, :, None, :]
    s = np.sin(t)[None, :, None, :]
    if inverse:
        s = -s
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
