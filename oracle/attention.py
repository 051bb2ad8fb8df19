"""Plain fp64 standard attention on the CPU (test infrastructure, see the package header).

Notation follows the pages: S = scale * Q K^T, P = softmax(S) row by row,
O = P V; m is a row's maximum score, l the sum of exp(S - m) over the row.
The log-sum-exp LSE = m + ln(l) is the single statistic the library returns in
place of the separate (l, m) pair that the [FA-notes] kernel sketch stores.

Everything is computed in float64 from exactly-converted inputs; there is no
tiling, fusion or reordering beyond row-blocking the query rows (rows of
softmax are independent, so a row block is still the standard algorithm).
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import torch

f64 = torch.float64


def _as64(x) -> torch.Tensor:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(f64)
    return torch.as_tensor(x, dtype=f64)


def visible(i: int, j: int, Nq: int, Nk: int, causal: bool) -> bool:
    """Causal visibility of key j from query row i.

    [LLM-basics] ①-7 and ④-4: token i attends to tokens 1..i (itself and the
    past).  The pages only state the square case; for Nq != Nk the rows are
    aligned to the end of the key sequence (bottom-right), so key j is visible
    iff j <= i + (Nk - Nq).  With Nq == Nk this is exactly the pages' rule, and
    for a single decode query it means "every cached key".
    """
    return (not causal) or (j <= i + (Nk - Nq))


def safe_softmax(x) -> torch.Tensor:
    """Softmax along the last axis with the row maximum subtracted first.

    [LLM-basics] ③-1: exp(x_i - m) / sum_j exp(x_j - m) equals the plain
    softmax because the common factor exp(-m) cancels; subtracting the maximum
    keeps every exponent <= 0 so nothing overflows.  [FA-notes] §5.1 shows the
    same three steps (max, exp of the shifted row, divide by the sum).
    Entries equal to -inf (masked) get probability exactly 0.
    """
    x = _as64(x)
    m = torch.amax(x, dim=-1, keepdim=True)
    e = torch.exp(x - m)
    return e / torch.sum(e, dim=-1, keepdim=True)


def _scores(q_rows: torch.Tensor, k: torch.Tensor, scale: float, row0: int, Nq: int,
            causal: bool) -> torch.Tensor:
    """S = scale * Q K^T for query rows [row0, row0 + len) with the causal mask applied.

    [LLM-basics] ①-2 steps 1-2 (dot products, then divide by sqrt(d_k));
    masked entries are set to -inf ([LLM-basics] ④-4: future positions filled
    with negative infinity so softmax gives them exactly zero weight).
    """
    s = (q_rows @ k.transpose(0, 1)) * scale
    if causal:
        Nk = k.shape[0]
        rows = torch.arange(row0, row0 + q_rows.shape[0]).unsqueeze(1)
        cols = torch.arange(Nk).unsqueeze(0)
        s = s.masked_fill(cols > rows + (Nk - Nq), float("-inf"))
    return s


def attention(q, k, v, scale: float, causal: bool, row_block: Optional[int] = None,
              heads: Optional[Sequence[int]] = None,
              rows: Optional[Tuple[int, int]] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Standard attention, materialising S and P per (batch, head).

    q: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d] (any float dtype, converted exactly
    to fp64).  Returns O [B, Nq, Hq, d] and LSE [B, Hq, Nq] in float64.

    Steps, in the order of [LLM-basics] ①-2 and [FA-evo] "표준 Attention 연산 과정":
      1. S = scale * Q K^T (scale is the caller's, 1/sqrt(d) for the workloads);
      2. causal mask (see ``visible``);
      3. m = row max; E = exp(S - m); l = row sum of E; P = E / l  (safe softmax);
      4. O = P V;  LSE = m + ln(l).
    GQA ([LLM-basics] ②-7): Hq/Hkv consecutive query heads share one K/V head,
    kvh = h // (Hq // Hkv).

    ``heads`` restricts the work to some query heads and ``rows`` to a query-row
    range [r0, r1); entries outside are left as NaN.  ``row_block`` bounds the
    memory of S and P by processing that many query rows at a time.
    """
    if not isinstance(q, torch.Tensor):
        q, k, v = _as64(q), _as64(k), _as64(v)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    group = Hq // Hkv
    o = torch.full((B, Nq, Hq, d), float("nan"), dtype=f64)
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=f64)
    r0, r1 = rows if rows is not None else (0, Nq)
    step = row_block or (r1 - r0)
    for b in range(B):
        for h in (heads if heads is not None else range(Hq)):
            kvh = h // group
            kk = _as64(k[b, :, kvh, :])   # fp64 copies of just the slices in use
            vv = _as64(v[b, :, kvh, :])
            for a in range(r0, r1, step):
                e_ = min(a + step, r1)
                s = _scores(_as64(q[b, a:e_, h, :]), kk, scale, a, Nq, causal)
                m = torch.amax(s, dim=1, keepdim=True)
                ex = torch.exp(s - m)
                l = torch.sum(ex, dim=1, keepdim=True)
                p = ex / l
                o[b, a:e_, h, :] = p @ vv
                lse[b, h, a:e_] = (m + torch.log(l)).squeeze(1)
    return o, lse


def attention_probs(q, k, v, scale: float, causal: bool, b: int = 0, h: int = 0) -> torch.Tensor:
    """The probability matrix P [Nq, Nk] of one (batch, head), for invariant checks."""
    q, k = _as64(q), _as64(k)
    Hq, Hkv = q.shape[2], k.shape[2]
    kvh = h // (Hq // Hkv)
    s = _scores(q[b, :, h, :], k[b, :, kvh, :], scale, 0, q.shape[1], causal)
    return safe_softmax(s)


def decode_attention(q, k_cache, v_cache, lengths, scale: float,
                     heads: Optional[Sequence[int]] = None,
                     batches: Optional[Iterable[int]] = None):
    """One decode step: q [B, Hq, d] against the first lengths[b] rows of the cache.

    [LLM-basics] ②-3 / ②-4: the new token's query attends to every cached key
    and value of its sequence (the cache is read whole each step).  It is the
    same standard attention with Nq = 1 and Nk = lengths[b] (all keys visible);
    the cache rows at or beyond lengths[b] are never read.  Returns O [B, Hq, d]
    and LSE [B, Hq] in float64 (NaN where a head or batch was not requested).
    """
    q = _as64(q)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    o = torch.full((B, Hq, d), float("nan"), dtype=f64)
    lse = torch.full((B, Hq), float("nan"), dtype=f64)
    hs = list(heads) if heads is not None else list(range(Hq))
    for b in (batches if batches is not None else range(B)):
        L = int(lengths[b])
        kk = _as64(k_cache[b, :L])          # [L, Hkv, d]
        vv = _as64(v_cache[b, :L])
        oo, ll = attention(q[b].reshape(1, 1, Hq, d), kk.unsqueeze(0), vv.unsqueeze(0), scale,
                           causal=False, heads=hs)
        o[b, hs] = oo[0, 0, hs]
        lse[b, hs] = ll[0, hs, 0]
    return o, lse


def decode_attention_paged(q, k_pages, v_pages, block_table, lengths, page_size: int,
                           scale: float, heads: Optional[Sequence[int]] = None,
                           batches: Optional[Iterable[int]] = None):
    """One decode step over a paged KV cache.

    [LLM-basics] ②-8 (PagedAttention): the cache is kept in fixed-size physical
    blocks ("pages") and a per-sequence block table maps the sequence's logical
    block j -- its keys j*page_size .. (j+1)*page_size - 1 -- to a physical page;
    several sequences may point at the same page.  k_pages and v_pages are
    [num_pages, page_size, Hkv, d]; block_table is [B, max_pages].  The step is
    the decode attention of [LLM-basics] ②-3 / ②-4 over the first lengths[b]
    logical keys, gathered page by page through the table (rows of the last page
    at or beyond the length are never read).  Returns O [B, Hq, d] and LSE [B, Hq]
    in float64 (NaN where a head or batch was not requested).
    """
    q = _as64(q)
    B, Hq, d = q.shape
    o = torch.full((B, Hq, d), float("nan"), dtype=f64)
    lse = torch.full((B, Hq), float("nan"), dtype=f64)
    hs = list(heads) if heads is not None else list(range(Hq))
    for b in (batches if batches is not None else range(B)):
        L = int(lengths[b])
        rows_k, rows_v = [], []
        for j in range((L + page_size - 1) // page_size):
            page = int(block_table[b][j])
            n = min(page_size, L - j * page_size)
            rows_k.append(_as64(k_pages[page, :n]))
            rows_v.append(_as64(v_pages[page, :n]))
        kk = torch.cat(rows_k, dim=0)  # [L, Hkv, d]
        vv = torch.cat(rows_v, dim=0)
        oo, ll = attention(q[b].reshape(1, 1, Hq, d), kk.unsqueeze(0), vv.unsqueeze(0), scale,
                           causal=False, heads=hs)
        o[b, hs] = oo[0, 0, hs]
        lse[b, hs] = ll[0, hs, 0]
    return o, lse


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool,
                     heads: Optional[Sequence[int]] = None):
    """Attention over a batch of variable-length sequences packed along the token axis.

    [FA3-entry] §2 lists variable-length inputs among the supported attention forms;
    [FA-evo] "실전 구현" shows the per-batch [B, S, H, D] layout this packs.  q is
    [total_q, Hq, d] and k, v are [total_k, Hkv, d]; sequence b owns query rows
    cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 and key rows cu_seqlens_k[b] ..
    cu_seqlens_k[b+1] - 1, and attends only within itself: each sequence is the
    standard attention of ``attention`` (causal alignment per sequence, bottom-right).
    Returns O [total_q, Hq, d] and LSE [Hq, total_q] in float64.  A sequence with no
    keys has no softmax to take (the row max and the normaliser of [LLM-basics] ③-1
    are over an empty set): its rows are left NaN, as are causal rows that see no key.
    """
    total_q, Hq, d = q.shape
    o = torch.full((total_q, Hq, d), float("nan"), dtype=f64)
    lse = torch.full((Hq, total_q), float("nan"), dtype=f64)
    B = len(cu_seqlens_q) - 1
    for b in range(B):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        if q1 == q0 or k1 == k0:
            continue
        ob, lb = attention(q[q0:q1].unsqueeze(0), k[k0:k1].unsqueeze(0), v[k0:k1].unsqueeze(0),
                           scale, causal, heads=heads)
        o[q0:q1] = ob[0]
        lse[:, q0:q1] = lb[0]
    return o, lse


def attention_backward(q, k, v, do, scale: float, causal: bool,
                       kv_heads: Optional[Sequence[int]] = None,
                       rows: Optional[Tuple[int, int]] = None,
                       keys: Optional[Tuple[int, int]] = None,
                       row_block: Optional[int] = None):
    """Gradients of standard attention: dQ, dK, dV for an upstream gradient dO.

    [FA-notes] §5.2 sketches the backward pass: P is rebuilt from Q, K and the
    forward's softmax statistics, then dV = P^T dO and dP = dO V^T, the remaining
    steps being elided; [LLM-basics] ③-5 names the same recomputation for training.
    The steps after dP are the derivative of the row softmax (the Jacobian of
    p = softmax(s) is diag(p) - p p^T), written out per row i:
        D_i   = sum_j P_ij dP_ij
        dS_ij = P_ij (dP_ij - D_i)
        dQ    = scale * dS K,    dK = scale * dS^T Q,    dV = P^T dO.
    Here P is recomputed from scratch (the standard attention of ``attention``,
    causal mask included), so this function needs no forward output.  GQA: the
    dK and dV of a K/V head add up the contributions of its Hq/Hkv query heads.

    q, do: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d].  Returns (dq [B, Nq, Hq, d],
    dk, dv [B, Nk, Hkv, d]) in float64.  ``kv_heads`` restricts the work to some
    K/V heads (and their query heads), ``rows`` the dQ rows returned, ``keys`` the
    dK/dV keys returned (an empty key range skips dK/dV, and then only the rows
    asked for are visited; an empty row range skips dQ, and under the causal mask the
    rows that cannot see the keys asked for are then skipped); entries not computed
    are NaN.  ``row_block`` bounds
    memory by visiting that many query rows at a time (rows are independent, and
    dK, dV are sums over rows).
    """
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    group = Hq // Hkv
    dq = torch.full((B, Nq, Hq, d), float("nan"), dtype=f64)
    dk = torch.full((B, Nk, Hkv, d), float("nan"), dtype=f64)
    dv = torch.full((B, Nk, Hkv, d), float("nan"), dtype=f64)
    r0, r1 = rows if rows is not None else (0, Nq)
    k0, k1 = keys if keys is not None else (0, Nk)
    want_kv = k1 > k0
    a0, a1 = (0, Nq) if want_kv else (r0, r1)
    if want_kv and causal and r1 <= r0:
        # no dQ asked for: rows before k0 - (Nk - Nq) see none of the keys asked for (their
        # P and dS columns there are exactly 0), so they add nothing to dK and dV
        a0 = min(max(0, k0 - (Nk - Nq)), Nq)
    step = row_block or max(a1 - a0, 1)
    for b in range(B):
        for kvh in (kv_heads if kv_heads is not None else range(Hkv)):
            kk = _as64(k[b, :, kvh, :])
            vv = _as64(v[b, :, kvh, :])
            dk_acc = torch.zeros((k1 - k0, d), dtype=f64)
            dv_acc = torch.zeros((k1 - k0, d), dtype=f64)
            for h in range(kvh * group, (kvh + 1) * group):
                for a in range(a0, a1, step):
                    e_ = min(a + step, a1)
                    qq = _as64(q[b, a:e_, h, :])
                    dd = _as64(do[b, a:e_, h, :])
                    s = _scores(qq, kk, scale, a, Nq, causal)
                    m = torch.amax(s, dim=1, keepdim=True)
                    ex = torch.exp(s - m)
                    p = ex / torch.sum(ex, dim=1, keepdim=True)        # P
                    dp = dd @ vv.transpose(0, 1)                       # dP = dO V^T
                    dsum = torch.sum(p * dp, dim=1, keepdim=True)      # D
                    ds = p * (dp - dsum)                               # dS
                    lo, hi = max(a, r0), min(e_, r1)
                    if lo < hi:
                        dq[b, lo:hi, h, :] = scale * (ds[lo - a:hi - a] @ kk)
                    if want_kv:
                        dv_acc += p[:, k0:k1].transpose(0, 1) @ dd
                        dk_acc += scale * (ds[:, k0:k1].transpose(0, 1) @ qq)
            if want_kv:
                dk[b, k0:k1, kvh, :] = dk_acc
                dv[b, k0:k1, kvh, :] = dv_acc
    return dq, dk, dv


def block_state(s_block: torch.Tensor, v_block: torch.Tensor):
    """The softmax state of one block of keys taken on its own, per row.

    A state is the triple (m, l, acc) of [FA-notes] §4: m the largest score of the
    row in the block, l = sum_j exp(s_j - m) and acc = sum_j exp(s_j - m) V_j (the
    output before division by l).  Rows are the leading axis of ``s_block``.
    """
    s_block = _as64(s_block)
    m = torch.amax(s_block, dim=-1)
    w = torch.exp(s_block - m.unsqueeze(-1))
    return m, torch.sum(w, dim=-1), w @ _as64(v_block)


def merge_states(first, second):
    """Combine the softmax states of two disjoint key blocks of the same rows.

    [FA-notes] §4 and [LLM-basics] ③-2: with the larger of the two maxima as the
    common reference, m = max(m1, m2), each block's sum is brought to that
    reference by the factor e^(m_i - m) and the two are added,
        l = e^(m1 - m) l1 + e^(m2 - m) l2;
    the unnormalised outputs take the same factors ([FA-notes] §5.2 rescales its
    output accumulator the same way),
        acc = e^(m1 - m) acc1 + e^(m2 - m) acc2.
    The merge is symmetric in its two arguments.
    """
    m1, l1, acc1 = first
    m2, l2, acc2 = second
    m = torch.maximum(m1, m2)
    f1 = torch.exp(m1 - m)
    f2 = torch.exp(m2 - m)
    return m, f1 * l1 + f2 * l2, f1.unsqueeze(-1) * acc1 + f2.unsqueeze(-1) * acc2


def online_attention_rows(s: torch.Tensor, v: torch.Tensor, block_edges: List[int]):
    """Attention of score rows s [R, N] with values v [N, dv], consuming the keys in the
    contiguous blocks [e0, e1), [e1, e2), ... given by ``block_edges`` (e0 = 0,
    last = N): the state of the keys seen so far is merged with each new block's
    state (``merge_states``), and the final output is acc / l ([FA-notes] §5.2:
    P = exp(S - m) / l).  Returns (O, LSE) with LSE = m + ln l.
    """
    s, v = _as64(s), _as64(v)
    blocks = list(zip(block_edges[:-1], block_edges[1:]))
    state = block_state(s[:, blocks[0][0]:blocks[0][1]], v[blocks[0][0]:blocks[0][1]])
    for a, e in blocks[1:]:
        state = merge_states(state, block_state(s[:, a:e], v[a:e]))
    m, l, acc = state
    return acc / l.unsqueeze(-1), m + torch.log(l)


def lse_merge(o_parts, lse_parts) -> Tuple[torch.Tensor, torch.Tensor]:
    """Combine per-chunk normalised outputs O_c and log-sum-exps lse_c of one row.

    This is the [FA-notes] §4 two-block merge applied to any number of blocks,
    written with LSE in place of (m, l): each chunk's l_c = e^(lse_c - M) up to
    the common factor e^M with M = max_c lse_c, so
        LSE = M + ln sum_c e^(lse_c - M),   O = sum_c e^(lse_c - LSE) O_c.
    o_parts: [C, ..., dv]; lse_parts: [C, ...].
    """
    o_parts, lse_parts = _as64(o_parts), _as64(lse_parts)
    M = torch.amax(lse_parts, dim=0)
    w = torch.exp(lse_parts - M)
    lse = M + torch.log(torch.sum(w, dim=0))
    wn = torch.exp(lse_parts - lse)
    o = torch.sum(wn.unsqueeze(-1) * o_parts, dim=0)
    return o, lse
