"""Pins of the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes an oracle-like module (the real ``oracle`` or a
copy with a planted mistake) and raises AssertionError when the module
disagrees with what the pages or the mathematics fix.  ``test_oracle.py`` runs
them on the real oracle; ``test_oracle_mutants.py`` runs them on mutated copies
and requires every planted mistake to be caught by at least one pin.

Page titles (cited by section below):
  [FA-notes]   "flash-attn" notes, minjae-portfolio.vercel.app/notes/flash-attn
  [LLM-basics] "LLM 기초 — Attention부터 FlashAttention까지", gylee815.github.io/llmso/w1
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
f64 = torch.float64


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, tol, what=""):
    a = torch.as_tensor(a, dtype=f64)
    b = torch.as_tensor(b, dtype=f64)
    err = (a - b).abs().max().item() if a.numel() else 0.0
    assert a.shape == b.shape, f"{what}: shape {tuple(a.shape)} vs {tuple(b.shape)}"
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _rand(shape, seed, scale=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=f64) * scale


def _example_tensors():
    ex = _golden("worked_example.json")
    q = torch.tensor(ex["query"], dtype=f64).reshape(1, 1, 1, 2)
    k = torch.tensor(ex["keys"], dtype=f64).reshape(1, 3, 1, 2)
    v = torch.tensor(ex["values"], dtype=f64).reshape(1, 3, 1, 2)
    return ex, q, k, v


# ---------------------------------------------------------------------------
# the pages' worked numbers
# ---------------------------------------------------------------------------

def pin_worked_example_printed(orc):
    """[LLM-basics] ①-2 worked example: the page's printed numbers, at the page's rounding."""
    ex, q, k, v = _example_tensors()
    scale = 1.0 / math.sqrt(ex["d_k"])
    o, lse = orc.attention(q, k, v, scale, causal=False)
    p = orc.attention_probs(q, k, v, scale, causal=False)[0]
    pr, dec = ex["printed"], ex["printed_decimals"]

    def at(x, key):
        _close(x, pr[key], 0.5 * 10 ** (-dec[key]) + 1e-12, f"worked example {key}")

    # scaled scores: LSE - ln p_j recovers s_j for every key (s_j = LSE + ln P_j)
    s = lse[0, 0, 0] + torch.log(p)
    at(s, "scaled_scores")
    at(s * math.sqrt(ex["d_k"]), "raw_scores")
    at(torch.exp(s), "exp_scaled")
    at(torch.exp(lse[0, 0, 0]), "exp_sum")   # sum_j e^{s_j} since no shift is needed here
    at(p, "softmax")
    at(o[0, 0, 0], "output")


def pin_worked_example_closed_form(orc):
    """Same example, exact: with a = e^{1/sqrt 2}, P = [a, 1, a]/(2a+1),
    O = [2a, a + 2]/(2a+1), LSE = ln(2a+1)."""
    ex, q, k, v = _example_tensors()
    a = math.exp(1.0 / math.sqrt(2.0))
    den = 2 * a + 1
    o, lse = orc.attention(q, k, v, 1.0 / math.sqrt(2.0), causal=False)
    p = orc.attention_probs(q, k, v, 1.0 / math.sqrt(2.0), causal=False)[0]
    _close(p, [a / den, 1 / den, a / den], 1e-15, "closed-form P")
    _close(o[0, 0, 0], [2 * a / den, (a + 2) / den], 1e-15, "closed-form O")
    _close(lse[0, 0, 0], math.log(den), 1e-15, "closed-form LSE")


def pin_softmax_examples(orc):
    """[LLM-basics] ①-3: softmax([1,2]) ~ [0.27, 0.73], softmax([10,20]) ~ [0.00005, 0.99995];
    exactly [1, e]/(1+e) and [1, e^10]/(1+e^10)."""
    g = _golden("softmax_examples.json")
    for case in g["cases"]:
        got = orc.safe_softmax(torch.tensor(case["x"], dtype=f64))
        _close(got, case["printed"], 0.5 * 10 ** (-case["decimals"]) + 1e-12, f"softmax {case['x']}")
        d = case["x"][1] - case["x"][0]
        exact = [1 / (1 + math.exp(d)), math.exp(d) / (1 + math.exp(d))]
        _close(got, exact, 1e-15, f"softmax closed form {case['x']}")


def pin_overflow(orc):
    """[LLM-basics] ③-1: exp overflows fp16 near x = 11.1 and fp32 near x = 88.7 (page's
    table), and a score of 100 already overflows fp32; the safe (max-subtracted)
    softmax stays finite and exact.  In fp64 the same holds at 1000 > ln(DBL_MAX)."""
    g = _golden("overflow_thresholds.json")
    for row in g["rows"]:
        fmax = float(np.finfo(getattr(np, row["dtype"])).max)
        assert abs(fmax - row["max_printed"]) <= 0.01 * row["max_printed"]
        assert round(math.log(fmax), row["x_decimals"]) == row["overflow_x_printed"]
    with np.errstate(over="ignore"):
        assert np.isinf(np.exp(np.float32(g["example_score"])))
    for big in (g["example_score"], 1000.0):
        x = torch.tensor([big, big - 1.0, 0.0], dtype=f64)
        got = orc.safe_softmax(x)
        assert torch.isfinite(got).all(), f"safe softmax not finite at {big}"
        e1 = math.exp(-1.0)
        den = 1 + e1 + math.exp(-big)
        _close(got, [1 / den, e1 / den, math.exp(-big) / den], 1e-15, f"softmax at {big}")
    # attention whose scores reach ~1000: finite, LSE = max score + ln(sum of shifted exps)
    q = torch.tensor([[[[10.0, 0.0]]]], dtype=f64)
    k = torch.tensor([[[[100.0, 0.0]], [[99.9, 0.0]]]], dtype=f64)
    v = torch.tensor([[[[1.0, -1.0]], [[3.0, 5.0]]]], dtype=f64)
    o, lse = orc.attention(q, k, v, 1.0, causal=False)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    w = math.exp(-1.0)
    _close(lse[0, 0, 0], 1000.0 + math.log(1 + w), 1e-12, "LSE at score 1000")
    _close(o[0, 0, 0], [(1 + 3 * w) / (1 + w), (-1 + 5 * w) / (1 + w)], 1e-14, "O at score 1000")


def pin_causal_visibility(orc):
    """[LLM-basics] ①-7 / ④-4: with five tokens, token n (1-based) sees tokens 1..n."""
    g = _golden("causal_visibility.json")
    n = g["tokens"]
    for i in range(n):
        seen = [j + 1 for j in range(n) if orc.visible(i, j, n, n, True)]
        assert seen == g["visible_1based"][str(i + 1)], f"row {i + 1}: {seen}"
    # the same through the probability matrix: masked weights are exactly zero
    q, k, v = _rand((1, n, 1, 4), 1), _rand((1, n, 1, 4), 2), _rand((1, n, 1, 4), 3)
    p = orc.attention_probs(q, k, v, 0.5, causal=True)
    for i in range(n):
        vis = [j + 1 for j in range(n) if p[i, j] > 0]
        assert vis == g["visible_1based"][str(i + 1)], f"P row {i + 1}: {vis}"


# ---------------------------------------------------------------------------
# invariants that hold at any size
# ---------------------------------------------------------------------------

_SHAPES = [  # B, Nq, Nk, Hq, Hkv, d, causal
    (1, 37, 37, 2, 2, 8, True),
    (2, 19, 45, 4, 2, 16, True),
    (1, 23, 31, 3, 1, 8, False),
]


def _qkv(shape, seed, gain=1.0):
    B, Nq, Nk, Hq, Hkv, d, _ = shape
    return (_rand((B, Nq, Hq, d), seed, gain), _rand((B, Nk, Hkv, d), seed + 1, gain),
            _rand((B, Nk, Hkv, d), seed + 2))


def pin_rows_sum_to_one(orc):
    """Every row of P is a probability distribution ([LLM-basics] ①-2 step 3, ③-1)."""
    for t, shape in enumerate(_SHAPES):
        q, k, v = _qkv(shape, 10 * t)
        for h in range(shape[3]):
            p = orc.attention_probs(q, k, v, 0.3, shape[6], b=0, h=h)
            assert (p >= 0).all()
            _close(p.sum(dim=1), torch.ones(p.shape[0], dtype=f64), 1e-12, "row sums")


def pin_constant_v(orc):
    """V_j = c for every key j  =>  O_i = c for every row (weights sum to one)."""
    for t, shape in enumerate(_SHAPES):
        B, Nq, Nk, Hq, Hkv, d, causal = shape
        q, k, _ = _qkv(shape, 20 * t)
        c = _rand((B, 1, Hkv, d), 99)
        v = c.expand(B, Nk, Hkv, d).clone()
        o, _ = orc.attention(q, k, v, 0.4, causal)
        want = torch.repeat_interleave(c, Hq // Hkv, dim=2).expand(B, Nq, Hq, d)
        _close(o, want, 1e-13, "constant V")


def pin_dominant_score(orc):
    """One key whose score exceeds every other visible score by >= 50 takes all the
    weight: O_i = V_j up to e^-50 ([LLM-basics] ①-3's [10,20] example taken to the limit)."""
    Nq = Nk = 16
    d = 4
    q = torch.zeros((1, Nq, 1, d), dtype=f64)
    q[..., 0] = 1.0
    k = _rand((1, Nk, 1, d), 5, 0.1)
    k[..., 0] = 0.0
    star = 3
    k[0, star, 0, 0] = 60.0
    v = _rand((1, Nk, 1, d), 6)
    o, lse = orc.attention(q, k, v, 1.0, causal=False)
    _close(o[0, :, 0, :], v[0, star, 0, :].expand(Nq, d), 1e-15 + 20 * math.exp(-50), "dominant key")
    # causal: rows before the dominant key cannot see it
    o2, _ = orc.attention(q, k, v, 1.0, causal=True)
    _close(o2[0, star:, 0, :], v[0, star, 0, :].expand(Nq - star, d), 1e-15 + 20 * math.exp(-50),
           "dominant key, causal")
    assert (o2[0, :star, 0, :] - v[0, star, 0, :]).abs().max() > 1e-3


def pin_causal_row0(orc):
    """Causal, Nq = Nk: row 0 sees only key 0, so O_0 = V_0 and LSE_0 = scale * q_0 . k_0."""
    for t, shape in enumerate(_SHAPES[:1]):
        B, Nq, Nk, Hq, Hkv, d, _ = shape
        q, k, v = _qkv(shape, 30)
        o, lse = orc.attention(q, k, v, 0.7, causal=True)
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            _close(o[0, 0, h], v[0, 0, kvh], 0.0, "row 0 = V[0]")
            _close(lse[0, h, 0], 0.7 * float((q[0, 0, h] * k[0, 0, kvh]).sum()), 1e-14, "LSE_0")


def pin_uniform_closed_form(orc):
    """K = 0 makes every visible score 0: causal O_i = mean(V_0..V_{i+Nk-Nq}) with
    LSE_i = ln(i + Nk - Nq + 1); non-causal O_i = mean(V), LSE_i = ln Nk."""
    for (Nq, Nk) in ((12, 12), (5, 17)):
        q = _rand((1, Nq, 2, 6), 40)
        k = torch.zeros((1, Nk, 1, 6), dtype=f64)
        v = _rand((1, Nk, 1, 6), 41)
        o, lse = orc.attention(q, k, v, 0.125, causal=True)
        for i in range(Nq):
            last = i + Nk - Nq
            for h in range(2):
                _close(o[0, i, h], v[0, :last + 1, 0].mean(dim=0), 1e-15, "uniform causal O")
                _close(lse[0, h, i], math.log(last + 1), 1e-15, "uniform causal LSE")
        o, lse = orc.attention(q, k, v, 0.125, causal=False)
        _close(o[0, :, 0], v[0, :, 0].mean(dim=0).expand(Nq, 6), 1e-15, "uniform O")
        _close(lse, torch.full((1, 2, Nq), math.log(Nk), dtype=f64), 1e-15, "uniform LSE")


def pin_gqa_repeat(orc):
    """[LLM-basics] ②-7: 14 query heads share 2 K/V heads in groups of 7.  Equal to
    MHA over K/V heads repeated 7 times consecutively."""
    g = _golden("gqa_example.json")
    Hq, Hkv, d = g["num_attention_heads"], g["num_key_value_heads"], 8
    assert Hq // Hkv == g["num_key_value_groups"]
    q, k, v = _rand((1, 9, Hq, d), 50), _rand((1, 9, Hkv, d), 51), _rand((1, 9, Hkv, d), 52)
    o, lse = orc.attention(q, k, v, 0.3, causal=True)
    kr = torch.repeat_interleave(k, Hq // Hkv, dim=2)
    vr = torch.repeat_interleave(v, Hq // Hkv, dim=2)
    o2, lse2 = orc.attention(q, kr, vr, 0.3, causal=True)
    _close(o, o2, 0.0, "GQA O")
    _close(lse, lse2, 0.0, "GQA LSE")
    # and head h really uses K/V head h // 7 (not h % 2): compare one head by hand
    for h in (0, 6, 7, 13):
        oh, lh = orc.attention(q[:, :, h:h + 1], k[:, :, h // 7:h // 7 + 1], v[:, :, h // 7:h // 7 + 1],
                               0.3, causal=True)
        _close(o[:, :, h], oh[:, :, 0], 0.0, f"GQA head {h}")


def pin_key_permutation(orc):
    """Non-causal attention is a function of the set of (key, value) pairs: permuting
    them jointly leaves O and LSE unchanged."""
    shape = _SHAPES[2]
    q, k, v = _qkv(shape, 60)
    perm = torch.randperm(shape[2], generator=torch.Generator().manual_seed(61))
    o, lse = orc.attention(q, k, v, 0.3, causal=False)
    o2, lse2 = orc.attention(q, k[:, perm], v[:, perm], 0.3, causal=False)
    _close(o, o2, 1e-14, "permuted O")
    _close(lse, lse2, 1e-14, "permuted LSE")


# ---------------------------------------------------------------------------
# the online softmax merge, brute-forced
# ---------------------------------------------------------------------------

def _compositions(n):
    """All ways to cut range(n) into contiguous non-empty blocks, as edge lists."""
    for cuts in itertools.product((0, 1), repeat=n - 1):
        edges = [0] + [i + 1 for i, c in enumerate(cuts) if c] + [n]
        yield edges


def pin_online_merge_bruteforce(orc):
    """[FA-notes] §4 / §5.2, [LLM-basics] ③-2: block-by-block online softmax with output
    rescaling equals the one-shot softmax for EVERY split of a row into contiguous
    blocks (rows of length 1..8, all 2^(n-1) splits)."""
    for n in range(1, 9):
        s = _rand((3, n), 70 + n, 3.0)
        s[1, n // 2] = 40.0             # a late large score forces a max change
        v = _rand((n, 5), 80 + n)
        p = torch.exp(s - s.max(dim=1, keepdim=True).values)
        o_ref = (p / p.sum(dim=1, keepdim=True)) @ v
        lse_ref = torch.logsumexp(s, dim=1)
        for edges in _compositions(n):
            o, lse = orc.online_attention_rows(s, v, edges)
            _close(o, o_ref, 1e-14, f"online O n={n} edges={edges}")
            _close(lse, lse_ref, 1e-14, f"online LSE n={n} edges={edges}")
    # one merge reproduces the two-block formulas on scalars: a state (m1, l1, acc1) stated
    # directly, and the state of a two-key block [3, 2] with V = (1, 10)
    m1, l1, a1 = 1.5, 2.0, 0.25
    x2 = torch.tensor([[3.0, 2.0]], dtype=f64)
    vals = torch.tensor([[1.0], [10.0]], dtype=f64)
    m2, l2, a2 = 3.0, 1.0 + math.exp(-1.0), 1.0 + 10.0 * math.exp(-1.0)
    bm, bl, bacc = orc.block_state(x2, vals)
    _close(bm, [m2], 0.0, "block max")
    _close(bl, [l2], 1e-15, "block sum")
    _close(bacc, [[a2]], 1e-15, "block numerator")
    first = (torch.tensor([m1], dtype=f64), torch.tensor([l1], dtype=f64),
             torch.tensor([[a1]], dtype=f64))
    for order in ((first, (bm, bl, bacc)), ((bm, bl, bacc), first)):
        m, l, acc = orc.merge_states(*order)
        _close(m, [3.0], 0.0, "m_new = max(m1, m2)")
        _close(l, [math.exp(m1 - 3.0) * l1 + math.exp(m2 - 3.0) * l2], 1e-15, "l_new")
        _close(acc, [[math.exp(m1 - 3.0) * a1 + a2]], 1e-15, "acc_new")


def pin_lse_merge_decode(orc):
    """Splitting one decode row's keys into 256-key chunks, attending to each chunk and
    merging the (O_c, lse_c) pairs gives the unsplit result (the two-block merge of
    [FA-notes] §4 applied across chunks)."""
    for L in (1, 255, 256, 257, 700):
        q = _rand((1, 1, 2, 8), 90 + L)
        k = _rand((1, L, 1, 8), 91 + L, 2.0)
        v = _rand((1, L, 1, 8), 92 + L)
        o_ref, lse_ref = orc.attention(q, k, v, 0.35, causal=False)
        parts_o, parts_l = [], []
        for a in range(0, L, 256):
            oc, lc = orc.attention(q, k[:, a:a + 256], v[:, a:a + 256], 0.35, causal=False)
            parts_o.append(oc[0, 0])
            parts_l.append(lc[0, :, 0])
        o, lse = orc.lse_merge(torch.stack(parts_o), torch.stack(parts_l))
        _close(o, o_ref[0, 0], 1e-14, f"merged O L={L}")
        _close(lse, lse_ref[0, :, 0], 1e-14, f"merged LSE L={L}")


def pin_decode_matches_prefill(orc):
    """Decode = the same attention with one query row over the first L_b cache rows;
    cache rows beyond L_b (NaN) are never touched."""
    B, Hq, Hkv, d, Nmax = 3, 4, 2, 8, 40
    lengths = [1, 17, 40]
    q = _rand((B, Hq, d), 100)
    kc = _rand((B, Nmax, Hkv, d), 101)
    vc = _rand((B, Nmax, Hkv, d), 102)
    for b, L in enumerate(lengths):
        kc[b, L:] = float("nan")
        vc[b, L:] = float("nan")
    o, lse = orc.decode_attention(q, kc, vc, lengths, 0.25)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    for b, L in enumerate(lengths):
        o2, l2 = orc.attention(q[b].reshape(1, 1, Hq, d), kc[b:b + 1, :L], vc[b:b + 1, :L], 0.25,
                               causal=True)
        _close(o[b], o2[0, 0], 0.0, "decode O")
        _close(lse[b], l2[0, :, 0], 0.0, "decode LSE")
    # L = 1: the single cached value, LSE = its score
    _close(o[0], vc[0, 0].repeat_interleave(Hq // Hkv, dim=0), 0.0, "L=1 decode")


def _paged_pool(num_pages, page_size, Hkv, d):
    kp = torch.full((num_pages, page_size, Hkv, d), float("nan"), dtype=f64)
    vp = torch.full((num_pages, page_size, Hkv, d), float("nan"), dtype=f64)
    return kp, vp


def pin_paged_constant_pages(orc):
    """[LLM-basics] ②-8: logical block j of a sequence lives in the physical page its
    block table names.  With K = 0 every valid key has score 0, so each query head's
    output is the plain mean of the valid V rows and LSE = ln L.  Every physical page
    holds one constant V row value, so the mean is the page constants weighted by how
    many of the sequence's keys fall in each page (the last page partly).  Tables are
    permuted, two sequences share a page, rows past the length and unused pages are NaN."""
    page_size, Hkv, d, Hq = 4, 2, 3, 4
    num_pages = 7
    kp, vp = _paged_pool(num_pages, page_size, Hkv, d)
    const = {p: torch.tensor([[p + 1.0, -2.0 * p, 0.5 * p * p], [3.0 - p, p / 4.0, 1.0]],
                             dtype=f64) for p in range(num_pages)}
    table = [[5, 2, 0, -1], [2, 6, -1, -1], [3, -1, -1, -1]]
    lengths = [10, 5, 1]
    for b, L in enumerate(lengths):
        for j in range((L + page_size - 1) // page_size):
            page = table[b][j]
            n = min(page_size, L - j * page_size)
            kp[page, :n] = 0.0
            vp[page, :n] = const[page].unsqueeze(0).expand(n, Hkv, d)
    q = _rand((3, Hq, d), 130)
    o, lse = orc.decode_attention_paged(q, kp, vp, table, lengths, page_size, 0.7)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    G = Hq // Hkv
    for b, L in enumerate(lengths):
        want = torch.zeros((Hkv, d), dtype=f64)
        for j in range((L + page_size - 1) // page_size):
            n = min(page_size, L - j * page_size)
            want += n * const[table[b][j]]
        want /= L
        for h in range(Hq):
            _close(o[b, h], want[h // G], 1e-14, f"paged mean b={b} h={h}")
            _close(lse[b, h:h + 1], [math.log(L)], 1e-14, f"paged LSE b={b}")


def pin_paged_dominant_key(orc):
    """One logical key position t gets a score 60 above every other key, so O is that key's
    V row (to ~1e-26): checks that logical position t is read from row t mod page_size of
    page table[t div page_size], for t at the first and last row of a page and inside the
    partial last page."""
    page_size, Hkv, d, Hq = 4, 1, 2, 2
    table = [[3, 0, 4]]
    L = 11
    for t in (0, 3, 4, 7, 8, 10):
        kp, vp = _paged_pool(5, page_size, Hkv, d)
        for j in range(3):
            n = min(page_size, L - j * page_size)
            kp[table[0][j], :n] = 0.0
            vp[table[0][j], :n] = _rand((n, Hkv, d), 140 + 10 * t + j)
        page, row = table[0][t // page_size], t % page_size
        kp[page, row] = 100.0
        q = torch.full((1, Hq, d), 0.3, dtype=f64)       # score(t) = 0.3 * 100 * d * scale = 60
        o, lse = orc.decode_attention_paged(q, kp, vp, table, [L], page_size, 1.0)
        for h in range(Hq):
            _close(o[0, h], vp[page, row, 0], 1e-20, f"dominant paged key t={t}")
            _close(lse[0, h:h + 1], [60.0 + 0.0], 1e-12, f"dominant paged LSE t={t}")


def pin_varlen_constant_v(orc):
    """Packed variable-length batch: every value row of sequence b equals a constant
    vector c_b, so every output row of sequence b is c_b whatever the scores — any
    read of another sequence's keys or values, or a wrong row offset, shows."""
    lens_q = [3, 1, 5, 2]
    lens_k = [4, 1, 5, 7]
    Hq, Hkv, d = 4, 2, 3
    cu_q = [0] + list(torch.cumsum(torch.tensor(lens_q), 0).tolist())
    cu_k = [0] + list(torch.cumsum(torch.tensor(lens_k), 0).tolist())
    q = _rand((cu_q[-1], Hq, d), 150)
    k = _rand((cu_k[-1], Hkv, d), 151, 2.0)
    v = torch.empty((cu_k[-1], Hkv, d), dtype=f64)
    consts = [_rand((Hkv, d), 152 + b) for b in range(4)]
    for b in range(4):
        v[cu_k[b]:cu_k[b + 1]] = consts[b]
    for causal in (False, True):
        o, lse = orc.attention_varlen(q, k, v, cu_q, cu_k, 0.5, causal)
        for b in range(4):
            for r in range(cu_q[b], cu_q[b + 1]):
                for h in range(Hq):
                    _close(o[r, h], consts[b][h // (Hq // Hkv)], 1e-14, f"varlen const b={b}")
        assert torch.isfinite(lse).all()


def pin_varlen_empty_sequences(orc):
    """Sequences with no queries or no keys inside a pack: a sequence without queries
    still moves the key offsets of those after it, and a sequence without keys has no
    defined softmax (its rows stay NaN).  Constant per-sequence V rows make every
    defined output row known in closed form."""
    lens_q = [2, 0, 3, 4, 1]
    lens_k = [0, 4, 3, 1, 2]
    Hq, Hkv, d = 2, 1, 3
    cu_q = [0, 2, 2, 5, 9, 10]
    cu_k = [0, 0, 4, 7, 8, 10]
    q = _rand((10, Hq, d), 170)
    k = _rand((10, Hkv, d), 171)
    v = torch.empty((10, Hkv, d), dtype=f64)
    consts = [_rand((Hkv, d), 172 + b) for b in range(5)]
    for b in range(5):
        v[cu_k[b]:cu_k[b + 1]] = consts[b]
    o, lse = orc.attention_varlen(q, k, v, cu_q, cu_k, 0.7, False)
    assert torch.isnan(o[0:2]).all() and torch.isnan(lse[:, 0:2]).all(), "keyless rows must stay NaN"
    for b in (2, 3, 4):
        for r in range(cu_q[b], cu_q[b + 1]):
            for h in range(Hq):
                _close(o[r, h], consts[b][0], 1e-14, f"varlen empty-seq offsets b={b}")
    assert torch.isfinite(lse[:, 2:]).all()
    # a one-key sequence: LSE is that key's score exactly
    r = cu_q[3]
    for h in range(Hq):
        want = 0.7 * float(q[r, h] @ k[cu_k[3], 0])
        _close(lse[h, r:r + 1], [want], 1e-13, "varlen single-key LSE")


def pin_varlen_causal_alignment(orc):
    """With K = 0 every visible key scores 0, so a row's output is the mean of the V rows
    it sees and LSE = ln(count).  Per sequence, causal row i sees keys 0 .. i + (Nk_b - Nq_b)
    (bottom-right alignment inside the sequence, not across the pack)."""
    lens_q = [2, 4, 1]
    lens_k = [5, 4, 3]
    Hq, Hkv, d = 2, 1, 2
    cu_q = [0, 2, 6, 7]
    cu_k = [0, 5, 9, 12]
    q = _rand((7, Hq, d), 160)
    k = torch.zeros((12, Hkv, d), dtype=f64)
    v = _rand((12, Hkv, d), 161)
    o, lse = orc.attention_varlen(q, k, v, cu_q, cu_k, 1.0, True)
    for b in range(3):
        nq, nk = lens_q[b], lens_k[b]
        for i in range(nq):
            cnt = i + (nk - nq) + 1
            want = v[cu_k[b]:cu_k[b] + cnt, 0].mean(dim=0)
            for h in range(Hq):
                _close(o[cu_q[b] + i, h], want, 1e-14, f"varlen causal b={b} i={i}")
                _close(lse[h, cu_q[b] + i:cu_q[b] + i + 1], [math.log(cnt)], 1e-14, "varlen LSE")


# ---------------------------------------------------------------------------
# independent re-computations
# ---------------------------------------------------------------------------

def pin_bruteforce_loops(orc):
    """Tiny shapes against scalar Python loops written from the definition
    (dot products, mask, max, exp, sum, weighted sum), both causal alignments."""
    for (B, Nq, Nk, Hq, Hkv, d, causal) in ((2, 3, 5, 4, 2, 3, True), (1, 4, 4, 2, 1, 2, True),
                                            (1, 3, 2, 3, 3, 2, False)):
        q = _rand((B, Nq, Hq, d), 110)
        k = _rand((B, Nk, Hkv, d), 111)
        v = _rand((B, Nk, Hkv, d), 112)
        scale = 0.6
        o, lse = orc.attention(q, k, v, scale, causal)
        ql, kl, vl = q.tolist(), k.tolist(), v.tolist()
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                g = h // G
                for i in range(Nq):
                    sc = []
                    for j in range(Nk):
                        if causal and j > i + (Nk - Nq):
                            continue
                        sc.append((j, scale * sum(ql[b][i][h][c] * kl[b][j][g][c] for c in range(d))))
                    mx = max(s for _, s in sc)
                    w = [(j, math.exp(s - mx)) for j, s in sc]
                    tot = sum(x for _, x in w)
                    for c in range(d):
                        want = sum(x * vl[b][j][g][c] for j, x in w) / tot
                        assert abs(o[b, i, h, c].item() - want) < 1e-13, (b, i, h, c)
                    assert abs(lse[b, h, i].item() - (mx + math.log(tot))) < 1e-13


def pin_sdpa_crosscheck(orc):
    """A library routine: torch's scaled_dot_product_attention on the CPU in fp64
    ([FA-notes] §6 names it as where FlashAttention is used), K/V heads repeated
    for GQA; LSE against torch.logsumexp of the masked scores."""
    import torch.nn.functional as F
    for (B, Nq, Nk, Hq, Hkv, d, causal) in ((1, 128, 128, 1, 1, 64, False), (2, 64, 64, 4, 2, 16, True),
                                            (1, 33, 70, 4, 1, 16, True)):
        q = _rand((B, Nq, Hq, d), 120)
        k = _rand((B, Nk, Hkv, d), 121)
        v = _rand((B, Nk, Hkv, d), 122)
        scale = 1.0 / math.sqrt(d)
        o, lse = orc.attention(q, k, v, scale, causal)
        qt = q.permute(0, 2, 1, 3)
        kt = torch.repeat_interleave(k, Hq // Hkv, dim=2).permute(0, 2, 1, 3)
        vt = torch.repeat_interleave(v, Hq // Hkv, dim=2).permute(0, 2, 1, 3)
        mask = None
        if causal:
            i = torch.arange(Nq).unsqueeze(1)
            j = torch.arange(Nk).unsqueeze(0)
            mask = j <= i + (Nk - Nq)
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        _close(o.permute(0, 2, 1, 3), ref, 1e-12, "SDPA O")
        s = (qt @ kt.transpose(-1, -2)) * scale
        if mask is not None:
            s = s.masked_fill(~mask, float("-inf"))
        _close(lse, torch.logsumexp(s, dim=-1), 1e-12, "logsumexp LSE")


def _sdpa_grads(q, k, v, do, scale, causal):
    """Gradients of torch's fp64 CPU scaled_dot_product_attention through autograd (K/V
    heads repeated for GQA, so autograd adds the group's contributions itself)."""
    import torch.nn.functional as F
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
    qt = qq.permute(0, 2, 1, 3)
    kt = torch.repeat_interleave(kk, Hq // Hkv, dim=2).permute(0, 2, 1, 3)
    vt = torch.repeat_interleave(vv, Hq // Hkv, dim=2).permute(0, 2, 1, 3)
    mask = None
    if causal:
        i = torch.arange(Nq).unsqueeze(1)
        j = torch.arange(Nk).unsqueeze(0)
        mask = j <= i + (Nk - Nq)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return torch.autograd.grad((o.permute(0, 2, 1, 3) * do).sum(), (qq, kk, vv))


def pin_bwd_autograd(orc):
    """The backward against autograd of a library routine (torch's SDPA, fp64 CPU):
    MHA and GQA, causal with Nq == Nk and Nq < Nk (bottom-right), non-causal."""
    for (B, Nq, Nk, Hq, Hkv, d, causal, sc) in ((1, 6, 6, 1, 1, 4, False, 0.5),
                                                (2, 9, 9, 4, 2, 5, True, 0.4),
                                                (1, 5, 11, 6, 2, 3, True, 0.9),
                                                (1, 12, 7, 4, 1, 8, False, 0.35)):
        q = _rand((B, Nq, Hq, d), 180)
        k = _rand((B, Nk, Hkv, d), 181)
        v = _rand((B, Nk, Hkv, d), 182)
        do = _rand((B, Nq, Hq, d), 183)
        dq, dk, dv = orc.attention_backward(q, k, v, do, sc, causal)
        gq, gk, gv = _sdpa_grads(q, k, v, do, sc, causal)
        _close(dq, gq, 1e-12, "bwd dQ vs autograd")
        _close(dk, gk, 1e-12, "bwd dK vs autograd")
        _close(dv, gv, 1e-12, "bwd dV vs autograd")


def pin_bwd_finite_differences(orc):
    """Brute force: central differences of L = sum(O * dO) through the (pinned) forward,
    for every input entry of a tiny causal GQA case."""
    B, Nq, Nk, Hq, Hkv, d, sc = 1, 3, 4, 2, 1, 2, 0.8
    q = _rand((B, Nq, Hq, d), 190)
    k = _rand((B, Nk, Hkv, d), 191)
    v = _rand((B, Nk, Hkv, d), 192)
    do = _rand((B, Nq, Hq, d), 193)
    grads = orc.attention_backward(q, k, v, do, sc, True)

    def loss(qq, kk, vv):
        o, _ = orc.attention(qq, kk, vv, sc, True)
        return float((o * do).sum())
    h = 1e-5
    for which, x in enumerate((q, k, v)):
        for idx in range(x.numel()):
            xp, xm = x.clone(), x.clone()
            xp.view(-1)[idx] += h
            xm.view(-1)[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grads[which].reshape(-1)[idx].item()) < 1e-8, (which, idx)


def pin_bwd_closed_forms(orc):
    """Closed forms.  K = 0 and every V row equal to c: every visible key has weight
    1/n_i, O = c whatever the scores, so dQ = dK = 0 and dV_j = sum over the rows i that
    see key j of dO_i / n_i.  A single key: P = 1, dQ = dK = 0, dV = sum_i dO_i."""
    B, Nq, Nk, Hq, Hkv, d = 1, 5, 7, 2, 1, 3
    q = _rand((B, Nq, Hq, d), 200)
    k = torch.zeros((B, Nk, Hkv, d), dtype=f64)
    c = _rand((d,), 201)
    v = c.expand(B, Nk, Hkv, d).clone()
    do = _rand((B, Nq, Hq, d), 202)
    dq, dk, dv = orc.attention_backward(q, k, v, do, 0.7, True)
    _close(dq, torch.zeros_like(dq), 1e-14, "K=0, const V: dQ")
    _close(dk, torch.zeros_like(dk), 1e-14, "K=0, const V: dK")
    want = torch.zeros((Nk, d), dtype=f64)
    for h in range(Hq):
        for i in range(Nq):
            n = i + (Nk - Nq) + 1
            want[:n] += do[0, i, h] / n
    _close(dv[0, :, 0], want, 1e-13, "K=0: dV row means")
    q1 = _rand((2, 4, 2, 3), 203)
    k1 = _rand((2, 1, 2, 3), 204)
    v1 = _rand((2, 1, 2, 3), 205)
    do1 = _rand((2, 4, 2, 3), 206)
    dq, dk, dv = orc.attention_backward(q1, k1, v1, do1, 1.3, False)
    _close(dq, torch.zeros_like(dq), 1e-14, "one key: dQ")
    _close(dk, torch.zeros_like(dk), 1e-14, "one key: dK")
    _close(dv[:, 0], do1.sum(dim=1), 1e-13, "one key: dV")
    # Scores hundreds apart ([LLM-basics] ③-1: exp of large scores overflows without the
    # max shift): P is one-hot on each row's last visible key, so that key's dV is the sum
    # of the dO rows it wins, every other dV row is 0, and dQ = dK = 0.
    Nq, Nk = 3, 5
    qb = torch.zeros((1, Nq, 1, 2), dtype=f64)
    qb[..., 0] = 30.0
    kb = torch.zeros((1, Nk, 1, 2), dtype=f64)
    kb[0, :, 0, 0] = 30.0 * torch.arange(Nk, dtype=f64)
    vb = _rand((1, Nk, 1, 2), 207)
    dob = _rand((1, Nq, 1, 2), 208)
    dq, dk, dv = orc.attention_backward(qb, kb, vb, dob, 1.0, True)
    want = torch.zeros((Nk, 2), dtype=f64)
    for i in range(Nq):
        want[i + (Nk - Nq)] += dob[0, i, 0]
    _close(dv[0, :, 0], want, 1e-14, "one-hot P: dV")
    _close(dq, torch.zeros_like(dq), 1e-14, "one-hot P: dQ")
    _close(dk, torch.zeros_like(dk), 1e-14, "one-hot P: dK")


def pin_bwd_invariants(orc):
    """Invariants of the softmax gradient: every row of dS sums to 0, so the dK rows of a
    head add up to 0; and adding one vector w to every key adds Q_i.w to a whole score
    row, which changes neither P nor (since rows of dS sum to 0) dQ, dK or dV."""
    B, Nq, Nk, Hq, Hkv, d = 2, 6, 9, 4, 2, 5
    q = _rand((B, Nq, Hq, d), 210)
    k = _rand((B, Nk, Hkv, d), 211)
    v = _rand((B, Nk, Hkv, d), 212)
    do = _rand((B, Nq, Hq, d), 213)
    w = _rand((d,), 214)
    for causal in (False, True):
        dq, dk, dv = orc.attention_backward(q, k, v, do, 0.45, causal)
        _close(dk.sum(dim=1), torch.zeros((B, Hkv, d), dtype=f64), 1e-13, "sum of dK rows")
        dq2, dk2, dv2 = orc.attention_backward(q, k + w, v, do, 0.45, causal)
        _close(dq2, dq, 1e-12, "key shift: dQ")
        _close(dk2, dk, 1e-12, "key shift: dK")
        _close(dv2, dv, 1e-12, "key shift: dV")
        # restricted calls return the same numbers
        rq, rk, rv = orc.attention_backward(q, k, v, do, 0.45, causal, kv_heads=[1], rows=(2, 5),
                                            keys=(3, 8), row_block=4)
        _close(rq[:, 2:5, 2:4], dq[:, 2:5, 2:4], 1e-13, "restricted dQ")
        _close(rk[:, 3:8, 1], dk[:, 3:8, 1], 1e-13, "restricted dK")
        _close(rv[:, 3:8, 1], dv[:, 3:8, 1], 1e-13, "restricted dV")
        oq, _, _ = orc.attention_backward(q, k, v, do, 0.45, causal, rows=(1, 4), keys=(0, 0))
        _close(oq[:, 1:4], dq[:, 1:4], 1e-13, "rows-only dQ")
        _, ok_, ov = orc.attention_backward(q, k, v, do, 0.45, causal, rows=(0, 0), keys=(6, 9))
        _close(ok_[:, 6:9], dk[:, 6:9], 1e-13, "keys-only dK")
        _close(ov[:, 6:9], dv[:, 6:9], 1e-13, "keys-only dV")


ALL_PINS = [
    pin_bwd_autograd,
    pin_bwd_finite_differences,
    pin_bwd_closed_forms,
    pin_bwd_invariants,
    pin_varlen_constant_v,
    pin_varlen_causal_alignment,
    pin_varlen_empty_sequences,
    pin_paged_constant_pages,
    pin_paged_dominant_key,
    pin_worked_example_printed,
    pin_worked_example_closed_form,
    pin_softmax_examples,
    pin_overflow,
    pin_causal_visibility,
    pin_rows_sum_to_one,
    pin_constant_v,
    pin_dominant_score,
    pin_causal_row0,
    pin_uniform_closed_form,
    pin_gqa_repeat,
    pin_key_permutation,
    pin_online_merge_bruteforce,
    pin_lse_merge_decode,
    pin_decode_matches_prefill,
    pin_bruteforce_loops,
    pin_sdpa_crosscheck,
]
