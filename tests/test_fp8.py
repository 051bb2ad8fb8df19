"""GPU parity of the FP8 forward (fa_forward_fp8) against the fp64 oracle.

Inputs: seeded E4M3 codes with per-tensor descales (``workloads.fp8_inputs``); the
oracle runs standard attention on the exact values code * descale.

Tolerance, derived from the kernel's arithmetic.  The score products are exact (E4M3
codes have 4 significant bits) and accumulate in fp32, so the only coarse rounding is of
the weights p_j = 2^(S_j c - m) to E4M3 for P V: |p^_j - p_j| <= max(2^-4 p_j, 2^-10)
(half an ulp of a 3-bit mantissa; half the subnormal step below 2^-6).  O is normalised
by the sum of the rounded weights, so O^ - O = sum_j (p^_j - p_j)(v_j - O) / sum_j p^_j.
The reference m is at most the row max (it is a score the row has seen), and taking it
equal to the row max is the worst case for the subnormal term: with P_j the exact
probabilities,
    |err| <= 1.12 * sum_j max(2^-4 P_j, 2^-10 P_max) |v_j - O| + 1e-4 sum_j P_j |v_j - O| + 1e-5
(1.12 covers sum p^ >= 0.9 sum p; the 1e-4 term the fp32 scores and exp2).  Independent
rounding errors add in quadrature, so the rms error must stay below
rms(sqrt(sum_j (max(2^-4 P_j, 2^-10 P_max)(v_j - O))^2)) (expected ~0.58 of it).  The
LSE comes from fp32 sums of the unrounded weights: max abs error <= 1e-3, as for bf16.
The bound terms are computed here in fp64 (test-side, for the tolerance only).
"""
import math

import pytest
import torch

import io_aware_attention_attn_amd as fa
import oracle
import workloads as W

pytestmark = pytest.mark.gpu
f64 = torch.float64


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def _values(q8, k8, v8, qd, kd, vd):
    return q8.to(f64) * qd, k8.to(f64) * kd, v8.to(f64) * vd


def _run(q8, k8, v8, qd, kd, vd, scale, causal):
    dev = _dev()
    B, Nq, Hq, d = q8.shape
    o = torch.full((B, Nq, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=dev)
    fa.fa_forward_fp8(q8.to(dev), k8.to(dev), v8.to(dev), qd, kd, vd, scale=scale, causal=causal,
                      o=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _check_rows(name, o, lse, q, k, v, o_ref, lse_ref, scale, causal, b, h, r0, r1):
    """Rows [r0, r1) of (b, h): O against the derived bound, LSE within 1e-3."""
    Nq, Hq = q.shape[1], q.shape[2]
    Nk, Hkv = k.shape[1], k.shape[2]
    kvh = h // (Hq // Hkv)
    s = scale * (q[b, r0:r1, h] @ k[b, :, kvh].T)
    if causal:
        i = torch.arange(r0, r1).unsqueeze(1)
        j = torch.arange(Nk).unsqueeze(0)
        s = s.masked_fill(j > i + (Nk - Nq), float("-inf"))
    p = torch.softmax(s, dim=1)                                  # [R, Nk]
    pmax = p.max(dim=1, keepdim=True).values
    w = torch.maximum(p * 2.0 ** -4, pmax * 2.0 ** -10) * (p > 0)
    bound = torch.empty((r1 - r0, q.shape[3]), dtype=f64)
    quad = torch.empty_like(bound)
    for c0 in range(0, r1 - r0, 16):  # 16 rows at a time: |v_j - O| is [rows, Nk, d]
        c1 = min(c0 + 16, r1 - r0)
        dev_ = (v[b, :, kvh].unsqueeze(0) - o_ref[b, r0 + c0:r0 + c1, h].unsqueeze(1)).abs()
        bound[c0:c1] = 1.12 * torch.einsum("rj,rjc->rc", w[c0:c1], dev_) \
            + 1e-4 * torch.einsum("rj,rjc->rc", p[c0:c1], dev_) + 1e-5
        quad[c0:c1] = torch.sqrt(torch.einsum("rj,rjc->rc", w[c0:c1] ** 2, dev_ * dev_))
    err = (o[b, r0:r1, h].to(f64) - o_ref[b, r0:r1, h]).abs()
    el = (lse[b, h, r0:r1].to(f64) - lse_ref[b, h, r0:r1]).abs()
    ratio = (err / bound).max().item()
    rms = err.pow(2).mean().sqrt().item()
    rms_lim = quad.pow(2).mean().sqrt().item()
    msg = (f"{name} b{b} h{h} rows {r0}:{r1}: O max {err.max().item():.3e} (err/bound {ratio:.3f}), "
           f"rms {rms:.3e} vs {rms_lim:.3e}, LSE max {el.max().item():.3e}")
    print(msg, flush=True)
    assert torch.isfinite(o[b, r0:r1, h]).all() and torch.isfinite(lse[b, h, r0:r1]).all(), msg
    assert ratio <= 1.0, msg
    assert rms <= rms_lim, msg
    assert el.max().item() <= 1e-3, msg


SMALL = [
    # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 2, 1, 128, 128, 64, True),
    (2, 4, 2, 200, 200, 128, True),
    (1, 4, 4, 100, 300, 64, False),
    (1, 8, 2, 77, 333, 128, True),
    (1, 2, 2, 1, 65, 64, True),
    (2, 2, 1, 257, 190, 128, False),
    (1, 8, 2, 1024, 1024, 128, True),  # snake assignment of work to XCDs
]


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
def test_fp8_small(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    print(f"fp8 case {case}", flush=True)
    scale = 1.0 / math.sqrt(d)
    q8, k8, v8, qd, kd, vd = W.fp8_inputs(B, Hq, Hkv, Nq, Nk, d, seed=21)
    o, lse = _run(q8, k8, v8, qd, kd, vd, scale, causal)
    q, k, v = _values(q8, k8, v8, qd, kd, vd)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    for b in range(B):
        for h in range(Hq):
            _check_rows("fp8", o, lse, q, k, v, o_ref, lse_ref, scale, causal, b, h, 0, Nq)


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_fp8_full_size_sampled(name):
    """The long causal shapes (c3: MHA N=8192 with peaky Q,K x1.5; c4: GQA N=32768) as
    E4M3 codes, in the launch the benchmark times; sampled heads and row blocks."""
    cfg = W.CONFIGS[name]
    q8, k8, v8, qd, kd, vd = W.fp8_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq, cfg.Nk, cfg.d, seed=0,
                                          qk_gain=cfg.qk_gain)
    o, lse = _run(q8, k8, v8, qd, kd, vd, cfg.scale, cfg.causal)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    q, k, v = _values(q8, k8, v8, qd, kd, vd)
    N = cfg.Nq
    heads = [0, 13] if name == "c3" else [0, 37]
    for h in heads:
        for (r0, r1) in ((0, 64), (N // 2, N // 2 + 48), (N - 64, N)):
            o_ref, lse_ref = oracle.attention(q, k, v, cfg.scale, cfg.causal, heads=[h],
                                              rows=(r0, r1), row_block=64)
            _check_rows(name, o, lse, q, k, v, o_ref, lse_ref, cfg.scale, cfg.causal, 0, h, r0, r1)


def test_fp8_descales_exact():
    """Descales enter as plain factors: doubling v_descale doubles O bit for bit, and
    moving a factor 2 from scale into q_descale changes nothing."""
    B, Hq, Hkv, N, d = 1, 4, 2, 300, 128
    q8, k8, v8, qd, kd, vd = W.fp8_inputs(B, Hq, Hkv, N, N, d, seed=22)
    s = 1.0 / math.sqrt(d)
    o1, l1 = _run(q8, k8, v8, qd, kd, vd, s, True)
    o2, l2 = _run(q8, k8, v8, qd, kd, 2 * vd, s, True)
    o3, l3 = _run(q8, k8, v8, 2 * qd, kd, vd, s / 2, True)
    assert torch.equal(o2, 2 * o1) and torch.equal(l2, l1)
    assert torch.equal(o3, o1) and torch.equal(l3, l1)


def test_fp8_deterministic():
    q8, k8, v8, qd, kd, vd = W.fp8_inputs(1, 8, 2, 700, 700, 128, seed=23)
    a = _run(q8, k8, v8, qd, kd, vd, 0.088, True)
    b = _run(q8, k8, v8, qd, kd, vd, 0.088, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
