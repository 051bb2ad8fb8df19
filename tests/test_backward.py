"""GPU parity of the backward pass (fa_backward) against the fp64 oracle.

Inputs: seeded bf16 Q, K, V and dO (``workloads.backward_inputs``); the forward's O
and LSE that fa_backward takes are the oracle's (rounded to fp32), so both sides
start from the same data and the comparison isolates the backward kernels.

Tolerance, derived from the kernels' arithmetic.  Every gradient is a sum of
products in which one factor is rounded to bf16 on the GPU: P for dV = P^T dO, dS
for dK = scale dS^T Q and dQ = scale dS K (relative error <= 2^-8 each); the other
operands are exact bf16 inputs, and everything else is fp32 (P and dS carry at most
~1e-4 relative error from fp32 scores and exp2; dP and D carry fp32 dot-product
error <= d 2^-24 times the sums of absolute products; the final sums over N rows or
keys add N 2^-24 relative).  So element by element
    |err| <= (2^-8 + 1e-4 + N 2^-24) * sum |term| + d 2^-24 * scale * sum P (A + E) |x|
with the sums over the same index as the gradient's own sum (A = sum_c |dO_c V_c|,
E = sum_c |dO_c O_c|, x = the other operand), plus 1e-6 absolute.  Rounding errors of
independent terms also add in quadrature, so the root-mean-square error must stay
below 2^-8 * rms(sqrt(sum term^2)) (expected ~0.58 of that).  The bound terms are
computed here in fp64 from the inputs (test-side, for the tolerance only); the
expected gradients are the oracle's.
"""
import math

import pytest
import torch

import io_aware_attention_attn_amd as fa
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

U = 2.0 ** -8
F32 = 2.0 ** -24
f64 = torch.float64


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def _row_terms(q, k, v, do, o, scale, causal, b, h, r0, r1):
    """P, dS, A (= |dO| |V|^T) and E (= sum |dO O|) for query rows [r0, r1) of (b, h),
    in fp64 (for error bounds only)."""
    Nq, Hq = q.shape[1], q.shape[2]
    Nk, Hkv = k.shape[1], k.shape[2]
    kvh = h // (Hq // Hkv)
    qq = q[b, r0:r1, h].to(f64)
    kk = k[b, :, kvh].to(f64)
    vv = v[b, :, kvh].to(f64)
    dd = do[b, r0:r1, h].to(f64)
    s = scale * (qq @ kk.T)
    if causal:
        i = torch.arange(r0, r1).unsqueeze(1)
        j = torch.arange(Nk).unsqueeze(0)
        s = s.masked_fill(j > i + (Nk - Nq), float("-inf"))
    p = torch.softmax(s, dim=1)
    dp = dd @ vv.T
    ds = p * (dp - (p * dp).sum(1, keepdim=True))
    a = dd.abs() @ vv.abs().T
    e = (dd.abs() * o[b, r0:r1, h].to(f64).abs()).sum(1, keepdim=True)
    return p, ds, a, e


def _check(name, got, ref, worst, quad, N):
    got = got.to(f64)
    err = (got - ref).abs()
    assert torch.isfinite(got).all(), f"{name}: non-finite"
    rel = (U + 1e-4 + N * F32)
    bound = rel * worst[0] + F32 * worst[1] + 1e-6
    over = (err - bound).max().item()
    ratio = (err / bound).max().item()
    rms_err = err.pow(2).mean().sqrt().item()
    rms_lim = U * quad.pow(2).mean().sqrt().item()
    msg = (f"{name}: max err {err.max().item():.3e}, largest err / worst-case bound "
           f"{ratio:.3f}, rms err {rms_err:.3e} vs limit {rms_lim:.3e}")
    print(msg, flush=True)
    assert over <= 0, msg
    assert rms_err <= rms_lim, msg


def _bounds_dq(q, k, v, do, o, scale, causal, b, h, r0, r1):
    Hkv = k.shape[2]
    kvh = h // (q.shape[2] // Hkv)
    p, ds, a, e = _row_terms(q, k, v, do, o, scale, causal, b, h, r0, r1)
    kk = k[b, :, kvh].to(f64)
    d = q.shape[3]
    w0 = scale * (ds.abs() @ kk.abs())
    w1 = d * scale * ((p * (a + e)) @ kk.abs())
    quad = scale * torch.sqrt((ds * ds) @ (kk * kk))
    return (w0, w1), quad


def _bounds_dkdv(q, k, v, do, o, scale, causal, b, kvh, k0, k1, row_block=1024):
    Nq, Hq, d = q.shape[1], q.shape[2], q.shape[3]
    G = Hq // k.shape[2]
    wk0 = torch.zeros((k1 - k0, d), dtype=f64)
    wk1 = torch.zeros_like(wk0)
    qk2 = torch.zeros_like(wk0)
    wv0 = torch.zeros_like(wk0)
    qv2 = torch.zeros_like(wk0)
    Nk = k.shape[1]
    a0 = max(0, k0 - (Nk - Nq)) if causal else 0
    for h in range(kvh * G, (kvh + 1) * G):
        for r0 in range(a0, Nq, row_block):
            r1 = min(r0 + row_block, Nq)
            p, ds, a, e = _row_terms(q, k, v, do, o, scale, causal, b, h, r0, r1)
            qq = q[b, r0:r1, h].to(f64)
            dd = do[b, r0:r1, h].to(f64)
            pc, dsc, ac = p[:, k0:k1], ds[:, k0:k1], a[:, k0:k1]
            wk0 += scale * (dsc.abs().T @ qq.abs())
            wk1 += d * scale * ((pc * (ac + e)).T @ qq.abs())
            qk2 += scale * scale * ((dsc * dsc).T @ (qq * qq))
            wv0 += pc.T @ dd.abs()
            qv2 += (pc * pc).T @ (dd * dd)
    return ((wk0, wk1), qk2.sqrt()), ((wv0, torch.zeros_like(wv0)), qv2.sqrt())


def _oracle_fwd(q, k, v, scale, causal):
    o, lse = oracle.attention(q, k, v, scale, causal, row_block=1024)
    return o.to(torch.float32), lse.to(torch.float32)


def _run_bwd(q, k, v, do, o, lse, scale, causal):
    dev = _dev()
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    dq = torch.full((B, Nq, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    dk = torch.full((B, Nk, Hkv, d), float("nan"), dtype=torch.float32, device=dev)
    dv = torch.full((B, Nk, Hkv, d), float("nan"), dtype=torch.float32, device=dev)
    fa.fa_backward(q.to(dev), k.to(dev), v.to(dev), o.to(dev), lse.to(dev), do.to(dev),
                   scale=scale, causal=causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


SMALL = [
    # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 2, 1, 128, 128, 64, True),
    (2, 4, 2, 200, 200, 128, True),
    (1, 4, 4, 100, 300, 64, False),
    (1, 8, 2, 77, 333, 128, True),
    (1, 2, 2, 1, 65, 64, True),
    (1, 16, 1, 130, 130, 64, True),
    (2, 2, 1, 257, 190, 128, False),
    # groups that do not divide over the 8 XCDs while the key / query blocks do (snake
    # assignment of work to XCDs in both gradient kernels)
    (1, 8, 2, 1024, 1024, 128, True),
    (1, 3, 1, 1000, 1000, 64, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
def test_backward_small(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    print(f"backward case {case}", flush=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = W.backward_inputs(B, Hq, Hkv, Nq, Nk, d, seed=11)
    o, lse = _oracle_fwd(q, k, v, scale, causal)
    dq, dk, dv = _run_bwd(q, k, v, do, o, lse, scale, causal)
    rq, rk, rv = oracle.attention_backward(q, k, v, do, scale, causal)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            w, quad = _bounds_dq(q, k, v, do, o, scale, causal, b, h, 0, Nq)
            _check(f"dQ b{b} h{h}", dq[b, :, h], rq[b, :, h], w, quad, Nk)
        for kvh in range(Hkv):
            (wk, qk), (wv, qv) = _bounds_dkdv(q, k, v, do, o, scale, causal, b, kvh, 0, Nk)
            _check(f"dK b{b} kvh{kvh}", dk[b, :, kvh], rk[b, :, kvh], wk, qk, Nq * G)
            _check(f"dV b{b} kvh{kvh}", dv[b, :, kvh], rv[b, :, kvh], wv, qv, Nq * G)


@pytest.mark.parametrize("case", [(1, 4, 2, 200, 200, 128, True, 4.0),
                                  (1, 2, 1, 96, 300, 64, False, 6.0)],
                         ids=["causal gain 4", "noncausal gain 6"])
def test_backward_peaky(case):
    """Q and K scaled up so that the scores are tens to hundreds apart: P is close to
    one-hot, exp2(S c - lse2) would overflow without the LSE shift, and dS concentrates on
    a few keys per row."""
    B, Hq, Hkv, Nq, Nk, d, causal, gain = case
    print(f"backward peaky case {case}", flush=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = W.backward_inputs(B, Hq, Hkv, Nq, Nk, d, seed=12, qk_gain=gain)
    o, lse = _oracle_fwd(q, k, v, scale, causal)
    dq, dk, dv = _run_bwd(q, k, v, do, o, lse, scale, causal)
    rq, rk, rv = oracle.attention_backward(q, k, v, do, scale, causal)
    G = Hq // Hkv
    for h in range(Hq):
        w, quad = _bounds_dq(q, k, v, do, o, scale, causal, 0, h, 0, Nq)
        _check(f"dQ h{h}", dq[0, :, h], rq[0, :, h], w, quad, Nk)
    for kvh in range(Hkv):
        (wk, qk), (wv, qv) = _bounds_dkdv(q, k, v, do, o, scale, causal, 0, kvh, 0, Nk)
        _check(f"dK kvh{kvh}", dk[0, :, kvh], rk[0, :, kvh], wk, qk, Nq * G)
        _check(f"dV kvh{kvh}", dv[0, :, kvh], rv[0, :, kvh], wv, qv, Nq * G)


def test_backward_c2_full():
    """The causal MHA workload (B=2, H=12, N=2048, d=64) in full."""
    cfg = W.CONFIGS["c2"]
    q, k, v, do = W.backward_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq, cfg.Nk, cfg.d, seed=0)
    o, lse = _oracle_fwd(q, k, v, cfg.scale, cfg.causal)
    dq, dk, dv = _run_bwd(q, k, v, do, o, lse, cfg.scale, cfg.causal)
    rq, rk, rv = oracle.attention_backward(q, k, v, do, cfg.scale, cfg.causal, row_block=512)
    for b in range(cfg.B):
        for h in (0, 7, 11):
            w, quad = _bounds_dq(q, k, v, do, o, cfg.scale, True, b, h, 0, cfg.Nq)
            _check(f"c2 dQ b{b} h{h}", dq[b, :, h], rq[b, :, h], w, quad, cfg.Nk)
            (wk, qk), (wv, qv) = _bounds_dkdv(q, k, v, do, o, cfg.scale, True, b, h, 0, cfg.Nk)
            _check(f"c2 dK b{b} h{h}", dk[b, :, h], rk[b, :, h], wk, qk, cfg.Nq)
            _check(f"c2 dV b{b} h{h}", dv[b, :, h], rv[b, :, h], wv, qv, cfg.Nq)
    # every head: against the oracle with the loosest per-head worst case
    for t, r in ((dq, rq), (dk, rk), (dv, rv)):
        assert torch.isfinite(t).all()
        assert (t.to(f64) - r).abs().max().item() < 5e-2


def test_backward_c4_sampled():
    """The long-context GQA shape (B=1, Hq=64, Hkv=8, N=32768, d=128, causal) at full
    size: dQ of sampled row blocks, dK/dV of sampled key blocks near the end (the
    sums over all the group's query heads and every row that sees them)."""
    cfg = W.CONFIGS["c4"]
    q, k, v, do = W.backward_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq, cfg.Nk, cfg.d, seed=0)
    N = cfg.Nq
    heads = (0, 37)
    # O and LSE for every row (the backward reads them for all rows); oracle rows in blocks
    o = torch.empty((1, N, cfg.Hq, cfg.d), dtype=torch.float32)
    lse = torch.empty((1, cfg.Hq, N), dtype=torch.float32)
    # the rows' forward statistics are needed for every head the sampled dK/dV sum over
    # and for the sampled dQ heads; other heads get the GPU forward's O and LSE (they
    # only feed rows that are not compared)
    dev = _dev()
    og, lg = fa.fa_forward(q.to(dev), k.to(dev), v.to(dev), scale=cfg.scale, causal=True)
    o.copy_(og.cpu())
    lse.copy_(lg.cpu())
    need_heads = sorted(set(heads) | set(range(0, 8)) | set(range(56, 64)))
    for h in need_heads:
        oo, ll = oracle.attention(q, k, v, cfg.scale, True, heads=[h], row_block=2048,
                                  rows=(N - 1024, N) if h not in heads else None)
        r0 = 0 if h in heads else N - 1024
        o[0, r0:, h] = oo[0, r0:, h].float()
        lse[0, h, r0:] = ll[0, h, r0:].float()
    dq, dk, dv = _run_bwd(q, k, v, do, o, lse, cfg.scale, True)
    for h in heads:
        for (r0, r1) in ((0, 128), (N // 2, N // 2 + 96), (N - 128, N)):
            rq, _, _ = oracle.attention_backward(q, k, v, do, cfg.scale, True, kv_heads=[h // 8],
                                                 rows=(r0, r1), keys=(0, 0), row_block=128)
            w, quad = _bounds_dq(q, k, v, do, o, cfg.scale, True, 0, h, r0, r1)
            _check(f"c4 dQ h{h} rows {r0}:{r1}", dq[0, r0:r1, h], rq[0, r0:r1, h], w, quad, N)
    for kvh in (0, 7):
        for (k0, k1) in ((N - 640, N - 512), (N - 96, N)):
            _, rk, rv = oracle.attention_backward(q, k, v, do, cfg.scale, True, kv_heads=[kvh],
                                                  rows=(0, 0), keys=(k0, k1), row_block=256)
            (wk, qk), (wv, qv) = _bounds_dkdv(q, k, v, do, o, cfg.scale, True, 0, kvh, k0, k1,
                                             row_block=256)
            _check(f"c4 dK kvh{kvh} keys {k0}:{k1}", dk[0, k0:k1, kvh], rk[0, k0:k1, kvh], wk,
                   qk, N * 8)
            _check(f"c4 dV kvh{kvh} keys {k0}:{k1}", dv[0, k0:k1, kvh], rv[0, k0:k1, kvh], wv,
                   qv, N * 8)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()


def test_backward_deterministic():
    """No atomics: two runs give identical bits."""
    B, Hq, Hkv, N, d = 1, 8, 2, 700, 128
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = W.backward_inputs(B, Hq, Hkv, N, N, d, seed=12)
    o, lse = _oracle_fwd(q, k, v, scale, True)
    a = _run_bwd(q, k, v, do, o, lse, scale, True)
    b = _run_bwd(q, k, v, do, o, lse, scale, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_after_gpu_forward():
    """End to end: the GPU forward's O and LSE into the GPU backward.  The forward's own
    O error (<= 1e-2 by its tolerance, ~1e-3 in practice) enters D, so the check here
    is the worst-case bound above plus that error's effect: |dP - D| changes by at most
    max|O error| * sum |dO| per row."""
    B, Hq, Hkv, N, d = 1, 4, 2, 384, 128
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = W.backward_inputs(B, Hq, Hkv, N, N, d, seed=13)
    dev = _dev()
    og, lg = fa.fa_forward(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=True)
    o_ref, _ = oracle.attention(q, k, v, scale, True)
    o_err = (og.cpu().to(f64) - o_ref).abs().max().item()
    dq, dk, dv = fa.fa_backward(q.to(dev), k.to(dev), v.to(dev), og, lg, do.to(dev), scale=scale,
                                causal=True)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(q, k, v, do, scale, True)
    dsum = do.to(f64).abs().sum(-1)  # [B, N, Hq]
    for h in range(Hq):
        w, quad = _bounds_dq(q, k, v, do, o_ref.float(), scale, True, 0, h, 0, N)
        kk = k[0, :, h // 2].to(f64)
        p, _, _, _ = _row_terms(q, k, v, do, o_ref.float(), scale, True, 0, h, 0, N)
        extra = scale * o_err * dsum[0, :, h].unsqueeze(1) * (p @ kk.abs())
        got = dq[0, :, h].cpu().to(f64)
        err = (got - rq[0, :, h]).abs()
        bound = (U + 1e-4 + N * F32) * w[0] + F32 * w[1] + extra + 1e-6
        assert (err <= bound).all(), f"dQ h{h}: max err {err.max().item():.3e}"
    assert torch.isfinite(dk.cpu()).all() and torch.isfinite(dv.cpu()).all()
    assert (dv.cpu().to(f64) - rv).abs().max().item() < 1e-2
