"""Every entry point enqueues on the caller's stream and is bitwise reproducible.

Each call runs twice on the default stream and once on a second (default-priority)
stream; the three results must be identical bit for bit.  Accuracy against the oracle
is covered by the parity test files; this file checks stream handling and determinism
(no atomics, no dependence on scheduling) for all of them.
"""
import math

import pytest
import torch

import io_aware_attention_attn_amd as fa
import workloads as W

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def _three_runs(call):
    """call(stream) -> tuple of output tensors (allocated inside)."""
    torch.cuda.synchronize()
    a = [t.clone() for t in call(None)]
    b = [t.clone() for t in call(None)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = call(s)
    s.synchronize()
    c = [t.clone() for t in c]
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y), "not reproducible on one stream"
        assert torch.equal(x, z), "different result on a side stream"


def test_forward_streams():
    dev = _dev()
    q, k, v = (t.to(dev) for t in W.prefill_inputs(2, 8, 2, 300, 300, 128, seed=31))
    _three_runs(lambda s: fa.fa_forward(q, k, v, causal=True, stream=s))


def test_forward_f32_streams():
    dev = _dev()
    q, k, v = (t.to(dev) for t in W.prefill_inputs(1, 2, 1, 130, 130, 64, "f32", seed=32))
    _three_runs(lambda s: fa.fa_forward_f32(q, k, v, causal=False, stream=s))


def test_varlen_streams():
    dev = _dev()
    lens = [100, 1, 257, 64]
    cu_q, cu_k, q, k, v = W.varlen_inputs(lens, lens, 8, 8, 128, seed=33)
    q, k, v, cu_q, cu_k = q.to(dev), k.to(dev), v.to(dev), cu_q.to(dev), cu_k.to(dev)
    _three_runs(lambda s: fa.fa_forward_varlen(q, k, v, cu_q, cu_k, max(lens), max(lens),
                                               causal=True, stream=s))


def test_fp8_streams():
    dev = _dev()
    q8, k8, v8, qd, kd, vd = W.fp8_inputs(1, 4, 2, 333, 333, 128, seed=34)
    q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
    _three_runs(lambda s: fa.fa_forward_fp8(q8, k8, v8, qd, kd, vd, causal=True, stream=s))


def test_backward_streams():
    dev = _dev()
    q, k, v, do = (t.to(dev) for t in W.backward_inputs(1, 4, 2, 200, 200, 64, seed=35))
    o, lse = fa.fa_forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    _three_runs(lambda s: fa.fa_backward(q, k, v, o, lse, do, causal=True, stream=s))


def test_decode_streams():
    dev = _dev()
    lengths, q, kc, vc = W.decode_inputs(4, 16, 2, 128, 1500, 1, 1500, seed=36)
    q, kc, vc, ld = q.to(dev), kc.to(dev), vc.to(dev), lengths.to(dev)
    _three_runs(lambda s: fa.fa_decode_splitkv(q, kc, vc, ld, chunk=256, stream=s))


def test_decode_paged_streams():
    dev = _dev()
    lengths, q, kc, vc = W.decode_inputs(3, 8, 1, 64, 1024, 1, 1024, seed=37)
    kp, vp, table = W.paged_from_contiguous(kc, vc, lengths, 128, seed=38, spare_pages=3)
    q, kp, vp, table, ld = q.to(dev), kp.to(dev), vp.to(dev), table.to(dev), lengths.to(dev)
    _three_runs(lambda s: fa.fa_decode_paged(q, kp, vp, table, ld, chunk=128, stream=s))


def test_stream_argument_without_making_it_current():
    """stream=s while torch's current stream stays the default one.  A long prefill is
    queued on s first, so the decode and backward queued behind it run well after the
    wrappers return and free their workspaces; the current stream meanwhile allocates
    blocks of the same sizes and fills them with NaN.  The workspaces were allocated in
    s's stream order, so those blocks are not the ones the kernels still read, and the
    results equal the same calls made on the current stream."""
    dev = _dev()
    lengths, q, kc, vc = W.decode_inputs(4, 16, 2, 128, 3000, 1, 3000, seed=39)
    q, kc, vc, ld = q.to(dev), kc.to(dev), vc.to(dev), lengths.to(dev)
    qb, kb, vb, dob = (t.to(dev) for t in W.backward_inputs(1, 4, 2, 300, 300, 64, seed=40))
    ob, lb = fa.fa_forward(qb, kb, vb, causal=True)
    ref_dec = [t.clone() for t in fa.fa_decode_splitkv(q, kc, vc, ld, chunk=256)]
    ref_bwd = [t.clone() for t in fa.fa_backward(qb, kb, vb, ob, lb, dob, causal=True)]
    qp, kp, vp = (t.to(dev) for t in W.prefill_inputs(1, 32, 4, 8192, 8192, 128, seed=41))
    torch.cuda.synchronize()
    ws_dec = fa.fa_decode_splitkv_workspace_bytes(4, 16, 3000, 128, 256)
    ws_bwd = fa.fa_backward_workspace_bytes(1, 4, 300)
    s = torch.cuda.Stream()
    assert torch.cuda.current_stream() != s
    for _ in range(3):
        fa.fa_forward(qp, kp, vp, causal=True, stream=s)  # keeps s busy for ~1.5 ms
        dec = fa.fa_decode_splitkv(q, kc, vc, ld, chunk=256, stream=s)
        bwd = fa.fa_backward(qb, kb, vb, ob, lb, dob, causal=True, stream=s)
        junk = [torch.full((n,), 255, dtype=torch.uint8, device=dev) for n in (ws_dec, ws_bwd)]
        s.synchronize()
        torch.cuda.synchronize()
        del junk
        for x, y in zip(ref_dec + ref_bwd, list(dec) + list(bwd)):
            assert torch.equal(x, y), "result changed when the stream was not current"
