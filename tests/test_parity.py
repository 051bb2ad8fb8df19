"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (stated for the bf16 workloads, derived for fp32 in the design notes):
  bf16 inputs: O max abs <= 1e-2, O mean abs <= 1e-3, LSE max abs <= 1e-3;
  fp32 inputs: O and LSE max abs <= 1e-5.
Both sides see the same seeded inputs (``workloads``); the oracle upcasts the
exact bf16/fp32 values to fp64.  Large workloads are checked on sampled
(head, row-block) slices the oracle computes directly, at full size and in the
same launch configuration the benchmark times.
"""
import math

import pytest
import torch

import io_aware_attention_attn_amd as fa
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL_BF16 = dict(o_max=1e-2, o_mean=1e-3, lse_max=1e-3)
TOL_F32 = dict(o_max=1e-5, o_mean=1e-5, lse_max=1e-5)


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def _cmp(o_gpu, lse_gpu, o_ref, lse_ref, tol, what):
    o_gpu = o_gpu.double()
    lse_gpu = lse_gpu.double()
    assert torch.isfinite(o_gpu).all(), f"{what}: non-finite O"
    assert torch.isfinite(lse_gpu).all(), f"{what}: non-finite LSE"
    e = (o_gpu - o_ref).abs()
    el = (lse_gpu - lse_ref).abs()
    msg = (f"{what}: O max {e.max().item():.3e} mean {e.mean().item():.3e}, "
           f"LSE max {el.max().item():.3e}")
    print(msg, flush=True)
    assert e.max().item() <= tol["o_max"], msg
    assert e.mean().item() <= tol["o_mean"], msg
    assert el.max().item() <= tol["lse_max"], msg


def _run_forward(q, k, v, scale, causal, f32=False, poison=True):
    dev = _dev()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    B, Nq, Hq, d = q.shape
    o = torch.full((B, Nq, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=dev)
    if not poison:
        o.zero_()
        lse.zero_()
    fn = fa.fa_forward_f32 if f32 else fa.fa_forward
    fn(qd, kd, vd, scale=scale, causal=causal, o=o, lse=lse)
    torch.cuda.synchronize()
    return o, lse


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def test_c1_fp32_full():
    cfg = W.CONFIGS["c1"]
    q, k, v = W.prefill_inputs_for(cfg)
    o, lse = _run_forward(q, k, v, cfg.scale, cfg.causal, f32=True)
    o_ref, lse_ref = oracle.attention(q, k, v, cfg.scale, cfg.causal)
    _cmp(o.cpu(), lse.cpu(), o_ref, lse_ref, TOL_F32, "c1")


def test_c2_full():
    cfg = W.CONFIGS["c2"]
    q, k, v = W.prefill_inputs_for(cfg)
    o, lse = _run_forward(q, k, v, cfg.scale, cfg.causal)
    o_ref, lse_ref = oracle.attention(q, k, v, cfg.scale, cfg.causal)
    _cmp(o.cpu(), lse.cpu(), o_ref, lse_ref, TOL_BF16, "c2")


def _sampled(cfg, heads, row_blocks):
    q, k, v = W.prefill_inputs_for(cfg)
    o, lse = _run_forward(q, k, v, cfg.scale, cfg.causal)
    o, lse = o.cpu(), lse.cpu()
    for h in heads:
        for (r0, r1) in row_blocks:
            o_ref, lse_ref = oracle.attention(q, k, v, cfg.scale, cfg.causal, heads=[h],
                                              rows=(r0, r1), row_block=512)
            _cmp(o[:, r0:r1, h], lse[:, h, r0:r1], o_ref[:, r0:r1, h], lse_ref[:, h, r0:r1],
                 TOL_BF16, f"{cfg.name} head {h} rows {r0}:{r1}")
    # every element written and finite
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_c3_full():
    """The peaky 8K causal MHA workload (Q, K x1.5: scores spread widely, so the exponent
    reference moves often) compared on every element of O and LSE: the oracle's full
    standard attention, row-blocked, on all 32 heads."""
    cfg = W.CONFIGS["c3"]
    q, k, v = W.prefill_inputs_for(cfg)
    o, lse = _run_forward(q, k, v, cfg.scale, cfg.causal)
    print("[c3] GPU done, oracle running", flush=True)
    o_ref, lse_ref = oracle.attention(q, k, v, cfg.scale, cfg.causal, row_block=2048)
    _cmp(o.cpu(), lse.cpu(), o_ref, lse_ref, TOL_BF16, "c3 (every element)")


def test_c4_sampled():
    cfg = W.CONFIGS["c4"]
    N = cfg.Nq
    _sampled(cfg, heads=[0, 7, 8, 37, 63],
             row_blocks=[(0, 256), (16320, 16450), (N - 256, N)])


def test_c4_every_head_sampled_rows():
    """Every one of c4's 64 query heads (so every GQA head-to-K/V-head pairing) at eight row
    ranges of four rows spread over the whole sequence (first and last tiles, a 128-row tile
    boundary, the middle, the ragged end of the causal span), against the oracle on that
    head's slice."""
    cfg = W.CONFIGS["c4"]
    N, G = cfg.Nq, cfg.Hq // cfg.Hkv
    q, k, v = W.prefill_inputs_for(cfg)
    o, lse = _run_forward(q, k, v, cfg.scale, cfg.causal)
    o, lse = o.cpu(), lse.cpu()
    starts = (0, 60, 124, 8188, 16380, 24572, N - 132, N - 4)
    for h in range(cfg.Hq):
        qh, kh, vh = q[:, :, h:h + 1], k[:, :, h // G:h // G + 1], v[:, :, h // G:h // G + 1]
        for r0 in starts:
            o_ref, lse_ref = oracle.attention(qh, kh, vh, cfg.scale, cfg.causal, rows=(r0, r0 + 4))
            _cmp(o[:, r0:r0 + 4, h], lse[:, h, r0:r0 + 4], o_ref[:, r0:r0 + 4, 0],
                 lse_ref[:, 0, r0:r0 + 4], TOL_BF16, f"c4 head {h} rows {r0}:{r0 + 4}")


def test_prefill_max_offsets():
    """The longest sequence the host accepts for Hq = 64, Hkv = 8, d = 128: one batch
    slice of O just under 2^31 bytes (N = 65279, odd, so the last tile is ragged).  Rows at
    both ends of the first and the last query head, causal, against the oracle on that
    head's slice."""
    B, Hq, Hkv, d = 1, 64, 8, 128
    N = (2 ** 31 - 1) // (Hq * d * 4) - 256
    assert N == 65279
    scale = 1.0 / math.sqrt(d)
    q, k, v = W.prefill_inputs(B, Hq, Hkv, N, N, d, "bf16", seed=41)
    o, lse = _run_forward(q, k, v, scale, True)
    o, lse = o.cpu(), lse.cpu()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    G = Hq // Hkv
    for h in (0, Hq - 1):
        qh, kh, vh = q[:, :, h:h + 1], k[:, :, h // G:h // G + 1], v[:, :, h // G:h // G + 1]
        for (r0, r1) in ((0, 64), (N - 64, N)):
            o_ref, lse_ref = oracle.attention(qh, kh, vh, scale, True, rows=(r0, r1),
                                              row_block=64)
            _cmp(o[:, r0:r1, h], lse[:, h, r0:r1], o_ref[:, r0:r1, 0], lse_ref[:, 0, r0:r1],
                 TOL_BF16, f"N={N} head {h} rows {r0}:{r1}")


def test_decode_max_offsets():
    """One sequence filling the largest contiguous cache the host accepts for Hkv = 8,
    d = 128: (Nk_max + 64) * Hkv * d * 2 just under 2^31 bytes, so the last K/V head's last
    rows sit at byte offsets just below 2^31.  K/V heads 0 and 7 against the oracle on
    their slices."""
    B, Hq, Hkv, d = 1, 8, 8, 128
    Nk_max = (2 ** 31 - 1) // (Hkv * d * 2) - 64
    assert Nk_max == 1048511
    scale = 1.0 / math.sqrt(d)
    lengths, q, kc, vc = W.decode_inputs(B, Hq, Hkv, d, Nk_max, 0, 0, seed=42,
                                         lengths=torch.tensor([Nk_max], dtype=torch.int32))
    dev = _dev()
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    fa.fa_decode_splitkv(q.to(dev), kc.to(dev), vc.to(dev), lengths.to(dev), scale=scale,
                         chunk=256, o=o, lse=lse)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    for h in (0, Hkv - 1):
        o_ref, lse_ref = oracle.decode_attention(q[:, h:h + 1], kc[:, :, h:h + 1],
                                                 vc[:, :, h:h + 1], lengths, scale)
        _cmp(o[:, h:h + 1], lse[:, h:h + 1], o_ref, lse_ref, TOL_BF16,
             f"decode Nk_max={Nk_max} K/V head {h}")


def test_c5_decode_full():
    cfg = W.CONFIGS["c5"]
    lengths, q, kc, vc = W.decode_inputs_for(cfg)
    dev = _dev()
    o = torch.full((cfg.B, cfg.Hq, cfg.d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((cfg.B, cfg.Hq), float("nan"), dtype=torch.float32, device=dev)
    fa.fa_decode_splitkv(q.to(dev), kc.to(dev), vc.to(dev), lengths.to(dev), scale=cfg.scale,
                         chunk=cfg.chunk, o=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_attention(q, kc, vc, lengths, cfg.scale)
    _cmp(o.cpu(), lse.cpu(), o_ref, lse_ref, TOL_BF16, "c5")


# ---------------------------------------------------------------------------
# edge shapes, full oracle
# ---------------------------------------------------------------------------

# These grids hold at most two workgroups per CU, so every shape with Nk > 128 runs the
# kernel's two-key-group form (alternate key blocks per group, states merged at the end);
# the Nk <= 128 shapes and the larger c2-c4 workloads run the plain form.
EDGE = [  # B, Nq, Nk, Hq, Hkv, d, causal, gain
    (1, 1, 1, 1, 1, 64, True, 1.0),
    (1, 1, 1000, 2, 1, 128, False, 1.0),
    (1, 1, 1000, 2, 1, 128, True, 1.0),
    (1, 200, 200, 2, 2, 64, True, 1.0),
    (1, 200, 200, 2, 2, 128, False, 1.0),
    (2, 77, 300, 4, 2, 128, True, 1.0),
    (1, 300, 77, 2, 1, 64, False, 1.0),
    (1, 129, 129, 8, 1, 128, True, 1.0),
    (1, 255, 513, 16, 2, 64, True, 1.0),
    (1, 384, 384, 2, 2, 128, True, 3.0),   # very peaky scores: many max changes
    (3, 64, 64, 3, 3, 64, False, 2.0),
    (1, 1100, 1100, 2, 1, 128, True, 1.0),
    # scores hundreds apart: exp would overflow without the reference shift, rows are
    # close to one-hot, and nearly every block moves the reference
    (1, 256, 256, 2, 1, 128, True, 10.0),
    (2, 100, 500, 2, 2, 64, False, 10.0),
    # (batch, K/V head) groups that do not divide over the 8 XCDs while their query blocks
    # do: the workgroups take the snake assignment of bundles to XCDs
    (1, 1024, 1024, 8, 2, 128, True, 1.0),
    (2, 512, 700, 6, 3, 64, True, 1.0),
    (1, 1000, 1000, 4, 1, 128, True, 1.0),
]


@pytest.mark.parametrize("shape", EDGE, ids=[str(s) for s in EDGE])
def test_edge_bf16(shape):
    B, Nq, Nk, Hq, Hkv, d, causal, gain = shape
    q, k, v = W.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", seed=7, qk_gain=gain)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_forward(q, k, v, scale, causal)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    _cmp(o.cpu(), lse.cpu(), o_ref, lse_ref, TOL_BF16, f"bf16 {shape}")


@pytest.mark.parametrize("shape", EDGE[:9], ids=[str(s) for s in EDGE[:9]])
def test_edge_f32(shape):
    B, Nq, Nk, Hq, Hkv, d, causal, gain = shape
    q, k, v = W.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, "f32", seed=8, qk_gain=gain)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_forward(q, k, v, scale, causal, f32=True)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal)
    _cmp(o.cpu(), lse.cpu(), o_ref, lse_ref, TOL_F32, f"f32 {shape}")


def test_worked_example_on_gpu():
    """The pages' three-token example (d_k = 2) cannot run at d = 2; embedded in d = 64 with
    zero padding it must give the same P-weighted output [0.802, 0.797]."""
    q = torch.zeros((1, 1, 1, 64), dtype=torch.float32)
    k = torch.zeros((1, 3, 1, 64), dtype=torch.float32)
    v = torch.zeros((1, 3, 1, 64), dtype=torch.float32)
    q[0, 0, 0, :2] = torch.tensor([1.0, 0.0])
    k[0, :, 0, :2] = torch.tensor([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    v[0, :, 0, :2] = torch.tensor([[1.0, 0.0], [0.0, 2.0], [1.0, 1.0]])
    a = math.exp(1 / math.sqrt(2))
    want = torch.tensor([2 * a / (2 * a + 1), (a + 2) / (2 * a + 1)], dtype=torch.float64)
    for f32 in (True, False):
        qq, kk, vv = (q, k, v) if f32 else (q.bfloat16(), k.bfloat16(), v.bfloat16())
        o, lse = _run_forward(qq, kk, vv, 1 / math.sqrt(2), False, f32=f32)
        tol = 1e-5 if f32 else 1e-2
        assert (o.cpu()[0, 0, 0, :2].double() - want).abs().max() <= tol
        assert abs(lse.cpu()[0, 0, 0].item() - math.log(2 * a + 1)) <= tol


# ---------------------------------------------------------------------------
# decode edge cases
# ---------------------------------------------------------------------------

DEC = [  # B, Hq, Hkv, d, Nk_max, lengths, chunk
    (4, 8, 1, 128, 1024, [1, 255, 256, 257], 256),
    (3, 16, 2, 128, 600, [511, 512, 600], 256),
    (2, 8, 8, 64, 700, [1, 700], 64),
    (2, 32, 1, 128, 2048, [2048, 1000], 512),   # 32 heads per K/V head: two head groups
    (2, 4, 2, 64, 300, [300, 63], 128),
    (3, 8, 2, 128, 3000, [2000, 3000, 1500], 1024),  # pieces of at least 16 steps
    # many short sequences: one wave's run of steps crosses several (batch, head) segments
    (40, 8, 2, 64, 200, [1 + (37 * i) % 200 for i in range(40)], 64),
    # more than 64 sequences (lengths read from memory, not kept one per lane)
    (70, 4, 1, 64, 130, [1 + (53 * i) % 130 for i in range(70)], 64),
]


@pytest.mark.parametrize("case", DEC, ids=[str(c[:5]) for c in DEC])
def test_decode_edges(case):
    B, Hq, Hkv, d, Nk_max, lens, chunk = case
    lengths = torch.tensor(lens, dtype=torch.int32)
    lengths, q, kc, vc = W.decode_inputs(B, Hq, Hkv, d, Nk_max, 0, 0, seed=11, lengths=lengths)
    dev = _dev()
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    scale = 1 / math.sqrt(d)
    fa.fa_decode_splitkv(q.to(dev), kc.to(dev), vc.to(dev), lengths.to(dev), scale=scale,
                         chunk=chunk, o=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_attention(q, kc, vc, lengths, scale)
    _cmp(o.cpu(), lse.cpu(), o_ref, lse_ref, TOL_BF16, f"decode {case}")


def test_decode_empty_sequences():
    """A sequence with no cached key gets O = 0 and LSE = -inf (the header's documented
    clamp); the work of the other sequences is unaffected."""
    lens = [0, 300, 0, 1, 0]
    B, Hq, Hkv, d, Nk_max = len(lens), 8, 2, 128, 512
    lengths = torch.tensor(lens, dtype=torch.int32)
    lengths, q, kc, vc = W.decode_inputs(B, Hq, Hkv, d, Nk_max, 0, 0, seed=12, lengths=lengths)
    dev = _dev()
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    scale = 1 / math.sqrt(d)
    fa.fa_decode_splitkv(q.to(dev), kc.to(dev), vc.to(dev), lengths.to(dev), scale=scale,
                         chunk=64, o=o, lse=lse)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    live = [b for b, L in enumerate(lens) if L > 0]
    o_ref, lse_ref = oracle.decode_attention(q, kc, vc, lengths, scale, batches=live)
    _cmp(o[live], lse[live], o_ref[live], lse_ref[live], TOL_BF16, "decode live rows")
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.all(o[b] == 0) and torch.all(lse[b] == float("-inf")), b


# ---------------------------------------------------------------------------
# paged KV-cache decode ([LLM-basics] ②-8, PagedAttention)
# ---------------------------------------------------------------------------

def _run_paged(q, kp, vp, table, lengths, scale, chunk):
    dev = _dev()
    B, Hq, d = q.shape
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    fa.fa_decode_paged(q.to(dev), kp.to(dev), vp.to(dev), table.to(dev), lengths.to(dev),
                       scale=scale, chunk=chunk, o=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def test_c5_decode_paged_full():
    """The c5 decode with its cache scattered over a permuted pool of 256-key pages."""
    cfg = W.CONFIGS["c5"]
    lengths, q, kc, vc = W.decode_inputs_for(cfg)
    kp, vp, table = W.paged_from_contiguous(kc, vc, lengths, 256, seed=7, spare_pages=9)
    o, lse = _run_paged(q, kp, vp, table, lengths, cfg.scale, cfg.chunk)
    o_ref, lse_ref = oracle.decode_attention_paged(q, kp, vp, table, lengths, 256, cfg.scale)
    _cmp(o, lse, o_ref, lse_ref, TOL_BF16, "c5 paged")


def test_c5_decode_kv_cache_empty():
    """The c5 decode on caches (contiguous, then a page pool) laid out by the library's
    allocation helper, one buffer with V 256 bytes past K's 1 KiB congruence class: the
    same results as the oracle (and bitwise the same as on separate allocations)."""
    cfg = W.CONFIGS["c5"]
    lengths, q, kc, vc = W.decode_inputs_for(cfg)
    dev = _dev()
    k2, v2 = fa.kv_cache_empty(kc.shape, device=dev)
    k2.copy_(kc.to(dev))
    v2.copy_(vc.to(dev))
    assert (v2.data_ptr() - k2.data_ptr()) % 1024 == 256
    qd, ld = q.to(dev), lengths.to(dev)
    o, lse = fa.fa_decode_splitkv(qd, k2, v2, ld, scale=cfg.scale, chunk=cfg.chunk)
    o_sep, lse_sep = fa.fa_decode_splitkv(qd, kc.to(dev), vc.to(dev), ld, scale=cfg.scale,
                                          chunk=cfg.chunk)
    torch.cuda.synchronize()
    assert torch.equal(o, o_sep) and torch.equal(lse, lse_sep)
    o_ref, lse_ref = oracle.decode_attention(q, kc, vc, lengths, cfg.scale)
    _cmp(o.cpu(), lse.cpu(), o_ref, lse_ref, TOL_BF16, "c5 kv_cache_empty")
    del k2, v2
    kp, vp, table = W.paged_from_contiguous(kc, vc, lengths, 256, seed=7, spare_pages=9)
    kp2, vp2 = fa.kv_cache_empty(kp.shape, device=dev)
    kp2.copy_(kp.to(dev))
    vp2.copy_(vp.to(dev))
    o, lse = fa.fa_decode_paged(qd, kp2, vp2, table.to(dev), ld, scale=cfg.scale,
                                chunk=cfg.chunk)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_attention_paged(q, kp, vp, table, lengths, 256, cfg.scale)
    _cmp(o.cpu(), lse.cpu(), o_ref, lse_ref, TOL_BF16, "c5 paged kv_cache_empty")


PAGED = [  # B, Hq, Hkv, d, page_size, lengths, chunk
    (3, 8, 2, 128, 64, [1, 64, 130], 64),
    (4, 16, 2, 64, 128, [127, 128, 129, 600], 256),
    (2, 8, 1, 128, 1024, [1000, 2500], 256),          # pages longer than a chunk
    (70, 4, 1, 64, 64, [1 + (41 * i) % 300 for i in range(70)], 64),   # > 64 sequences
]


@pytest.mark.parametrize("case", PAGED, ids=[str(c[:5]) for c in PAGED])
def test_decode_paged_edges(case):
    B, Hq, Hkv, d, ps, lens, chunk = case
    lengths = torch.tensor(lens, dtype=torch.int32)
    Nk_max = ((max(lens) + ps - 1) // ps) * ps
    lengths, q, kc, vc = W.decode_inputs(B, Hq, Hkv, d, Nk_max, 0, 0, seed=21, lengths=lengths)
    kp, vp, table = W.paged_from_contiguous(kc, vc, lengths, ps, seed=22, spare_pages=3)
    scale = 1 / math.sqrt(d)
    o, lse = _run_paged(q, kp, vp, table, lengths, scale, chunk)
    o_ref, lse_ref = oracle.decode_attention_paged(q, kp, vp, table, lengths, ps, scale)
    _cmp(o, lse, o_ref, lse_ref, TOL_BF16, f"paged {case[:5]}")


def test_decode_paged_shared_pages():
    """Sequences that share physical pages (a common prefix, as in the pages' block-table
    figure) and an empty sequence (O = 0, LSE = -inf)."""
    ps, Hq, Hkv, d = 64, 8, 2, 128
    g = torch.Generator("cpu").manual_seed(31)
    num_pages = 12
    kp = torch.randn((num_pages, ps, Hkv, d), generator=g).to(torch.bfloat16)
    vp = torch.randn((num_pages, ps, Hkv, d), generator=g).to(torch.bfloat16)
    table = torch.tensor([[4, 9, 1, 7, -1], [4, 9, 2, -1, -1], [4, 9, 1, 7, 11], [0, -1, -1, -1, -1],
                          [5, 3, -1, -1, -1]], dtype=torch.int32)
    lens = [230, 150, 300, 0, 128]
    lengths = torch.tensor(lens, dtype=torch.int32)
    q = torch.randn((len(lens), Hq, d), generator=g).to(torch.bfloat16)
    o, lse = _run_paged(q, kp, vp, table, lengths, 1 / math.sqrt(d), 64)
    live = [b for b, L in enumerate(lens) if L > 0]
    o_ref, lse_ref = oracle.decode_attention_paged(q, kp, vp, table, lengths, ps, 1 / math.sqrt(d),
                                                   batches=live)
    _cmp(o[live], lse[live], o_ref[live], lse_ref[live], TOL_BF16, "paged shared")
    assert torch.all(o[3] == 0) and torch.all(lse[3] == float("-inf"))


def test_decode_paged_matches_contiguous():
    """Same keys through a page table and through the contiguous cache: the two entry points
    agree to fp32 rounding (the split and the merge are the same; only addressing differs)."""
    cfg = W.CONFIGS["c5"]
    lengths, q, kc, vc = W.decode_inputs(4, 64, 8, 128, 4096, 1000, 4096, seed=41)
    kp, vp, table = W.paged_from_contiguous(kc, vc, lengths, 128, seed=42)
    o1, l1 = _run_paged(q, kp, vp, table, lengths, cfg.scale, 256)
    dev = _dev()
    o2, l2 = fa.fa_decode_splitkv(q.to(dev), kc.to(dev), vc.to(dev), lengths.to(dev),
                                  scale=cfg.scale, chunk=256)
    torch.cuda.synchronize()
    assert (o1 - o2.cpu()).abs().max().item() <= 1e-6
    assert (l1 - l2.cpu()).abs().max().item() <= 1e-6


# ---------------------------------------------------------------------------
# determinism and stream behaviour
# ---------------------------------------------------------------------------

def test_bitwise_deterministic():
    q, k, v = W.prefill_inputs(1, 4, 2, 700, 700, 128, "bf16", seed=3)
    o1, l1 = _run_forward(q, k, v, 0.09, True)
    o2, l2 = _run_forward(q, k, v, 0.09, True, poison=False)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    lengths, qd, kc, vc = W.decode_inputs(2, 8, 1, 128, 900, 0, 0, seed=4,
                                          lengths=torch.tensor([900, 333], dtype=torch.int32))
    dev = _dev()
    args = (qd.to(dev), kc.to(dev), vc.to(dev), lengths.to(dev))
    a = fa.fa_decode_splitkv(*args)
    b = fa.fa_decode_splitkv(*args)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_runs_on_caller_stream():
    q, k, v = W.prefill_inputs(1, 2, 2, 256, 256, 64, "bf16", seed=5)
    dev = _dev()
    s = torch.cuda.Stream()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, lse = fa.fa_forward(qd, kd, vd, causal=True)
    s.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, 1 / 8, True)
    _cmp(o.cpu(), lse.cpu(), o_ref, lse_ref, TOL_BF16, "side stream")
