"""GPU parity of the packed variable-length prefill (fa_forward_varlen) against the oracle.

Tolerances are those of the bf16 prefill (O max abs <= 1e-2, mean <= 1e-3, LSE max
abs <= 1e-3).  Query rows that see no key (a sequence without keys, or causal rows
ahead of every key when a sequence has more queries than keys) have no softmax in
the oracle (it leaves them NaN); the library's convention for them is O = 0 and
LSE = -inf, checked exactly.  Outputs are poisoned with NaN before each call, so an
element the kernel never writes shows up.
"""
import pytest
import torch

import io_aware_attention_attn_amd as fa
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = dict(o_max=1e-2, o_mean=1e-3, lse_max=1e-3)


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def _run(q, k, v, cu_q, cu_k, max_q, max_k, causal, scale=None):
    dev = _dev()
    tq, Hq, d = q.shape
    o = torch.full((tq, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((Hq, tq), float("nan"), dtype=torch.float32, device=dev)
    fa.fa_forward_varlen(q, k, v, cu_q.to(dev), cu_k.to(dev), max_q, max_k, scale=scale,
                         causal=causal, o=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _to_dev_views(qkv_views):
    """Move q, k, v to the GPU keeping their token strides (views of one tensor stay views)."""
    dev = _dev()
    base = qkv_views[0]._base if qkv_views[0]._base is not None else None
    if base is not None and all(t._base is base for t in qkv_views):
        based = base.to(dev)
        out = []
        for t in qkv_views:
            off = t.storage_offset() - base.storage_offset()
            out.append(based.as_strided(t.shape, t.stride(), based.storage_offset() + off))
        return out
    return [t.to(dev) for t in qkv_views]


def _sees_a_key(lens_q, lens_k, causal):
    """Per packed query row: does it see at least one key (from the sizes alone)."""
    rows = []
    for nq, nk in zip(lens_q, lens_k):
        for i in range(nq):
            rows.append(nk > 0 and (not causal or i + (nk - nq) >= 0))
    return torch.tensor(rows, dtype=torch.bool)


def _check(o, lse, o_ref, lse_ref, has_key, what):
    # the oracle's undefined rows are exactly the rows without a visible key
    ref_nan = torch.isnan(lse_ref).any(dim=0)
    assert torch.equal(ref_nan, ~has_key), f"{what}: oracle NaN rows differ from keyless rows"
    if (~has_key).any():
        assert (o[~has_key] == 0).all(), f"{what}: keyless rows must have O = 0"
        assert torch.isneginf(lse[:, ~has_key]).all(), f"{what}: keyless rows need LSE = -inf"
    if has_key.any():
        og, orf = o[has_key].double(), o_ref[has_key]
        lg, lrf = lse[:, has_key].double(), lse_ref[:, has_key]
        assert torch.isfinite(og).all() and torch.isfinite(lg).all(), f"{what}: non-finite"
        e, el = (og - orf).abs(), (lg - lrf).abs()
        msg = (f"{what}: O max {e.max().item():.3e} mean {e.mean().item():.3e}, "
               f"LSE max {el.max().item():.3e}")
        print(msg, flush=True)
        assert e.max().item() <= TOL["o_max"], msg
        assert e.mean().item() <= TOL["o_mean"], msg
        assert el.max().item() <= TOL["lse_max"], msg


MIXED = [
    # (lens_q, lens_k, Hq, Hkv, d, causal)
    ([1, 63, 0, 128, 129, 300, 7, 257], None, 4, 2, 64, True),
    ([1, 63, 0, 128, 129, 300, 7, 257], None, 4, 2, 64, False),
    ([200, 1, 0, 0, 385, 64, 65], None, 4, 1, 128, True),
    ([200, 1, 0, 0, 385, 64, 65], None, 2, 2, 128, False),
    # queries and keys of different lengths, keyless sequences, causal rows ahead of keys
    ([5, 100, 64, 0, 200, 3, 130], [300, 100, 0, 50, 130, 1, 0], 4, 2, 64, False),
    ([5, 100, 64, 0, 200, 3, 130], [300, 100, 0, 50, 130, 1, 0], 4, 2, 64, True),
    ([5, 100, 64, 0, 200, 3, 130], [300, 100, 0, 50, 130, 1, 0], 8, 2, 128, True),
    # K/V heads a multiple of the XCD count (the K/V-head-major work order)
    ([100, 300, 1, 129, 0, 64], None, 16, 8, 64, True),
    ([100, 300, 1, 129, 0, 64], [90, 310, 0, 129, 5, 64], 8, 8, 128, False),
]


@pytest.mark.parametrize("case", MIXED, ids=[f"{i}" for i in range(len(MIXED))])
def test_varlen_mixed(case):
    lens_q, lens_k, Hq, Hkv, d, causal = case
    lens_k = lens_q if lens_k is None else lens_k
    print(f"varlen case lens_q={lens_q} lens_k={lens_k} Hq={Hq} Hkv={Hkv} d={d} "
          f"causal={causal}", flush=True)
    cu_q, cu_k, q, k, v = W.varlen_inputs(lens_q, lens_k, Hq, Hkv, d, seed=3)
    dev = _dev()
    o, lse = _run(q.to(dev), k.to(dev), v.to(dev), cu_q, cu_k, max(lens_q), max(lens_k), causal)
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, cu_q, cu_k, d ** -0.5, causal)
    _check(o, lse, o_ref, lse_ref, _sees_a_key(lens_q, lens_k, causal), f"varlen {case}")


def test_varlen_packed_qkv_view():
    """q, k, v as head-range views of one [total, Hq + 2 Hkv, d] tensor (the fused QKV
    layout of the pages' packed example, H = 12, d = 64), several ragged sequences."""
    lens = [2048, 1000, 17, 513]
    Hq = Hkv = 12
    d = 64
    cu_q, cu_k, q, k, v = W.varlen_inputs(lens, lens, Hq, Hkv, d, seed=4, packed_qkv=True)
    qd, kd, vd = _to_dev_views([q, k, v])
    assert qd.stride(0) == (Hq + 2 * Hkv) * d and qd.data_ptr() + Hq * d * 2 == kd.data_ptr()
    o, lse = _run(qd, kd, vd, cu_q, cu_k, max(lens), max(lens), True)
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, cu_q, cu_k, d ** -0.5, True)
    _check(o, lse, o_ref, lse_ref, _sees_a_key(lens, lens, True), "packed qkv")


@pytest.mark.parametrize("d,causal", [(128, True), (64, False)])
def test_varlen_equals_fixed_length_bitwise(d, causal):
    """Equal lengths: the packed launch runs the same blocks with the same arithmetic as
    fa_forward, so O and LSE agree bit for bit (only the layout differs).  The grid (576
    workgroups) is above two per CU, where fa_forward would split the key loop of each
    workgroup over two key groups."""
    B, N, Hq, Hkv = 3, 2048, 12, 4
    dev = _dev()
    q, k, v = W.prefill_inputs(B, Hq, Hkv, N, N, d, seed=5)
    o_f, lse_f = fa.fa_forward(q.to(dev), k.to(dev), v.to(dev), causal=causal)
    cu = W.cu_seqlens([N] * B)
    o_v, lse_v = _run(q.reshape(B * N, Hq, d).to(dev), k.reshape(B * N, Hkv, d).to(dev),
                      v.reshape(B * N, Hkv, d).to(dev), cu, cu, N, N, causal)
    torch.cuda.synchronize()
    assert torch.equal(o_f.cpu().reshape(B * N, Hq, d), o_v)
    assert torch.equal(lse_f.cpu().permute(1, 0, 2).reshape(Hq, B * N), lse_v)


def test_varlen_rejects_bad_views():
    dev = _dev()
    q = torch.zeros((10, 4, 64), dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, 10], dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):   # heads not dense
        fa.fa_forward_varlen(q[:, ::2], q[:, :2], q[:, :2], cu, cu, 10, 10)
    with pytest.raises(fa.FAError):   # longest sequence longer than the pack
        fa.fa_forward_varlen(q, q[:, :2], q[:, :2], cu, cu, 11, 10)


def test_v1_sampled():
    """The full-size packed workload (16 long-context GQA sequences, lengths
    U[512, 16384], causal), in the launch the benchmark times; sampled heads and row
    blocks of the shortest, the longest and a middle sequence against the oracle."""
    cfg = W.VARLEN["v1"]
    lengths, cu_q, cu_k, q, k, v = W.varlen_inputs_for(cfg)
    dev = _dev()
    Lmax = int(lengths.max())
    o, lse = _run(q.to(dev), k.to(dev), v.to(dev), cu_q, cu_k, Lmax, Lmax, cfg.causal)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    Ls = [int(x) for x in lengths]
    picks = sorted({Ls.index(min(Ls)), Ls.index(max(Ls)), 4})
    for b in picks:
        s0, L = int(cu_q[b]), Ls[b]
        qs, ks, vs = q[s0:s0 + L].unsqueeze(0), k[s0:s0 + L].unsqueeze(0), v[s0:s0 + L].unsqueeze(0)
        for h in (0, 37, 63):
            for (r0, r1) in [(0, 200), (L // 2 - 64, L // 2 + 70), (L - 200, L)]:
                o_ref, lse_ref = oracle.attention(qs, ks, vs, cfg.scale, cfg.causal, heads=[h],
                                                  rows=(r0, r1), row_block=512)
                e = (o[s0 + r0:s0 + r1, h].double() - o_ref[0, r0:r1, h]).abs()
                el = (lse[h, s0 + r0:s0 + r1].double() - lse_ref[0, h, r0:r1]).abs()
                msg = (f"v1 seq {b} (L={L}) head {h} rows {r0}:{r1}: O max {e.max().item():.3e} "
                       f"mean {e.mean().item():.3e} LSE max {el.max().item():.3e}")
                print(msg, flush=True)
                assert e.max().item() <= TOL["o_max"], msg
                assert e.mean().item() <= TOL["o_mean"], msg
                assert el.max().item() <= TOL["lse_max"], msg
