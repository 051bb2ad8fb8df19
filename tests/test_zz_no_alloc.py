"""The allocation-free decode entry point (fa_decode_splitkv_noalloc) through the C ABI.

It must give what fa_decode_splitkv gives with a caller workspace: the kernels are the
same and deterministic, so the outputs are compared bit for bit (which is within the
decode's tolerance against the oracle, checked here too).  Two calls run back to back
with the second one smaller, then the first again: the scratch array keeps the last
call's partial results, and none of them may leak into the next call.
"""
import ctypes
import math

import pytest
import torch

import io_aware_attention_attn_amd as fa
import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def _case(B, Hq, Hkv, d, Nk_max, lo, hi, seed, chunk):
    dev = _dev()
    lengths, q, kc, vc = W.decode_inputs(B, Hq, Hkv, d, Nk_max, lo, hi, seed=seed)
    return dict(lengths=lengths, q=q, kc=kc, vc=vc, chunk=chunk, scale=1.0 / math.sqrt(d),
                dq=q.to(dev), dkc=kc.to(dev), dvc=vc.to(dev), dl=lengths.to(dev))


def _noalloc(c):
    """One call of the C entry point on torch's current stream; outputs poisoned first."""
    dev = _dev()
    B, Hq, d = c["q"].shape
    _, Nk_max, Hkv, _ = c["kc"].shape
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    st = fa.lib().fa_decode_splitkv_noalloc(
        c["dq"].data_ptr(), c["dkc"].data_ptr(), c["dvc"].data_ptr(), c["dl"].data_ptr(),
        o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nk_max, d, ctypes.c_float(c["scale"]),
        c["chunk"], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == fa.FA_OK, fa.fa_status_str(st)
    return o, lse


def _with_workspace(c):
    o, lse = fa.fa_decode_splitkv(c["dq"], c["dkc"], c["dvc"], c["dl"], scale=c["scale"],
                                  chunk=c["chunk"])
    return o, lse


def _check(c, what):
    print(f"[no_alloc] {what}: B={c['q'].shape[0]} Hq={c['q'].shape[1]} "
          f"Hkv={c['kc'].shape[2]} d={c['q'].shape[2]} Nk_max={c['kc'].shape[1]} "
          f"chunk={c['chunk']}", flush=True)
    o1, l1 = _noalloc(c)
    o2, l2 = _with_workspace(c)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all() and torch.isfinite(l1).all(), what
    assert torch.equal(o1, o2), f"{what}: O differs from fa_decode_splitkv"
    assert torch.equal(l1, l2), f"{what}: LSE differs from fa_decode_splitkv"
    o_ref, l_ref = oracle.decode_attention(c["q"], c["kc"], c["vc"], c["lengths"], c["scale"])
    e = (o1.cpu().double() - o_ref).abs()
    el = (l1.cpu().double() - l_ref).abs()
    assert e.max().item() <= 1e-2 and e.mean().item() <= 1e-3 and el.max().item() <= 1e-3, \
        f"{what}: O max {e.max().item():.3e} mean {e.mean().item():.3e} LSE {el.max().item():.3e}"


def test_noalloc_matches_workspace_entry_point_twice():
    big = _case(8, 32, 4, 128, 12000, 1, 12000, seed=51, chunk=256)
    small = _case(3, 8, 2, 64, 700, 1, 700, seed=52, chunk=128)
    _check(big, "first call")
    _check(small, "second call, smaller")
    _check(big, "first shape again")


def test_noalloc_rejects_oversized_request():
    """A request whose partial results exceed the 80 MiB scratch is refused (status only;
    validation returns before anything is launched)."""
    dev = _dev()
    t = torch.zeros(16, dtype=torch.float32, device=dev)
    p = t.data_ptr()
    st = fa.lib().fa_decode_splitkv_noalloc(p, p, p, p, p, p, 20, 64, 8, 32768, 128,
                                            ctypes.c_float(0.1), 256, None)
    assert st == fa.FA_ERR_SCRATCH
