"""The C-ABI library on the CPU: it loads, exports every symbol include/fa.h declares,
and rejects invalid arguments with the documented status before any HIP call.

Only calls that fail validation are made here (no device is needed for those);
nothing is launched.  Pointer arguments are fake, aligned, non-null addresses:
validation returns before they could ever be dereferenced.
"""
import ctypes
import os
import re

import pytest

import io_aware_attention_attn_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

P = 0x10000          # fake, 16-byte aligned, never dereferenced
MIS = 0x10004        # 4-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.LIB_PATH):
        pytest.skip("libfa.so not built (run python -m io_aware_attention_attn_amd._build)")
    return fa.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == {"fa_forward", "fa_forward_f32", "fa_forward_fp8", "fa_forward_varlen",
                          "fa_backward_workspace_bytes", "fa_backward",
                          "fa_decode_splitkv_workspace_bytes",
                          "fa_decode_splitkv", "fa_decode_splitkv_noalloc", "fa_decode_paged",
                          "fa_status_str", "fa_probe_mfma_bf16_operand_bytes",
                          "fa_probe_mfma_bf16", "fa_probe_stream_read"}
    for n in names:
        assert hasattr(L, n), f"libfa.so does not export {n}"


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        s = fa.fa_status_str(st)
        assert s.startswith("FA_"), s
    assert "unknown" in fa.fa_status_str(-99)


def _fwd(L, entry, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=64, scale=0.125,
         causal=0):
    return getattr(L, entry)(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, None)


@pytest.mark.parametrize("entry", ["fa_forward", "fa_forward_f32"])
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL),
    (dict(k=None), fa.FA_ERR_NULL),
    (dict(v=None), fa.FA_ERR_NULL),
    (dict(o=None), fa.FA_ERR_NULL),
    (dict(lse=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE),
    (dict(Hq=-1), fa.FA_ERR_SHAPE),
    (dict(Hkv=0), fa.FA_ERR_SHAPE),
    (dict(Nq=0), fa.FA_ERR_SHAPE),
    (dict(Nk=0), fa.FA_ERR_SHAPE),
    (dict(Hq=3, Hkv=2), fa.FA_ERR_SHAPE),
    (dict(Nq=9, Nk=8, causal=1), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(q=MIS), fa.FA_ERR_ALIGN),
    (dict(v=MIS), fa.FA_ERR_ALIGN),
    (dict(o=MIS), fa.FA_ERR_ALIGN),
    (dict(B=1 << 20, Nq=1 << 12, Hq=1 << 10, Hkv=1 << 10, Nk=8), fa.FA_ERR_SHAPE),
    # one batch slice of O at 2^31 bytes: (65280 + 256) x 64 heads x 128 x 4 B (65279 passes)
    (dict(B=1, Hq=64, Hkv=8, Nq=65280, Nk=65280, d=128), fa.FA_ERR_SHAPE),
])
def test_forward_rejects(L, entry, kw, status):
    assert _fwd(L, entry, **kw) == status


def _fp8(L, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=128, scale=0.125,
         causal=0, qd=0.01, kd=0.02, vd=0.03):
    return L.fa_forward_fp8(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, qd, kd, vd,
                            None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL),
    (dict(lse=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE),
    (dict(Nq=9, causal=1), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(k=MIS), fa.FA_ERR_ALIGN),
    (dict(qd=0.0), fa.FA_ERR_SHAPE),
    (dict(kd=-1.0), fa.FA_ERR_SHAPE),
    (dict(vd=float("nan")), fa.FA_ERR_SHAPE),
    (dict(vd=float("inf")), fa.FA_ERR_SHAPE),
])
def test_fp8_rejects(L, kw, status):
    assert _fp8(L, **kw) == status


def _varlen(L, q=P, k=P, v=P, o=P, lse=P, cq=P, ck=P, B=2, Hq=4, Hkv=2, max_q=64, max_k=70,
            total_q=100, total_k=120, d=64, scale=0.125, causal=0, qs=None, ks=None, vs=None):
    qs = Hq * d if qs is None else qs
    ks = Hkv * d if ks is None else ks
    vs = ks if vs is None else vs
    return L.fa_forward_varlen(q, k, v, o, lse, cq, ck, B, Hq, Hkv, max_q, max_k, total_q,
                               total_k, d, scale, causal, qs, ks, vs, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL),
    (dict(v=None), fa.FA_ERR_NULL),
    (dict(lse=None), fa.FA_ERR_NULL),
    (dict(cq=None), fa.FA_ERR_NULL),
    (dict(ck=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE),
    (dict(max_q=0), fa.FA_ERR_SHAPE),
    (dict(total_q=0, max_q=0), fa.FA_ERR_SHAPE),
    (dict(max_q=101), fa.FA_ERR_SHAPE),          # longer than the whole pack
    (dict(max_k=121), fa.FA_ERR_SHAPE),
    (dict(max_k=-1), fa.FA_ERR_SHAPE),
    (dict(total_k=-1), fa.FA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(qs=4 * 64 - 8), fa.FA_ERR_SHAPE),      # row narrower than its heads
    (dict(ks=2 * 64 - 8, vs=2 * 64 - 8), fa.FA_ERR_SHAPE),
    (dict(vs=3 * 64), fa.FA_ERR_SHAPE),          # K and V strides differ
    (dict(qs=4 * 64 + 4), fa.FA_ERR_ALIGN),      # rows not 16-byte aligned
    (dict(ks=2 * 64 + 4, vs=2 * 64 + 4), fa.FA_ERR_ALIGN),
    (dict(k=MIS), fa.FA_ERR_ALIGN),
    (dict(lse=MIS), fa.FA_ERR_ALIGN),
    (dict(cq=0x10002), fa.FA_ERR_ALIGN),
    # one sequence's rows past 2^31 bytes
    (dict(total_q=1 << 22, max_q=1 << 17, Hq=64, Hkv=8, d=128), fa.FA_ERR_SHAPE),
    (dict(total_k=1 << 22, max_k=1 << 20, Hq=64, Hkv=8, d=128), fa.FA_ERR_SHAPE),
])
def test_varlen_rejects(L, kw, status):
    assert _varlen(L, **kw) == status


def _bwd(L, q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Hq=4, Hkv=2, Nq=64, Nk=64,
         d=128, scale=0.1, causal=1, ws=P, ws_bytes=1 << 20):
    return L.fa_backward(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                         ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL),
    (dict(o=None), fa.FA_ERR_NULL),
    (dict(lse=None), fa.FA_ERR_NULL),
    (dict(do=None), fa.FA_ERR_NULL),
    (dict(dq=None), fa.FA_ERR_NULL),
    (dict(dk=None), fa.FA_ERR_NULL),
    (dict(dv=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_SHAPE),
    (dict(Nq=65, Nk=64), fa.FA_ERR_SHAPE),      # causal with more queries than keys
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(do=MIS), fa.FA_ERR_ALIGN),
    (dict(dk=MIS), fa.FA_ERR_ALIGN),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), fa.FA_ERR_WORKSPACE),
    (dict(ws=MIS), fa.FA_ERR_ALIGN),
])
def test_backward_rejects(L, kw, status):
    assert _bwd(L, **kw) == status


def test_backward_workspace_bytes(L):
    assert fa.fa_backward_workspace_bytes(2, 3, 100) == 2 * ((2 * 3 * 100 * 4 + 255) // 256) * 256
    assert fa.fa_backward_workspace_bytes(0, 3, 100) == 0


def test_workspace_bytes(L):
    n = fa.fa_decode_splitkv_workspace_bytes(16, 64, 32768, 128, 256)
    # a (batch, K/V head) of 512 steps of 64 keys, split in runs of at least 4 steps
    # that may start or end inside it: at most 128 + 1 pieces
    pieces = 32768 // 256 + 1
    want_o = 16 * 64 * pieces * 128 * 4
    want_l = 16 * 64 * pieces * 4
    assert n == ((want_o + 255) // 256) * 256 + ((want_l + 255) // 256) * 256
    assert fa.fa_decode_splitkv_workspace_bytes(1, 1, 1, 64, 64) > 0
    for bad in [(0, 1, 1, 64, 256), (1, 1, 0, 64, 256), (1, 1, 1, 80, 256), (1, 1, 1, 64, 100),
                (1, 1, 1, 64, 0)]:
        assert fa.fa_decode_splitkv_workspace_bytes(*bad) == 0, bad


def _dec(L, q=P, kc=P, vc=P, sl=P, o=P, lse=P, B=2, Hq=8, Hkv=2, Nk_max=512, d=128, scale=0.1,
         chunk=256, ws=P, ws_bytes=1 << 30):
    return L.fa_decode_splitkv(q, kc, vc, sl, o, lse, B, Hq, Hkv, Nk_max, d, scale, chunk, ws,
                               ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL),
    (dict(kc=None), fa.FA_ERR_NULL),
    (dict(sl=None), fa.FA_ERR_NULL),
    (dict(lse=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_SHAPE),
    (dict(Nk_max=0), fa.FA_ERR_SHAPE),
    # one sequence's K rows past 2^31 bytes (32-bit offsets): (1048513 + 64) keys x 8 heads
    # x 256 B
    (dict(B=1, Hq=8, Hkv=8, Nk_max=1048513), fa.FA_ERR_SHAPE),
    (dict(d=100), fa.FA_ERR_UNSUPPORTED),
    (dict(chunk=100), fa.FA_ERR_UNSUPPORTED),
    (dict(chunk=0), fa.FA_ERR_UNSUPPORTED),
    (dict(q=MIS), fa.FA_ERR_ALIGN),
    (dict(kc=MIS), fa.FA_ERR_ALIGN),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=16), fa.FA_ERR_WORKSPACE),
    (dict(ws=MIS), fa.FA_ERR_ALIGN),
])
def test_decode_rejects(L, kw, status):
    assert _dec(L, **kw) == status


def _dec_noalloc(L, q=P, kc=P, vc=P, sl=P, o=P, lse=P, B=2, Hq=8, Hkv=2, Nk_max=512, d=128,
                 scale=0.1, chunk=256):
    return L.fa_decode_splitkv_noalloc(q, kc, vc, sl, o, lse, B, Hq, Hkv, Nk_max, d, scale, chunk,
                                       None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL),
    (dict(vc=None), fa.FA_ERR_NULL),
    (dict(o=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_SHAPE),
    (dict(B=1, Hq=8, Hkv=8, Nk_max=1048513), fa.FA_ERR_SHAPE),
    (dict(d=100), fa.FA_ERR_UNSUPPORTED),
    (dict(chunk=100), fa.FA_ERR_UNSUPPORTED),
    (dict(lse=0x10001), fa.FA_ERR_ALIGN),
    (dict(vc=MIS), fa.FA_ERR_ALIGN),
    # partial results beyond the 80 MiB scratch: 64 heads at 32768 keys and chunk 256 need
    # 4.26 MB per sequence (129 pieces x (128 + 1) floats per head), so 20 sequences do not
    # fit; with chunk 64 (513 pieces) 5 sequences do not
    (dict(B=20, Hq=64, Hkv=8, Nk_max=32768), fa.FA_ERR_SCRATCH),
    (dict(B=5, Hq=64, Hkv=8, Nk_max=32768, chunk=64), fa.FA_ERR_SCRATCH),
])
def test_decode_noalloc_rejects(L, kw, status):
    """Invalid requests, and requests larger than the fixed scratch, are refused before any
    HIP call (so also here, without a GPU)."""
    assert _dec_noalloc(L, **kw) == status


def test_decode_noalloc_scratch_limit_matches_workspace_query():
    """The scratch limit is stated in workspace bytes: the largest accepted requests are
    those whose fa_decode_splitkv workspace fits 80 MiB."""
    limit = 80 << 20
    assert fa.fa_decode_splitkv_workspace_bytes(16, 64, 32768, 128, 256) <= limit
    assert fa.fa_decode_splitkv_workspace_bytes(19, 64, 32768, 128, 256) <= limit
    assert fa.fa_decode_splitkv_workspace_bytes(20, 64, 32768, 128, 256) > limit
    assert fa.fa_decode_splitkv_workspace_bytes(5, 64, 32768, 128, 64) > limit


def _paged(L, q=P, kp=P, vp=P, bt=P, sl=P, o=P, lse=P, B=2, Hq=8, Hkv=2, num_pages=16,
           page_size=256, max_pages=4, d=128, scale=0.1, chunk=256, ws=P, ws_bytes=1 << 30):
    return L.fa_decode_paged(q, kp, vp, bt, sl, o, lse, B, Hq, Hkv, num_pages, page_size,
                             max_pages, d, scale, chunk, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(kp=None), fa.FA_ERR_NULL),
    (dict(vp=None), fa.FA_ERR_NULL),
    (dict(bt=None), fa.FA_ERR_NULL),
    (dict(sl=None), fa.FA_ERR_NULL),
    (dict(num_pages=0), fa.FA_ERR_SHAPE),
    (dict(page_size=0), fa.FA_ERR_SHAPE),
    (dict(max_pages=0), fa.FA_ERR_SHAPE),
    (dict(page_size=100), fa.FA_ERR_UNSUPPORTED),
    (dict(page_size=32), fa.FA_ERR_UNSUPPORTED),
    (dict(max_pages=1 << 30, page_size=64), fa.FA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_SHAPE),
    (dict(d=100), fa.FA_ERR_UNSUPPORTED),
    (dict(chunk=96), fa.FA_ERR_UNSUPPORTED),
    (dict(kp=MIS), fa.FA_ERR_ALIGN),
    (dict(bt=0x10002), fa.FA_ERR_ALIGN),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), fa.FA_ERR_WORKSPACE),
])
def test_paged_decode_rejects(L, kw, status):
    assert _paged(L, **kw) == status


def test_binding_raises_without_gpu_tensors(L):
    torch = pytest.importorskip("torch")
    q = torch.zeros((1, 4, 1, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_forward(q, q, q)
    with pytest.raises(TypeError):
        fa.fa_forward(q.float(), q, q)


def test_product_does_not_import_oracle():
    """The product package and the oracle share no code: no import either way."""
    pkg = os.path.join(ROOT, "io_aware_attention_attn_amd")
    imp_oracle = re.compile(r"^\s*(from\s+oracle\b|import\s+oracle\b)|#include\s+\"[^\"]*oracle", re.M)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not imp_oracle.search(src), f
    imp_pkg = re.compile(r"^\s*(from|import)\s+io_aware_attention_attn_amd\b", re.M)
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            src = open(os.path.join(ROOT, "oracle", f)).read()
            assert not imp_pkg.search(src), f


@pytest.mark.parametrize("shape", [(16, 32768, 8, 128), (2, 700, 2, 64), (3, 100, 1, 64),
                                   (1311, 256, 8, 128)])
def test_kv_cache_empty_layout(shape):
    """The allocation helper: two contiguous caches of the requested shape in one buffer,
    not overlapping, both 16-byte aligned relative to the buffer, and the V cache 256 bytes
    past the K cache's 1 KiB congruence class (on the CPU here; the device only changes
    where the buffer lives)."""
    torch = pytest.importorskip("torch")
    k, v = fa.kv_cache_empty(shape, device="cpu")
    assert tuple(k.shape) == shape and tuple(v.shape) == shape
    assert k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16
    assert k.is_contiguous() and v.is_contiguous()
    nbytes = k.numel() * 2
    delta = v.data_ptr() - k.data_ptr()
    assert delta >= nbytes                      # no overlap
    assert delta % 16 == 0                      # V keeps K's 16-byte alignment
    assert delta % 1024 == fa.KV_V_OFFSET_MOD_1K == 256
    assert delta - nbytes < 1024                # at most one KiB of padding


def test_binding_allocates_on_the_launch_stream(monkeypatch):
    """Every tensor a wrapper allocates (outputs, workspace) is allocated in the stream
    order of the stream the library is handed, not torch's current stream: a workspace
    freed on return is then only reused by work ordered after the kernels.  Checked on
    the CPU with the library and the stream replaced by recorders."""
    torch = pytest.importorskip("torch")

    class FakeStream:
        cuda_stream = 0x5150

    seen_alloc, seen_launch = [], []

    def fake_empty(shape, dtype, device, ts):
        seen_alloc.append(ts)
        return torch.zeros(shape, dtype=dtype)

    class FakeLib:
        def __getattr__(self, name):
            if name.endswith("_workspace_bytes"):
                return lambda *a: 4096
            if name == "fa_status_str":
                return lambda st: b"x"

            def entry(*args):
                seen_launch.append(args[-1])
                return 0
            entry.__name__ = name
            return entry

    def no_direct_alloc(*a, **k):
        raise AssertionError("wrapper allocated outside the launch stream")

    monkeypatch.setattr(fa, "_torch_stream", lambda s: FakeStream())
    monkeypatch.setattr(fa, "_empty", fake_empty)
    monkeypatch.setattr(fa, "lib", lambda: FakeLib())
    monkeypatch.setattr(fa, "_check_tensor", lambda *a, **k: None)
    monkeypatch.setattr(fa, "_check_token_rows", lambda *a, **k: None)
    monkeypatch.setattr(torch, "empty", no_direct_alloc)
    bf = torch.bfloat16
    q = torch.zeros((1, 4, 2, 64), dtype=bf)
    k = torch.zeros((1, 4, 1, 64), dtype=bf)
    o32 = torch.zeros((1, 4, 2, 64))
    l32 = torch.zeros((1, 2, 4))
    calls = [
        lambda: fa.fa_forward(q, k, k, causal=True),
        lambda: fa.fa_forward_f32(q.float(), k.float(), k.float()),
        lambda: fa.fa_forward_fp8(q, k, k, 1.0, 1.0, 1.0),
        lambda: fa.fa_forward_varlen(q[0], k[0], k[0], torch.tensor([0, 4], dtype=torch.int32),
                                     torch.tensor([0, 4], dtype=torch.int32), 4, 4),
        lambda: fa.fa_backward(q, k, k, o32, l32, q, causal=True),
        lambda: fa.fa_decode_splitkv(q[:, 0], k, k, torch.tensor([4], dtype=torch.int32)),
        lambda: fa.fa_decode_paged(q[:, 0], k, k, torch.zeros((1, 1), dtype=torch.int32),
                                   torch.tensor([4], dtype=torch.int32)),
    ]
    for i, call in enumerate(calls):
        seen_alloc.clear()
        seen_launch.clear()
        call()
        assert seen_alloc, f"call {i} allocated nothing"
        assert all(isinstance(t, FakeStream) for t in seen_alloc), i
        assert seen_launch == [FakeStream.cuda_stream], i


def test_bench_traffic_lookups_name_profiled_kernels():
    """The kernel instantiations bench.py reads HBM traffic for (roofline.traffic, the decode
    traffic) are keys of profiles/hbm_traffic.json, i.e. the names rocprofv3 reports for the
    current kernels; a renamed instantiation would otherwise turn the figure into null."""
    import ast
    import json
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    tree = ast.parse(open(os.path.join(root, "bench.py")).read())
    names = [n.args[0].value for n in ast.walk(tree)
             if isinstance(n, ast.Call) and getattr(n.func, "id", None) == "profiled_traffic"
             and n.args and isinstance(n.args[0], ast.Constant)]
    assert names, "bench.py reads no profiled traffic"
    profiled = json.load(open(os.path.join(root, "profiles", "hbm_traffic.json")))
    for name in names:
        assert name in profiled, name


def test_bench_parses_amd_smi_power_and_clocks():
    """bench.py's power leg reads the socket power and the per-XCD GFX clocks from the text
    `amd-smi metric -p -c` prints (layout of ROCm 7.2's amd-smi: a POWER block, then one
    GFX_k block per XCD whose first line is its current clock); other clock blocks and the
    MIN/MAX lines are not taken."""
    import bench
    text = """GPU: 0
    POWER:
        SOCKET_POWER: 1349 W
        GFX_VOLTAGE: N/A
        THROTTLE_STATUS: N/A
    CLOCK:
        GFX_0:
            CLK: 1751 MHz
            MIN_CLK: 157 MHz
            MAX_CLK: 2400 MHz
            CLK_LOCKED: DISABLED
        GFX_1:
            CLK: 1655 MHz
            MIN_CLK: 157 MHz
            MAX_CLK: 2400 MHz
        MEM_0:
            CLK: 2000 MHz
            MIN_CLK: 900 MHz
        VCLK_0:
            CLK: 59 MHz
"""
    assert bench.parse_smi_metric(text) == (1349.0, [1751.0, 1655.0])
    assert bench.parse_smi_metric("GPU: 0\n    POWER:\n        SOCKET_POWER: N/A\n") is None


def test_probe_validation(L):
    """The matrix-core probe checks its arguments before any HIP call."""
    need = L.fa_probe_mfma_bf16_operand_bytes(4)
    assert need == 4 * 256 * 8 * 16
    assert L.fa_probe_mfma_bf16_operand_bytes(0) == 0
    ok = dict(operands=P, nbytes=need, out=P, blocks=4, iters=10)
    def call(**kw):
        a = dict(ok, **kw)
        return L.fa_probe_mfma_bf16(a["operands"], a["nbytes"], a["out"], a["blocks"],
                                    a["iters"], None)
    assert call(operands=None) == fa.FA_ERR_NULL
    assert call(out=None) == fa.FA_ERR_NULL
    assert call(blocks=0) == fa.FA_ERR_SHAPE
    assert call(iters=0) == fa.FA_ERR_SHAPE
    assert call(blocks=(1 << 20) + 1, nbytes=1 << 40) == fa.FA_ERR_SHAPE
    assert call(nbytes=need - 1) == fa.FA_ERR_SHAPE
    assert call(operands=MIS) == fa.FA_ERR_ALIGN
    assert call(out=MIS) == fa.FA_ERR_ALIGN


def test_stream_probe_validation(L):
    """The streaming-read probe checks its arguments before any HIP call."""
    ok = dict(buf=P, nbytes=1 << 20, out=P, blocks=8)
    def call(**kw):
        a = dict(ok, **kw)
        return L.fa_probe_stream_read(a["buf"], a["nbytes"], a["out"], a["blocks"], None)
    assert call(buf=None) == fa.FA_ERR_NULL
    assert call(out=None) == fa.FA_ERR_NULL
    assert call(blocks=0) == fa.FA_ERR_SHAPE
    assert call(blocks=(1 << 16) + 1) == fa.FA_ERR_SHAPE
    assert call(nbytes=0) == fa.FA_ERR_SHAPE
    assert call(nbytes=(1 << 20) + 8) == fa.FA_ERR_SHAPE
    assert call(nbytes=(1 << 31) + 16) == fa.FA_ERR_SHAPE
    assert call(buf=MIS) == fa.FA_ERR_ALIGN
    assert call(out=P + 2) == fa.FA_ERR_ALIGN
