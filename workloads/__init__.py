"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and bench.py.

This module holds the workload table and the random-input recipe only.  It does
no attention arithmetic of any kind: it draws normal variates, rounds them to
the storage dtype and (for decode) poisons the unused cache rows with NaN.

Recipe (the pages give shapes but no generator, so this is a stated choice):
  * one ``torch.Generator('cpu')`` seeded with ``seed`` (0 for every workload);
  * prefill draws Q, then K, then V as fp32 ``randn`` in the [B, N, H, d] layout;
    the "peaky" workload multiplies Q and K by 1.5 in fp32; bf16 workloads then
    round to bfloat16 (round-to-nearest-even, torch's conversion);
  * decode draws the per-sequence key counts first (``randint(lo, hi + 1)``,
    both ends inclusive), then q [B, Hq, d], then the K cache and the V cache
    [B, Nk_max, Hkv, d]; cache rows at or beyond a sequence's length are set to
    NaN so that any read of them shows up in the result.

Shapes follow the pages' workloads: the packed-QKV usage example of the
"Attention is All You Need부터 FlashAttention-3까지" page (section "실전 구현")
is B=2, S=2048, H=12, D=64; the d=128 / GQA-8 long-context shapes stand in for
the Llama-class 32K-context runs that page quotes (section "실무 활용"); the
decode workload follows the KV-cache / GQA sections (②-3, ②-7) of
"LLM 기초 — Attention부터 FlashAttention까지".  No dataset is involved.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    workload: str           # human-readable description with sizes
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    dtype: str              # "f32" or "bf16"
    qk_gain: float = 1.0    # Q and K multiplied by this before rounding

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self) -> float:
        """Algorithmic FLOPs: 4*B*Hq*Nq*Nk*d, halved when causal."""
        f = 4.0 * self.B * self.Hq * self.Nq * self.Nk * self.d
        return f / 2.0 if self.causal else f


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    workload: str
    B: int
    Hq: int
    Hkv: int
    d: int
    Nk_max: int
    len_lo: int
    len_hi: int
    chunk: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


CONFIGS: Dict[str, object] = {
    "c1": PrefillConfig("c1", "noncausal single-head fp32 B=1 H=1 N=128 d=64",
                        B=1, Hq=1, Hkv=1, Nq=128, Nk=128, d=64, causal=False, dtype="f32"),
    "c2": PrefillConfig("c2", "causal MHA prefill bf16 B=2 H=12 N=2048 d=64",
                        B=2, Hq=12, Hkv=12, Nq=2048, Nk=2048, d=64, causal=True, dtype="bf16"),
    "c3": PrefillConfig("c3", "causal MHA prefill bf16 B=1 H=32 N=8192 d=128 (Q,K x1.5)",
                        B=1, Hq=32, Hkv=32, Nq=8192, Nk=8192, d=128, causal=True, dtype="bf16",
                        qk_gain=1.5),
    "c4": PrefillConfig("c4", "causal GQA prefill bf16 B=1 Hq=64 Hkv=8 N=32768 d=128",
                        B=1, Hq=64, Hkv=8, Nq=32768, Nk=32768, d=128, causal=True, dtype="bf16"),
    "c5": DecodeConfig("c5", "GQA split-KV decode bf16 B=16 Hq=64 Hkv=8 d=128 "
                       "L~U[4096,32768] chunk=256",
                       B=16, Hq=64, Hkv=8, d=128, Nk_max=32768, len_lo=4096, len_hi=32768,
                       chunk=256),
}


@dataclasses.dataclass(frozen=True)
class VarlenConfig:
    """A packed batch of B sequences whose lengths are uniform on [len_lo, len_hi]
    (queries and keys of a sequence equally long, as in a prefill)."""
    name: str
    workload: str
    B: int
    Hq: int
    Hkv: int
    d: int
    len_lo: int
    len_hi: int
    causal: bool

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


def varlen_flops(lens_q, lens_k, Hq: int, d: int, causal: bool) -> float:
    """Algorithmic FLOPs of a packed batch: 4*Hq*d*sum_b(Nq_b*Nk_b), halved when causal
    (the convention of PrefillConfig.flops, sequence by sequence)."""
    f = 4.0 * Hq * d * sum(int(a) * int(b) for a, b in zip(lens_q, lens_k))
    return f / 2.0 if causal else f


# The packed variable-length prefill: a length mix of long-context GQA sequences in one launch.
VARLEN: Dict[str, VarlenConfig] = {
    "v1": VarlenConfig("v1", "causal GQA varlen prefill bf16 16 sequences L~U[512,16384] "
                       "Hq=64 Hkv=8 d=128", B=16, Hq=64, Hkv=8, d=128, len_lo=512,
                       len_hi=16384, causal=True),
}


def _round(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def prefill_inputs(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, dtype: str = "bf16",
                   seed: int = 0, qk_gain: float = 1.0):
    """Q [B,Nq,Hq,d], K and V [B,Nk,Hkv,d] on the CPU, drawn in the order Q, K, V."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, Nq, Hq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Nk, Hkv, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Nk, Hkv, d), generator=g, dtype=torch.float32)
    if qk_gain != 1.0:
        q.mul_(qk_gain)
        k.mul_(qk_gain)
    return _round(q, dtype), _round(k, dtype), _round(v, dtype)


def backward_inputs(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, seed: int = 0,
                    qk_gain: float = 1.0):
    """bf16 Q, K, V as ``prefill_inputs`` (same draws), then the upstream gradient dO
    [B,Nq,Hq,d] drawn next from the same generator as fp32 ``randn`` rounded to bf16."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, Nq, Hq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Nk, Hkv, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Nk, Hkv, d), generator=g, dtype=torch.float32)
    do = torch.randn((B, Nq, Hq, d), generator=g, dtype=torch.float32)
    if qk_gain != 1.0:
        q.mul_(qk_gain)
        k.mul_(qk_gain)
    return tuple(t.to(torch.bfloat16) for t in (q, k, v, do))


def fp8_inputs(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, seed: int = 0,
               qk_gain: float = 1.0):
    """FP8 (torch.float8_e4m3fn, OCP E4M3) Q, K, V with per-tensor descales, from the
    same fp32 draws as ``prefill_inputs``: descale = max|x| / 448 (E4M3's largest
    finite value), code = round-to-nearest-even(x / descale).  Returns
    (q8, k8, v8, q_descale, k_descale, v_descale); the values are code * descale."""
    g = torch.Generator("cpu").manual_seed(seed)
    xs = [torch.randn((B, Nq, Hq, d), generator=g, dtype=torch.float32),
          torch.randn((B, Nk, Hkv, d), generator=g, dtype=torch.float32),
          torch.randn((B, Nk, Hkv, d), generator=g, dtype=torch.float32)]
    if qk_gain != 1.0:
        xs[0].mul_(qk_gain)
        xs[1].mul_(qk_gain)
    codes, desc = [], []
    for x in xs:
        ds = float(x.abs().max()) / 448.0
        codes.append((x / ds).to(torch.float8_e4m3fn))
        desc.append(ds)
    return (*codes, *desc)


def prefill_inputs_for(cfg: PrefillConfig, seed: int = 0):
    return prefill_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq, cfg.Nk, cfg.d, cfg.dtype, seed,
                          cfg.qk_gain)


def decode_lengths(B: int, lo: int, hi: int, seed: int = 0,
                   g: Optional[torch.Generator] = None) -> torch.Tensor:
    """Per-sequence key counts, uniform on [lo, hi] inclusive (int32)."""
    if g is None:
        g = torch.Generator("cpu").manual_seed(seed)
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)


def decode_inputs(B: int, Hq: int, Hkv: int, d: int, Nk_max: int, lo: int, hi: int,
                  seed: int = 0, nan_pad: bool = True, lengths: Optional[torch.Tensor] = None):
    """(lengths int32 [B], q bf16 [B,Hq,d], k_cache, v_cache bf16 [B,Nk_max,Hkv,d]).

    Draw order: lengths (unless given), q, K cache, V cache.  Rows at or beyond
    a sequence's length are NaN when ``nan_pad`` is set.
    """
    g = torch.Generator("cpu").manual_seed(seed)
    if lengths is None:
        lengths = decode_lengths(B, lo, hi, g=g)
    else:
        lengths = lengths.to(torch.int32).clone()
    q = torch.randn((B, Hq, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    kc = torch.randn((B, Nk_max, Hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    vc = torch.randn((B, Nk_max, Hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    if nan_pad:
        for b in range(B):
            L = int(lengths[b])
            kc[b, L:] = float("nan")
            vc[b, L:] = float("nan")
    return lengths, q, kc, vc


def decode_inputs_for(cfg: DecodeConfig, seed: int = 0, nan_pad: bool = True):
    return decode_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.Nk_max, cfg.len_lo, cfg.len_hi,
                         seed, nan_pad)


def cu_seqlens(lengths) -> torch.Tensor:
    """Offsets [0, L0, L0+L1, ...] (int32, B + 1 entries) of sequences packed end to end."""
    out = [0]
    for L in lengths:
        out.append(out[-1] + int(L))
    return torch.tensor(out, dtype=torch.int32)


def varlen_inputs(lens_q, lens_k, Hq: int, Hkv: int, d: int, seed: int = 0,
                  packed_qkv: bool = False):
    """A packed variable-length batch on the CPU (bf16):
    (cu_q, cu_k int32 [B+1], q [total_q, Hq, d], k and v [total_k, Hkv, d]).

    Draw order: q, then k, then v, each fp32 ``randn`` in the packed layout.  With
    ``packed_qkv`` (needs lens_q == lens_k) one [total, Hq + 2*Hkv, d] tensor is drawn
    instead and q, k, v are views of its head ranges, the layout of a fused QKV
    projection (their token stride is (Hq + 2*Hkv) * d).
    """
    cu_q, cu_k = cu_seqlens(lens_q), cu_seqlens(lens_k)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    g = torch.Generator("cpu").manual_seed(seed)
    if packed_qkv:
        if [int(x) for x in lens_q] != [int(x) for x in lens_k]:
            raise ValueError("packed QKV needs equal query and key lengths")
        qkv = torch.randn((tq, Hq + 2 * Hkv, d), generator=g, dtype=torch.float32)
        qkv = qkv.to(torch.bfloat16)
        return cu_q, cu_k, qkv[:, :Hq], qkv[:, Hq:Hq + Hkv], qkv[:, Hq + Hkv:]
    q = torch.randn((tq, Hq, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((tk, Hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((tk, Hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return cu_q, cu_k, q, k, v


def varlen_inputs_for(cfg: VarlenConfig, seed: int = 0):
    """(lengths int32 [B], cu_q, cu_k, q, k, v) of a VarlenConfig: lengths drawn with
    ``decode_lengths`` from the same seed, then the packed tensors (seed + 1)."""
    lengths = decode_lengths(cfg.B, cfg.len_lo, cfg.len_hi, seed=seed)
    cu_q, cu_k, q, k, v = varlen_inputs(lengths, lengths, cfg.Hq, cfg.Hkv, cfg.d, seed=seed + 1)
    return (lengths, cu_q, cu_k, q, k, v)


def decode_bytes(lengths, Hq: int, Hkv: int, d: int) -> float:
    """Compulsory HBM bytes of one decode step: K and V of the valid keys (bf16),
    plus q (bf16), O (fp32) and LSE (fp32), each counted once."""
    total_keys = int(sum(int(x) for x in lengths))
    B = len(lengths)
    kv = 2.0 * total_keys * Hkv * d * 2
    return kv + B * Hq * d * 2 + B * Hq * d * 4 + B * Hq * 4


def paged_from_contiguous(k_cache: torch.Tensor, v_cache: torch.Tensor, lengths, page_size: int,
                          seed: int = 0, spare_pages: int = 0, nan_pad: bool = True):
    """Scatter a contiguous cache [B, Nk_max, Hkv, d] into a page pool.

    Returns (k_pages, v_pages [num_pages, page_size, Hkv, d], block_table int32
    [B, ceil(Nk_max / page_size)]).  Sequence b's logical page j goes to a
    physical page drawn from a seeded permutation of the pool (so the table is
    not the identity); `spare_pages` unused pages are added to the pool.  Rows
    of a page past the sequence's length, and the spare pages, are NaN when
    ``nan_pad`` is set; table entries past a sequence's last page are -1.
    """
    B, Nk_max, Hkv, d = k_cache.shape
    maxp = (Nk_max + page_size - 1) // page_size
    npg = [(int(L) + page_size - 1) // page_size for L in lengths]
    num_pages = sum(npg) + spare_pages
    g = torch.Generator("cpu").manual_seed(seed)
    perm = torch.randperm(max(num_pages, 1), generator=g).tolist()
    fill = float("nan") if nan_pad else 0.0
    kp = torch.full((max(num_pages, 1), page_size, Hkv, d), fill, dtype=k_cache.dtype)
    vp = torch.full((max(num_pages, 1), page_size, Hkv, d), fill, dtype=v_cache.dtype)
    table = torch.full((B, maxp), -1, dtype=torch.int32)
    nxt = 0
    for b in range(B):
        L = int(lengths[b])
        for j in range(npg[b]):
            page = perm[nxt]
            nxt += 1
            n = min(page_size, L - j * page_size)
            kp[page, :n] = k_cache[b, j * page_size:j * page_size + n]
            vp[page, :n] = v_cache[b, j * page_size:j * page_size + n]
            table[b, j] = page
    return kp, vp, table
