"""Plant plausible mistakes in copies of the oracle and require the pins to catch each.

Each mutant is the oracle's own source with one textual change (a dropped term,
a wrong sign, index, axis or operand), loaded as a separate module on the CPU.
A mutant "survives" if every pin still passes; no mutant may survive.
"""
import importlib.util
import os
import sys
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "attention.py")

MUTANTS = {
    "scale dropped": ("s = (q_rows @ k.transpose(0, 1)) * scale", "s = (q_rows @ k.transpose(0, 1))"),
    "mask off by one": ("cols > rows + (Nk - Nq)", "cols >= rows + (Nk - Nq)"),
    "mask top-left": ("cols > rows + (Nk - Nq)", "cols > rows"),
    "visible off by one": ("(j <= i + (Nk - Nq))", "(j < i + (Nk - Nq))"),
    "gqa modulo": ("kvh = h // group", "kvh = h % Hkv"),
    "lse without ln l": ("(m + torch.log(l)).squeeze(1)", "m.squeeze(1)"),
    "wrong value operand": ("o[b, a:e_, h, :] = p @ vv", "o[b, a:e_, h, :] = p @ kk"),
    "max over wrong axis": ("m = torch.amax(s, dim=1, keepdim=True)\n                ex = torch.exp(s - m)\n                l = ",
                            "m = torch.amax(s, dim=0, keepdim=True)\n                ex = torch.exp(s - m)\n                l = "),
    "sum over wrong axis": ("l = torch.sum(ex, dim=1, keepdim=True)",
                            "l = torch.sum(ex, dim=0, keepdim=True)"),
    "no max shift in attention": ("ex = torch.exp(s - m)\n                l = ", "ex = torch.exp(s)\n                l = "),
    "bwd no max shift": ("ex = torch.exp(s - m)\n                    p = ", "ex = torch.exp(s)\n                    p = "),
    "softmax without max shift": ("e = torch.exp(x - m)", "e = torch.exp(x)"),
    "merge factor sign": ("f1 = torch.exp(m1 - m)", "f1 = torch.exp(m - m1)"),
    "merge drops the second factor on acc": ("f2.unsqueeze(-1) * acc2", "acc2"),
    "merge drops the second factor on l": ("f1 * l1 + f2 * l2", "f1 * l1 + l2"),
    "merge keeps the first max": ("m = torch.maximum(m1, m2)", "m = m1"),
    "block sum without max shift": ("w = torch.exp(s_block - m.unsqueeze(-1))", "w = torch.exp(s_block)"),
    "merge weight vs M": ("wn = torch.exp(lse_parts - lse)", "wn = torch.exp(lse_parts - M)"),
    "final O not normalised": ("return acc / l.unsqueeze(-1), m + torch.log(l)",
                               "return acc, m + torch.log(l)"),
    "decode reads one row short": ("L = int(lengths[b])\n        kk = _as64(k_cache[b, :L])",
                                   "L = max(int(lengths[b]) - 1, 1)\n        kk = _as64(k_cache[b, :L])"),
    "decode reads past length": ("kk = _as64(k_cache[b, :L])", "kk = _as64(k_cache[b, :L + 1])"),
    "varlen keys from the query offsets": ("ob, lb = attention(q[q0:q1].unsqueeze(0), k[k0:k1].unsqueeze(0), v[k0:k1]",
                                          "ob, lb = attention(q[q0:q1].unsqueeze(0), k[q0:q1].unsqueeze(0), v[q0:q1]"),
    "varlen values of the next sequence": ("v[k0:k1].unsqueeze(0),\n                           scale, causal, heads=heads)",
                                           "v[k1:k1 + (k1 - k0)].unsqueeze(0),\n                           scale, causal, heads=heads)"),
    "varlen whole-pack causal alignment": ("ob, lb = attention(q[q0:q1].unsqueeze(0), k[k0:k1].unsqueeze(0), v[k0:k1].unsqueeze(0),\n                           scale, causal, heads=heads)",
                                           "ob, lb = attention(q[q0:q1].unsqueeze(0), k[:k1].unsqueeze(0), v[:k1].unsqueeze(0),\n                           scale, causal, heads=heads)"),
    "varlen key count from the query count": ("k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])",
                                              "k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b]) + (q1 - q0)"),
    "varlen keyless sequence not skipped": ("if q1 == q0 or k1 == k0:", "if q1 == q0:"),
    "bwd drops the D term": ("ds = p * (dp - dsum)", "ds = p * dp"),
    "bwd D over the wrong axis": ("dsum = torch.sum(p * dp, dim=1, keepdim=True)",
                                  "dsum = torch.sum(p * dp, dim=0, keepdim=True)"),
    "bwd dQ without scale": ("dq[b, lo:hi, h, :] = scale * (ds[lo - a:hi - a] @ kk)",
                             "dq[b, lo:hi, h, :] = (ds[lo - a:hi - a] @ kk)"),
    "bwd dQ from V": ("dq[b, lo:hi, h, :] = scale * (ds[lo - a:hi - a] @ kk)",
                      "dq[b, lo:hi, h, :] = scale * (ds[lo - a:hi - a] @ vv)"),
    "bwd dP from K": ("dp = dd @ vv.transpose(0, 1)", "dp = dd @ kk.transpose(0, 1)"),
    "bwd dV from dS": ("dv_acc += p[:, k0:k1].transpose(0, 1) @ dd",
                       "dv_acc += ds[:, k0:k1].transpose(0, 1) @ dd"),
    "bwd dK from dO": ("dk_acc += scale * (ds[:, k0:k1].transpose(0, 1) @ qq)",
                       "dk_acc += scale * (ds[:, k0:k1].transpose(0, 1) @ dd)"),
    "bwd GQA keeps the last head only": ("dv_acc += p[:, k0:k1].transpose(0, 1) @ dd",
                                          "dv_acc = p[:, k0:k1].transpose(0, 1) @ dd"),
    "bwd unnormalised P": ("p = ex / torch.sum(ex, dim=1, keepdim=True)        # P",
                           "p = ex        # P"),
    "paged ignores block table": ("page = int(block_table[b][j])", "page = j"),
    "paged reads whole last page": ("n = min(page_size, L - j * page_size)", "n = page_size"),
    "paged misses partial last page": ("for j in range((L + page_size - 1) // page_size):",
                                       "for j in range(L // page_size):"),
    "paged takes the next table entry": ("page = int(block_table[b][j])",
                                         "page = int(block_table[b][j + 1])"),
}


def _load_mutant(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name!r} not unique/found"
    mod = types.ModuleType(f"oracle_mutant_{abs(hash(name))}")
    mod.__file__ = SRC
    exec(compile(src.replace(old, new), SRC, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load_mutant(name, *MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or the mutant crashing on a shape
            caught.append(pin.__name__)
    assert caught, f"mutant {name!r} passed every pin"
