"""The matrix-core rate probe on the GPU: its arithmetic (what the benchmark's ceiling
figure counts as FLOP is really computed) and its argument checks through the binding."""
import pytest
import torch

import io_aware_attention_attn_amd as fa

pytestmark = pytest.mark.gpu


def test_probe_counts_its_products():
    # all operands bf16 1.0: each 32x32x16 product adds 16 to every accumulator element;
    # a thread holds 4 accumulators x 16 elements, so its sum is 64 * 16 * iters
    dev = torch.device("cuda", 0)
    blocks, iters = 3, 5
    nb = fa.fa_probe_mfma_bf16_operand_bytes(blocks)
    ops = torch.ones(nb // 2, dtype=torch.bfloat16, device=dev)
    out = torch.full((blocks * 256,), float("nan"), device=dev)
    flop = fa.fa_probe_mfma_bf16(ops, out, blocks, iters)
    torch.cuda.synchronize()
    assert flop == blocks * 4 * iters * 4 * 2 * 32 * 32 * 16
    assert torch.equal(out.cpu(), torch.full((blocks * 256,), 64.0 * 16 * iters))


def test_probe_rejects_a_short_operand_buffer():
    dev = torch.device("cuda", 0)
    nb = fa.fa_probe_mfma_bf16_operand_bytes(2)
    ops = torch.ones(nb // 2 - 8, dtype=torch.bfloat16, device=dev)
    out = torch.empty(512, device=dev)
    with pytest.raises(fa.FAError):
        fa.fa_probe_mfma_bf16(ops, out, 2, 1)
