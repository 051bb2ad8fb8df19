"""The measurement probes on the GPU: the matrix-core probe's arithmetic (what the
benchmark's ceiling figure counts as FLOP is really computed), the streaming probe's
coverage (every word of the buffer read exactly once, a ragged tail included), and their
argument checks through the binding."""
import numpy as np
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


@pytest.mark.parametrize("nbytes,blocks", [(1 << 20, 8), ((1 << 20) + 4096 + 48, 7),
                                           (16, 1), (3 * 32768 + 16, 2)])
def test_stream_probe_reads_every_word_once(nbytes, blocks):
    # the XOR over all per-thread results equals the XOR of every 32-bit word of the
    # buffer: a word skipped or read twice changes it (random words, so with overwhelming
    # probability)
    dev = torch.device("cuda", 0)
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    buf = host.to(dev)
    out = torch.full((blocks * 256,), -1, dtype=torch.int32, device=dev)
    got = fa.fa_probe_stream_read(buf, out, blocks)
    torch.cuda.synchronize()
    assert got == nbytes
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)) == want


def test_stream_probe_rejects_a_ragged_size():
    dev = torch.device("cuda", 0)
    buf = torch.zeros(1026, dtype=torch.int32, device=dev)  # 4104 bytes, not a multiple of 16
    out = torch.empty(256, dtype=torch.int32, device=dev)
    with pytest.raises(fa.FAError):
        fa.fa_probe_stream_read(buf, out, 1)
