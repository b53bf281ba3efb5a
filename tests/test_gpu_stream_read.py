"""The streaming-read yardstick (sfi_stream_read) reads every 16-byte word of its buffer.

Its only visible effect is the sink word it writes when a thread's XOR of the words it read
equals the fixed constant.  Over a zeroed buffer with the constant planted in one word, the
thread that reads that word (and only it) sees the constant, so exactly one sink word, the one
of the workgroup whose chunk holds the planted word, must change: this checks the chunking,
the tail of a ragged last chunk and idle workgroups past the end.
"""
import pytest
import torch

from sparse_kv_attention_dense_amd import binding as B

from gpu_util import DEV, say

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9 - (1 << 32)          # the kernel's constant as an int32


@pytest.mark.parametrize("nbytes,wg", [(1 << 24, 1024), ((1 << 24) + 48, 1000), (4096, 4096)])
def test_stream_read_reads_every_word(nbytes, wg):
    say(f"[stream_read] bytes={nbytes} workgroups={wg}")
    n16 = nbytes // 16
    per = -(-n16 // wg)
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
    sink = torch.zeros(64, dtype=torch.int32, device=DEV)
    for k16 in sorted({0, 1, n16 // 2, per - 1, min(per, n16 - 1), 12345 % n16, n16 - 1}):
        word = 4 * k16 + k16 % 4
        buf.zero_()
        buf[word] = MAGIC
        sink.zero_()
        B.sfi_stream_read(buf, wg, sink)
        torch.cuda.synchronize()
        expect = torch.zeros_like(sink)
        expect[(k16 // per) % 64] = MAGIC
        assert torch.equal(sink, expect), f"planted word {word}"
    # a zeroed buffer leaves the sink alone
    buf.zero_()
    sink.fill_(5)
    B.sfi_stream_read(buf, wg, sink)
    torch.cuda.synchronize()
    assert torch.equal(sink, torch.full_like(sink, 5))
