"""The streaming-read probe reads exactly the windows it names: a fixed word
placed in one window's first chunk reaches the sink only when that window is
among the ones read (launch i reads window i mod (span / window))."""
import pytest
import torch

import w4a16_bit_matmul_amd as wq
from parity import say

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9  # the probe's fixed value (a thread's XOR of its words)


@pytest.mark.parametrize("nontemporal", [False, True])
@pytest.mark.parametrize("chunks", [1, 2, 4, 8, 16])
def test_read_probe_reads_the_named_windows(chunks, nontemporal):
    say(f"read probe chunks={chunks} nontemporal={nontemporal}")
    window = 256 * chunks * 16 * 3  # three workgroups per window
    span_windows = 3
    for target in range(span_windows):
        for count in (1, 2, 3, 4):
            buf = torch.zeros(window * span_windows // 4, dtype=torch.int32, device="cuda")
            # second workgroup of the target window, thread 5: its first chunk
            # holds the fixed word, its other chunks are zero
            word = (target * window + 256 * chunks * 16 + 5 * 16) // 4
            buf[word] = MAGIC - (1 << 32)
            sink = torch.zeros(1, dtype=torch.int32, device="cuda")
            wq.wq_read_probe(buf, window, count, chunks=chunks, nontemporal=nontemporal, sink=sink)
            torch.cuda.synchronize()
            read = {i % span_windows for i in range(count)}
            got = int(sink.item()) & 0xFFFFFFFF
            assert got == (MAGIC if target in read else 0), (chunks, target, count, hex(got))


def test_read_probe_window_tail_is_clamped():
    # a window of 2080 chunks (not a whole number of 2048-chunk workgroups):
    # loads past the end re-read the final chunk, which holds the fixed word.
    # Threads 0-30 of the second workgroup read one zero chunk and seven
    # clamped copies of the final chunk, an odd count, so their XOR is the word.
    say("read probe ragged window")
    window = 256 * 8 * 16 + 512
    buf = torch.zeros(window // 4, dtype=torch.int32, device="cuda")
    buf[window // 4 - 4] = MAGIC - (1 << 32)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    wq.wq_read_probe(buf, window, 1, chunks=8, sink=sink)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == MAGIC
