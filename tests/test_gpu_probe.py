"""The streaming-read probe (a measurement helper of the library): it reads
every 16-byte word of the buffer, which a word planted at the head, in the
body and in the ragged tail of the grid-stride walk shows."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words,at", [(1, 0), (4096, 17), (1 << 20, (1 << 20) - 1), ((1 << 20) + 5, (1 << 20) + 4)])
def test_probe_reads_every_word(words, at):
    import torch

    import spmspv_graph_traversal_amd as dbs

    buf = torch.zeros(words * 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    dbs.dbs_probe_read(buf, sink, never=0x5A5A5A5A)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0  # all-zero data folds to 0 in every thread
    buf[4 * at + 2] = 0x5A5A5A5A  # one planted word: the thread that reads it folds to `never`
    dbs.dbs_probe_read(buf, sink, never=0x5A5A5A5A)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0x5A5A5A5A
