"""The read-ceiling probe (gqa_stream_read) reads everything it is given: its
single write happens exactly when a thread's xor fold of its 16-byte pieces
equals 0x12345678, so a fold split over a thread's first piece and its piece
in the ragged tail shows that both were read."""
import pytest
import torch

import grouped_query_kv_decode_amd as gqa

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    gqa.load_library()
    yield


@pytest.mark.parametrize("nontemporal", [True, False])
@pytest.mark.parametrize("grid", [0, 1])
def test_stream_read_reads_every_piece(nontemporal, grid):
    stride = (2048 if grid == 0 else grid) * 256        # pieces between a thread's reads
    n16 = 3 * 524288 + 5                                # 3 full passes of the default grid and a ragged tail
    pieces = torch.zeros((n16, 4), dtype=torch.int32, device=DEV)
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    gqa.stream_read(pieces, nontemporal, grid, sink)
    torch.cuda.synchronize()
    assert int(sink) == 7                                # all zero: no fold hits the sentinel

    t = 3                                                # a thread that owns a piece of the tail
    tail = 3 * 524288 + t
    assert tail % stride == t and tail < n16
    pieces[t, 0] = 0x12340000
    pieces[tail, 2] = 0x00005678
    gqa.stream_read(pieces, nontemporal, grid, sink)
    torch.cuda.synchronize()
    assert int(sink) == 0x12345678

    pieces[tail, 2] = 0                                  # half the sentinel: no write
    sink.fill_(7)
    gqa.stream_read(pieces, nontemporal, grid, sink)
    torch.cuda.synchronize()
    assert int(sink) == 7
