"""The read-only streaming ceiling kernel (nvfp4_stream_read) reads every 16-byte chunk of both
arrays: with all bytes zero except one chunk whose four words fold (XOR) to a marker, the one
lane that loads that chunk, and no other, writes the marker to the sink."""
import pytest
import torch

import gpu_util as U
from nvfp4_w4a4_block_amd import binding as B

pytestmark = pytest.mark.gpu
MAGIC = 0x5A17C0DE


@pytest.fixture(scope="module", autouse=True)
def _lib():
    U.require_gpu_lib()


def _probe(a_bytes, b_bytes, where, chunk):
    a = torch.zeros((max(a_bytes, 16) // 4,), dtype=torch.int32, device=U.DEV)
    b = torch.zeros((max(b_bytes, 16) // 4,), dtype=torch.int32, device=U.DEV)
    words = torch.tensor([0x11111111, 0x22222222, 0x44444444, MAGIC ^ 0x11111111 ^ 0x22222222 ^ 0x44444444],
                         dtype=torch.int64).to(torch.int32)
    (a if where == "a" else b)[4 * chunk:4 * chunk + 4] = words.to(U.DEV)
    sink = torch.full((1,), -1, dtype=torch.int32, device=U.DEV)
    lib = B.load()
    st = lib.nvfp4_stream_read(a.data_ptr(), a_bytes, b.data_ptr(), b_bytes, sink.data_ptr(), MAGIC,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    return int(sink.item()) & 0xFFFFFFFF


@pytest.mark.parametrize("a_bytes,b_bytes", [(65536000, 8192000), (4096, 16), (1 << 20, 0), (16 * 12345, 16 * 777)])
def test_stream_read_reaches_every_chunk(a_bytes, b_bytes):
    for where, n in (("a", a_bytes), ("b", b_bytes)):
        if n == 0:
            continue
        chunks = n // 16
        for c in sorted({0, 1, 63, 64, chunks // 2, chunks - 65, chunks - 2, chunks - 1} & set(range(chunks))):
            assert _probe(a_bytes, b_bytes, where, c) == MAGIC, (where, c)


def test_stream_read_writes_nothing_without_the_marker():
    a = torch.zeros((1 << 18,), dtype=torch.int32, device=U.DEV)
    sink = torch.full((1,), -1, dtype=torch.int32, device=U.DEV)
    B.nvfp4_stream_read(a, a[:4], sink=sink, magic=MAGIC)
    torch.cuda.synchronize()
    assert int(sink.item()) == -1
