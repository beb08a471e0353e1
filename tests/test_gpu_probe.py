"""GPU checks of the probes (the measurement aids behind bench.py's measured
peaks). The read probe must visit every 16-byte piece of the buffer it is
given; the copy probe must copy every byte, onto another buffer and onto
itself.

The probe sums two words of each of its loads per lane and writes the sum to
the sink only when it equals 1234.5. A single nonzero float placed in the last
word of the last load of the last lane of the last wavefront therefore reaches
the sink exactly when that piece was read, and a zero buffer leaves the sink
alone.
"""
import pytest
import torch

from gdn_harness import DEV, log

pytestmark = pytest.mark.gpu

MAGIC = 1234.5


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_ssm_amd as m
    return m


def test_probe_leaves_sink_on_zeros(gdn):
    src = torch.zeros(3 * 32768 // 4, dtype=torch.float32, device=DEV)
    sink = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    gdn.gdn_hbm_read_probe(src, sink)
    torch.cuda.synchronize()
    assert sink.item() == -1.0


@pytest.mark.parametrize("item,load,lane,word", [(11, 7, 63, 3), (0, 0, 0, 0), (5, 3, 17, 0)])
def test_probe_reads_every_piece(gdn, item, load, lane, word):
    """12 wavefront items of 8 KiB: the piece at (item, load, lane) holds
    MAGIC in word 0 or 3 (the two words summed)."""
    src = torch.zeros(3 * 32768 // 4, dtype=torch.float32, device=DEV)
    off = (item * 8192 + load * 1024 + lane * 16) // 4 + word
    src[off] = MAGIC
    sink = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    gdn.gdn_hbm_read_probe(src, sink)
    torch.cuda.synchronize()
    log(f"[probe] item {item} load {load} lane {lane} word {word}: sink {sink.item()}")
    assert sink.item() == MAGIC


@pytest.mark.parametrize("nbytes", [32768, 5 * 32768])
def test_copy_probe_copies_every_byte(gdn, nbytes):
    g = torch.Generator(device=DEV)
    g.manual_seed(nbytes)
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device=DEV, generator=g)
    keep = src.clone()
    dst = torch.zeros_like(src)
    gdn.gdn_hbm_copy_probe(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, keep), "copy differs"
    assert torch.equal(src, keep), "source changed"
    gdn.gdn_hbm_copy_probe(dst, dst)          # onto itself
    torch.cuda.synchronize()
    assert torch.equal(dst, keep), "in-place copy changed the buffer"
