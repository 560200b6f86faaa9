"""The streaming-read probe (pkv_hbm_read_probe): it reads the range and
stores nothing for data that does not fold to its fixed word, and refuses
unaligned ranges and empty grids."""

import pytest

pytestmark = pytest.mark.gpu


def test_read_probe_reads_and_leaves_the_sink(dev):
    import torch
    import paged_kv_cache_204_amd as pkv
    src = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    for blocks in (1, 64, 1024):
        pkv.pkv_hbm_read_probe(src, src.numel(), sink, blocks)
    # a ragged tail: 16-byte chunks that do not fill the last grid stride
    pkv.pkv_hbm_read_probe(src, 16 * 1001, sink, 3)
    torch.cuda.synchronize()
    assert sink.cpu().tolist() == [7, 7, 7, 7]
    for nbytes, blocks in ((15, 1), (1 << 20, 0)):
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_hbm_read_probe(src, nbytes, sink, blocks)
        assert e.value.code == pkv.PKV_ERR_ARG
