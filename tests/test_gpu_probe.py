"""The HBM read probe reads the pages its id list names: a page whose first
16 bytes hold the probe's sink constant (and zeros elsewhere) makes the xor
of lane 0 equal that constant, so the sink is written exactly when that page
is in the list."""

import pytest
import torch

from decode_attention_amd import probe as P

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


def test_probe_reads_the_listed_pages(gpu_lib):
    P.load_probe_library()
    buf = torch.zeros(8 * P.PAGE_BYTES, dtype=torch.uint8, device="cuda")
    words = buf.view(torch.int32)
    words[5 * P.PAGE_BYTES // 4] = MAGIC - (1 << 32)  # the constant's bits as int32
    before = buf.clone()
    for ids, wg, hit in (([3], 1, False), ([5], 1, True), ([0, 1, 2, 3, 4, 6, 7], 3, False),
                         ([7, 6, 5], 2, True), ([], 4, False)):
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        P.read_pages(buf, torch.tensor(ids, dtype=torch.int32, device="cuda"), wg, sink)
        torch.cuda.synchronize()
        print(f"[probe] ids={ids} workgroups={wg} sink={int(sink.item()) & 0xFFFFFFFF:#x}", flush=True)
        assert (int(sink.item()) & 0xFFFFFFFF) == (MAGIC if hit else 0)
    assert torch.equal(buf, before)
    with pytest.raises(ValueError):
        P.read_pages(buf, torch.tensor([8], dtype=torch.int32, device="cuda"), 1, sink)
