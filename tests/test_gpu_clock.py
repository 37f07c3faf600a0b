"""The clock probe reads the shader clock while the matrix cores are busy
(needs a GPU): a plausible clock, and every block's products written."""
import struct

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_clock_probe_reads_a_plausible_clock():
    from sparse_attention_video_means_amd import svgear as S
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 8 * cus
    out = S.svgear_clock_probe(blocks, 512)
    torch.cuda.synchronize()
    khz = S.svgear_realtime_khz()
    o = out.cpu().tolist()
    assert khz > 0 and o[1] > o[0] and o[3] > o[2]
    mhz = (o[1] - o[0]) / (o[3] - o[2]) * khz / 1000.0
    assert 300.0 < mhz < 3000.0, mhz
    # every block runs the same products: one checksum, positive
    sums = {struct.unpack("f", struct.pack("I", v & 0xFFFFFFFF))[0] for v in o[4:]}
    assert len(sums) == 1 and next(iter(sums)) > 0.0, sums
