"""The HBM streaming-read probe (paged_hbm_read), a measurement aid: every pattern
runs to completion on sizes that do and do not fill whole per-wave steps (the
per-wave direct-to-LDS pattern reads the bytes past the waves' shares in a
grid-stride tail), and leaves its sink untouched (it is written only when the
folded data equals a value random data does not produce)."""
import pytest
import torch

from tests import gpu_util as U

pytestmark = pytest.mark.gpu

# 16 bytes; one 8 KiB step; 512 workgroups x 4 waves x one 8 KiB step, plus 48
# bytes; 64 MiB plus 16 bytes
SIZES = [16, 8192, 512 * 4 * 8192 + 48, (64 << 20) + 16]


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("nbytes", SIZES)
def test_hbm_read_patterns_complete(mode, nbytes):
    o = U.ops()
    g = torch.Generator(device=U.DEV).manual_seed(nbytes + mode)
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=U.DEV)
    buf.random_(generator=g)
    sink = torch.zeros(1, dtype=torch.int32, device=U.DEV)
    for wgs in (0, 3):
        o.hbm_read(buf, sink, workgroups=wgs, mode=mode)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
