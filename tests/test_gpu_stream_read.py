"""svlm_stream_read (the measurement helper the bench takes its achievable
streaming rate from): every workgroup's range is read, as its sink word
shows (the first float of the range), including a ragged last range, and the
zero-byte form is one empty workgroup."""
import pytest

from tests._util import log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("nfloats,wgs", [(1 << 20, 216), (3 * 1024 * 1024 + 20, 7), (256, 1), (1000, 3)])
def test_stream_read_touches_every_range(nfloats, wgs):
    from visual_kv_pruning_amd import ops
    src = torch.arange(nfloats, dtype=torch.float32, device="cuda:0")
    sink = torch.full((wgs,), -1.0, device="cuda:0")
    log(f"stream_read case {nfloats} floats over {wgs} workgroups")
    ops.stream_read(src, wgs, sink)
    torch.cuda.synchronize()
    per = -(-nfloats * 4 // wgs)
    per = -(-per // 1024) * 1024 // 4                     # floats per workgroup (1 KB multiples)
    n_wg = -(-nfloats // per)
    want = []
    for w in range(n_wg):
        n = min(per, nfloats - w * per) * 4                # bytes of this range
        last0 = -(-(-(-n // 1024)) // 4) - 1               # the first wave's last 1 KB transfer
        want.append(float(w * per + last0 * 1024))         # its first float: byte 4096 * last0
    want += [-1.0] * (wgs - n_wg)
    assert sink.cpu().tolist() == want


def test_stream_read_empty_launch():
    from visual_kv_pruning_amd import ops
    sink = torch.full((1,), -1.0, device="cuda:0")
    ops.stream_read(None, 1, sink)
    torch.cuda.synchronize()
    assert sink.item() == 0.0
