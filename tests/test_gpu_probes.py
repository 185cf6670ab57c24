"""The measurement probes (include/apex4_probe.h) run on the GPU, report the
documented amount of work, and give rates in a plausible range for this chip
(well below the datasheet peaks' upper bounds, well above zero)."""
import pytest

torch = pytest.importorskip("torch")

from w4a4_group_quantized_amd import apex4  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    apex4.lib()
    return torch.device("cuda:0")


def timed(fn):
    s = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    work = fn()
    e1.record(s)
    torch.cuda.synchronize()
    return work, e0.elapsed_time(e1) * 1e-3


def test_probe_mfma(dev):
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    ops, t = timed(lambda: apex4.probe_mfma_i8(500, sink))
    assert ops == 1024 * 4 * 500 * 4 * 2 * 32 ** 3
    assert 100e12 < ops / t < 5.5e15


def test_probe_mfma_f6(dev):
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    ops, t = timed(lambda: apex4.probe_mfma_f6(500, sink))
    assert ops == 1024 * 4 * 500 * 4 * 2 * 32 * 32 * 64
    assert 100e12 < ops / t < 11e15
    assert int(sink.item()) == 0


def test_probe_hbm_read(dev):
    buf = torch.zeros(1 << 28, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    nbytes, t = timed(lambda: apex4.probe_hbm_read(buf, sink))
    assert nbytes == 1 << 28
    assert 0.5e12 < nbytes / t < 20e12      # (256 MB may partly hit the last-level cache)
    assert int(sink.item()) == 0            # zeros never hit the sentinel


def test_probe_valu(dev):
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    flops, t = timed(lambda: apex4.probe_valu_f32(1000, sink))
    assert flops == 1024 * 256 * 1000 * 16
    assert 5e12 < flops / t < 400e12


def test_probe_lds_read(dev):
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    nbytes, t = timed(lambda: apex4.probe_lds_read(2000, sink))
    assert nbytes == 1024 * 256 * 2000 * 8 * 16
    # 256 CUs x 128 or 256 bytes per clock at ~2 GHz: tens to ~160 TB/s
    assert 5e12 < nbytes / t < 400e12
