"""GPU check of w8a16_hbm_read, the plain-read helper bench.py times as the
floor of the decode GEMV's weight stream: it reads and writes nothing, at
every launch shape it accepts, on a ragged size."""
import pytest
import torch

from gemm_mamba_ssm_amd import binding

pytestmark = pytest.mark.gpu


def test_hbm_read_writes_nothing():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    binding.load()
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    buf = torch.randint(0, 256, (3 * (1 << 20) + 48,), dtype=torch.uint8, device=dev, generator=g)
    keep = buf.clone()
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    for threads in (64, 128, 256, 512, 1024):
        for loads in (1, 2, 4, 8, 16):
            print(f"w8a16_hbm_read threads={threads} loads={loads}", flush=True)
            assert binding.hbm_read_raw(buf.data_ptr(), buf.numel(), threads, loads, sink.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert not bool(sink.any())
    assert torch.equal(buf, keep)
