"""The two measurement aids of the C ABI on the GPU (needs an MI355X): the
streaming-read probe and the prefill passes' compute-mix probe run, return
H2O_OK, and leave their sink untouched (it is written on one chance in 2^32
only)."""
import pytest
import torch

from kv_cache_eviction_prefill_amd import h2o as H

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda", 0)


def _stream():
    return torch.cuda.current_stream(DEV).cuda_stream


@pytest.mark.parametrize("nbytes", [16, 4096, (64 << 20), (64 << 20) + 48])
def test_probe_read_runs(nbytes):
    """Whole runs and a ragged end (a buffer that is no multiple of a block's
    32 KiB run) both complete."""
    buf = torch.ones((nbytes + 3) // 4, dtype=torch.float32, device=DEV)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    assert H.h2o_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), _stream()) == H.H2O_OK
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_probe_mix_runs(mode):
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    for iters in (1, 16):
        assert H.h2o_probe_mix(mode, iters, sink.data_ptr(), _stream()) == H.H2O_OK
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
