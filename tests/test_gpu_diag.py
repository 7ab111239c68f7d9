"""The streaming-read ceiling the bench reports next to the HBM datasheet peak (needs an
MI355X): a plain read kernel over device buffers, through the C ABI."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_read_bandwidth_of_a_large_buffer_is_plausible(gpu_lib):
    buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB, beyond the 256 MB cache
    gbps = gpu_lib.read_bandwidth(buf, passes=5)
    assert 1000.0 < gbps < 8800.0, gbps


def test_read_bandwidth_ragged_tail():
    from rank_compressed_kv_ap_amd import binding
    buf = torch.zeros(4 * 1000003, dtype=torch.float32, device="cuda")   # not a multiple of a grid's stride
    assert binding.read_bandwidth(buf, passes=2) > 0.0
