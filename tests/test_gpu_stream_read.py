"""mla_stream_read, the measurement helper behind the achievable-read figure
that bench.py sets beside the decode roofline and the kernel of known bytes
the traffic counters are calibrated on: it must read every byte once.  Its
XOR of all 16-byte chunks is integer arithmetic, so it is checked bit for bit
against numpy's XOR reduction of the same bytes, in both modes (loads into
registers; direct-to-LDS copies), for sizes that leave ragged tails against
the 8-chunk passes and the 65,536-thread grid, against the 1 KiB copies and
the 256 workgroups' ranges (fewer pieces than workgroups, a tail under
1 KiB), and twice in a row into one sink (which must then be back to zero)."""
import numpy as np
import pytest
import torch

from mla_latent_kv_36_amd import binding as mla

from gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load()


def _xor16(a: np.ndarray) -> np.ndarray:
    return np.bitwise_xor.reduce(a.view(np.uint32).reshape(-1, 4), axis=0)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("chunks", [1, 7, 64 * 100 + 5, 65536, 65536 * 8 + 3, 5_000_003])
def test_stream_read_xor_is_exact(chunks, mode):
    note(f"stream_read chunks={chunks} mode={mode}")
    rng = np.random.default_rng(chunks)
    host = rng.integers(0, 2**32, size=4 * chunks, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    mla.mla_stream_read(src, sink, mode)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, _xor16(host))
    # a second read into the same sink XORs again: back to zero
    mla.mla_stream_read(src, sink, mode)
    torch.cuda.synchronize()
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), np.zeros(4, np.uint32))
