"""The measurement probes on the GPU (velox_mfma_probe, velox_hbm_read_probe).

* The read probe reads every 16-byte word exactly once: over a buffer of
  float32 ones the per-thread sums add up to the element count (exact in
  float32 at these sizes), for grids that leave ragged grid-stride tails.
* The MFMA probe writes positive shader and reference clock counts whose
  ratio is a plausible shader clock, and finite sums.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import geometry_routed_block_velox_amd as velox
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    velox.lib()


@pytest.mark.parametrize("n,grid", [(16 << 20, 2048), (1_000_004, 7), (4, 1), (12_345_676, 513)])
def test_read_probe_reads_every_word_once(n, grid):
    say(f"velox_hbm_read_probe: {n} floats, grid {grid}")
    buf = torch.ones(n, dtype=torch.float32, device="cuda")
    sink = velox.hbm_read_probe(buf, grid=grid)
    torch.cuda.synchronize()
    s = sink.double().cpu().numpy()
    assert s.shape == (grid * 256,)
    assert float(s.sum()) == float(n)
    assert np.all(s == np.floor(s)) and s.min() >= 0


def test_read_probe_rejects_ragged_bytes():
    buf = torch.ones(5, dtype=torch.float32, device="cuda")  # 20 bytes, not a multiple of 16
    with pytest.raises(velox.VeloxError):
        velox.hbm_read_probe(buf, grid=4)


def test_mfma_probe_clocks():
    say("velox_mfma_probe: grid 8, 200 iterations")
    clocks = velox.mfma_probe(8, 200)
    torch.cuda.synchronize()
    c = clocks.cpu().numpy()
    assert np.all(c > 0)
    ghz = c[:, 0] / c[:, 1] * 0.1  # shader clocks per 100 MHz reference tick
    say(f"shader clock {ghz.min():.2f}..{ghz.max():.2f} GHz")
    assert np.all((ghz > 0.3) & (ghz < 3.5))
