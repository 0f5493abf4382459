"""GPU: mla_stream_probe (the decode's tile stream without its arithmetic)
moves the source bytes into LDS: with every source byte equal to one value,
each workgroup's sink holds that value, for private and paired streams and
for tile counts below, at and above the ring of four buffers."""

import sys

import pytest
import torch

import mla_latent_kv_15_amd as mla

pytestmark = pytest.mark.gpu

TILE = 32 * 1152  # one 32-row bf16 tile


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


@pytest.mark.parametrize("paired", [False, True])
@pytest.mark.parametrize("tiles", [1, 2, 4, 9])
def test_stream_probe_moves_the_bytes(paired, tiles):
    wg = 512  # two rounds of the 256 CUs
    n = (wg // 2 if paired else wg) * tiles * TILE
    src = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    sink = torch.full((wg,), -1, dtype=torch.int32, device="cuda")
    print(f"stream probe paired={paired} tiles={tiles}", file=sys.stderr, flush=True)
    mla.mla_stream_probe(src, wg, tiles, paired, sink)
    torch.cuda.synchronize()
    assert bool((sink == 0x5A).all()), sink.unique()
