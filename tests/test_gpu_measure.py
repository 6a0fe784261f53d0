"""GPU checks of the streaming-read measurement kernel (pkv_stream_read):
the partial sums of the words read add up to the sum of every 32-bit word of
the buffer modulo 2^32, so every byte was read exactly once (a missed or
repeated 16-byte chunk changes the total)."""

import numpy as np
import pytest
import torch

import pagedattention_pkv_store_amd as pkv
from conftest import ensure_library

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


@pytest.mark.parametrize("nbytes,n_partials", [(0, 4), (16, 1), (16, 37), (3 * (1 << 20) + 48, 37),
                                               ((1 << 26) + 16 * 1000, 2048), (1 << 24, 65535)])
def test_stream_read_sums_every_word_once(nbytes, n_partials):
    print(f"stream_read bytes={nbytes} partials={n_partials}", flush=True)
    rng = np.random.default_rng(nbytes % 1000 + n_partials)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV) if nbytes else torch.empty(0, dtype=torch.int32, device=DEV)
    sums = torch.full((n_partials,), -1, dtype=torch.int32, device=DEV)
    pkv.stream_read(buf, sums)
    torch.cuda.synchronize()
    got = int(sums.cpu().numpy().view(np.uint32).astype(np.uint64).sum()) % (1 << 32)
    expect = int(host.astype(np.uint64).sum()) % (1 << 32)
    assert got == expect
    if nbytes == 0:
        assert (sums.cpu() == 0).all()
