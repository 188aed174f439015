"""The HBM read probe (include/spin_probe.h): every wave's checksum equals
the XOR of the bytes it is documented to read, so the probe reads exactly
the listed pages with the score kernel's lane layout."""
import numpy as np
import pytest
import torch

from tests.gpu_util import DEV, banner

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_ids", [1, 63, 5000])
def test_read_probe_checksums(n_ids):
    banner(f"read probe n_ids={n_ids}")
    from sparse_attention_indexer_spin_amd import api, _lib
    rng = np.random.default_rng(n_ids)
    n_pages = 300
    pages = rng.integers(0, 256, (n_pages, 8192), dtype=np.uint8)
    ids = rng.integers(-3, n_pages + 3, n_ids).astype(np.int32)     # out-of-range ids read page 0
    sink = torch.zeros(_lib.SPIN_READ_PROBE_SINK_WORDS, dtype=torch.int32, device=DEV)
    api.spin_read_pages(torch.from_numpy(pages).to(DEV), torch.from_numpy(ids).to(DEV), sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32).reshape(_lib.SPIN_READ_PROBE_WAVES, 64)
    words = pages.view(np.uint32).reshape(n_pages, 8, 16, 4, 4)   # [page][KB][16-B chunk][4 words]
    lane = np.arange(64)
    chunk = (lane & 7) * 8 + ((lane >> 3) & 1) * 4 + (lane >> 4)  # 16-B chunk index within a KB
    per_page = np.bitwise_xor.reduce(words.reshape(n_pages, 8, 64, 4)[:, :, chunk, :],
                                     axis=(1, 3))                # [page][lane]
    W = _lib.SPIN_READ_PROBE_WAVES
    want = np.zeros((W, 64), dtype=np.uint32)
    for w in range(W):
        lo, hi = w * n_ids // W, (w + 1) * n_ids // W
        for i in ids[lo:hi]:
            want[w] ^= per_page[i if 0 <= i < n_pages else 0]
    assert np.array_equal(got, want)
