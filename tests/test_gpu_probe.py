"""The read-bandwidth probe (pa_read_probe) reads exactly the tiles it is
given: the XOR of its per-worker checksums equals the XOR, computed on the
host, of every 32-bit word of every listed tile."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def expected_xor(words: np.ndarray, tile_bytes: int, ids) -> int:
    tiles = words.reshape(-1, tile_bytes // 4)
    per_tile = np.bitwise_xor.reduce(tiles, axis=1)
    return int(np.bitwise_xor.reduce(per_tile[ids])) if len(ids) else 0


@pytest.mark.parametrize("tile_bytes", [4096, 8192])
@pytest.mark.parametrize("nontemporal", [False, True])
@pytest.mark.parametrize("workers", [1, 7, 64, 0])
def test_probe_reads_every_listed_tile_once(tile_bytes, nontemporal, workers):
    import paged_kv_cache_310_amd as pa
    rng = np.random.default_rng(3120 + tile_bytes + workers)
    nbytes = 6 << 20
    words = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint32)
    base = torch.from_numpy(words.view(np.int32)).cuda()
    ntiles = nbytes // tile_bytes
    cases = {
        "permutation": rng.permutation(ntiles),
        "with repeats": rng.integers(0, ntiles, ntiles // 3 + 5),
        "ragged prefix": rng.permutation(ntiles)[:ntiles // 2 + 3],
        "one tile": np.array([ntiles - 1]),
    }
    for name, ids in cases.items():
        print(f"probe tile {tile_bytes} nt {nontemporal} workers {workers} case {name}", flush=True)
        t_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
        cs = pa.pa_read_probe(base, t_ids, tile_bytes, nontemporal, num_workers=workers)
        got = int(np.bitwise_xor.reduce(cs.cpu().numpy().view(np.uint32)))
        assert got == expected_xor(words, tile_bytes, ids), name
    # address order: every whole tile, then a prefix of them
    for n in (ntiles, ntiles // 3 + 1):
        cs = pa.pa_read_probe(base, None, tile_bytes, nontemporal, num_tiles=n, num_workers=workers)
        got = int(np.bitwise_xor.reduce(cs.cpu().numpy().view(np.uint32)))
        assert got == expected_xor(words, tile_bytes, np.arange(n))
