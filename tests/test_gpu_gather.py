"""abs_gather_tiles (the measurement probe that reads K/V-shaped tiles as the
decode does, with none of its arithmetic) through the C ABI: every listed
tile is read once, checked by the XOR of all its 32-bit words against numpy,
for several launch shapes, runs of more than 64 tiles per wavefront and
tile counts that do not divide evenly."""
import numpy as np
import pytest
import torch

from block_sparse_attention_abs_amd import abs as A

pytestmark = pytest.mark.gpu

TILE = 4096


def _xor_words(words):
    return int(np.bitwise_xor.reduce(words.ravel())) if words.size else 0


@pytest.mark.parametrize("n,workgroups,in_flight", [(1, 1, 1), (257, 1, 2), (257, 3, 4), (1000, 64, 8),
                                                    (4096, 256, 4), (5000, 1024, 8), (300, 1024, 2)])
def test_gather_reads_every_listed_tile_once(n, workgroups, in_flight):
    rng = np.random.default_rng(n * 7 + workgroups)
    pool_tiles = n + 37
    host = rng.integers(0, 2**32, size=(pool_tiles, TILE // 4), dtype=np.uint64).astype(np.uint32)
    pool = torch.from_numpy(host.view(np.int32)).cuda()
    pick = rng.permutation(pool_tiles)[:n]                       # scattered, each tile once
    addr = torch.from_numpy((pool.data_ptr() + pick.astype(np.uint64) * TILE).astype(np.uint64).view(np.int64)).cuda()
    out = torch.full((workgroups,), -1, dtype=torch.int32, device="cuda")
    print(f"[gpu gather] n={n} workgroups={workgroups} in_flight={in_flight}", flush=True)
    A.abs_gather_tiles(addr.data_ptr(), n, TILE, workgroups, in_flight, out.data_ptr(), A.current_stream())
    torch.cuda.synchronize()
    got = _xor_words(out.cpu().numpy().view(np.uint32))
    assert got == _xor_words(host[pick])


def test_gather_listed_twice_cancels():
    rng = np.random.default_rng(5)
    host = rng.integers(0, 2**32, size=(8, TILE // 4), dtype=np.uint64).astype(np.uint32)
    pool = torch.from_numpy(host.view(np.int32)).cuda()
    pick = np.array([0, 3, 3, 5, 7, 7, 7], dtype=np.uint64)     # 3 twice (cancels), 7 three times (stays)
    addr = torch.from_numpy((pool.data_ptr() + pick * TILE).astype(np.uint64).view(np.int64)).cuda()
    out = torch.zeros((2,), dtype=torch.int32, device="cuda")
    A.abs_gather_tiles(addr.data_ptr(), len(pick), TILE, 2, 2, out.data_ptr(), A.current_stream())
    torch.cuda.synchronize()
    got = _xor_words(out.cpu().numpy().view(np.uint32))
    assert got == _xor_words(host[[0, 5, 7]])


def test_gather_addresses_with_the_low_word_top_bit_set():
    """Tile addresses whose low 32 bits are at or above 2^31 (a pool of just
    over 2 GiB holds such addresses and others, whatever its base): the lane
    reads of the address halves must not sign-extend the low half.  Words are
    a counter hash, w[i] = i x 0x9E3779B1 mod 2^32, made on the device and
    recomputed on the host for the tiles read."""
    mul = 0x9E3779B1
    nwords = (1 << 31) // 4 + 2 * TILE // 4
    i = torch.arange(nwords, dtype=torch.int64, device="cuda")
    w = (i * mul) & 0xFFFFFFFF
    pool = torch.where(w >= (1 << 31), w - (1 << 32), w).to(torch.int32)
    del i, w
    base = pool.data_ptr()
    ntiles = nwords * 4 // TILE
    t = np.arange(ntiles, dtype=np.uint64)
    low = (np.uint64(base) + t * np.uint64(TILE)) & np.uint64(0xFFFFFFFF)
    hi_tiles = t[low >= np.uint64(1 << 31)]
    lo_tiles = t[low < np.uint64(1 << 31)]
    assert len(hi_tiles) and len(lo_tiles)
    pick = np.concatenate([hi_tiles[:: max(1, len(hi_tiles) // 20)][:20], lo_tiles[:: max(1, len(lo_tiles) // 20)][:20]])
    addr = torch.from_numpy((np.uint64(base) + pick * np.uint64(TILE)).view(np.int64)).cuda()
    out = torch.zeros((4,), dtype=torch.int32, device="cuda")
    print(f"[gpu gather] 2 GiB pool at {base:#x}: {len(pick)} tiles", flush=True)
    A.abs_gather_tiles(addr.data_ptr(), len(pick), TILE, 4, 2, out.data_ptr(), A.current_stream())
    torch.cuda.synchronize()
    idx = (pick[:, None] * np.uint64(TILE // 4) + np.arange(TILE // 4, dtype=np.uint64)[None, :])
    want = _xor_words(((idx * np.uint64(mul)) & np.uint64(0xFFFFFFFF)).astype(np.uint32))
    assert _xor_words(out.cpu().numpy().view(np.uint32)) == want
    del pool
    torch.cuda.empty_cache()
