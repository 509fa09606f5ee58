"""Host-side plan construction (onebit_plan_host_tables; no device involved).

Checks the tile table against a direct numpy model: 2048-element tiles cut from
each chunk's start (one empty tile for an empty chunk), packed-word offsets, the
merged masked intervals (maximal runs of masked elements) and each tile's mask
classification (none / all / the intervals that touch it).
"""
import numpy as np
import pytest

from error_compensated_bit_amd import onebit as ob
from error_compensated_bit_amd import workloads as W

TILE = 2048


def model_tiles(chunk_off):
    rows = []
    word = 0
    for j in range(chunk_off.size - 1):
        o, ln = int(chunk_off[j]), int(chunk_off[j + 1] - chunk_off[j])
        nt = max(1, -(-ln // TILE))
        for k in range(nt):
            rows.append((o + k * TILE, word + k * (TILE // 32), max(0, min(TILE, ln - k * TILE)), j))
        word += -(-ln // 32)
    return np.array(rows, dtype=np.int64).reshape(-1, 4), word


def masked_elements(n, tensor_off, keep):
    mk = np.zeros(n, bool)
    for t in range(keep.size):
        if not keep[t]:
            mk[tensor_off[t]:tensor_off[t + 1]] = True
    return mk


def runs(mk):
    d = np.diff(np.concatenate([[0], mk.astype(np.int8), [0]]))
    return np.stack([np.nonzero(d == 1)[0], np.nonzero(d == -1)[0]], axis=1)


def check(chunk_off, tensor_off=None, keep=None, sample=None):
    tiles, words, iv = ob.onebit_plan_host_tables(chunk_off, tensor_off, keep)
    ref, ref_words = model_tiles(np.asarray(chunk_off))
    np.testing.assert_array_equal(tiles[:, :4], ref)
    assert words == ref_words
    n = int(chunk_off[-1])
    if tensor_off is None:
        assert iv.shape[0] == 0 and np.all(tiles[:, 4:] == 0)
        return tiles
    mk = masked_elements(n, tensor_off, keep)
    np.testing.assert_array_equal(iv, runs(mk).reshape(-1, 2))
    rows = tiles
    if sample is not None and tiles.shape[0] > sample:
        touched = np.nonzero(tiles[:, 5] != tiles[:, 4])[0]
        pick = np.random.default_rng(0).choice(tiles.shape[0], sample, replace=False)
        rows = tiles[np.union1d(touched, pick)]
    for start, _, ln, _, lo, hi in rows:
        seg = mk[start:start + ln]
        if ln == 0:
            assert lo == 0 and hi == 0
        elif lo == -1:
            assert seg.all()
        else:
            cover = np.zeros(ln, bool)
            for a, b in iv[lo:hi]:
                assert a < start + ln and b > start, "interval listed for a tile it does not touch"
                cover[max(a, start) - start:min(b, start + ln) - start] = True
            np.testing.assert_array_equal(cover, seg)
            assert not (seg.all() and hi - lo == 1), "a fully covered tile must be flagged"
    return tiles


def test_bert_tables():
    for wl in (W.bert_small(), W.bert_like()):
        tiles = check(wl.chunk_off, wl.tensor_off, wl.tensor_keep, sample=3000)
        assert tiles.shape[0] == sum(max(1, -(-int(x) // TILE)) for x in np.diff(wl.chunk_off))


def test_fixed_chunks_and_ragged_tail():
    check(W.fixed_chunks(1_557_611_200 // 1000, 1 << 20))
    check(W.fixed_chunks(10_000, 4096))


@pytest.mark.parametrize("seed", range(12))
def test_random_tables(seed):
    rng = np.random.default_rng(seed)
    n_t = int(rng.integers(1, 40))
    sizes = rng.integers(0, 9000, n_t)
    sizes[rng.random(n_t) < 0.15] = 0                 # empty tensors
    t_off = W.offsets_from_sizes(sizes)
    n = int(t_off[-1])
    cuts = np.sort(rng.integers(0, n + 1, int(rng.integers(0, 12))))
    c_off = np.unique(np.concatenate([[0], cuts, [n]])).astype(np.int64)
    if rng.random() < 0.3:                             # an empty chunk
        c_off = np.sort(np.concatenate([c_off, [c_off[len(c_off) // 2]]]))
    keep = (rng.random(n_t) < 0.6).astype(np.uint8)
    check(c_off, t_off, keep)
    check(c_off)


def test_validation():
    for bad in ([1, 4], [0, 5, 2]):
        with pytest.raises(ob.OnebitError) as ei:
            ob.onebit_plan_host_tables(np.array(bad))
        assert ei.value.status == ob.ONEBIT_ERR_INVALID
    with pytest.raises(ob.OnebitError):
        ob.onebit_plan_host_tables(np.array([0, 10]), np.array([0, 9]), np.array([1], np.uint8))
    tiles, words, iv = ob.onebit_plan_host_tables(np.array([0]))
    assert tiles.shape == (0, 6) and words == 0
