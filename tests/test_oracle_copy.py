"""Pins for the oracle's collective-shaped copies and checkers: per-byte loops, the block
transpose's involution and fixed diagonal, and planted mistakes the checkers must flag."""
import numpy as np
import pytest

from concurrent_gemm_dma_amd import workloads as wl


def _bytewise_gather(shards):
    out = []
    for s in shards:
        for b in s.tobytes():
            out.append(b)
    return np.array(out, dtype=np.uint8)


def _bytewise_a2a(src, grid, bb):
    dst = np.zeros_like(src)
    for i in range(grid):
        for j in range(grid):
            for b in range(bb):
                dst[(j * grid + i) * bb + b] = src[(i * grid + j) * bb + b]
    return dst


@pytest.mark.parametrize("n,sb", [(8, 37), (1, 5), (3, 16), (8, 1)])
def test_gather_bytewise(orc, n, sb):
    shards = [wl.gen_bytes(sb, 50 + i) for i in range(n)]
    np.testing.assert_array_equal(orc.gather(shards), _bytewise_gather(shards))


def test_gather_empty(orc):
    assert orc.gather([]).size == 0
    assert orc.gather([np.empty(0, np.uint8)] * 3).size == 0


@pytest.mark.parametrize("grid,bb", [(3, 5), (8, 4), (1, 9), (2, 1)])
def test_a2a_bytewise(orc, grid, bb):
    src = wl.gen_bytes(grid * grid * bb, 60 + grid)
    np.testing.assert_array_equal(orc.all2all_block(src, grid, bb), _bytewise_a2a(src, grid, bb))


def test_a2a_involution_and_diagonal(orc):
    grid, bb = 8, 64
    src = wl.gen_bytes(grid * grid * bb, 70)
    dst = orc.all2all_block(src, grid, bb)
    np.testing.assert_array_equal(orc.all2all_block(dst, grid, bb), src)
    for i in range(grid):
        off = (i * grid + i) * bb
        np.testing.assert_array_equal(dst[off:off + bb], src[off:off + bb])
    assert not np.array_equal(dst, src)


def test_first_diff_locates_planted_byte(orc):
    a = wl.gen_bytes(4096, 80)
    assert orc.first_diff(a, a.copy()) == -1
    for off in (0, 1, 17, 4095):
        b = a.copy()
        b[off] ^= 0x01
        assert orc.first_diff(a, b) == off


def test_checker_flags_dropped_swapped_stale(orc):
    shards = [wl.gen_bytes(256, 90 + i) for i in range(8)]
    good = orc.gather(shards)
    dropped = good.copy()
    dropped[3 * 256:4 * 256] = 0xA5          # shard 3 never arrived: poison remains
    assert orc.first_diff(good, dropped) == 3 * 256 + int(
        np.flatnonzero(good[3 * 256:4 * 256] != 0xA5)[0])
    swapped = orc.gather([shards[1], shards[0]] + shards[2:])
    assert orc.first_diff(good, swapped) != -1
    stale = np.full_like(good, 0x5A)
    assert orc.first_diff(good, stale) != -1


def test_gemm_compare_flags(orc):
    rng = np.random.Generator(np.random.PCG64(11))
    ref = wl.gen_bf16((1000,), ("normal", 0.0, 1.0), 12)
    rep = orc.gemm_compare(ref, ref.copy())
    assert rep["n_violations"] == 0 and rep["n_diff"] == 0 and rep["frob_rel"] == 0.0
    # one large error: elementwise violation
    bad = ref.copy()
    bad[123] ^= 0x4000
    rep = orc.gemm_compare(ref, bad)
    assert rep["n_violations"] >= 1 and rep["first_violation"] == 123
    # NaN output counts as a violation and as non-finite
    bad = ref.copy()
    bad[5] = 0x7FC0
    rep = orc.gemm_compare(ref, bad)
    assert rep["n_violations"] >= 1 and rep["n_nonfinite"] == 1
    # many 1-ulp changes pass elementwise but trip nothing else unless too many
    one_ulp = (ref.astype(np.int32) + rng.integers(0, 2, size=ref.size)).astype(np.uint16)
    rep = orc.gemm_compare(ref, one_ulp)
    assert rep["n_violations"] == 0
    assert rep["frob_rel"] > 1e-3  # ~half the elements off by one ulp is too much in aggregate


def test_tagged_pattern_and_attribution(orc):
    """The diagnostic gather pattern: every 8-byte word names its shard and the place it belongs,
    so a misplaced, swapped or missing word is attributed. The checker is pinned on planted
    mistakes in the oracle's own gather."""
    n, sb = 8, 4096
    shards = wl.gen_tagged_shards(n, sb)
    good = orc.gather(shards)
    assert orc.explain_tagged_gather(good, n, sb) == []
    # word 5 of shard 2 as a plain number: shard 2 in the top byte, destination 2*4096 + 40
    assert int(shards[2][40:48].view("<u8")[0]) == (2 << 56) | (2 * sb + 40)

    swapped = good.copy()
    a, b = 2 * sb + 64, 5 * sb + 8                      # two words exchanged across shards
    swapped[a:a + 8], swapped[b:b + 8] = good[b:b + 8].copy(), good[a:a + 8].copy()
    assert orc.explain_tagged_gather(swapped, n, sb) == [(a, 5, b), (b, 2, a)]

    dropped = good.copy()
    dropped[3 * sb + 16:3 * sb + 24] = 0xA5             # never written: poison remains
    assert orc.explain_tagged_gather(dropped, n, sb) == [(3 * sb + 16, -1, -1)]

    shifted = good.copy()
    shifted[4 * sb:5 * sb] = good[3 * sb:4 * sb]        # shard 3 landed in shard 4's slot
    rep = orc.explain_tagged_gather(shifted, n, sb, limit=4)
    assert rep == [(4 * sb + 8 * w, 3, 3 * sb + 8 * w) for w in range(4)]

    torn = good.copy()
    torn[6 * sb + 3] ^= 0x10                            # one byte flipped inside a word
    assert orc.explain_tagged_gather(torn, n, sb) == [(6 * sb, -1, -1)]  # no valid tag left
    with pytest.raises(ValueError):
        orc.explain_tagged_gather(good[:-8], n, sb)
    with pytest.raises(ValueError):
        wl.gen_tagged_shards(2, 12)
