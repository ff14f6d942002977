"""Second route to the oracle's tile classifier (O3, oracle_classify).

The GPU tile counters are compared bit-exactly with O3, so O3 itself is
pinned here by a classifier written a different way: no loop over pairs,
only the corners of each tile. Under the causal rule (web page "Sequence
parallelism -- splitting the token dimension across GPUs", section "Causal
attention gives us another optimization": a query sees the keys at or before
its own position) a tile of query positions [p0, p1] and key positions
[k0, k1] is
  * skipped   iff its first key lies after its last query   (k0 > p1),
  * full      iff its last key lies at or before its first query (k1 <= p0),
  * masked    otherwise,
and the allowed pairs of the tile are sum over p of clamp(p - k0 + 1, 0,
k1 - k0 + 1), a closed form per row. Bidirectional tiles are all full.
The cases put the diagonal anywhere inside a tile (random query offsets,
block starts and lengths that are not multiples of the tile sizes), and one
tile is counted by hand with exactly one masked pair.
"""
import numpy as np
import pytest

import oracle

TQ, TK = 32, 64   # the tile the kernels count


def _corner_classify(Tq, q_off, starts, lens, causal, tq=TQ, tk=TK):
    """Per block: class (0 full, 1 diag, 2 skip) and allowed pairs; tile counts
    [full, masked, skip] for one (batch, head)."""
    tiles = [0, 0, 0]
    cls, pairs = [], []
    for s, n in zip(starts, lens):
        bp = 0
        for i0 in range(0, Tq, tq):
            p0, p1 = q_off + i0, q_off + min(i0 + tq, Tq) - 1
            for j0 in range(0, n, tk):
                k0, k1 = s + j0, s + min(j0 + tk, n) - 1
                if not causal or k1 <= p0:
                    tiles[0] += 1
                    bp += (p1 - p0 + 1) * (k1 - k0 + 1)
                elif k0 > p1:
                    tiles[2] += 1
                else:
                    tiles[1] += 1
                    bp += sum(min(max(p - k0 + 1, 0), k1 - k0 + 1) for p in range(p0, p1 + 1))
        total = Tq * n
        cls.append(2 if bp == 0 else (0 if bp == total else 1))
        pairs.append(bp)
    return np.array(cls, np.int8), np.array(pairs, np.int64), np.array(tiles, np.int64)


def test_one_masked_pair_by_hand():
    """32 queries at positions 100..131 against one 64-key block at 38..101:
    only query 100 misses a key (101), so the single tile is masked with
    32*64 - 1 = 2047 allowed pairs, and the block is DIAG."""
    cls, pairs, tiles = oracle.classify(32, 100, [38], [64], causal=True, tile_q=TQ, tile_k=TK)
    assert list(cls) == [1] and list(pairs) == [2047] and list(tiles) == [0, 1, 0]
    # one key earlier, every pair is allowed: FULL
    cls, pairs, tiles = oracle.classify(32, 100, [37], [64], causal=True, tile_q=TQ, tile_k=TK)
    assert list(cls) == [0] and list(pairs) == [2048] and list(tiles) == [1, 0, 0]
    # the mirror case: query 131 alone sees key 131 = the block's first key
    cls, pairs, tiles = oracle.classify(32, 100, [131], [64], causal=True, tile_q=TQ, tile_k=TK)
    assert list(cls) == [1] and list(pairs) == [1] and list(tiles) == [0, 1, 0]
    cls, _, tiles = oracle.classify(32, 100, [132], [64], causal=True, tile_q=TQ, tile_k=TK)
    assert list(cls) == [2] and list(tiles) == [0, 0, 1]


def _case(rng):
    Tq = int(rng.integers(1, 300))
    q_off = int(rng.integers(0, 600))
    nb = int(rng.integers(1, 6))
    starts = [int(x) for x in rng.integers(0, 900, nb)]
    lens = [int(x) for x in rng.integers(0, 260, nb)]
    return Tq, q_off, starts, lens


@pytest.mark.parametrize("seed", range(24))
def test_oracle_tiles_match_corner_rule(seed):
    rng = np.random.default_rng(9000 + seed)
    Tq, q_off, starts, lens = _case(rng)
    for causal in (True, False):
        want = _corner_classify(Tq, q_off, starts, lens, causal)
        got = oracle.classify(Tq, q_off, starts, lens, causal=causal, tile_q=TQ, tile_k=TK)
        for g, w_, name in zip(got, want, ("class", "pairs", "tiles")):
            np.testing.assert_array_equal(g, w_, err_msg=f"{name}: Tq={Tq} q_off={q_off} "
                                          f"starts={starts} lens={lens} causal={causal}")


def test_oracle_tiles_scale_with_batch_and_heads():
    rng = np.random.default_rng(9100)
    Tq, q_off, starts, lens = _case(rng)
    _, _, one = oracle.classify(Tq, q_off, starts, lens, causal=True, tile_q=TQ, tile_k=TK)
    _, _, many = oracle.classify(Tq, q_off, starts, lens, causal=True, B=3, Hq=5,
                                 tile_q=TQ, tile_k=TK)
    np.testing.assert_array_equal(many, 15 * one)


def test_some_cases_cut_tiles_off_the_grid():
    """The seeded cases do exercise diagonals that cross a tile's interior
    with a single masked pair or a single allowed pair somewhere."""
    seen_masked = seen_one_masked = seen_one_allowed = 0
    for seed in range(24):
        rng = np.random.default_rng(9000 + seed)
        Tq, q_off, starts, lens = _case(rng)
        for s, n in zip(starts, lens):
            for i0 in range(0, Tq, TQ):
                p0, p1 = q_off + i0, q_off + min(i0 + TQ, Tq) - 1
                for j0 in range(0, n, TK):
                    k0, k1 = s + j0, s + min(j0 + TK, n) - 1
                    allowed = sum(min(max(p - k0 + 1, 0), k1 - k0 + 1)
                                  for p in range(p0, p1 + 1))
                    tot = (p1 - p0 + 1) * (k1 - k0 + 1)
                    seen_masked += 0 < allowed < tot
                    seen_one_masked += allowed == tot - 1 and tot > 1
                    seen_one_allowed += allowed == 1 and tot > 1
    assert seen_masked >= 50 and seen_one_masked > 0 and seen_one_allowed > 0
