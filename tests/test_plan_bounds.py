"""Host-side checks of the balanced split's arithmetic (no GPU).

The plan kernel lays every entry's tiles on a cost axis (an entry first takes
kEntryCost units, then kTileCost per tile), cuts it into R runs (R = W
workgroups, or fewer so that a run holds at least kMinRunTiles tiles) and
gives run r the tiles that start in [C r / R, C (r + 1) / R).  Each workgroup
has room for balanced_capacity records, and the workspace holds W of those
regions for any W up to the bound.  This re-derives the split from that
definition for many tables and checks that no run exceeds the capacity, that
the runs cover every tile once, that workgroups map one-to-one onto runs, and
that the workspace bound holds.  The constants are read from the header the
kernels are built with."""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = open(os.path.join(ROOT, "paged_kv_decode_pkv_amd", "csrc", "pkv_launch.h")).read()


def const(name):
    return int(re.search(rf"constexpr int {name} = (\d+);", HDR).group(1))


TILE, ENTRY, MINRUN = const("kTileCost"), const("kEntryCost"), const("kMinRunTiles")
MAX_CUS, MAX_WAVES_CU = const("kMaxComputeUnits"), const("kMaxWavesPerCU")


def capacity(max_tiles, batch, blocks):
    full = -(-max_tiles // blocks) + (ENTRY * batch + TILE * blocks - 1) // (TILE * blocks) + 2
    return max(full, 2 * MINRUN + 2)


def block_region_bound(max_tiles, batch, wb):
    full = max_tiles + (ENTRY * batch + TILE - 1) // TILE + 5 * wb
    return max(full, wb * (3 + 2 * MINRUN))


def run_of_block(w, W, R):
    if W % 8:
        return w if w < R else R
    x, i = w % 8, w // 8
    r0, r1 = R * x // 8, R * (x + 1) // 8
    return r0 + i if r0 + i < r1 else R


def split(tiles, W):
    """Run of every tile, from the cost-axis definition."""
    tiles = np.asarray(tiles, dtype=np.int64)
    T, Z = int(tiles.sum()), int((tiles > 0).sum())
    C = TILE * T + ENTRY * Z
    R = max(1, min(W, C // (TILE * MINRUN)))
    start = np.concatenate([[0], np.cumsum(tiles)])
    nz = np.concatenate([[0], np.cumsum(tiles > 0)])
    pos = []
    for b, n in enumerate(tiles):
        base = TILE * start[b] + ENTRY * nz[b] + ENTRY
        pos.extend(base + TILE * np.arange(n))
    pos = np.asarray(pos, dtype=np.int64)
    runs = ((pos + 1) * R - 1) // C   # the largest r with C r / R <= p
    # the same from the run boundaries
    lo = (C * runs) // R
    hi = (C * (runs + 1)) // R
    assert np.all((lo <= pos) & (pos < hi))
    return runs, R


CASES = [
    ("one tile", [1], 256),
    ("single entry", [33], 256),
    ("tiny batch", [40, 37], 256),
    ("batch 8", [33, 12, 60, 2, 64, 17, 40, 0], 256),
    ("uneven W", [500, 3, 1, 77], 250),
    ("many short", [1] * 4096, 256),
    ("many short, small W", [1] * 4096, 8),
]


@pytest.mark.parametrize("name,tiles,W", CASES, ids=[c[0] for c in CASES])
def test_split_fits_capacity(name, tiles, W):
    runs, R = split(tiles, W)
    counts = np.bincount(runs, minlength=R)
    max_tiles = len(tiles) * max(max(tiles), 1)
    assert counts.max(initial=0) <= capacity(max_tiles, len(tiles), W)
    assert counts.sum() == sum(tiles)


def test_split_random_tables():
    rng = np.random.default_rng(7)
    for _ in range(300):
        batch = int(rng.integers(1, 300))
        maxp = int(rng.integers(1, 300))
        tiles = rng.integers(0, 2 * maxp + 1, size=batch)
        W = int(rng.choice([8, 64, 250, 256, 512, 1024]))
        runs, R = split(tiles, W)
        counts = np.bincount(runs, minlength=R)
        assert counts.max(initial=0) <= capacity(batch * 2 * maxp, batch, W)
        assert R <= W


@pytest.mark.parametrize("W", [1, 7, 8, 250, 256, 1024])
def test_blocks_map_one_to_one_onto_runs(W):
    for R in sorted(r for r in {1, 2, 5, 8, 9, W // 3 or 1, W - 1 or 1, W} if r <= W):
        got = [run_of_block(w, W, R) for w in range(W)]
        taken = [r for r in got if r < R]
        assert sorted(taken) == list(range(R))
        if W % 8 == 0 and R >= 8:
            # every XCD (ids congruent mod 8) holds a share of the runs
            assert all(any(got[w] < R for w in range(x, W, 8)) for x in range(8))


@pytest.mark.parametrize("waves", [1, 2, 4, 8])
def test_workspace_holds_every_block_region(waves):
    wb = (MAX_CUS * MAX_WAVES_CU + waves - 1) // waves
    for batch, max_tiles in [(1, 2), (64, 64 * 512), (4096, 4096 * 2), (4096, 4096 * 4096)]:
        bound = block_region_bound(max_tiles, batch, wb)
        for W in {1, 8, 100, wb // 2, wb - 1, wb}:
            assert W * (1 + capacity(max_tiles, batch, W)) <= bound


# ------------------------------------------------------------- fixed runs
RANKED = const("kRankedBatch")


def fixed_deal(tiles, ct, W):
    """Workgroup of every (entry, chunk), from the fixed-mode definition: the
    full chunks in entry order, then the shorter last chunks largest first
    (ties, and all of them above the ranked batch size, in entry order),
    dealt in snake order over W workgroups."""
    tiles = [int(t) for t in tiles]
    full = [(b, c, ct) for b, t in enumerate(tiles) for c in range(t // ct)]
    part = [(b, t // ct, t % ct) for b, t in enumerate(tiles) if t % ct]
    if len(tiles) <= RANKED:
        part.sort(key=lambda x: (-x[2], x[0]))
    order = full + part
    deal = {}
    for r, (b, c, n) in enumerate(order):
        k, i = divmod(r, W)
        deal[(b, c)] = (i if k % 2 == 0 else W - 1 - i, n)
    return deal


def fixed_capacity(chunks, ct, entry_tiles, W):
    return -(-chunks // W) * max(1, min(ct, entry_tiles))


@pytest.mark.parametrize("ct", [1, 2, 8, 32, 128])
def test_fixed_deal_covers_every_chunk_once_within_capacity(ct):
    rng = np.random.default_rng(11 + ct)
    for _ in range(60):
        batch = int(rng.integers(1, 300))
        maxt = int(rng.integers(1, 40 * ct + 1 if ct < 8 else 600))
        tiles = rng.integers(0, maxt + 1, size=batch)
        W = int(rng.choice([1, 8, 250, 256, 512]))
        deal = fixed_deal(tiles, ct, W)
        # each entry's chunks are exactly those of its own length: the split
        # does not depend on the rest of the batch
        for b, t in enumerate(tiles):
            assert sorted(c for (bb, c) in deal if bb == b) == list(range(-(-int(t) // ct)))
        load = np.zeros(W, np.int64)
        for (b, c), (w, n) in deal.items():
            assert 0 <= w < W and 0 < n <= ct
            load[w] += n
        assert load.sum() == tiles.sum()
        max_chunks = max(1, -(-maxt // ct))
        assert load.max() <= fixed_capacity(batch * max_chunks, ct, maxt, W)


def test_fixed_deal_balances_the_qwen3_4b_like_step():
    """16-page runs of the Qwen3-4B-like batch (lengths log-uniform in
    [64, 4096], 8-token tiles) over 256 workgroups: the busiest workgroup
    holds at most one run more than the mean share."""
    import workloads
    spec = workloads.CONFIGS[3]
    table = workloads.make_table(spec)
    tiles = -(-np.asarray(table.lengths) // 8)
    ct, W = 32, 256
    deal = fixed_deal(tiles, ct, W)
    load = np.zeros(W, np.int64)
    for (w, n) in deal.values():
        load[w] += n
    assert load.max() <= tiles.sum() / W + ct


@pytest.mark.parametrize("waves", [1, 8])
def test_workspace_holds_every_fixed_block_region(waves):
    wb = (MAX_CUS * MAX_WAVES_CU + waves - 1) // waves
    for batch, entry_tiles, ct in [(1, 2, 2), (64, 438, 32), (8, 4096, 2), (4200, 48, 32),
                                   (256, 64, 131072)]:
        chunks = batch * -(-entry_tiles // ct)
        c = min(ct, entry_tiles)
        bound = wb * (1 + c) + chunks * c
        for W in {1, 8, 100, wb // 2, wb}:
            assert W * (1 + fixed_capacity(chunks, ct, entry_tiles, W)) <= bound
