"""Host model of the GEMM's work-item order (no GPU).

The persistent GEMM runs work items b, b + G, b + 2G, ... on workgroup b, and with
G = 256 workgroups the items that run together on one XCD are those with the same
item % 8 in one round of 256.  Each item is a (K split, output tile) pair with a K
rotation.  This model replays the two item orders of `tile_of` as the kernel source
writes them and checks, for the layer's weight-gradient plans and a few more:
- every (split, tile) pair is one item, exactly once;
- the rotation is within the split's slice count;
- in the blocked order, the 32 items of one XCD and round are one split of a 4 x 8
  group of tiles with one rotation (they walk K in lockstep and share 12 panels);
- in the row-tile walk with a row-tile count divisible by 8, an XCD's items also share
  their rotation;
- in the row-band order (one unsplit launch over 8 column tiles whose A operand exceeds
  128 MiB), each round is a band of 32 row tiles, each XCD's items are 4 x 8 tiles, and
  every tile keeps the walk's rotation.
The host sets the blocked order only when the whole grid, times the splits, fills
rounds of 256 items and the tile counts divide by 4 (rows) and 8 (columns); the
conditions are checked here as the host code states them.
"""
import pytest


def blocked_ok(tiles_m, tiles_n, splits):
    return tiles_m % 4 == 0 and tiles_n % 8 == 0 and (tiles_m * tiles_n * splits) % 256 == 0


def band_tile(tile, tiles_m):
    b, j = tile >> 8, tile & 255
    h = min(32, tiles_m - 32 * b)
    return 32 * b + j % h, j // h


def tile_of(item, tiles_m, tiles_n, splits, nk, blocked, banded=False, tile0=0, ntiles=None):
    spl = -(-nk // splits)
    if ntiles is None:
        ntiles = tiles_m * tiles_n
    if banded:
        split = item // ntiles
        tm, tn = band_tile(tile0 + item - split * ntiles, tiles_m)
        xk = tm & 7
    elif blocked:
        x = item & 7
        w = (item >> 3) & 31
        blk = ((item >> 8) << 3) | x
        bpm = tiles_m >> 2
        bps = bpm * (tiles_n >> 3)
        split = blk // bps
        bb = blk - split * bps
        tm = (bb % bpm) * 4 + (w & 3)
        tn = (bb // bpm) * 8 + (w >> 2)
        xk = x
    else:
        ntiles = tiles_m * tiles_n
        split = item // ntiles
        tile = item - split * ntiles
        tm, tn = tile % tiles_m, tile // tiles_m
        xk = tm & 7
    kb_begin = split * spl
    kb_end = min(nk, kb_begin + spl)
    rot = (xk * (kb_end - kb_begin)) // 8
    return split, tm, tn, rot, kb_end - kb_begin


# (tiles_m, tiles_n, splits, nk): the layer's weight gradients at 16384 tokens
# (qkv 4096 x 2048 split 2, o 2048 x 2048 split 4, down 2048 x 6144 in 192-column
# tiles) and other grids that qualify
PLANS = [(16, 8, 2, 128), (8, 8, 4, 128), (8, 32, 1, 128), (4, 64, 1, 16), (32, 8, 1, 8), (4, 8, 8, 64),
         (8, 16, 2, 40), (12, 16, 4, 17)]


@pytest.mark.parametrize("blocked", [True, False])
@pytest.mark.parametrize("tiles_m,tiles_n,splits,nk", PLANS)
def test_item_order_covers_every_pair_once(tiles_m, tiles_n, splits, nk, blocked):
    assert blocked_ok(tiles_m, tiles_n, splits)
    items = tiles_m * tiles_n * splits
    seen = set()
    for i in range(items):
        split, tm, tn, rot, n = tile_of(i, tiles_m, tiles_n, splits, nk, blocked)
        assert 0 <= split < splits and 0 <= tm < tiles_m and 0 <= tn < tiles_n
        assert 0 <= rot < max(n, 1)
        seen.add((split, tm, tn))
    assert len(seen) == items


@pytest.mark.parametrize("tiles_m,tiles_n,splits,nk", PLANS)
def test_blocked_order_groups_each_xcd(tiles_m, tiles_n, splits, nk):
    items = tiles_m * tiles_n * splits
    for r in range(items // 256):
        for x in range(8):
            group = [tile_of(256 * r + 8 * w + x, tiles_m, tiles_n, splits, nk, True) for w in range(32)]
            assert len({g[0] for g in group}) == 1, "one split per XCD and round"
            assert len({g[3] for g in group}) == 1, "one rotation per XCD and round"
            tms, tns = {g[1] for g in group}, {g[2] for g in group}
            assert len(tms) == 4 and len(tns) == 8, "a 4 x 8 group of tiles: 12 panels"
            assert max(tms) - min(tms) == 3 and max(tns) - min(tns) == 7


@pytest.mark.parametrize("tiles_m,tiles_n,splits,nk", [(64, 8, 1, 16), (16, 8, 2, 128), (8, 32, 1, 128)])
def test_row_tile_walk_shares_rotation_per_xcd(tiles_m, tiles_n, splits, nk):
    """The order the other launches keep: with tiles_m % 8 == 0 an XCD's items share tm % 8,
    hence the rotation (but, with few row tiles, not many panels)."""
    items = tiles_m * tiles_n * splits
    for r in range(-(-items // 256)):
        for x in range(8):
            group = [tile_of(i, tiles_m, tiles_n, splits, nk, False)
                     for i in range(256 * r + x, min(items, 256 * (r + 1)), 8)]
            for split in {g[0] for g in group}:
                assert len({g[3] for g in group if g[0] == split}) == 1


def test_blocked_order_needs_whole_rounds():
    """Grids that do not fill rounds of 256 items, or whose tile counts do not divide,
    keep the row-tile walk."""
    assert not blocked_ok(48, 8, 1)        # gate_up weight gradient: 384 tiles
    assert not blocked_ok(8, 6, 4)
    assert not blocked_ok(6, 8, 8)
    assert not blocked_ok(4, 8, 1)


@pytest.mark.parametrize("tiles_m,nk", [(64, 16), (64, 96), (32, 48), (96, 7), (48, 128), (16, 300), (45, 20)])
def test_banded_order(tiles_m, nk):
    """One unsplit launch over 8 column tiles and a multiple of 32 row tiles: bands of 32 row
    tiles x 8 column tiles, one per round.  Every tile once; each XCD and round holds 4 row
    tiles x 8 column tiles with one rotation (the row tile's, as in the walk); each row tile's
    items all run in one round."""
    items = tiles_m * 8
    seen, round_of_tm = set(), {}
    for i in range(items):
        split, tm, tn, rot, n = tile_of(i, tiles_m, 8, 1, nk, False, banded=True)
        assert split == 0 and 0 <= tm < tiles_m and 0 <= tn < 8
        assert rot == tile_of(tn * tiles_m + tm, tiles_m, 8, 1, nk, False)[3], "the walk's rotation"
        seen.add((tm, tn))
        assert round_of_tm.setdefault(tm, i // 256) == i // 256
    assert len(seen) == items
    for r in range(items // 256):
        if tiles_m - 32 * r < 32:
            break
        for x in range(8):
            group = [tile_of(256 * r + 8 * w + x, tiles_m, 8, 1, nk, False, banded=True) for w in range(32)]
            assert len({g[3] for g in group}) == 1
            assert len({g[1] for g in group}) == 4 and len({g[2] for g in group}) == 8


@pytest.mark.parametrize("tiles_m,whole,splits,nk", [(48, 256, 2, 128), (40, 256, 3, 64), (96, 512, 2, 40)])
def test_banded_whole_then_split(tiles_m, whole, splits, nk):
    """A plan that computes its first tiles whole and splits the rest: in the row-band
    numbering the two launches cover every tile once, the split launch's tiles are whole row
    tiles (every column tile of each), and all of a tile's splits cover its K range once."""
    tiles = tiles_m * 8
    cover = {}
    for i in range(whole):
        _, tm, tn, _, n = tile_of(i, tiles_m, 8, 1, nk, False, banded=True, tile0=0, ntiles=whole)
        cover.setdefault((tm, tn), []).append((0, n))
    split_rows = set()
    for i in range((tiles - whole) * splits):
        split, tm, tn, _, n = tile_of(i, tiles_m, 8, splits, nk, False, banded=True, tile0=whole,
                                      ntiles=tiles - whole)
        cover.setdefault((tm, tn), []).append((split, n))
        split_rows.add(tm)
    assert len(cover) == tiles
    for (tm, tn), parts in cover.items():
        assert sum(n for _, n in parts) == nk and len({s for s, _ in parts}) == len(parts)
    assert all(len(cover[(tm, tn)]) == splits for tm in split_rows for tn in range(8))
